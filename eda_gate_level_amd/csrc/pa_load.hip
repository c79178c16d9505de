// pa_load.hip -- load-time kernels: design tables and the event layout.
//
// The design load derives per-gate constants once: the segment and fraction
// of the gate's output load on its cell's cap axis (the load side of the
// bilinear NLDM lookup of "GPU-Accelerated Gate-Level Time-Based Power
// Analysis via Event-Density-Aware Partitioning and Kernel Fusion",
// Sec. 2.4.1) and the switching energy 0.5 c Vdd^2 of its output (Eq. 1).
//
// The event load validates the per-pin streams (sorted, alternating values,
// inside the window, positive slews) and lays them out: a radix sort puts
// the events in (time chunk, gate, pin kind, clock cycle, time, pin) order,
// the kind telling the gate's input pins from its output pin, and every
// gate's part of a chunk is cut into windows whose length follows the gate's
// event density (the paper's event-density-aware per-gate cycle
// partitioning), the input and the output events of a gate in windows of
// their own.  The first event of an input window carries the gate's input
// state at the window start, found from per-pin event-count parities (the
// state reconstruction at a window start of Sec. 2.4.2); output events need
// no state.  Windows start on cycle boundaries, so the per-pin glitch
// counter never crosses one.
#include <hip/hip_runtime.h>

#include <cstring>
#include <utility>

#include <rocprim/device/device_radix_sort.hpp>
#include <rocprim/device/device_scan.hpp>

#include "pa_common.h"
#include "pa_load.h"

namespace pa {
namespace {

constexpr int kLT = 256;
// per-gate rows from the walk kernel's window sums: kRowLanes lanes add a
// gate's windows, or, for a gate of more than kRowSmall windows, its pieces
// of kRowPiece windows, each summed by a block first
constexpr uint32_t kRowLanes = 2, kRowSmall = 64, kRowPiece = 1024;

inline int grid_for(int64_t n) {
  int64_t g = (n + kLT - 1) / kLT;
  if (g < 1) g = 1;
  if (g > 65535 * 16) g = 65535 * 16;
  return (int)g;
}

// ------------------------------------------------------------------ design

// per internal gate g (caller gate perm[g])
__global__ void k_gate_tables(int64_t G, const int32_t *perm, const int32_t *gate_cell, const double *gate_cap,
                              int32_t n_cells, const int32_t *cell_k, const double *cap_axis, int32_t n_cap, double vdd,
                              uint32_t *gate_info, uint4 *gate_rec, int32_t *gate_k, uint32_t *err) {
  for (int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; g < G; g += (int64_t)gridDim.x * blockDim.x) {
    const int32_t cell = gate_cell[perm[g]];
    const double cap = gate_cap[perm[g]];
    if (cell < 0 || cell >= n_cells) {
      atomicOr(err, ERR_CELL_ID);
      gate_k[g] = 0;
      continue;
    }
    if (!isfinite(cap)) atomicOr(err, ERR_CAP);
    const double *ca = cap_axis + (size_t)cell * n_cap;
    int seg = 0;
    for (int j = 1; j < n_cap - 1; ++j) seg += (cap >= ca[j]) ? 1 : 0;
    gate_info[g] = (uint32_t)cell | ((uint32_t)seg << 24);
    const uint64_t cb = (uint64_t)__double_as_longlong(cap);
    gate_rec[g] = make_uint4((uint32_t)cb, (uint32_t)(cb >> 32), gate_info[g], 0u);
    gate_k[g] = cell_k[cell];
  }
}

// pin -> (internal gate, local index) from the gates' first pins
__global__ void k_pin_owner(int64_t G, const int64_t *pin_base, const int32_t *gate_k, int32_t *pin_gate,
                            uint8_t *pin_local) {
  for (int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; g < G; g += (int64_t)gridDim.x * blockDim.x) {
    const int64_t p0 = pin_base[g], p1 = p0 + gate_k[g] + 1;
    for (int64_t p = p0; p < p1; ++p) {
      pin_gate[p] = (int32_t)g;
      pin_local[p] = (uint8_t)(p - p0);
    }
  }
}

// ------------------------------------------------------------------ events

__global__ void k_pin_check(int64_t P, int64_t E, const int64_t *pin_ptr, const uint8_t *pin_init, uint32_t *err) {
  if (blockIdx.x == 0 && threadIdx.x == 0 && (pin_ptr[0] != 0 || pin_ptr[P] != E)) atomicOr(err, ERR_ENDS);
  for (int64_t p = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; p < P; p += (int64_t)gridDim.x * blockDim.x) {
    if (pin_ptr[p + 1] < pin_ptr[p]) atomicOr(err, ERR_PIN_PTR);
    if (pin_init[p] > 1) atomicOr(err, ERR_INIT);
  }
}

// Owning pin of every event, the last p with pin_ptr[p] <= e: every pin with
// events writes its index at its first event (those positions are distinct),
// the rest of the array holding 0, and a running maximum over the events
// spreads each index over its pin's range.  This runs before the pin checks
// are read back, so a position outside [0, E) is skipped (the load then
// fails on those checks).
__global__ void k_pin_starts(int64_t P, int64_t E, const int64_t *pin_ptr, uint32_t *mark) {
  for (int64_t p = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; p < P; p += (int64_t)gridDim.x * blockDim.x) {
    const int64_t a = pin_ptr[p];
    if (a < pin_ptr[p + 1] && a >= 0 && a < E) mark[a] = (uint32_t)p;
  }
}

// validation of every event against its pin
__global__ void k_event_check(int64_t E, const int64_t *pin_ptr, const uint8_t *pin_init, const int64_t *evt_t,
                              const uint8_t *evt_val, const float *evt_slew, int64_t t_max, const uint32_t *ev_pin,
                              uint32_t *err) {
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < E; e += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t lo = ev_pin[e];
    const int64_t idx = e - pin_ptr[lo];
    const int64_t t = evt_t[e];
    uint32_t bad = 0;
    if (t < 0 || t >= t_max) bad |= ERR_TIME_RANGE;
    if (idx > 0 && e > 0 && !(t > evt_t[e - 1])) bad |= ERR_TIME_ORDER;
    const uint8_t init = pin_init[lo] & 1u;
    if (evt_val[e] != (uint8_t)(init ^ ((idx + 1) & 1))) bad |= ERR_VALUE;
    const float s = evt_slew[e];
    if (!(s > 0.0f) || !isfinite(s)) bad |= ERR_SLEW;
    if (bad) atomicOr(err, bad);
  }
}

// Window level of every gate: a gate of density rho = N_evt / N_cyc gets
// windows of Cc / 2^s cycles, the smallest s with rho * Cc / 2^s <= target
// (the paper sizes its per-gate windows to a target event count per thread;
// here the chunk is the upper bound on a window, which plays the part of its
// parallelism floor).
__global__ void k_gate_levels(int64_t G, const int64_t *pin_base, const int32_t *gate_k, const int64_t *pin_ptr,
                              int64_t C, int32_t Cc, int32_t lc, double target, int32_t fixed_level,
                              uint8_t *level) {
  for (int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; g < G; g += (int64_t)gridDim.x * blockDim.x) {
    if (fixed_level >= 0) {  // the same window length for every gate
      level[g] = (uint8_t)fixed_level;
      continue;
    }
    const double n_evt = (double)(pin_ptr[pin_base[g] + gate_k[g] + 1] - pin_ptr[pin_base[g]]);
    const double rho = n_evt / (double)C;
    int sl = 0;
    while (sl < lc && rho * (double)(Cc >> sl) > target) ++sl;
    level[g] = (uint8_t)sl;
  }
}

// Fields of an event in the layout order.
struct EvPos {
  uint64_t q;     // chunk
  uint32_t g;     // gate
  uint32_t cyc;   // cycle inside the chunk
  uint32_t code;  // pin code
  uint32_t tic;   // time inside the cycle
};

__device__ __forceinline__ EvPos ev_pos(int64_t e, const int64_t *evt_t, const uint32_t *ev_pin,
                                        const int32_t *pin_gate, const uint8_t *pin_local, const int32_t *gate_k,
                                        const LayoutFmt &f) {
  EvPos r;
  const int64_t t = evt_t[e];
  const uint32_t p = ev_pin[e];
  r.g = (uint32_t)pin_gate[p];
  const uint32_t i = pin_local[p];
  const int64_t cg = t / f.T;
  r.q = (uint64_t)(cg >> f.lc);
  r.cyc = (uint32_t)(cg & ((int64_t(1) << f.lc) - 1));
  r.tic = (uint32_t)(t - cg * f.T);
  r.code = i == (uint32_t)gate_k[r.g] ? out_code(f.pb) : i;
  return r;
}

// (cycle, time, pin code) as one integer of lc + pb + tb bits
__device__ __forceinline__ uint64_t lk_of(const EvPos &p, const LayoutFmt &f) {
  return ((uint64_t)p.cyc << (f.pb + f.tb)) | ((uint64_t)p.tic << f.pb) | p.code;
}

// sort keys: (chunk, gate, kind, lk) in one word, or (gate, kind, lk) with the
// chunk apart; kind = 1 for the output pin
__global__ void k_sort_keys(int64_t E, const int64_t *evt_t, const uint32_t *ev_pin, const int32_t *pin_gate,
                            const uint8_t *pin_local, const int32_t *gate_k, LayoutFmt f, uint64_t *key,
                            uint32_t *chunk, uint32_t *idx) {
  const uint32_t lkb = f.lc + f.pb + f.tb + 1;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < E; e += (int64_t)gridDim.x * blockDim.x) {
    const EvPos p = ev_pos(e, evt_t, ev_pin, pin_gate, pin_local, gate_k, f);
    const uint64_t kind = p.code == out_code(f.pb) ? 1u : 0u;
    const uint64_t low = ((uint64_t)p.g << lkb) | (kind << (lkb - 1)) | lk_of(p, f);
    if (chunk) {
      key[e] = low;
      chunk[e] = (uint32_t)p.q;
    } else {
      key[e] = (p.q << (f.gb + lkb)) | low;
    }
    idx[e] = (uint32_t)e;
  }
}

// chunk of every event in the order of perm (input of the second sort stage)
__global__ void k_chunk_of(int64_t E, const uint32_t *perm, const uint32_t *chunk, uint32_t *chunk_sorted) {
  for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < E; x += (int64_t)gridDim.x * blockDim.x)
    chunk_sorted[x] = chunk[perm[x]];
}

// an event's fields from its sort key (chunk, gate, kind, cycle, time, pin code)
__device__ __forceinline__ EvPos key_pos(uint64_t K, const LayoutFmt &f) {
  const uint32_t lkb = f.lc + f.pb + f.tb + 1;
  EvPos r;
  r.q = K >> (f.gb + lkb);
  r.g = (uint32_t)(K >> lkb) & ((1u << f.gb) - 1u);
  const uint64_t lk = K & ((uint64_t(1) << (lkb - 1)) - 1u);
  r.code = (uint32_t)lk & ((1u << f.pb) - 1u);
  r.tic = (uint32_t)(lk >> f.pb) & (uint32_t)((uint64_t(1) << f.tb) - 1u);
  r.cyc = (uint32_t)(lk >> (f.pb + f.tb));
  return r;
}

// Packed keys of the sorted events, window heads and their start states.
// With skey (the sorted one-word keys) an event's fields and its
// predecessor's come from the keys; without, from the caller's arrays.
__global__ void k_layout(int64_t E, const uint32_t *perm, const uint64_t *skey, const int64_t *evt_t,
                         const float *evt_slew, const uint8_t *evt_val, const uint32_t *ev_pin,
                         const int32_t *pin_gate, const uint8_t *pin_local, const int32_t *gate_k,
                         const uint8_t *level, LayoutFmt f, uint64_t *key_out, float *slew_out, uint32_t *orig_out,
                         uint32_t *chunk_out) {
  for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < E; x += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = perm[x];
    const EvPos p = skey ? key_pos(skey[x], f) : ev_pos(e, evt_t, ev_pin, pin_gate, pin_local, gate_k, f);
    const uint32_t sl = level[p.g];
    const uint32_t w = p.cyc >> (f.lc - sl);
    const uint32_t outc = out_code(f.pb);
    bool head = true;
    if (x > 0) {
      const EvPos pp = skey ? key_pos(skey[x - 1], f) : ev_pos(perm[x - 1], evt_t, ev_pin, pin_gate, pin_local, gate_k, f);
      head = !(pp.q == p.q && pp.g == p.g && (pp.code == outc) == (p.code == outc) && (pp.cyc >> (f.lc - sl)) == w);
    }
    // an input window's start state is added by k_window_s0, once the windows are known
    const uint64_t lk = lk_of(p, f);
    const uint32_t hs = kKeyGateShift + f.gb;  // the cycle's high bits go above the gate id (none at hs = 64)
    key_out[x] = (hs < 64 ? (lk >> 32) << hs : 0ull) | ((uint64_t)p.g << kKeyGateShift) |
                 ((uint64_t)head << kKeyHeadShift) | ((uint64_t)(evt_val[e] & 1u) << kKeyValShift) |
                 (lk & 0xFFFFFFFFull);
    slew_out[x] = evt_slew[e];
    orig_out[x] = (uint32_t)e;
    chunk_out[x] = (uint32_t)p.q;
  }
}

// The input state at the start of every input window, into its first
// event's key: a pin's value there is its initial value XOR the parity of
// its events before the window start (a binary search in the pin's events).
// One thread per window, after the windows' first events are known.
__global__ void k_window_s0(uint32_t W, const uint32_t *ws, const uint32_t *chunk_sorted, const uint8_t *level,
                            const int32_t *gate_k, const int64_t *pin_base, const int64_t *pin_ptr,
                            const uint8_t *pin_init, const int64_t *evt_t, LayoutFmt f, uint64_t *skey) {
  const uint32_t outc = out_code(f.pb);
  for (int64_t w = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; w < W; w += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t x = ws[w];
    const uint64_t K = skey[x];
    const uint32_t g = (uint32_t)(K >> kKeyGateShift) & ((1u << f.gb) - 1u);
    // the cycle's high bits above the gate id (none when the gate id fills the word)
    const uint32_t hs = kKeyGateShift + f.gb;
    const uint64_t lk = (K & 0xFFFFFFFFull) | (hs < 64 ? (K >> hs) << 32 : 0ull);
    if (((uint32_t)lk & outc) == outc) continue;  // an output window needs no state
    const uint32_t cyc = (uint32_t)(lk >> (f.pb + f.tb));
    const uint32_t sh = f.lc - level[g];
    const int64_t tw = ((int64_t)chunk_sorted[x] * f.Cc + (int64_t)((cyc >> sh) << sh)) * f.T;
    const int64_t pb = pin_base[g];
    const int32_t k = gate_k[g];
    // the pins' binary searches (first event at or after tw) step together,
    // so their loads go out side by side
    int64_t lo[kMaxInputs], hi[kMaxInputs], base[kMaxInputs];
#pragma unroll
    for (int j = 0; j < kMaxInputs; ++j) {
      base[j] = j < k ? pin_ptr[pb + j] : 0;
      hi[j] = j < k ? pin_ptr[pb + j + 1] : 0;
      lo[j] = base[j];
    }
    bool more = true;
    while (more) {
      more = false;
      int64_t t[kMaxInputs];
#pragma unroll
      for (int j = 0; j < kMaxInputs; ++j) t[j] = lo[j] < hi[j] ? evt_t[(lo[j] + hi[j]) >> 1] : 0;
#pragma unroll
      for (int j = 0; j < kMaxInputs; ++j) {
        if (lo[j] < hi[j]) {
          const int64_t mid = (lo[j] + hi[j]) >> 1;
          if (t[j] < tw) lo[j] = mid + 1; else hi[j] = mid;
          more |= lo[j] < hi[j];
        }
      }
    }
    uint64_t S0 = 0;
#pragma unroll
    for (int j = 0; j < kMaxInputs; ++j)
      if (j < k) S0 |= (uint64_t)((pin_init[pb + j] ^ (uint8_t)((lo[j] - base[j]) & 1)) & 1u) << j;
    skey[x] = K | (S0 << kKeyS0Shift);
  }
}

// first sorted event of every chunk: cb[q] = first x with chunk(x) >= q
__global__ void k_chunk_base(int64_t E, int32_t Q, const uint32_t *chunk_sorted, uint32_t *cb) {
  for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x <= E; x += (int64_t)gridDim.x * blockDim.x) {
    const int64_t qa = x > 0 ? (int64_t)chunk_sorted[x - 1] : -1;
    const int64_t qb = x < E ? (int64_t)chunk_sorted[x] : (int64_t)Q;
    for (int64_t q = qa + 1; q <= qb; ++q) cb[q] = (uint32_t)x;
  }
}


// ------------------------------------------------------ lane streams of the pass
//
// The sorted events (window order) are dealt to the pass's lanes in phases:
// every block owns a range of whole windows of one chunk; its input windows,
// longest first, are cut into groups of 64, and so are its output windows; a
// group is a phase, in which each of a wave's 64 lanes walks one window of
// the group (lane i the group's i-th window), all starting at the phase's
// first slot, and the phase lasts as long as its longest window (rounded up
// to an even count).  So every lane of a wave meets a window start at the same
// step and walks windows of one kind.  The phases, costliest first, go to the
// block's 16 waves, each to the wave that would finish it first given the
// work it holds and its measured relative speed (the longest-processing-time
// rule); a wave's phases follow one another in its stream, and a wave's 64
// streams are interleaved in pairs.

constexpr int kLaneNT = 1024;  // lanes of a block of the pass
constexpr int kLaneNW = kLaneNT / 64;
constexpr int kPlanNT = 1024;  // threads of a block of the phase plan

__global__ void k_head_flags(int64_t E, const uint64_t *skey, uint32_t *flag) {
  for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < E; x += (int64_t)gridDim.x * blockDim.x)
    flag[x] = (uint32_t)(skey[x] >> kKeyHeadShift) & 1u;
}

// ws[w] = first sorted event of window w (winc = inclusive count of heads); ws[W] = E
__global__ void k_win_starts(int64_t E, const uint64_t *skey, const uint32_t *winc, uint32_t *ws) {
  for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < E; x += (int64_t)gridDim.x * blockDim.x) {
    if ((skey[x] >> kKeyHeadShift) & 1ull) ws[winc[x] - 1] = (uint32_t)x;
    if (x == E - 1) ws[winc[x]] = (uint32_t)E;
  }
}

// first window of every block: the first window starting at or after the
// block's nominal first event (E: none)
__global__ void k_block_windows(int32_t nr, int64_t E, const uint32_t *rstart, const uint64_t *skey,
                                const uint32_t *winc, uint32_t W, uint32_t *bwin) {
  for (int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; b <= nr; b += (int64_t)gridDim.x * blockDim.x) {
    const int64_t x = rstart[b];
    bwin[b] = x < E ? winc[x] - (uint32_t)((skey[x] >> kKeyHeadShift) & 1ull) : W;
  }
}

// per window: (block << 32 | kind << 31 | ~length), so a stable sort orders
// every block's input windows longest first, then its output windows
// longest first; wlen = the window's event count
__global__ void k_win_keys(uint32_t W, const uint32_t *ws, const uint32_t *bwin, int32_t nr, const uint64_t *skey,
                           uint32_t outc, uint64_t *wkey, uint32_t *widx, uint32_t *wlen) {
  for (int64_t w = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; w < W; w += (int64_t)gridDim.x * blockDim.x) {
    int lo = 0, hi = nr;  // last block with bwin[b] <= w
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (bwin[mid] <= (uint32_t)w) lo = mid; else hi = mid;
    }
    const uint32_t n = ws[w + 1] - ws[w];
    const uint64_t kind = ((uint32_t)skey[ws[w]] & outc) == outc ? 1u : 0u;
    wlen[w] = n;
    wkey[w] = ((uint64_t)lo << 32) | (kind << 31) | (uint64_t)(0x7FFFFFFFu - n);
    widx[w] = (uint32_t)w;
  }
}

// Relative walk times of a block's waves 4 i .. 4 i + 3 given equal work,
// measured on the 10M-event, skewed and 200M-event workloads: the i-th oldest
// wave of every SIMD issues after the older ones
__constant__ uint32_t kWaveSlow[4] = {72u, 92u, 110u, 126u};

// One block per block of the pass.  Its windows come in worder (input
// windows longest first, then output windows longest first; sorted keys in
// wkey); phase i of a kind is that kind's windows 64 i .. 64 i + 63.  One
// wave deals the phases, costliest first, to the waves, each to the wave
// that would finish it first (its cost so far plus the phase's, times its
// relative walk time; a phase costs its slots times w_in or w_out, the
// relative cost of a slot of its kind in the pass); ph gets the phase's
// wave and first slot, in this block's part [floor(w0 / 64) + 2 b, ...) of
// the array, which holds at least its phases.  Before that all threads count
// the input windows and read the phases' lengths into LDS.  Then every window
// gets its place: wlane[w] = (global wave << 6 | lane, first slot).  wave_len
// = the slots of every wave's stream.

constexpr int kPlanLen = 4096;  // phases whose lengths the phase plan keeps in LDS

__global__ __launch_bounds__(kPlanNT) void k_phase_plan(const uint32_t *bwin, const uint32_t *worder,
                                                        const uint64_t *wkey, const uint32_t *wlen, uint32_t hp,
                                                        uint32_t w_in, uint32_t w_out, uint2 *ph, uint2 *wlane,
                                                        uint32_t *wave_len) {
  __shared__ uint32_t s_cnt[kPlanNT / 64];
  __shared__ uint32_t s_len[kPlanLen];
  const int b = blockIdx.x, u = threadIdx.x;
  const uint32_t w0 = bwin[b], nb = bwin[b + 1] - w0;
  uint2 *php = ph + (w0 >> 6) + 2u * (uint32_t)b;
  // input windows: the keys without the kind bit (they come first), counted by all threads
  uint32_t cnt = 0;
  for (uint32_t r0 = 0; r0 < nb; r0 += 4 * kPlanNT) {
    uint64_t kk[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t r = r0 + t * kPlanNT + u;
      kk[t] = r < nb ? wkey[w0 + r] : (1ull << 31);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) cnt += ((kk[t] >> 31) & 1u) ? 0u : 1u;
  }
  for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
  if ((u & 63) == 0) s_cnt[u >> 6] = cnt;
  __syncthreads();
  uint32_t nin = 0;
  for (int i = 0; i < kPlanNT / 64; ++i) nin += s_cnt[i];
  const uint32_t nout = nb - nin;
  const uint32_t pin_ = (nin + 63) >> 6, pout = (nout + 63) >> 6, np = pin_ + pout;
  // a phase's slots: the header pair and its longest (first) window rounded up to even
  auto plen = [&](uint32_t i) {
    const uint32_t first = i < pin_ ? i * 64 : nin + (i - pin_) * 64;
    return hp + ((wlen[worder[w0 + first]] + 1u) & ~1u);
  };
  for (uint32_t i = u; i < np && i < (uint32_t)kPlanLen; i += kPlanNT) s_len[i] = plen(i);
  __syncthreads();
  if (u < 64) {
    // wave 0 deals: lane v < 16 holds wave v's slots and cost; each phase goes
    // to the lane with the least (cost + the phase's) x slowness, the lowest
    // such lane on ties, found by a butterfly over the 16 lanes
    const int lane = u;
    uint32_t load = 0;
    uint64_t cost = 0;
    const uint64_t slow = kWaveSlow[(lane & (kLaneNW - 1)) >> 2];
    uint32_t i = 0, o = 0;
    while (i < pin_ || o < pout) {
      const uint32_t xi = i, xo = pin_ + o;
      const uint32_t li = i < pin_ ? (xi < (uint32_t)kPlanLen ? s_len[xi] : plen(xi)) : 0u;
      const uint32_t lo2 = o < pout ? (xo < (uint32_t)kPlanLen ? s_len[xo] : plen(xo)) : 0u;
      const uint64_t ci = (uint64_t)li * w_in, co = (uint64_t)lo2 * w_out;
      const bool take_in = i < pin_ && (o >= pout || ci >= co);
      const uint64_t cc = take_in ? ci : co;
      uint64_t f = lane < kLaneNW ? (cost + cc) * slow : ~0ull;
      uint32_t v = (uint32_t)lane;
      for (int off = kLaneNW / 2; off > 0; off >>= 1) {
        const uint64_t f2 = __shfl_xor(f, off, kLaneNW);
        const uint32_t v2 = __shfl_xor(v, off, kLaneNW);
        if (f2 < f || (f2 == f && v2 < v)) f = f2, v = v2;
      }
      const uint32_t lv = __shfl(load, (int)v);
      if (lane == 0) php[take_in ? i : pin_ + o] = make_uint2(v, lv);
      if ((uint32_t)lane == v) {
        load += take_in ? li : lo2;
        cost += cc;
      }
      if (take_in) ++i; else ++o;
    }
    if (lane < kLaneNW) wave_len[(size_t)b * kLaneNW + lane] = load;
  }
  __syncthreads();
  for (uint32_t r0 = 0; r0 < nb; r0 += 4 * kPlanNT) {
    uint2 p[4];
    uint32_t wo[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t r = min(r0 + t * kPlanNT + u, nb - 1);
      const uint32_t i = r < nin ? r : r - nin;
      p[t] = php[(r < nin ? 0u : pin_) + (i >> 6)];
      wo[t] = worder[w0 + r];
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t r = r0 + t * kPlanNT + u;
      const uint32_t i = r < nin ? r : r - nin;
      if (r < nb) wlane[wo[t]] = make_uint2(((uint32_t)b * kLaneNW + p[t].x) << 6 | (i & 63u), p[t].y + hp);
    }
  }
}

// The walk kernel's stream, 8 bytes a slot (the lane streams above, slot for
// slot).  An event: key = cycle << (tbc + ck) | tic << ck | pin code >> 1, and
// the slew's bits with the sign bit (always 0 in a slew) holding the pin
// code's low bit (input pins) or the pin's new value (output pin).  tbc =
// bits of the clock period, so the tic field is never all ones in an event.
// An empty slot: key ~0, slew 1.0.
__global__ void k_compact(int64_t n, const uint64_t *key, const float *slew, uint64_t pad_key, uint32_t pb,
                          uint32_t tb, uint32_t gb, uint32_t tbc, uint32_t ck, uint32_t *ckey, uint32_t *cslew) {
  const uint32_t outc = out_code(pb), cs = pb + tb, ysh = 10u + gb;
  const uint32_t tmask = (1u << tb) - 1u;
  for (int64_t y = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; y < n; y += (int64_t)gridDim.x * blockDim.x) {
    const uint64_t K = key[y];
    uint32_t kw = 0xFFFFFFFFu, sw = 0x3F800000u;
    if (K != pad_key) {
      const uint32_t lk = (uint32_t)K, hw = (uint32_t)(K >> 32);
      const uint32_t code = lk & outc;
      const uint32_t tic = (lk >> pb) & tmask;
      const uint32_t hi = ysh < 32 ? hw >> ysh : 0u;  // the cycle's bits above the gate id
      const uint32_t cyc = (uint32_t)((((uint64_t)hi) << 32 | lk) >> cs);
      const bool out = code == outc;
      kw = (cyc << (tbc + ck)) | (tic << ck) | (out ? 0u : (code >> 1));
      sw = __float_as_uint(slew[y]) | ((out ? ((hw >> 8) & 1u) : (code & 1u)) << 31);
    }
    ckey[y] = kw;
    cslew[y] = sw;
  }
}

// Every window's header pair, the two slots in front of its first event in
// the compact stream: keys (hdr | output << (tbc + ck), cell | cap segment <<
// 20 | start state << 24 for an input window, 0 for an output window), slews
// the gate's load (fp64 bits, low word first).  hdr has an all-ones tic field.
__global__ void k_headers(uint32_t W, const uint2 *wlane, const uint2 *wdesc, const uint32_t *ws, const uint64_t *skey,
                          const uint4 *gate_rec, const uint32_t *rank, uint32_t gb, uint32_t outc, uint32_t hdr,
                          uint32_t out_bit, uint32_t *ckey, uint32_t *cslew, uint32_t *wpos) {
  for (int64_t w = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; w < W; w += (int64_t)gridDim.x * blockDim.x) {
    const uint2 wl = wlane[w];
    const uint32_t j = wl.y - 2u;  // the header pair: an even slot of the lane's stream
    const uint32_t y = wdesc[wl.x >> 6].x + (j >> 1) * 128u + 2u * (wl.x & 63u);
    const uint64_t K = skey[ws[w]];
    const uint32_t hw = (uint32_t)(K >> 32);
    const uint32_t g = (hw >> 10) & ((1u << gb) - 1u);
    const bool out = ((uint32_t)K & outc) == outc;
    const uint4 r = gate_rec[g];
    ckey[y] = hdr | (out ? out_bit : 0u);
    ckey[y + 1] = out ? 0u : ((r.z & 0xFFFFFu) | ((r.z >> 24) << 20) | ((hw & 0xFFu) << 24));
    cslew[y] = r.x;
    cslew[y + 1] = r.y;
    wpos[rank[w]] = y >> 1;  // the header's pair: where the walk kernel stores the window's sums
  }
}

// Every sorted event's cost in the pass, for cutting the chunks into blocks
// of equal cost: w_in for an input-pin event, w_out for an output-pin
// event, plus w_head for the first event of a window (its set-up).
__global__ void k_event_cost(int64_t E, const uint64_t *skey, uint32_t outc, uint32_t w_in, uint32_t w_out,
                             uint32_t w_head, const int32_t *gate_k, uint32_t gb, uint64_t *cost) {
  for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < E; x += (int64_t)gridDim.x * blockDim.x) {
    const uint64_t K = skey[x];
    const bool out = ((uint32_t)K & outc) == outc;
    uint32_t wi = w_in;
    if (gate_k != nullptr && !out) {
      // an input event of a gate with few inputs costs less (its LUT rows
      // spread over fewer LDS banks): w_in - 2 for one input, - 1 for two,
      // + 1 from five
      const int k = gate_k[(uint32_t)(K >> 42) & ((1u << gb) - 1u)];
      wi = (uint32_t)max(1, (int)w_in + (k < 3 ? k - 3 : 0) + (k >= 5 ? 1 : 0));
    }
    cost[x] = (out ? w_out : wi) + (((K >> kKeyHeadShift) & 1ull) ? w_head : 0u);
  }
}

// pos[i] = the first sorted event whose inclusive cost prefix exceeds
// target[i] (E if none); pref is nondecreasing
__global__ void k_cost_cuts(int32_t n, const uint64_t *target, const uint64_t *pref, int64_t E, uint32_t *pos) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const uint64_t t = target[i];
    int64_t lo = 0, hi = E;
    while (lo < hi) {
      const int64_t mid = (lo + hi) >> 1;
      if (pref[mid] <= t) lo = mid + 1; else hi = mid;
    }
    pos[i] = (uint32_t)lo;
  }
}

// out[i] = inclusive prefix before sorted event at[i] (0 for event 0)
__global__ void k_gather_prefix(int32_t n, const uint32_t *at, const uint64_t *pref, uint64_t *out) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = at[i] > 0 ? pref[at[i] - 1] : 0ull;
}

// every sorted event to its slot in its lane's stream
__global__ void k_scatter(int64_t E, const uint64_t *skey, const float *sslew, const uint32_t *sorig,
                          const uint32_t *winc, const uint32_t *ws, const uint2 *wlane, const uint2 *wdesc,
                          uint64_t *key, float *slew, uint32_t *orig) {
  for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < E; x += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t w = winc[x] - 1u;
    const uint2 wl = wlane[w];
    const uint32_t j = wl.y + ((uint32_t)x - ws[w]);
    const uint32_t y = wdesc[wl.x >> 6].x + (j >> 1) * 128u + 2u * (wl.x & 63u) + (j & 1u);
    key[y] = skey[x];
    slew[y] = sslew[x];
    orig[y] = sorig[x];
  }
}

}  // namespace

// ------------------------------------------------------------- launchers

// Leakage power at t = 0 (every gate in its initial input state), in two
// fixed-order steps: kL0B partial sums, then their sum.
constexpr int kL0B = 256;

__global__ __launch_bounds__(kLT) void k_leak0_part(int64_t G, const uint32_t *gate_info, const uint2 *cell_meta,
                                                     const double *leak, const int64_t *pin_base,
                                                     const uint8_t *pin_init, double *part) {
  __shared__ double s_w[kLT / 64];
  double l = 0.0;
  for (int64_t g = blockIdx.x * (int64_t)kLT + threadIdx.x; g < G; g += (int64_t)kL0B * kLT) {
    const uint2 m = cell_meta[gate_info[g] & 0xFFFFFFu];
    const int k = (int)(m.x & 15u);
    const int64_t p0 = pin_base[g];
    uint32_t S = 0;
    for (int j = 0; j < k; ++j) S |= uint32_t(pin_init[p0 + j]) << j;
    l += leak[(m.x >> 4) + S];
  }
  for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
  if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = l;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int w = 0; w < kLT / 64; ++w) t += s_w[w];
    part[blockIdx.x] = t;
  }
}

__global__ void k_leak0_sum(const double *part, double *l0) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    double t = 0.0;
    for (int i = 0; i < kL0B; ++i) t += part[i];
    *l0 = t;
  }
}

hipError_t launch_leak0(int64_t G, const uint32_t *gate_info, const uint2 *cell_meta, const double *leak,
                        const int64_t *pin_base, const uint8_t *pin_init, double *part, double *l0, hipStream_t s) {
  hipLaunchKernelGGL(k_leak0_part, dim3(kL0B), dim3(kLT), 0, s, G, gate_info, cell_meta, leak, pin_base, pin_init,
                     part);
  hipLaunchKernelGGL(k_leak0_sum, dim3(1), dim3(64), 0, s, part, l0);
  return hipGetLastError();
}
int leak0_parts() { return kL0B; }

// Per-gate output start: row perm[g] = (0, 0, 0, leak[S0] * window), the
// gate's leakage before any power change.
// A gate's leakage energy at its initial state over the window (internal gate g).
__device__ __forceinline__ double gate_leak_window(int64_t g, const uint32_t *gate_info, const uint2 *cell_meta,
                                                   const double *leak, const int64_t *pin_base,
                                                   const uint8_t *pin_init, double window) {
  const uint2 m = cell_meta[gate_info[g] & 0xFFFFFFu];
  const int k = (int)(m.x & 15u);
  const int64_t p0 = pin_base[g];
  uint32_t S = 0;
  for (int j = 0; j < k; ++j) S |= uint32_t(pin_init[p0 + j]) << j;
  return leak[(m.x >> 4) + S] * window;
}

// Every gate's row (caller's order): zero dynamic parts and the leakage at the
// initial state over the window (the general kernel adds the rest).
__global__ void k_gate_rows(int64_t G, const uint32_t *gate_info, const uint2 *cell_meta, const double *leak,
                            const int64_t *pin_base, const uint8_t *pin_init, const int32_t *perm, double window,
                            double *gate_J) {
  for (int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; g < G; g += (int64_t)gridDim.x * blockDim.x) {
    double *row = gate_J + 4 * (size_t)perm[g];
    row[0] = 0.0;
    row[1] = 0.0;
    row[2] = 0.0;
    row[3] = gate_leak_window(g, gate_info, cell_meta, leak, pin_base, pin_init, window);
  }
}

hipError_t launch_gate_rows(int64_t G, const uint32_t *gate_info, const uint2 *cell_meta, const double *leak,
                            const int64_t *pin_base, const uint8_t *pin_init, const int32_t *perm, double window,
                            double *gate_J, hipStream_t s) {
  if (G <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_gate_rows, dim3(grid_for(G)), dim3(kLT), 0, s, G, gate_info, cell_meta, leak, pin_base,
                     pin_init, perm, window, gate_J);
  return hipGetLastError();
}

// The pieces of the larger gates' rows (see k_gate_sums): block p sums piece
// p, kRowPiece ranks of gate pgate[p], in a fixed order.
__global__ __launch_bounds__(kLT) void k_piece_sums(const uint32_t *goff, const uint32_t *pfirst,
                                                     const uint32_t *pgate, const uint32_t *wpos, const double4 *rec,
                                                     double4 *part) {
  const uint32_t p = blockIdx.x, g = pgate[p];
  const uint32_t r0 = goff[g] + (p - pfirst[g]) * kRowPiece, r1 = min(goff[g + 1], r0 + kRowPiece);
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
  for (uint32_t r = r0 + threadIdx.x; r < r1; r += kLT) {
    const double4 x = rec[wpos[r]];
    s0 += x.x;
    s1 += x.y;
    s2 += x.z;
    s3 += x.w;
  }
  for (int off = 32; off > 0; off >>= 1) {
    s0 += __shfl_down(s0, off);
    s1 += __shfl_down(s1, off);
    s2 += __shfl_down(s2, off);
    s3 += __shfl_down(s3, off);
  }
  __shared__ double4 sw[kLT / 64];
  if ((threadIdx.x & 63) == 0) sw[threadIdx.x >> 6] = make_double4(s0, s1, s2, s3);
  __syncthreads();
  if (threadIdx.x != 0) return;
  double4 t = sw[0];
  for (int w = 1; w < kLT / 64; ++w) {
    t.x += sw[w].x;
    t.y += sw[w].y;
    t.z += sw[w].z;
    t.w += sw[w].w;
  }
  part[p] = t;
}

// Per-gate rows from the walk kernel's window sums (stored at each window's
// header pair, wpos[r] for the window of rank r: the windows ranked
// gate-major, internal gate order; goff[g] the first rank of gate g).  kRowLanes lanes take one gate: each adds every kRowLanes-th of
// the gate's window sums (at most kRowSmall windows), or of its pieces
// (k_piece_sums, before), and a fixed tree adds the lanes' sums.  So a row
// repeats bit for bit from run to run, and no gate waits on one lane walking
// all of its windows.
__global__ __launch_bounds__(kLT) void k_gate_sums(int64_t G, const uint32_t *goff, const uint32_t *pfirst,
                                                    const double *gleak, const int32_t *perm, const uint32_t *wpos,
                                                    const double4 *rec, const double4 *part, double *gate_J) {
  const int64_t g = (blockIdx.x * (int64_t)kLT + threadIdx.x) / kRowLanes;  // wave-aligned groups of lanes
  const uint32_t j = threadIdx.x % kRowLanes;
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0, lk = 0.0;
  int32_t c = 0;
  if (g < G) {
    if (j == 0) {
      lk = gleak[g];
      c = perm[g];
    }
    const uint32_t r0 = goff[g], r1 = goff[g + 1];
    if (r1 - r0 > kRowSmall) {
#pragma unroll 4
      for (uint32_t q = pfirst[g] + j; q < pfirst[g + 1]; q += kRowLanes) {
        const double4 x = part[q];
        s0 += x.x;
        s1 += x.y;
        s2 += x.z;
        s3 += x.w;
      }
    } else {
#pragma unroll 4
      for (uint32_t r = r0 + j; r < r1; r += kRowLanes) {
        const double4 x = rec[wpos[r]];
        s0 += x.x;
        s1 += x.y;
        s2 += x.z;
        s3 += x.w;
      }
    }
  }
  for (int off = kRowLanes / 2; off > 0; off >>= 1) {
    s0 += __shfl_xor(s0, off);
    s1 += __shfl_xor(s1, off);
    s2 += __shfl_xor(s2, off);
    s3 += __shfl_xor(s3, off);
  }
  if (g >= G || j != 0) return;
  s3 += lk;
  double2 *row = reinterpret_cast<double2 *>(gate_J + 4 * (size_t)c);
  row[0] = make_double2(s0, s1);
  row[1] = make_double2(s2, s3);
}

hipError_t launch_gate_sums(int64_t G, uint32_t n_pieces, const uint32_t *goff, const uint32_t *pfirst,
                            const uint32_t *pgate, const double *gleak, const int32_t *perm, const uint32_t *wpos,
                            const double *rec, double *part, double *gate_J, hipStream_t s) {
  if (G <= 0) return hipSuccess;
  const double4 *r4 = reinterpret_cast<const double4 *>(rec);
  double4 *p4 = reinterpret_cast<double4 *>(part);
  if (n_pieces > 0)
    hipLaunchKernelGGL(k_piece_sums, dim3(n_pieces), dim3(kLT), 0, s, goff, pfirst, pgate, wpos, r4, p4);
  const int64_t nb = (G * kRowLanes + kLT - 1) / kLT;
  hipLaunchKernelGGL(k_gate_sums, dim3((uint32_t)nb), dim3(kLT), 0, s, G, goff, pfirst, gleak, perm, wpos, r4, p4,
                     gate_J);
  return hipGetLastError();
}

// What the row sums read besides the window sums, once per event load: every
// gate's leakage energy at its initial state over the window, and every
// piece's gate.
__global__ void k_gate_prep(int64_t G, const uint32_t *gate_info, const uint2 *cell_meta, const double *leak,
                            const int64_t *pin_base, const uint8_t *pin_init, double window, const uint32_t *pfirst,
                            double *gleak, uint32_t *pgate) {
  for (int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; g < G; g += (int64_t)gridDim.x * blockDim.x) {
    gleak[g] = gate_leak_window(g, gate_info, cell_meta, leak, pin_base, pin_init, window);
    for (uint32_t q = pfirst[g]; q < pfirst[g + 1]; ++q) pgate[q] = (uint32_t)g;
  }
}

hipError_t launch_gate_prep(int64_t G, const uint32_t *gate_info, const uint2 *cell_meta, const double *leak,
                            const int64_t *pin_base, const uint8_t *pin_init, double window, const uint32_t *pfirst,
                            double *gleak, uint32_t *pgate, hipStream_t s) {
  if (G <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_gate_prep, dim3(grid_for(G)), dim3(kLT), 0, s, G, gate_info, cell_meta, leak, pin_base,
                     pin_init, window, pfirst, gleak, pgate);
  return hipGetLastError();
}

// Every window's internal gate (the sort key) and index (the value), for
// ranking the windows gate-major.
__global__ void k_win_gates(uint32_t W, const uint32_t *ws, const uint64_t *skey, uint32_t gb, uint32_t *key,
                            uint32_t *val) {
  for (int64_t w = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; w < W; w += (int64_t)gridDim.x * blockDim.x) {
    key[w] = (uint32_t)(skey[ws[w]] >> 32 >> 10) & ((1u << gb) - 1u);
    val[w] = (uint32_t)w;
  }
}

// From the windows sorted by gate (stable: window order within a gate):
// every window's rank.
__global__ void k_win_ranks(uint32_t W, const uint32_t *val, uint32_t *rank) {
  for (int64_t r = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; r < W; r += (int64_t)gridDim.x * blockDim.x)
    rank[val[r]] = (uint32_t)r;
}

// Every gate's first rank, the first sorted key not below the gate (a gate
// without windows gets the next gate's first rank; goff[G] = W), and its
// pieces for the row sums: none up to kRowSmall windows, else one per
// kRowPiece windows.
__global__ void k_gate_first(uint32_t W, int64_t G, const uint32_t *key, uint32_t *goff, uint32_t *npiece) {
  for (int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; g <= G; g += (int64_t)gridDim.x * blockDim.x) {
    auto first = [&](int64_t x) {
      uint32_t lo = 0, hi = W;
      while (lo < hi) {
        const uint32_t mid = lo + (hi - lo) / 2;
        if ((int64_t)key[mid] < x) lo = mid + 1;
        else hi = mid;
      }
      return lo;
    };
    const uint32_t a = first(g);
    goff[g] = a;
    if (g < G) {
      const uint32_t n = first(g + 1) - a;
      npiece[g] = n > kRowSmall ? (n + kRowPiece - 1) / kRowPiece : 0u;
    }
  }
}

hipError_t launch_win_gates(uint32_t W, const uint32_t *ws, const uint64_t *skey, uint32_t gb, uint32_t *key,
                            uint32_t *val, hipStream_t s) {
  if (W == 0) return hipSuccess;
  hipLaunchKernelGGL(k_win_gates, dim3(grid_for(W)), dim3(kLT), 0, s, W, ws, skey, gb, key, val);
  return hipGetLastError();
}

hipError_t launch_win_ranks(uint32_t W, int64_t G, const uint32_t *key, const uint32_t *val, uint32_t *rank,
                            uint32_t *goff, uint32_t *npiece, hipStream_t s) {
  if (W > 0) hipLaunchKernelGGL(k_win_ranks, dim3(grid_for(W)), dim3(kLT), 0, s, W, val, rank);
  hipLaunchKernelGGL(k_gate_first, dim3(grid_for(G + 1)), dim3(kLT), 0, s, W, G, key, goff, npiece);
  return hipGetLastError();
}

hipError_t launch_gate_tables(int64_t G, const int32_t *perm, const int32_t *gate_cell, const double *gate_cap,
                              int32_t n_cells, const int32_t *cell_k, const double *cap_axis, int32_t n_cap, double vdd,
                              uint32_t *gate_info, uint4 *gate_rec, int32_t *gate_k, uint32_t *err, hipStream_t s) {
  hipLaunchKernelGGL(k_gate_tables, dim3(grid_for(G)), dim3(kLT), 0, s, G, perm, gate_cell, gate_cap, n_cells, cell_k,
                     cap_axis, n_cap, vdd, gate_info, gate_rec, gate_k, err);
  return hipGetLastError();
}

hipError_t launch_pin_owner(int64_t G, const int64_t *pin_base, const int32_t *gate_k, int32_t *pin_gate,
                            uint8_t *pin_local, hipStream_t s) {
  hipLaunchKernelGGL(k_pin_owner, dim3(grid_for(G)), dim3(kLT), 0, s, G, pin_base, gate_k, pin_gate, pin_local);
  return hipGetLastError();
}

hipError_t launch_pin_check(int64_t P, int64_t E, const int64_t *pin_ptr, const uint8_t *pin_init, uint32_t *err,
                            hipStream_t s) {
  hipLaunchKernelGGL(k_pin_check, dim3(grid_for(P)), dim3(kLT), 0, s, P, E, pin_ptr, pin_init, err);
  return hipGetLastError();
}

hipError_t launch_event_check(int64_t E, int64_t P, const int64_t *pin_ptr, const uint8_t *pin_init,
                              const int64_t *evt_t, const uint8_t *evt_val, const float *evt_slew, int64_t t_max,
                              uint32_t *mark, uint32_t *ev_pin, uint32_t *err, void *tmp, size_t *tmp_bytes,
                              hipStream_t s) {
  if (E <= 0) return hipSuccess;
  if (!tmp) return rocprim::inclusive_scan(nullptr, *tmp_bytes, mark, ev_pin, (size_t)E, rocprim::maximum<uint32_t>(), s);
  hipError_t e = hipMemsetAsync(mark, 0, sizeof(uint32_t) * E, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_pin_starts, dim3(grid_for(P)), dim3(kLT), 0, s, P, E, pin_ptr, mark);
  e = rocprim::inclusive_scan(tmp, *tmp_bytes, mark, ev_pin, (size_t)E, rocprim::maximum<uint32_t>(), s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_event_check, dim3(grid_for(E)), dim3(kLT), 0, s, E, pin_ptr, pin_init, evt_t, evt_val, evt_slew,
                     t_max, ev_pin, err);
  return hipGetLastError();
}

hipError_t launch_gate_levels(int64_t G, const int64_t *pin_base, const int32_t *gate_k, const int64_t *pin_ptr,
                              int64_t C, int32_t Cc, int32_t lc, double target, int32_t fixed_level,
                              uint8_t *level, hipStream_t s) {
  hipLaunchKernelGGL(k_gate_levels, dim3(grid_for(G)), dim3(kLT), 0, s, G, pin_base, gate_k, pin_ptr, C, Cc, lc, target,
                     fixed_level, level);
  return hipGetLastError();
}

hipError_t launch_sort_keys(int64_t E, const int64_t *evt_t, const uint32_t *ev_pin, const int32_t *pin_gate,
                            const uint8_t *pin_local, const int32_t *gate_k, const LayoutFmt &f, uint64_t *key,
                            uint32_t *chunk, uint32_t *idx, hipStream_t s) {
  hipLaunchKernelGGL(k_sort_keys, dim3(grid_for(E)), dim3(kLT), 0, s, E, evt_t, ev_pin, pin_gate, pin_local, gate_k, f,
                     key, chunk, idx);
  return hipGetLastError();
}

hipError_t launch_chunk_of(int64_t E, const uint32_t *perm, const uint32_t *chunk, uint32_t *chunk_sorted,
                           hipStream_t s) {
  hipLaunchKernelGGL(k_chunk_of, dim3(grid_for(E)), dim3(kLT), 0, s, E, perm, chunk, chunk_sorted);
  return hipGetLastError();
}

hipError_t launch_layout(int64_t E, const uint32_t *perm, const uint64_t *skey, const int64_t *evt_t,
                         const float *evt_slew, const uint8_t *evt_val, const uint32_t *ev_pin,
                         const int32_t *pin_gate, const uint8_t *pin_local, const int32_t *gate_k,
                         const uint8_t *level, const LayoutFmt &f, uint64_t *key_out, float *slew_out,
                         uint32_t *orig_out, uint32_t *chunk_out, hipStream_t s) {
  hipLaunchKernelGGL(k_layout, dim3(grid_for(E)), dim3(kLT), 0, s, E, perm, skey, evt_t, evt_slew, evt_val, ev_pin,
                     pin_gate, pin_local, gate_k, level, f, key_out, slew_out, orig_out, chunk_out);
  return hipGetLastError();
}

hipError_t launch_window_s0(uint32_t W, const uint32_t *ws, const uint32_t *chunk_sorted, const uint8_t *level,
                            const int32_t *gate_k, const int64_t *pin_base, const int64_t *pin_ptr,
                            const uint8_t *pin_init, const int64_t *evt_t, const LayoutFmt &f, uint64_t *skey,
                            hipStream_t s) {
  if (W == 0) return hipSuccess;
  hipLaunchKernelGGL(k_window_s0, dim3(grid_for(W)), dim3(kLT), 0, s, W, ws, chunk_sorted, level, gate_k, pin_base,
                     pin_ptr, pin_init, evt_t, f, skey);
  return hipGetLastError();
}

hipError_t launch_chunk_base(int64_t E, int32_t Q, const uint32_t *chunk_sorted, uint32_t *cb, hipStream_t s) {
  hipLaunchKernelGGL(k_chunk_base, dim3(grid_for(E + 1)), dim3(kLT), 0, s, E, Q, chunk_sorted, cb);
  return hipGetLastError();
}

hipError_t launch_head_flags(int64_t E, const uint64_t *skey, uint32_t *flag, hipStream_t s) {
  hipLaunchKernelGGL(k_head_flags, dim3(grid_for(E)), dim3(kLT), 0, s, E, skey, flag);
  return hipGetLastError();
}
hipError_t launch_win_starts(int64_t E, const uint64_t *skey, const uint32_t *winc, uint32_t *ws, hipStream_t s) {
  hipLaunchKernelGGL(k_win_starts, dim3(grid_for(E)), dim3(kLT), 0, s, E, skey, winc, ws);
  return hipGetLastError();
}
hipError_t launch_block_windows(int32_t nr, int64_t E, const uint32_t *rstart, const uint64_t *skey,
                                const uint32_t *winc, uint32_t W, uint32_t *bwin, hipStream_t s) {
  hipLaunchKernelGGL(k_block_windows, dim3(grid_for(nr + 1)), dim3(kLT), 0, s, nr, E, rstart, skey, winc, W, bwin);
  return hipGetLastError();
}
hipError_t launch_win_keys(uint32_t W, const uint32_t *ws, const uint32_t *bwin, int32_t nr, const uint64_t *skey,
                           uint32_t outc, uint64_t *wkey, uint32_t *widx, uint32_t *wlen, hipStream_t s) {
  if (W == 0) return hipSuccess;
  hipLaunchKernelGGL(k_win_keys, dim3(grid_for(W)), dim3(kLT), 0, s, W, ws, bwin, nr, skey, outc, wkey, widx, wlen);
  return hipGetLastError();
}
size_t phase_plan_entries(uint32_t W, int32_t nr) { return (size_t)(W >> 6) + 2 * (size_t)nr + 2; }
hipError_t launch_phase_plan(int32_t nr, const uint32_t *bwin, const uint32_t *worder, const uint64_t *wkey,
                             const uint32_t *wlen, uint32_t hp, uint32_t w_in, uint32_t w_out, uint2 *ph,
                             uint2 *wlane, uint32_t *wave_len, hipStream_t s) {
  if (nr <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_phase_plan, dim3((unsigned)nr), dim3(kPlanNT), 0, s, bwin, worder, wkey, wlen, hp, w_in, w_out,
                     ph, wlane, wave_len);
  return hipGetLastError();
}
hipError_t launch_headers(uint32_t W, const uint2 *wlane, const uint2 *wdesc, const uint32_t *ws, const uint64_t *skey,
                          const uint4 *gate_rec, const uint32_t *rank, uint32_t gb, uint32_t outc, uint32_t hdr,
                          uint32_t out_bit, uint32_t *ckey, uint32_t *cslew, uint32_t *wpos, hipStream_t s) {
  if (W == 0) return hipSuccess;
  hipLaunchKernelGGL(k_headers, dim3(grid_for(W)), dim3(kLT), 0, s, W, wlane, wdesc, ws, skey, gate_rec, rank, gb, outc,
                     hdr, out_bit, ckey, cslew, wpos);
  return hipGetLastError();
}
hipError_t launch_compact(int64_t n, const uint64_t *key, const float *slew, uint64_t pad_key, uint32_t pb,
                          uint32_t tb, uint32_t gb, uint32_t tbc, uint32_t ck, uint32_t *ckey, uint32_t *cslew,
                          hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_compact, dim3(grid_for(n)), dim3(kLT), 0, s, n, key, slew, pad_key, pb, tb, gb, tbc, ck, ckey,
                     cslew);
  return hipGetLastError();
}
hipError_t launch_scatter(int64_t E, const uint64_t *skey, const float *sslew, const uint32_t *sorig,
                          const uint32_t *winc, const uint32_t *ws, const uint2 *wlane, const uint2 *wdesc,
                          uint64_t *key, float *slew, uint32_t *orig, hipStream_t s) {
  hipLaunchKernelGGL(k_scatter, dim3(grid_for(E)), dim3(kLT), 0, s, E, skey, sslew, sorig, winc, ws, wlane, wdesc,
                     key, slew, orig);
  return hipGetLastError();
}
int lane_plan_lanes() { return kLaneNT; }

namespace {
__global__ void k_fill_u64(int64_t n, uint64_t v, uint64_t *out) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = v;
}
}  // namespace

hipError_t launch_fill_u64(int64_t n, uint64_t v, uint64_t *out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_u64, dim3(grid_for(n)), dim3(kLT), 0, s, n, v, out);
  return hipGetLastError();
}

hipError_t launch_event_cost(int64_t E, const uint64_t *skey, uint32_t outc, uint32_t w_in, uint32_t w_out,
                             uint32_t w_head, const int32_t *gate_k, uint32_t gb, uint64_t *cost, hipStream_t s) {
  if (E <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_event_cost, dim3(grid_for(E)), dim3(kLT), 0, s, E, skey, outc, w_in, w_out, w_head, gate_k, gb,
                     cost);
  return hipGetLastError();
}
hipError_t launch_cost_cuts(int32_t n, const uint64_t *target, const uint64_t *pref, int64_t E, uint32_t *pos,
                            hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_cost_cuts, dim3(grid_for(n)), dim3(kLT), 0, s, n, target, pref, E, pos);
  return hipGetLastError();
}
hipError_t launch_gather_prefix(int32_t n, const uint32_t *at, const uint64_t *pref, uint64_t *out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_gather_prefix, dim3(grid_for(n)), dim3(kLT), 0, s, n, at, pref, out);
  return hipGetLastError();
}
hipError_t scan_inclusive_u64(const uint64_t *in, uint64_t *out, int64_t n, void *tmp, size_t *tmp_bytes,
                              hipStream_t s) {
  return rocprim::inclusive_scan(tmp, *tmp_bytes, in, out, (size_t)n, rocprim::plus<uint64_t>(), s);
}

hipError_t scan_inclusive_u32(const uint32_t *in, uint32_t *out, int64_t n, void *tmp, size_t *tmp_bytes,
                              hipStream_t s) {
  return rocprim::inclusive_scan(tmp, *tmp_bytes, in, out, (size_t)n, rocprim::plus<uint32_t>(), s);
}

// radix sorts that ping-pong between the two buffers given (no copy back):
// the sorted keys and values end in (*k0, *v0) or (*k1, *v1), and the
// pointers are swapped so that *k0 and *v0 hold them
hipError_t sort_pairs_u64(uint64_t **k0, uint64_t **k1, uint32_t **v0, uint32_t **v1, int64_t n, int end_bit,
                          void *tmp, size_t *tmp_bytes, hipStream_t s) {
  rocprim::double_buffer<uint64_t> kb(*k0, *k1);
  rocprim::double_buffer<uint32_t> vb(*v0, *v1);
  const hipError_t e = rocprim::radix_sort_pairs(tmp, *tmp_bytes, kb, vb, (size_t)n, 0u, (unsigned)end_bit, s);
  if (tmp && e == hipSuccess && kb.current() != *k0) {
    std::swap(*k0, *k1);
    std::swap(*v0, *v1);
  }
  return e;
}

hipError_t sort_pairs_u32(uint32_t **k0, uint32_t **k1, uint32_t **v0, uint32_t **v1, int64_t n, int end_bit,
                          void *tmp, size_t *tmp_bytes, hipStream_t s) {
  rocprim::double_buffer<uint32_t> kb(*k0, *k1);
  rocprim::double_buffer<uint32_t> vb(*v0, *v1);
  const hipError_t e = rocprim::radix_sort_pairs(tmp, *tmp_bytes, kb, vb, (size_t)n, 0u, (unsigned)end_bit, s);
  if (tmp && e == hipSuccess && kb.current() != *k0) {
    std::swap(*k0, *k1);
    std::swap(*v0, *v1);
  }
  return e;
}

}  // namespace pa
