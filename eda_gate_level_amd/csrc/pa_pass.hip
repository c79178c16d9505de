// pa_pass.hip -- the hot path of gate-level time-based power analysis on
// gfx950: one fused pass over the event layout plus a finalize.
//
// Method: "GPU-Accelerated Gate-Level Time-Based Power Analysis via
// Event-Density-Aware Partitioning and Kernel Fusion" (arXiv 2609.05960).
// Per event (Sec. 2.4.1, Fig. 2, Eqs. 1-3): the gate state before the event
// selects the internal-power LUT, bilinear on input slew and output load; a
// 0->1 output event draws 1/2 c v^2; the m-th event (m >= 2) of a pin in a
// clock cycle is a glitch scaled by r_gl; the energy lands in the event's
// cycle bin.  Per gate (Sec. 2.4.2, Fig. 3, Eq. 4): state-dependent leakage
// over every inter-event interval, spread over the cycle bins it overlaps.
// The paper fuses both parts into one thread per (gate, cycle window)
// (Fig. 7).  This pass keeps the fusion and maps it onto 64-lane waves:
//   * the events are laid out by (time chunk, gate, clock cycle, time, pin);
//     every gate's part of a chunk is cut into density-aware windows whose
//     first event carries the gate's input state at the window start;
//   * a block owns a range of whole windows inside one chunk and each of its
//     waves streams a share of them, 128 consecutive events per batch (two
//     per lane, 16-byte loads), the next batch prefetched into registers;
//   * the state before every event is a segmented XOR scan of the input
//     events' pin bits across the wave (DPP row shifts and broadcasts), the
//     segments being the windows: the k-way merge of Sec. 2.4.2, since the
//     layout is already in time order.  Events of one timestamp are
//     adjacent; each sees the state before the first of them, and the lowest
//     input pin among them charges the leakage change of the whole set;
//   * a glitch is an event whose pin has an earlier event in the same
//     (gate, cycle) run: a segmented OR scan of pin bits over the runs
//     (Fig. 7); its pulse width and the previous slew come from the pin's
//     previous event in the run: the event just before, or the one a max
//     scan of positions per pin finds (Eq. 2);
//   * one lane per event: state-selected LUT, bilinear on slew and load
//     (Sec. 2.4.1, Fig. 2), switching energy (Eq. 1), energies added to
//     per-cycle bins in LDS.  The LUTs of the cells most of a block's events
//     use are copied into the block's spare LDS at its start (chosen at load
//     from a sample of its events); the other cells are read through the
//     caches;
//   * leakage is charged as power changes: at every distinct input timestamp
//     the lowest switching input pin adds dP = leak[S+] - leak[S-]; its
//     partial bin gets dP * (bin end - t) and all later bins get dP * their
//     length through an in-LDS prefix sum per chunk and a per-chunk carry;
//     the leakage at t = 0 is the sum over gates of leak[S0].  This is the
//     paper's per-interval, per-overlapped-bin split (Sec. 2.4.2, Eq. 4)
//     summed in another order;
//   * every block writes its bins and totals to its own slots; the finalize
//     kernel adds them up in a fixed order (no global atomics).
#include <hip/hip_runtime.h>

#include "pa_common.h"

namespace pa {

namespace {

#ifndef PA_NT
#define PA_NT 1024
#endif
#ifndef PA_FUSED_ATTR
#define PA_FUSED_ATTR
#endif
constexpr int kNT = PA_NT;           // threads per block
constexpr int kNW = kNT / 64;        // waves per block, each working on its own batches
constexpr int kBPC = 1024 / kNT;     // blocks per compute unit (16 waves each)
constexpr int kB = 128;              // events per wave batch, two consecutive ones per lane
constexpr int kCCMAX = 2048;         // max cycles per chunk (LDS bins)
constexpr int kPlan = 8;             // cells per block whose LUTs may sit in LDS
constexpr uint32_t kLutLds = 0x80000000u;  // LUT base flag in a block's cell table: offset into its LDS copy
typedef __attribute__((address_space(3))) double lds_f64;
constexpr size_t kLdsMax = 160 * 1024 / kBPC;  // LDS of a block (gfx950: 160 KB per compute unit)
static_assert(kB - 1 >= kGroupMax, "a (gate, cycle) run fits in one batch after an odd start");

typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t key_head(uint64_t k) { return uint32_t(k >> kKeyHeadShift) & 1u; }

// first window head at or after position x (E if none); one whole wave
__device__ int find_head(const uint64_t *key, int64_t E, int64_t x) {
  const int lane = threadIdx.x & 63;
  for (;;) {
    if (x >= E) return (int)E;
    const int64_t y = x + lane;
    const bool h = (y >= E) || key_head(key[y]);
    const unsigned long long m = __ballot(h);
    if (m) return (int)(x + __ffsll((long long)m) - 1);
    x += 64;
  }
}

__device__ __forceinline__ double wave_sum(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// LDS ordering between the lanes of one wave (no block barrier)
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// value of another lane by a DPP move; lanes without a source read 0 (the
// bound control writes 0 there, so no zeroed old value is needed)
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, true);
}

// another lane's value by a DPP move inside a scan step: lanes without a
// source (outside the row, or rows the broadcast does not write) read 0
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp_src(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, true);
}

// inclusive XOR and max scans over the 64 lanes (row shifts 1, 2, 4, 8, then
// row broadcasts 15 and 31); 0 is the identity of both
__device__ __forceinline__ uint32_t xor_scan(uint32_t w) {
  w ^= dpp_src<0x111>(w);
  w ^= dpp_src<0x112>(w);
  w ^= dpp_src<0x114>(w);
  w ^= dpp_src<0x118>(w);
  w ^= dpp_src<0x142, 0xA>(w);
  w ^= dpp_src<0x143, 0xC>(w);
  return w;
}

__device__ __forceinline__ uint32_t max_scan(uint32_t w) {
  w = max(w, dpp_src<0x111>(w));
  w = max(w, dpp_src<0x112>(w));
  w = max(w, dpp_src<0x114>(w));
  w = max(w, dpp_src<0x118>(w));
  w = max(w, dpp_src<0x142, 0xA>(w));
  w = max(w, dpp_src<0x143, 0xC>(w));
  return w;
}

// Glitch-scan element: low 16 bits = pins with an event so far in the run,
// kRun = a (gate, cycle) run starts here.  a then b: b restarts or the sets join.
constexpr uint32_t kRun = 0x10000u;
__device__ __forceinline__ uint32_t or_combine(uint32_t a, uint32_t b) { return (b & kRun) ? b : (a | b); }

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t or_step(uint32_t w) {
  const uint32_t t = dpp_mov<CTRL, ROWS>(w) | w;
  return (w & kRun) ? w : t;
}

__device__ __forceinline__ uint32_t or_scan(uint32_t w) {
  w = or_step<0x111>(w);
  w = or_step<0x112>(w);
  w = or_step<0x114>(w);
  w = or_step<0x118>(w);
  w = or_step<0x142, 0xA>(w);
  w = or_step<0x143, 0xC>(w);
  return w;
}

struct CellLds {
  double2 *axw, *caxw;
  float *thr;
  double *bw, *bb;
  unsigned long long *bc;
  double *leak;
  uint2 *meta;
  double *lut;  // the block's LUT copies, 16-byte aligned after the cell meta
};

__host__ __device__ inline size_t cell_bytes(int n_cells, int n_slew, int n_cap, int n_thr, int64_t n_leak) {
  return 16 * (size_t)n_cells * (n_slew - 1 + n_cap - 1) + 4 * (size_t)n_cells * n_thr + 8 * (size_t)n_leak +
         8 * (size_t)n_cells;
}

// dynamic LDS: [slew (axis, 1/width) pairs][cap (axis, 1/width) pairs][slew thresholds][bins: wave,
// leakage change, counts][leakage][cell meta][LUT copies]
__device__ __forceinline__ CellLds carve(unsigned char *s, int Cc, int n_cells, int n_slew, int n_cap, int n_thr,
                                         int64_t n_leak, bool cells) {
  CellLds L;
  L.axw = reinterpret_cast<double2 *>(s);
  L.caxw = L.axw + (cells ? n_cells * (n_slew - 1) : 0);
  L.thr = reinterpret_cast<float *>(L.caxw + (cells ? n_cells * (n_cap - 1) : 0));
  L.bw = reinterpret_cast<double *>(L.thr + (cells ? n_cells * n_thr : 0));
  L.bb = L.bw + Cc;
  L.bc = reinterpret_cast<unsigned long long *>(L.bb + Cc);
  L.leak = reinterpret_cast<double *>(L.bc + Cc);
  L.meta = reinterpret_cast<uint2 *>(L.leak + (cells ? n_leak : 0));
  const size_t end = (size_t)(reinterpret_cast<unsigned char *>(L.meta + (cells ? n_cells : 0)) - s);
  L.lut = reinterpret_cast<double *>(s + ((end + 15) & ~size_t(15)));
  return L;
}

// NIN: number of inner slew-axis points when fixed at compile time (-1: any)
template <bool CELL_LDS, bool DIAG, int NIN>
__global__ __launch_bounds__(kNT) PA_FUSED_ATTR void k_fused(PassArgs a) {
  extern __shared__ __align__(16) unsigned char s_dyn[];
  __shared__ uint32_t st_lk[kNW][kB];  // batch events (lk) for the in-cycle walk
  __shared__ uint8_t st_gh[kNW][kB];   // tie flags of the batch events (same run, same time as the one before)
  __shared__ float st_sl[kNW][kB];     // slews of the batch events
  __shared__ double s_red[kNW][8];
  __shared__ double s_scan[kNW];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int b = blockIdx.x, nb = gridDim.x;
  const int Cc = a.Cc, ns = a.n_slew, nc = a.n_cap, nthr = a.n_thr;
  const CellLds L = carve(s_dyn, Cc, a.n_cells, ns, nc, nthr, a.n_leak, CELL_LDS);
  const bool has_range = b < a.n_ranges;

  auto meta_of = [&](uint32_t c) -> uint2 {
    if constexpr (CELL_LDS) return L.meta[c]; else return a.cell_meta[c];
  };
  auto thr_of = [&](uint32_t c, int j) -> float4 {
    // cells < 2^24 and short axes: every offset here is a full-rate 24-bit product
    if constexpr (CELL_LDS) return *reinterpret_cast<const float4 *>(L.thr + __umul24(c, nthr) + j);
    else return *reinterpret_cast<const float4 *>(a.cell_thr + __umul24(c, nthr) + j);
  };
  auto axw_of = [&](uint32_t c, uint32_t j) -> double2 {
    if constexpr (CELL_LDS) return L.axw[__umul24(c, ns - 1) + j]; else return a.cell_axw[__umul24(c, ns - 1) + j];
  };
  auto caxw_of = [&](uint32_t c, uint32_t j) -> double2 {
    if constexpr (CELL_LDS) return L.caxw[__umul24(c, nc - 1) + j]; else return a.cell_caxw[__umul24(c, nc - 1) + j];
  };
  auto leak_of = [&](uint32_t j) -> double {
    if constexpr (CELL_LDS) return L.leak[j]; else return a.leak[j];
  };

  // ---- the block's chunk and this wave's range (cut at window heads at load);
  // the first batch is fetched before the tables are staged
  int q = 0, pos = 0, wend = 0;
  if (has_range) {
    q = (int)a.rchunk[b];
    // wave-uniform, so the batch loop is steered by scalar branches
    pos = __builtin_amdgcn_readfirstlane(a.wbound[b * (kNW + 1) + wid]);
    wend = __builtin_amdgcn_readfirstlane(a.wbound[b * (kNW + 1) + wid + 1]);
  }
  u64x2 kp = {0ull, 0ull};
  f32x2 sp = {0.f, 0.f};
  // pairs past the wave's range belong to other waves (or to the two zeroed
  // entries after the last event); the batch ignores them
  const int xmax = (int)(((a.E + 2) & ~int64_t(1)) - 2);
  auto load_batch = [&](int p) {
    const int x0 = min((p & ~1) + 2 * lane, xmax);
    kp = __builtin_nontemporal_load(reinterpret_cast<const u64x2 *>(a.key + x0));
    sp = __builtin_nontemporal_load(reinterpret_cast<const f32x2 *>(a.slew + x0));
  };
  if (pos < wend) load_batch(pos);
  for (int c = tid; c < Cc; c += kNT) {
    L.bw[c] = 0.0;
    L.bb[c] = 0.0;
    L.bc[c] = 0ull;
  }
  if constexpr (CELL_LDS) {
    for (int j = tid; j < a.n_cells * (ns - 1); j += kNT) L.axw[j] = a.cell_axw[j];
    for (int j = tid; j < a.n_cells * (nc - 1); j += kNT) L.caxw[j] = a.cell_caxw[j];
    for (int j = tid; j < a.n_cells * nthr; j += kNT) L.thr[j] = a.cell_thr[j];
    for (int j = tid; j < a.n_leak; j += kNT) L.leak[j] = a.leak[j];
    // the cells whose LUTs this block reads from LDS: their table entries
    // point into the copy instead of the global LUT
    uint32_t pc[kPlan], po[kPlan];
#pragma unroll
    for (int e = 0; e < kPlan; ++e) {
      const uint2 v = (has_range && a.lut_lds > 0) ? a.lut_plan[(size_t)b * kPlan + e] : make_uint2(~0u, 0u);
      pc[e] = v.x;
      po[e] = v.y;
    }
    for (int j = tid; j < a.n_cells; j += kNT) {
      uint2 mv = a.cell_meta[j];
#pragma unroll
      for (int e = 0; e < kPlan; ++e)
        if (pc[e] == (uint32_t)j) mv.y = kLutLds | po[e];
      L.meta[j] = mv;
    }
    // LUT sizes 2^k k ns nc are even, so every table starts 16-byte aligned
#pragma unroll 1
    for (int e = 0; e < kPlan; ++e) {
      if (pc[e] == ~0u) break;
      const uint2 gm = a.cell_meta[pc[e]];
      const uint32_t k = gm.x & 15u;
      const int n2 = (int)((((1u << k) * k) * (uint32_t)(ns * nc)) >> 1);
      const double2 *src = reinterpret_cast<const double2 *>(a.lut + gm.y);
      double2 *dst = reinterpret_cast<double2 *>(L.lut + po[e]);
#pragma unroll 4
      for (int j = tid; j < n2; j += kNT) dst[j] = src[j];
    }
  }
  __syncthreads();

  double e_int = 0.0, e_sw = 0.0, e_gl = 0.0, e_lk = 0.0;
  unsigned n_gl = 0;

  const int64_t cstart = (int64_t)q * a.chunk_ticks;
  const int64_t clen = min(a.chunk_ticks, a.t_max - cstart);
  const int ncyc = (int)((clen + a.T - 1) / a.T);
  const bool last_chunk = (q == a.Q - 1);
  const uint32_t lastc = (uint32_t)(ncyc - 1);
  const uint32_t T = a.T;
  const double Td = (double)T;
  const double tail = (double)(a.t_max - cstart);  // t_max - t = tail - (cyc T + tic)
  const double tick = a.tick_s;
  const uint32_t tb = a.tb, pb = a.pb, cs = tb + pb;
  const uint32_t gmask = (1u << a.gb) - 1u, ysh = 10u + a.gb;  // gate id and high cycle bits in the key's high word
  const uint32_t tmask = (1u << tb) - 1u;
  const uint32_t outc = (1u << pb) - 1u;

  if (has_range) {
    uint32_t carry = 0;
    uint32_t *slk = st_lk[wid];
    uint8_t *sgh = st_gh[wid];

    while (pos < wend) {
      const int base = pos & ~1;
      const int first = pos - base;  // 0, or 1 when the batch starts on an odd event
      const int navail = min(kB, wend - base);
      const uint64_t K0 = kp.x, K1 = kp.y;
      const float s0 = sp.x, s1 = sp.y;
      const int i0 = 2 * lane, i1 = i0 + 1;
      const bool v0 = i0 >= first && i0 < navail;
      const bool v1 = i1 < navail;
      const uint32_t lk0 = (uint32_t)K0, lk1 = (uint32_t)K1;
      const uint32_t h0 = (uint32_t)(K0 >> 32), h1 = (uint32_t)(K1 >> 32);
      const bool hd0 = (h0 >> 9) & 1u, hd1 = (h1 >> 9) & 1u;
      // cycles in the chunk
      const uint32_t y0 = (uint32_t)((((uint64_t)h0 >> ysh) << 32 | lk0) >> cs);
      const uint32_t y1 = (uint32_t)((((uint64_t)h1 >> ysh) << 32 | lk1) >> cs);
      // the event before slot i0 is the previous lane's second one
      const uint32_t lkp0 = dpp_mov<0x138>(lk1);
      const uint32_t yp0 = dpp_mov<0x138>(y1);
      // run starts: a window head, the batch start, or a new clock cycle
      const bool gh0 = hd0 || i0 == first || y0 != yp0;
      const bool gh1 = hd1 || i1 == first || y1 != y0;
      // process up to the last run start, so that no (gate, cycle) run is split
      const unsigned long long M0 = __ballot(v0 && gh0), M1 = __ballot(v1 && gh1);
      int last = -1;
      if (M0) last = 2 * (63 - __clzll((long long)M0));
      if (M1) last = max(last, 2 * (63 - __clzll((long long)M1)) + 1);
      const int end = (base + navail < wend && last > first) ? last : navail;
      const bool a0 = v0 && i0 < end, a1 = v1 && i1 < end;
      const int npos = base + end;
      if (npos < wend) load_batch(npos);

      const uint32_t c0 = lk0 & outc, c1 = lk1 & outc;                    // pin codes
      const uint32_t t0 = (lk0 >> pb) & tmask, t1 = (lk1 >> pb) & tmask;  // time inside the cycle
      const bool in0 = c0 != outc, in1 = c1 != outc;
      // the gates' records; slot 1 reuses slot 0's when both events are of one gate
      const uint32_t g0 = (h0 >> 10) & gmask, g1 = (h1 >> 10) & gmask;
      const bool same_gate = a0 && g1 == g0;
      uint4 rec0 = make_uint4(0u, 0u, 0u, 0u), rec1 = make_uint4(0u, 0u, 0u, 0u);
      if (a0) rec0 = a.gate_rec[g0];
      if (a1 && !same_gate) rec1 = a.gate_rec[g1];

      // ---- state before every event (Sec. 2.4.2): the toggles of the input
      // events before it in the batch (an XOR scan, Q) on top of the state at
      // the last window head at or before it.  A head h carries
      // (h + 1) << 8 | (S0 ^ Q[h]), so a max scan finds the last one, and the
      // state before event i is that low byte ^ Q[i]; the state carried
      // from the previous batch acts as a head at position 0.
      const uint32_t tg0 = (a0 && in0) ? (1u << c0) : 0u;
      const uint32_t tg1 = (a1 && in1) ? (1u << c1) : 0u;
      const uint32_t Q0 = xor_scan(tg0 ^ tg1) ^ tg0 ^ tg1;  // toggles before slot i0
      const uint32_t Q1 = Q0 ^ tg0;
      const uint32_t V0 = (a0 && hd0) ? (((uint32_t)(i0 + 1) << 8) | ((h0 ^ Q0) & 0xFFu)) : 0u;
      const uint32_t V1 = (a1 && hd1) ? (((uint32_t)(i1 + 1) << 8) | ((h1 ^ Q1) & 0xFFu)) : 0u;
      uint32_t vm = max(V0, V1);
      if (lane == 0) vm = max(vm, carry);
      const uint32_t M = max_scan(vm);
      uint32_t Mx = dpp_mov<0x138>(M);
      if (lane == 0) Mx = carry;
      const uint32_t B0 = max(Mx, V0), B1 = max(B0, V1);
      uint32_t S0s = (B0 ^ Q0) & 0xFFu;
      uint32_t S1s = (B1 ^ Q1) & 0xFFu;
      // state after event end - 1 (a lane's slot 1 past the end adds nothing)
      carry = (uint32_t)__builtin_amdgcn_readlane((int)((B1 ^ Q1 ^ tg1) & 0xFFu), (end - 1) >> 1);

      // ---- glitches: the pin already has an event in this (gate, cycle) run
      // (Sec. 2.4.1, Fig. 7); runs never cross a batch, so no carry.  When no
      // run of the batch holds three or more events, the only earlier event
      // of a run is the one just before; otherwise an OR scan of pin bits
      // over the runs gives every event the pins seen before it.
      const uint32_t tp0 = (lkp0 >> pb) & tmask;  // time of the event before slot i0
      const uint32_t ghp = dpp_mov<0x138>((uint32_t)gh1);  // the event before slot i0 starts a run
      const float sp0 = __uint_as_float(dpp_mov<0x138>(__float_as_uint(s1)));  // its slew
      const bool slowgl = (__ballot(a0 && !gh0 && !ghp) | __ballot(a1 && !gh1 && !gh0)) != 0ull;
      bool gl0 = false, gl1 = false;
      uint32_t tq0 = tp0, tq1 = t0;  // time of the pin's previous event (glitches)
      float sq0 = sp0, sq1 = s0;     // its slew
      if (!slowgl) {
        gl0 = a0 && !gh0 && (c0 == (lkp0 & outc));
        gl1 = a1 && !gh1 && (c1 == c0);
      } else {
        const uint32_t u0 = a0 ? (1u << c0) : 0u, u1 = a1 ? (1u << c1) : 0u;
        const uint32_t Io = or_scan(or_combine(gh0 ? (kRun | u0) : u0, gh1 ? (kRun | u1) : u1));
        // (the lane move runs in every lane: a lane whose value is not taken
        // must still provide its own to the next one)
        const uint32_t Xo = dpp_mov<0x138>(Io) & 0xFFFFu;  // lane 0 reads 0: a batch starts a run
        const uint32_t seen0 = gh0 ? 0u : Xo;
        const uint32_t seen1 = gh1 ? 0u : (seen0 | u0);
        gl0 = a0 && ((seen0 >> c0) & 1u);
        gl1 = a1 && ((seen1 >> c1) & 1u);
      }

      // ---- events of one gate at one timestamp (ties), adjacent in the
      // layout: each sees the state before the first of them (the scan
      // counted the earlier ones, which are inputs: the output code is the
      // highest), and the first, the lowest input pin, charges the leakage
      // change of all their input pins together
      const bool tie0 = a0 && !gh0 && t0 == tp0;
      const bool tie1 = a1 && !gh1 && t1 == t0;
      uint32_t mk0 = 1u << c0, mk1 = 1u << c1;  // input pins switching at the event's timestamp
      const bool ow0 = !tie0, ow1 = !tie1;      // first of its timestamp
      if ((__ballot(tie0 || tie1) | (slowgl ? __ballot(gl0 || gl1) : 0ull)) != 0ull) {
        slk[i0] = lk0;
        slk[i1] = lk1;
        sgh[i0] = (uint8_t)tie0;
        sgh[i1] = (uint8_t)tie1;
        st_sl[wid][i0] = s0;
        st_sl[wid][i1] = s1;
        wave_sync();
        // glitches in runs of three or more events: the pin's previous event
        // in the run (it exists: the glitch's pin has an earlier event in the
        // run).  In pulse trains it is mostly the event just before; for the
        // rest it is the pin's last event before this one, found for every
        // pin left by a max scan of positions.
        if (slowgl) {
          bool need0 = gl0, need1 = gl1;
          int pp0 = 0, pp1 = 0;
          if (need0 && (lkp0 & outc) == c0) {  // (the event before a glitch is in its run)
            pp0 = i0 - 1;
            need0 = false;
          }
          if (need1 && c0 == c1) {
            pp1 = i0;
            need1 = false;
          }
          if ((__ballot(need0) | __ballot(need1)) != 0ull) {
            for (uint32_t c = 0; c <= outc; ++c) {
              if ((__ballot(need0 && c0 == c) | __ballot(need1 && c1 == c)) == 0ull) continue;
              const uint32_t v0 = (a0 && c0 == c) ? (uint32_t)(i0 + 1) : 0u;
              const uint32_t v1 = (a1 && c1 == c) ? (uint32_t)(i1 + 1) : 0u;
              const uint32_t Mx = dpp_mov<0x138>(max_scan(max(v0, v1)));  // last before slot i0
              if (need0 && c0 == c) pp0 = (int)Mx - 1;
              if (need1 && c1 == c) pp1 = (int)max(Mx, v0) - 1;
            }
          }
          if (gl0) {
            tq0 = (slk[pp0] >> pb) & tmask;
            sq0 = st_sl[wid][pp0];
          }
          if (gl1) {
            tq1 = (slk[pp1] >> pb) & tmask;
            sq1 = st_sl[wid][pp1];
          }
        }
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int p = r ? i1 : i0;
          const uint32_t cx = r ? c1 : c0;
          // back over the earlier events of the same timestamp: undo their toggles
          uint32_t corr = 0;
          bool bk = r ? tie1 : tie0;
          for (int y = p - 1; __ballot(bk) != 0ull; --y) {
            if (bk) {
              corr ^= 1u << (slk[y] & outc);
              bk = sgh[y] != 0;
            }
          }
          // forward over the later ones: the input pins switching with this event
          uint32_t mk = 1u << cx;
          bool fw = (r ? (a1 && in1) : (a0 && in0)) && p + 1 < end && sgh[p + 1];
          for (int y = p + 1; __ballot(fw) != 0ull; ++y) {
            if (fw) {
              const uint32_t j = slk[y] & outc;
              if (j != outc) mk |= 1u << j;
              fw = y + 1 < end && sgh[y + 1];
            }
          }
          if (r) { S1s ^= corr; mk1 = mk; } else { S0s ^= corr; mk0 = mk; }
        }
        wave_sync();
      }

      // ---- one event per lane slot: energy, glitch, leakage change, bins
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const bool act = r ? a1 : a0;
        if (!act) continue;
        const uint32_t lk = r ? lk1 : lk0, hw = r ? h1 : h0;
        const uint32_t code = r ? c1 : c0, cyc = r ? y1 : y0, tic = r ? t1 : t0;
        const bool input = r ? in1 : in0;
        const uint4 rec = (r && !same_gate) ? rec1 : rec0;
        const uint32_t info = rec.z;
        const double cap = __hiloint2double((int)rec.y, (int)rec.x);
        const float sl = r ? s1 : s0;
        const uint32_t cell = info & 0xFFFFFFu;
        const uint2 m = meta_of(cell);
        const uint32_t kk = m.x & 15u, lb = m.x >> 4;
        const uint32_t smask = (1u << kk) - 1u;
        const uint32_t Sm = (r ? S1s : S0s) & smask;
        // slew segment on the cell's axis: inner points at or below the slew (Sec. 2.4.1, Fig. 2)
        uint32_t si = 0;
        if constexpr (NIN >= 0) {
          // NIN inner points, fully unrolled
#pragma unroll
          for (int j = 0; j < NIN; j += 4) {
            const float4 th = thr_of(cell, j);
            si += sl >= th.x ? 1u : 0u;
            if (j + 1 < NIN) si += sl >= th.y ? 1u : 0u;
            if (j + 2 < NIN) si += sl >= th.z ? 1u : 0u;
            if (j + 3 < NIN) si += sl >= th.w ? 1u : 0u;
          }
        } else {
          // padding points are +inf and never counted
          for (int j = 0; j < nthr; j += 4) {
            const float4 th = thr_of(cell, j);
            si += (sl >= th.x ? 1u : 0u) + (sl >= th.y ? 1u : 0u) + (sl >= th.z ? 1u : 0u) + (sl >= th.w ? 1u : 0u);
          }
        }
        const double2 aw = axw_of(cell, si);
        const double fa = ((double)sl - aw.x) * aw.y;
        const uint32_t cl = input ? code : 0u;
        const uint32_t lo = __umul24(__umul24(__umul24(Sm, kk) + cl, ns) + si, nc) + (info >> 24);
        double L00, L01, L10, L11;
        if (CELL_LDS && (m.y & kLutLds) != 0u) {
          // an LDS-typed pointer, so the two branches' loads stay ds reads and
          // global loads instead of merging into flat loads
          const lds_f64 *Lp = (const lds_f64 *)(L.lut) + ((m.y & ~kLutLds) + lo);
          L00 = Lp[0], L01 = Lp[1], L10 = Lp[nc], L11 = Lp[nc + 1];
        } else {
          const double *Lp = a.lut + (m.y + lo);
          L00 = Lp[0], L01 = Lp[1], L10 = Lp[nc], L11 = Lp[nc + 1];
        }
        const double2 cx = caxw_of(cell, info >> 24);
        const double fc = (cap - cx.x) * cx.y;  // position on the gate's cap segment (Sec. 2.4.1, Fig. 2)
        const double v0 = L00 + fc * (L01 - L00);
        const double v1 = L10 + fc * (L11 - L10);
        const double Eint = v0 + fa * (v1 - v0);
        const double E = input ? Eint : (((hw >> 8) & 1u) ? a.hv2 * cap : 0.0);  // Eq. 1: 0->1 output events only
        const bool glitch = r ? gl1 : gl0;
        double contrib = E;
        double lk_gate = 0.0;  // leakage of this power change up to t_max (per-gate output)
        double dyn = 0.0;      // this event's dynamic energy after the glitch scale
        if (glitch) {
          const double pw = (double)(tic - (r ? tq1 : tq0));
          const double rr = pw / (0.5 * ((double)sl + (double)(r ? sq1 : sq0)));  // Eq. 2 (reading)
          contrib = (rr > 1.0 ? 1.0 : rr) * E;
          e_gl += contrib;
          ++n_gl;
        } else if (input) {
          e_int += E;
        } else {
          e_sw += E;
        }
        dyn = contrib;
        // leakage power change at this timestamp (owner = lowest switching input pin)
        // (read for every event, so that the reads can start early; output
        // events and later events of a timestamp keep dp = 0)
        const double lk1v = leak_of(lb + (Sm ^ ((r ? mk1 : mk0) & smask))), lk0v = leak_of(lb + Sm);
        {
          const double dp = (input && (r ? ow1 : ow0)) ? lk1v - lk0v : 0.0;
          if (dp != 0.0) {
            // rest of the event's bin (the flush corrects a partial last bin)
            const double part = dp * tick * (double)(T - tic);
            if constexpr (DIAG) {
              if (a.gate_J) {
                lk_gate = dp * tick * (double)(a.t_max - cstart - ((int64_t)cyc * T + tic));
                atomicAdd(a.gate_J + 4 * (size_t)a.gate_perm[(hw >> 10) & gmask] + 3, lk_gate);
              }
            }
            contrib += part;
            e_lk += part;
            atomicAdd(&L.bb[cyc], dp);
          }
        }
        if (contrib != 0.0) atomicAdd(&L.bw[cyc], contrib);
        atomicAdd(&L.bc[cyc], 1ull | ((unsigned long long)glitch << 32));
        if constexpr (DIAG) {
          const uint32_t o = a.orig[base + (r ? i1 : i0)];
          if (a.evt_glitch) a.evt_glitch[o] = glitch ? 1 : 0;
          if (a.evt_state) a.evt_state[o] = (uint8_t)(input ? Sm : 0u);
          // the gate's own energy: internal, switching or glitch (device atomics)
          if (a.gate_J && dyn != 0.0)
            atomicAdd(a.gate_J + 4 * (size_t)a.gate_perm[(hw >> 10) & gmask] + (glitch ? 2 : (input ? 0 : 1)), dyn);
        }
      }
      pos = npos;
    }
  }
  __syncthreads();

  // ---- the block's bins: in-chunk prefix of the leakage changes, then its own slots
  double dsum = 0.0;
  {
    constexpr int PER = (kCCMAX + kNT - 1) / kNT;
    double loc[PER];
    double s = 0.0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid * PER + u;
      loc[u] = (has_range && c < ncyc) ? L.bb[c] : 0.0;
      s += loc[u];
    }
    double incl = s;
    for (int o = 1; o < 64; o <<= 1) {
      const double v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    if (lane == 63) s_scan[wid] = incl;
    __syncthreads();
    double wbase = 0.0;
    for (int w = 0; w < kNW; ++w) {
      const double v = s_scan[w];
      if (w < wid) wbase += v;
      dsum += v;
    }
    double run = wbase + incl - s;
    double *ow = a.blk_wave + (size_t)b * Cc;
    unsigned long long *oc = a.blk_cnt + (size_t)b * Cc;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid * PER + u;
      if (c < Cc) {
        double v = 0.0;
        unsigned long long cn = 0ull;
        if (has_range && c < ncyc) {
          // leakage changes of earlier bins of the chunk; the changes of this
          // bin reach t_max from the bin end on (its own part is in bw)
          const bool partial = last_chunk && c == (int)lastc;
          const double len = partial ? (double)a.last_len : Td;
          v = L.bw[c] + run * len * tick;
          if (partial) {
            const double fix = loc[u] * tick * (Td - (double)a.last_len);
            v -= fix;
            e_lk -= fix;
          } else {
            e_lk += loc[u] * tick * (tail - Td * (double)(c + 1));
          }
          cn = L.bc[c];
          run += loc[u];
        }
        ow[c] = v;
        oc[c] = cn;
      }
    }
  }

  // ---- block totals
  {
    double v[6] = {e_int, e_sw, e_gl, e_lk, 0.0, (double)n_gl};
#pragma unroll
    for (int u = 0; u < 6; ++u) v[u] = wave_sum(v[u]);
    if (lane == 0) {
#pragma unroll
      for (int u = 0; u < 6; ++u) s_red[wid][u] = v[u];
    }
    __syncthreads();
    if (tid < 8) {
      double t = 0.0;
      if (tid < 5) {
        for (int w = 0; w < kNW; ++w) t += s_red[w][tid];
      } else if (tid == 5) {
        t = dsum;
      } else if (tid == 6) {
        for (int w = 0; w < kNW; ++w) t += s_red[w][5];
      }
      a.blk_part[(size_t)b * 8 + tid] = t;
    }
  }
}

// One wave per block range: the cuts between the block's waves, moved to window heads.
__global__ __launch_bounds__(64) void k_wave_bounds(const uint64_t *key, int64_t E, const uint32_t *rstart,
                                                     int32_t *wb) {
  const int64_t r0 = rstart[blockIdx.x], r1 = rstart[blockIdx.x + 1];
  for (int w = 0; w <= kNW; ++w) {
    const int h = find_head(key, E, r0 + (r1 - r0) * w / kNW);
    if (threadIdx.x == 0) wb[(size_t)blockIdx.x * (kNW + 1) + w] = h;
  }
}

// One wave per block range: 64 events sampled at the midpoints of 64 equal
// slices of the range give the cells present (nondecreasing, since gates
// are numbered in cell order) and each cell's share; the heaviest cells whose
// LUTs still fit in `budget` doubles are taken, heaviest first.
__global__ __launch_bounds__(64) void k_lut_plan(const uint64_t *key, const int32_t *wb, const uint4 *gate_rec,
                                                 const uint2 *cell_meta, uint32_t gb, int ns, int nc,
                                                 uint32_t budget, uint2 *plan) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int r0 = wb[(size_t)b * (kNW + 1)], r1 = wb[(size_t)b * (kNW + 1) + kNW];
  const uint32_t gmask = (1u << gb) - 1u;
  uint32_t cell = ~0u;
  if (r1 > r0) {
    const int p = r0 + (int)((int64_t)(r1 - r0) * (2 * lane + 1) / 128);
    const uint32_t g = (uint32_t)(key[p] >> (32 + 10)) & gmask;
    cell = gate_rec[g].z & 0xFFFFFFu;
  }
  const uint32_t prev = __shfl_up(cell, 1);
  const bool start = cell != ~0u && (lane == 0 || prev != cell);
  const unsigned long long st = __ballot(start);
  uint32_t len = 0, sz = 0;
  if (start) {
    const unsigned long long after = lane < 63 ? (st >> (lane + 1)) << (lane + 1) : 0ull;
    len = (after ? (uint32_t)(__ffsll((long long)after) - 1) : 64u) - (uint32_t)lane;
    const uint32_t k = cell_meta[cell].x & 15u;
    sz = ((1u << k) * k) * (uint32_t)(ns * nc);
  }
  bool cand = start && sz <= budget;
  uint32_t used = 0;
  int ne = 0;
  while (ne < kPlan) {
    uint32_t v = cand ? (len << 6 | (63u - (uint32_t)lane)) : 0u;
    for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
    if (v == 0u) break;
    const int bl = 63 - (int)(v & 63u);
    const uint32_t bsz = (uint32_t)__shfl((int)sz, bl), bcell = (uint32_t)__shfl((int)cell, bl);
    if (lane == bl) cand = false;
    if (used + bsz <= budget) {
      if (lane == 0) plan[(size_t)b * kPlan + ne] = make_uint2(bcell, used);
      used += bsz;
      ++ne;
    }
  }
  if (lane >= ne && lane < kPlan) plan[(size_t)b * kPlan + lane] = make_uint2(~0u, 0u);
}

constexpr int kFC = 64;             // finalize: cycles per block (one per lane)
constexpr int kFP = 8;              // finalize: waves per block, each adding up a share of the blocks
constexpr int kFT = kFC * kFP;

// Lane l of wave p adds up, for cycle l of the block's 64, the bins of the
// p-th share of the cycle's chunk's blocks; the waves also share the sums over
// all blocks' totals.  Wave 0 then adds the shares in order after the leakage
// carried into the chunk (L0 plus the changes of earlier chunks); block 0 also
// writes the totals (Eq. 3).  Every sum runs in a fixed order, and every loop
// keeps eight independent loads in flight.
__global__ __launch_bounds__(kFT) void k_finalize(FinalArgs f) {
  __shared__ double s_w[kFP][kFC];
  __shared__ unsigned long long s_n[kFP][kFC];
  __shared__ double s_t[kFP][8];
  const int lane = threadIdx.x & 63, wp = threadIdx.x >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * kFC;
  const int64_t chi = min(c0 + kFC, f.C) - 1;
  const int64_t c = c0 + lane;
  const int qa = (int)(c0 / f.Cc), qb = (int)(chi / f.Cc);
  const int q = (int)(min(c, chi) / f.Cc);
  const uint32_t ba = f.chunk_blk[qa];
  const bool totals = blockIdx.x == 0;
  {
    // this wave's share of the cycle's chunk's blocks
    const uint32_t b0 = f.chunk_blk[q], b1 = f.chunk_blk[q + 1];
    const uint32_t n = b1 - b0, s0 = b0 + n * wp / kFP, s1 = b0 + n * (wp + 1) / kFP;
    const int cin = (int)(min(c, chi) - (int64_t)q * f.Cc);
    double w = 0.0;
    unsigned long long cnt = 0;
    for (uint32_t bb = s0; bb < s1; bb += 8) {
      double v[8];
      unsigned long long m[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool ok = bb + u < s1;
        v[u] = ok ? f.blk_wave[(size_t)(bb + u) * f.Cc + cin] : 0.0;
        m[u] = ok ? f.blk_cnt[(size_t)(bb + u) * f.Cc + cin] : 0ull;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        w += v[u];
        cnt += m[u];
      }
    }
    s_w[wp][lane] = w;
    s_n[wp][lane] = cnt;
    // this wave's share of the blocks' totals: L0, the changes before chunk qa, and (block 0) the energies
    double t[7] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    for (int b8 = wp * 64 * 8; b8 < f.grid; b8 += kFT * 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int bb = b8 + u * 64 + lane;
        if (bb < f.grid) {
          const double *pp = f.blk_part + (size_t)bb * 8;
          if ((uint32_t)bb < ba) t[1] += pp[5];
          if (totals) {
            t[2] += pp[0];
            t[3] += pp[1];
            t[4] += pp[2];
            t[5] += pp[3];
            t[6] += pp[6];
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 7; ++u) t[u] = wave_sum(t[u]);
    if (lane == 0) {
#pragma unroll
      for (int u = 0; u < 7; ++u) s_t[wp][u] = t[u];
    }
  }
  __syncthreads();
  if (wp != 0) return;
  const double l0 = *f.l0;
  double pre = 0.0;
#pragma unroll
  for (int p = 0; p < kFP; ++p) pre += s_t[p][1];
  // the changes inside chunks qa .. qb-1 (qb - qa < 64), then their exclusive prefix
  double dq = 0.0;
  if (lane < qb - qa) {
    const uint32_t b0 = f.chunk_blk[qa + lane], b1 = f.chunk_blk[qa + lane + 1];
    for (uint32_t bb = b0; bb < b1; ++bb) dq += f.blk_part[(size_t)bb * 8 + 5];
  }
  double incl = dq;
  for (int o = 1; o < 64; o <<= 1) {
    const double v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  const double Pj = l0 + pre + (incl - dq);  // power carried into chunk qa + lane
  const double Pq = __shfl(Pj, q - qa, 64);
  if (c < f.C) {
    const double len = (c == f.C - 1) ? (double)f.last_len : (double)f.T;
    double w = Pq * len * f.tick_s;
    unsigned long long cnt = 0;
#pragma unroll
    for (int p = 0; p < kFP; ++p) {
      w += s_w[p][lane];
      cnt += s_n[p][lane];
    }
    f.wave_out[c] = w;
    f.cyc_events[c] = cnt & 0xFFFFFFFFull;
    f.cyc_glitches[c] = cnt >> 32;
  }
  if (totals && lane == 0) {
    double t[5] = {0.0, 0.0, 0.0, 0.0, 0.0};
    for (int p = 0; p < kFP; ++p)
      for (int u = 0; u < 5; ++u) t[u] += s_t[p][2 + u];
    const double window = (double)f.t_max * f.tick_s;
    const double e_leak = l0 * window + t[3];
    f.res[0] = t[0];
    f.res[1] = t[1];
    f.res[2] = t[2];
    f.res[3] = e_leak;
    f.res[4] = t[0] / window;  // Eq. 3
    f.res[5] = t[1] / window;
    f.res[6] = t[2] / window;
    f.res[7] = e_leak / window;
    f.res[8] = t[4];
  }
}

}  // namespace

int pass_block_threads() { return kNT; }
int pass_blocks_per_cu() { return kBPC; }
size_t pass_static_lds_bytes() {
  return (size_t)kNW * kB * (sizeof(uint32_t) + sizeof(uint8_t) + sizeof(float)) + (size_t)kNW * 9 * sizeof(double);
}
int pass_wave_bounds_per_block() { return kNW + 1; }

hipError_t launch_wave_bounds(const uint64_t *key, int64_t E, const uint32_t *rstart, int32_t n_ranges, int32_t *wb,
                              hipStream_t s) {
  if (n_ranges <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_wave_bounds, dim3(n_ranges), dim3(64), 0, s, key, E, rstart, wb);
  return hipGetLastError();
}
hipError_t launch_lut_plan(const uint64_t *key, const int32_t *wb, int32_t n_ranges, const uint4 *gate_rec,
                           const uint2 *cell_meta, uint32_t gb, int n_slew, int n_cap, int32_t lut_lds, uint2 *plan,
                           hipStream_t s) {
  if (n_ranges <= 0 || lut_lds <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_lut_plan, dim3(n_ranges), dim3(64), 0, s, key, wb, gate_rec, cell_meta, gb, n_slew, n_cap,
                     (uint32_t)lut_lds, plan);
  return hipGetLastError();
}
int pass_lut_plan_slots() { return kPlan; }
int pass_wave_batch() { return kB; }
int pass_max_chunk_cycles() { return kCCMAX; }

size_t pass_lds_bytes(int Cc, int n_cells, int n_slew, int n_cap, int n_thr, int64_t n_leak, bool cells) {
  return 24 * (size_t)Cc + (cells ? cell_bytes(n_cells, n_slew, n_cap, n_thr, n_leak) : 0);
}

bool pass_cells_fit_lds(int Cc, int n_cells, int n_slew, int n_cap, int n_thr, int64_t n_leak) {
  return pass_lds_bytes(Cc, n_cells, n_slew, n_cap, n_thr, n_leak, true) + pass_static_lds_bytes() <= kLdsMax;
}

static size_t lut_lds_offset(int Cc, int n_cells, int n_slew, int n_cap, int n_thr, int64_t n_leak) {
  return (pass_lds_bytes(Cc, n_cells, n_slew, n_cap, n_thr, n_leak, true) + 15) & ~size_t(15);
}

int32_t pass_lut_lds_doubles(int Cc, int n_cells, int n_slew, int n_cap, int n_thr, int64_t n_leak) {
  if (!pass_cells_fit_lds(Cc, n_cells, n_slew, n_cap, n_thr, n_leak)) return 0;
  const size_t used = lut_lds_offset(Cc, n_cells, n_slew, n_cap, n_thr, n_leak) + pass_static_lds_bytes();
  return used < kLdsMax ? (int32_t)((kLdsMax - used) / 16 * 2) : 0;
}

hipError_t launch_pass(const PassArgs &a, int grid_blocks, hipStream_t s) {
  const bool cells = pass_cells_fit_lds(a.Cc, a.n_cells, a.n_slew, a.n_cap, a.n_thr, a.n_leak);
  const bool diag = a.evt_glitch || a.evt_state || a.gate_J;
  size_t dyn = pass_lds_bytes(a.Cc, a.n_cells, a.n_slew, a.n_cap, a.n_thr, a.n_leak, cells);
  if (cells && a.lut_lds > 0) {
    if (!a.lut_plan) return hipErrorInvalidValue;
    dyn = lut_lds_offset(a.Cc, a.n_cells, a.n_slew, a.n_cap, a.n_thr, a.n_leak) + 8 * (size_t)a.lut_lds;
  }
  if (dyn + pass_static_lds_bytes() > kLdsMax) return hipErrorInvalidValue;
  const dim3 g(grid_blocks), t(kNT);
  if (cells && !diag) {
    if (a.n_slew == 7) hipLaunchKernelGGL((k_fused<true, false, 5>), g, t, dyn, s, a);
    else if (a.n_slew == 8) hipLaunchKernelGGL((k_fused<true, false, 6>), g, t, dyn, s, a);
    else hipLaunchKernelGGL((k_fused<true, false, -1>), g, t, dyn, s, a);
  } else if (cells) {
    hipLaunchKernelGGL((k_fused<true, true, -1>), g, t, dyn, s, a);
  } else if (!diag) {
    hipLaunchKernelGGL((k_fused<false, false, -1>), g, t, dyn, s, a);
  } else {
    hipLaunchKernelGGL((k_fused<false, true, -1>), g, t, dyn, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_finalize(const FinalArgs &f, hipStream_t s) {
  const int grid = (int)((f.C + kFC - 1) / kFC);
  hipLaunchKernelGGL(k_finalize, dim3(grid), dim3(kFT), 0, s, f);
  return hipGetLastError();
}

}  // namespace pa
