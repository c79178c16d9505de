// pa_load.hip -- load-time kernels: design tables and the event layout.
//
// The design load derives per-gate constants once: the segment and fraction
// of the gate's output load on its cell's cap axis (the load side of the
// bilinear NLDM lookup of "GPU-Accelerated Gate-Level Time-Based Power
// Analysis via Event-Density-Aware Partitioning and Kernel Fusion",
// Sec. 2.4.1) and the switching energy 0.5 c Vdd^2 of its output (Eq. 1).
//
// The event load validates the per-pin streams (sorted, alternating values,
// inside the window, positive slews) and lays them out chunk-major: time is
// cut into chunks of Cc clock cycles, every gate's chunk into density-aware
// windows, and inside a (chunk, gate, window) segment the events are ordered
// by pin and time.  Every segment is one contiguous run of packed keys that
// also carry the gate's input state at the window start (the state
// reconstruction at a window start of Sec. 2.4.2, from per-pin event-count
// parities).  Windows start on cycle boundaries, so the per-pin glitch
// counter never crosses one.
#include <hip/hip_runtime.h>

#include <hipcub/hipcub.hpp>

#include "pa_common.h"
#include "pa_load.h"

namespace pa {
namespace {

constexpr int kLT = 256;

inline int grid_for(int64_t n) {
  int64_t g = (n + kLT - 1) / kLT;
  if (g < 1) g = 1;
  if (g > 65535 * 16) g = 65535 * 16;
  return (int)g;
}

// ------------------------------------------------------------------ design

__global__ void k_gate_tables(int64_t G, const int32_t *gate_cell, const double *gate_cap, int32_t n_cells,
                              const int32_t *cell_k, const double *cap_axis, int32_t n_cap, double vdd,
                              uint32_t *gate_info, double *capfrac, double *esw, int32_t *gate_k, uint32_t *err) {
  for (int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; g < G; g += (int64_t)gridDim.x * blockDim.x) {
    const int32_t cell = gate_cell[g];
    const double cap = gate_cap[g];
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
    capfrac[g] = (cap - ca[seg]) / (ca[seg + 1] - ca[seg]);
    esw[g] = 0.5 * cap * vdd * vdd;
    gate_k[g] = cell_k[cell];
  }
}

// pin -> (gate, local index) from the gate pin bases
__global__ void k_pin_owner(int64_t G, const int64_t *pin_base, int32_t *pin_gate, uint8_t *pin_local) {
  for (int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; g < G; g += (int64_t)gridDim.x * blockDim.x) {
    const int64_t p0 = pin_base[g], p1 = pin_base[g + 1];
    for (int64_t p = p0; p < p1; ++p) {
      pin_gate[p] = (int32_t)g;
      pin_local[p] = (uint8_t)(p - p0);
    }
  }
}

// ------------------------------------------------------------------ events

__global__ void k_pin_check(int64_t P, const int64_t *pin_ptr, const uint8_t *pin_init, uint32_t *err) {
  for (int64_t p = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; p < P; p += (int64_t)gridDim.x * blockDim.x) {
    if (pin_ptr[p + 1] < pin_ptr[p]) atomicOr(err, ERR_PIN_PTR);
    if (pin_init[p] > 1) atomicOr(err, ERR_INIT);
  }
}

// owning pin of every event (last p with pin_ptr[p] <= e) and validation
__global__ void k_event_check(int64_t E, int64_t P, const int64_t *pin_ptr, const uint8_t *pin_init,
                              const int64_t *evt_t, const uint8_t *evt_val, const float *evt_slew, int64_t t_max,
                              uint32_t *ev_pin, uint32_t *err) {
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < E; e += (int64_t)gridDim.x * blockDim.x) {
    int64_t lo = 0, hi = P;  // pin_ptr[lo] <= e < pin_ptr[hi]
    while (hi - lo > 1) {
      const int64_t mid = (lo + hi) >> 1;
      if (pin_ptr[mid] <= e) lo = mid; else hi = mid;
    }
    ev_pin[e] = (uint32_t)lo;
    const int64_t idx = e - pin_ptr[lo];
    const int64_t t = evt_t[e];
    uint32_t bad = 0;
    if (t < 0 || t >= t_max) bad |= ERR_TIME_RANGE;
    if (idx > 0 && !(t > evt_t[e - 1])) bad |= ERR_TIME_ORDER;
    const uint8_t init = pin_init[lo] & 1u;
    if (evt_val[e] != (uint8_t)(init ^ ((idx + 1) & 1))) bad |= ERR_VALUE;
    const float s = evt_slew[e];
    if (!(s > 0.0f) || !isfinite(s)) bad |= ERR_SLEW;
    if (bad) atomicOr(err, bad);
  }
}

// ---- density-aware windows (paper Sec. 3, event-density-aware per-gate
// cycle partitioning): a gate of density rho = N_evt / N_cyc gets windows of
// about n_evt_tgt / rho cycles; here the window length is Cc / 2^s, the
// smallest s with rho * Cc / 2^s <= target (the density floor is the chunk
// itself), refined below until no window holds more than kSegMax events.
__global__ void k_gate_levels(int64_t G, const int64_t *pin_base, const int64_t *pin_ptr, int64_t C, int32_t Cc,
                              int32_t lc, double target, uint8_t *level) {
  for (int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; g < G; g += (int64_t)gridDim.x * blockDim.x) {
    const double n_evt = (double)(pin_ptr[pin_base[g + 1]] - pin_ptr[pin_base[g]]);
    const double rho = n_evt / (double)C;
    int sl = 0;
    while (sl < lc && rho * (double)(Cc >> sl) > target) ++sl;
    level[g] = (uint8_t)sl;
  }
}

// (k + 1) << level: (window, pin) pairs of a gate in one chunk
__global__ void k_pw_len(int64_t G, const int32_t *gate_k, const uint8_t *level, int64_t *pw_len) {
  for (int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; g < G; g += (int64_t)gridDim.x * blockDim.x)
    pw_len[g] = (int64_t)(gate_k[g] + 1) << level[g];
}

struct WinIdx {
  int64_t pair;  // (chunk, gate, window, pin) pair of the event
  int64_t base;  // pair of (chunk, gate, window, pin 0)
  int64_t q;
};

__device__ __forceinline__ WinIdx win_index(int64_t t, int64_t T, int32_t lc, int32_t sl, int64_t PW, int64_t pwb,
                                            int32_t k, int32_t i) {
  const int64_t cyc = t / T;
  const int64_t q = cyc >> lc;
  const int64_t cin = cyc & (((int64_t)1 << lc) - 1);
  const int64_t w = cin >> (lc - sl);
  WinIdx r;
  r.q = q;
  r.base = q * PW + pwb + w * (k + 1);
  r.pair = r.base + i;
  return r;
}

__global__ void k_count_w(int64_t E, const int64_t *evt_t, const uint32_t *ev_pin, const int32_t *pin_gate,
                          const uint8_t *pin_local, const int32_t *gate_k, const uint8_t *level,
                          const int64_t *pwbase, int64_t PW, int64_t T, int32_t lc, uint32_t *cnt) {
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < E; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t p = ev_pin[e];
    const int32_t g = pin_gate[p];
    const WinIdx wi = win_index(evt_t[e], T, lc, level[g], PW, pwbase[g], gate_k[g], pin_local[p]);
    atomicAdd(&cnt[wi.pair], 1u);
  }
}

// flags bit 0: some window exceeds kSegMax and its gate can be refined;
// bit 1: a one-cycle window exceeds kSegMax (cannot be refined)
__global__ void k_winmax(int64_t G, int32_t Q, const int32_t *gate_k, const uint8_t *level, const int64_t *pwbase,
                         int64_t PW, int32_t lc, const uint32_t *cnt, uint8_t *level_next, uint32_t *flags,
                         uint32_t *max_seg) {
  const int64_t n = G * (int64_t)Q;
  for (int64_t u = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; u < n; u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t q = u / G, g = u - q * G;
    const int32_t np = gate_k[g] + 1, sl = level[g];
    const int64_t b0 = q * PW + pwbase[g];
    uint32_t mx = 0;
    for (int64_t w = 0; w < ((int64_t)1 << sl); ++w) {
      uint32_t sum = 0;
      for (int32_t i = 0; i < np; ++i) sum += cnt[b0 + w * np + i];
      mx = sum > mx ? sum : mx;
    }
    atomicMax(max_seg, mx);
    if (mx > (uint32_t)kSegMax) {
      if (sl < lc) {
        atomicOr(flags, 1u);
        level_next[g] = (uint8_t)(sl + 1);  // every writer stores the same value
      } else {
        atomicOr(flags, 2u);
      }
    }
  }
}

// per pin, walking its (chunk, window) pairs in time order: the caller's index
// of its first event in each window and its value at each window start
__global__ void k_pin_windows(int64_t P, int32_t Q, const int64_t *pin_ptr, const uint8_t *pin_init,
                              const int32_t *pin_gate, const uint8_t *pin_local, const int32_t *gate_k,
                              const uint8_t *level, const int64_t *pwbase, int64_t PW, const uint32_t *cnt,
                              uint32_t *first, uint8_t *vstart) {
  for (int64_t p = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; p < P; p += (int64_t)gridDim.x * blockDim.x) {
    const int32_t g = pin_gate[p];
    const int32_t np = gate_k[g] + 1, i = pin_local[p];
    const int64_t nw = (int64_t)1 << level[g];
    uint32_t run = (uint32_t)pin_ptr[p];
    uint8_t v = pin_init[p] & 1u;
    for (int32_t q = 0; q < Q; ++q) {
      const int64_t b0 = (int64_t)q * PW + pwbase[g] + i;
      for (int64_t w = 0; w < nw; ++w) {
        const int64_t pr = b0 + w * np;
        const uint32_t c = cnt[pr];
        first[pr] = run;
        vstart[pr] = v;
        run += c;
        v ^= (uint8_t)(c & 1u);
      }
    }
  }
}

__global__ void k_scatter_w(int64_t E, const int64_t *evt_t, const float *evt_slew, const uint8_t *evt_val,
                            const uint32_t *ev_pin, const int32_t *pin_gate, const uint8_t *pin_local,
                            const int32_t *gate_k, const uint8_t *level, const int64_t *pwbase, int64_t PW, int64_t T,
                            int32_t lc, int64_t chunk_ticks, const uint32_t *first, const uint32_t *off,
                            const uint8_t *vstart, KeyFmt kf, uint64_t *key_out, float *slew_out, uint32_t *orig_out) {
  const uint32_t outc = out_code(kf.p_bits);
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < E; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t p = ev_pin[e];
    const int32_t g = pin_gate[p];
    const int32_t k = gate_k[g], i = pin_local[p];
    const int64_t t = evt_t[e];
    const WinIdx wi = win_index(t, T, lc, level[g], PW, pwbase[g], k, i);
    const int64_t dest = (int64_t)off[wi.pair] + (e - (int64_t)first[wi.pair]);
    uint32_t S0 = 0;
    for (int32_t j = 0; j < k; ++j) S0 |= uint32_t(vstart[wi.base + j]) << j;
    const uint64_t head = dest == (int64_t)off[wi.base] ? 1u : 0u;
    const uint64_t code = i == k ? outc : (uint32_t)i;
    const uint64_t trel = (uint64_t)(t - wi.q * chunk_ticks);
    const uint64_t lk = (code << kf.t_bits) | trel;
    key_out[dest] = ((uint64_t)g << kKeyGateShift) | (head << kKeyHeadShift) | (lk << kKeyLkShift) |
                    ((uint64_t)(evt_val[e] & 1u) << kKeyValShift) | (uint64_t)S0;
    slew_out[dest] = evt_slew[e];
    orig_out[dest] = (uint32_t)e;
  }
}

__global__ void k_chunk_base_w(int32_t Q, int64_t PW, const uint32_t *off, uint32_t *cb) {
  for (int32_t q = blockIdx.x * blockDim.x + threadIdx.x; q <= Q; q += gridDim.x * blockDim.x)
    cb[q] = off[(int64_t)q * PW];
}

}  // namespace

// ------------------------------------------------------------- launchers

hipError_t launch_gate_tables(int64_t G, const int32_t *gate_cell, const double *gate_cap, int32_t n_cells,
                              const int32_t *cell_k, const double *cap_axis, int32_t n_cap, double vdd,
                              uint32_t *gate_info, double *capfrac, double *esw, int32_t *gate_k, uint32_t *err,
                              hipStream_t s) {
  hipLaunchKernelGGL(k_gate_tables, dim3(grid_for(G)), dim3(kLT), 0, s, G, gate_cell, gate_cap, n_cells, cell_k,
                     cap_axis, n_cap, vdd, gate_info, capfrac, esw, gate_k, err);
  return hipGetLastError();
}

hipError_t launch_pin_owner(int64_t G, const int64_t *pin_base, int32_t *pin_gate, uint8_t *pin_local,
                            hipStream_t s) {
  hipLaunchKernelGGL(k_pin_owner, dim3(grid_for(G)), dim3(kLT), 0, s, G, pin_base, pin_gate, pin_local);
  return hipGetLastError();
}

hipError_t launch_pin_check(int64_t P, const int64_t *pin_ptr, const uint8_t *pin_init, uint32_t *err,
                            hipStream_t s) {
  hipLaunchKernelGGL(k_pin_check, dim3(grid_for(P)), dim3(kLT), 0, s, P, pin_ptr, pin_init, err);
  return hipGetLastError();
}

hipError_t launch_event_check(int64_t E, int64_t P, const int64_t *pin_ptr, const uint8_t *pin_init,
                              const int64_t *evt_t, const uint8_t *evt_val, const float *evt_slew, int64_t t_max,
                              uint32_t *ev_pin, uint32_t *err, hipStream_t s) {
  hipLaunchKernelGGL(k_event_check, dim3(grid_for(E)), dim3(kLT), 0, s, E, P, pin_ptr, pin_init, evt_t, evt_val,
                     evt_slew, t_max, ev_pin, err);
  return hipGetLastError();
}

hipError_t launch_gate_levels(int64_t G, const int64_t *pin_base, const int64_t *pin_ptr, int64_t C, int32_t Cc,
                              int32_t lc, double target, uint8_t *level, hipStream_t s) {
  hipLaunchKernelGGL(k_gate_levels, dim3(grid_for(G)), dim3(kLT), 0, s, G, pin_base, pin_ptr, C, Cc, lc, target, level);
  return hipGetLastError();
}

hipError_t launch_pw_len(int64_t G, const int32_t *gate_k, const uint8_t *level, int64_t *pw_len, hipStream_t s) {
  hipLaunchKernelGGL(k_pw_len, dim3(grid_for(G)), dim3(kLT), 0, s, G, gate_k, level, pw_len);
  return hipGetLastError();
}

hipError_t launch_count_w(int64_t E, const int64_t *evt_t, const uint32_t *ev_pin, const int32_t *pin_gate,
                          const uint8_t *pin_local, const int32_t *gate_k, const uint8_t *level,
                          const int64_t *pwbase, int64_t PW, int64_t T, int32_t lc, uint32_t *cnt, hipStream_t s) {
  hipLaunchKernelGGL(k_count_w, dim3(grid_for(E)), dim3(kLT), 0, s, E, evt_t, ev_pin, pin_gate, pin_local, gate_k,
                     level, pwbase, PW, T, lc, cnt);
  return hipGetLastError();
}

hipError_t launch_winmax(int64_t G, int32_t Q, const int32_t *gate_k, const uint8_t *level, const int64_t *pwbase,
                         int64_t PW, int32_t lc, const uint32_t *cnt, uint8_t *level_next, uint32_t *flags,
                         uint32_t *max_seg, hipStream_t s) {
  hipLaunchKernelGGL(k_winmax, dim3(grid_for(G * (int64_t)Q)), dim3(kLT), 0, s, G, Q, gate_k, level, pwbase, PW, lc,
                     cnt, level_next, flags, max_seg);
  return hipGetLastError();
}

hipError_t launch_pin_windows(int64_t P, int32_t Q, const int64_t *pin_ptr, const uint8_t *pin_init,
                              const int32_t *pin_gate, const uint8_t *pin_local, const int32_t *gate_k,
                              const uint8_t *level, const int64_t *pwbase, int64_t PW, const uint32_t *cnt,
                              uint32_t *first, uint8_t *vstart, hipStream_t s) {
  hipLaunchKernelGGL(k_pin_windows, dim3(grid_for(P)), dim3(kLT), 0, s, P, Q, pin_ptr, pin_init, pin_gate, pin_local,
                     gate_k, level, pwbase, PW, cnt, first, vstart);
  return hipGetLastError();
}

hipError_t launch_scatter_w(int64_t E, const int64_t *evt_t, const float *evt_slew, const uint8_t *evt_val,
                            const uint32_t *ev_pin, const int32_t *pin_gate, const uint8_t *pin_local,
                            const int32_t *gate_k, const uint8_t *level, const int64_t *pwbase, int64_t PW, int64_t T,
                            int32_t lc, int64_t chunk_ticks, const uint32_t *first, const uint32_t *off,
                            const uint8_t *vstart, const KeyFmt &kf, uint64_t *key_out, float *slew_out,
                            uint32_t *orig_out, hipStream_t s) {
  hipLaunchKernelGGL(k_scatter_w, dim3(grid_for(E)), dim3(kLT), 0, s, E, evt_t, evt_slew, evt_val, ev_pin, pin_gate,
                     pin_local, gate_k, level, pwbase, PW, T, lc, chunk_ticks, first, off, vstart, kf, key_out,
                     slew_out, orig_out);
  return hipGetLastError();
}

hipError_t launch_chunk_base_w(int32_t Q, int64_t PW, const uint32_t *off, uint32_t *cb, hipStream_t s) {
  hipLaunchKernelGGL(k_chunk_base_w, dim3(grid_for(Q + 1)), dim3(kLT), 0, s, Q, PW, off, cb);
  return hipGetLastError();
}

hipError_t scan_exclusive_u32(const uint32_t *in, uint32_t *out, int64_t n, void *tmp, size_t *tmp_bytes,
                              hipStream_t s) {
  return hipcub::DeviceScan::ExclusiveSum(tmp, *tmp_bytes, in, out, (size_t)n, s);
}

hipError_t scan_exclusive_i64(const int64_t *in, int64_t *out, int64_t n, void *tmp, size_t *tmp_bytes,
                              hipStream_t s) {
  return hipcub::DeviceScan::ExclusiveSum(tmp, *tmp_bytes, in, out, (size_t)n, s);
}

}  // namespace pa
