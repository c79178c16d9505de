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
// cut into chunks of Cc clock cycles, and inside a chunk the events are
// ordered by gate, pin and time.  Every (chunk, gate) segment is then one
// contiguous run of packed keys that also carry the gate's input state at the
// chunk start (the state reconstruction at a window start of Sec. 2.4.2,
// computed once from per-pin event-count parities).  Chunks start on cycle
// boundaries, so the per-pin glitch counter never crosses a chunk.
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

__global__ void k_count(int64_t E, int64_t P, const int64_t *evt_t, const uint32_t *ev_pin, int64_t chunk_ticks,
                        uint32_t *cnt) {
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < E; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t q = evt_t[e] / chunk_ticks;
    atomicAdd(&cnt[q * P + ev_pin[e]], 1u);
  }
}

// largest (chunk, gate) segment
__global__ void k_segmax(int64_t G, int64_t P, int32_t Q, const int64_t *pin_base, const uint32_t *cnt,
                         uint32_t *mx) {
  const int64_t n = G * (int64_t)Q;
  for (int64_t u = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; u < n; u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t q = u / G, g = u - q * G;
    uint32_t s = 0;
    for (int64_t p = pin_base[g]; p < pin_base[g + 1]; ++p) s += cnt[q * P + p];
    atomicMax(mx, s);
  }
}

// per pin, walking the chunks in order: the caller's index of its first event
// in each chunk and its value at each chunk start
__global__ void k_pin_chunks(int64_t P, int32_t Q, const int64_t *pin_ptr, const uint8_t *pin_init,
                             const uint32_t *cnt, uint32_t *first, uint8_t *pinval) {
  for (int64_t p = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; p < P; p += (int64_t)gridDim.x * blockDim.x) {
    uint32_t run = (uint32_t)pin_ptr[p];
    uint8_t v = pin_init[p] & 1u;
    for (int32_t q = 0; q < Q; ++q) {
      const uint32_t c = cnt[(int64_t)q * P + p];
      first[(int64_t)q * P + p] = run;
      pinval[(int64_t)q * P + p] = v;
      run += c;
      v ^= (uint8_t)(c & 1u);
    }
  }
}

// input-pin state of every gate at every chunk start
__global__ void k_seg_state(int64_t G, int64_t P, int32_t Q, const int64_t *pin_base, const int32_t *gate_k,
                            const uint8_t *pinval, uint8_t *st) {
  const int64_t n = G * (int64_t)Q;
  for (int64_t u = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; u < n; u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t q = u / G, g = u - q * G;
    const int64_t p0 = pin_base[g];
    uint32_t S = 0;
    for (int j = 0; j < gate_k[g]; ++j) S |= uint32_t(pinval[q * P + p0 + j]) << j;
    st[u] = (uint8_t)S;
  }
}

__global__ void k_scatter(int64_t E, int64_t P, int64_t G, const int64_t *evt_t, const float *evt_slew,
                          const uint8_t *evt_val, const uint32_t *ev_pin, const int32_t *pin_gate,
                          const uint8_t *pin_local, int64_t chunk_ticks, const uint32_t *first,
                          const uint32_t *pin_off, const uint8_t *st, KeyFmt kf, uint64_t *key_out,
                          float *slew_out, uint32_t *orig_out) {
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < E; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t p = ev_pin[e];
    const int64_t g = pin_gate[p];
    const uint64_t i = pin_local[p];
    const int64_t t = evt_t[e];
    const int64_t q = t / chunk_ticks;
    const uint64_t trel = (uint64_t)(t - q * chunk_ticks);
    const int64_t qp = q * P + p;
    const int64_t dest = (int64_t)pin_off[qp] + (e - (int64_t)first[qp]);
    const uint64_t lk = (i << kf.t_bits) | trel;
    const uint64_t k = ((uint64_t)g << kKeyGateShift) | (lk << kKeyLkShift) |
                       ((uint64_t)(evt_val[e] & 1u) << kKeyValShift) | (uint64_t)st[q * G + g];
    key_out[dest] = k;
    slew_out[dest] = evt_slew[e];
    orig_out[dest] = (uint32_t)e;
  }
}

__global__ void k_chunk_base(int32_t Q, int64_t P, int64_t E, const uint32_t *pin_off, uint32_t *cb) {
  for (int32_t q = blockIdx.x * blockDim.x + threadIdx.x; q <= Q; q += gridDim.x * blockDim.x)
    cb[q] = q < Q ? pin_off[(int64_t)q * P] : (uint32_t)E;
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

hipError_t launch_count(int64_t E, int64_t P, const int64_t *evt_t, const uint32_t *ev_pin, int64_t chunk_ticks,
                        uint32_t *cnt, hipStream_t s) {
  hipLaunchKernelGGL(k_count, dim3(grid_for(E)), dim3(kLT), 0, s, E, P, evt_t, ev_pin, chunk_ticks, cnt);
  return hipGetLastError();
}

hipError_t launch_segmax(int64_t G, int64_t P, int32_t Q, const int64_t *pin_base, const uint32_t *cnt,
                         uint32_t *mx, hipStream_t s) {
  hipLaunchKernelGGL(k_segmax, dim3(grid_for(G * (int64_t)Q)), dim3(kLT), 0, s, G, P, Q, pin_base, cnt, mx);
  return hipGetLastError();
}

hipError_t launch_pin_chunks(int64_t P, int32_t Q, const int64_t *pin_ptr, const uint8_t *pin_init,
                             const uint32_t *cnt, uint32_t *first, uint8_t *pinval, hipStream_t s) {
  hipLaunchKernelGGL(k_pin_chunks, dim3(grid_for(P)), dim3(kLT), 0, s, P, Q, pin_ptr, pin_init, cnt, first, pinval);
  return hipGetLastError();
}

hipError_t launch_seg_state(int64_t G, int64_t P, int32_t Q, const int64_t *pin_base, const int32_t *gate_k,
                            const uint8_t *pinval, uint8_t *st, hipStream_t s) {
  hipLaunchKernelGGL(k_seg_state, dim3(grid_for(G * (int64_t)Q)), dim3(kLT), 0, s, G, P, Q, pin_base, gate_k,
                     pinval, st);
  return hipGetLastError();
}

hipError_t launch_scatter(int64_t E, int64_t P, int64_t G, const int64_t *evt_t, const float *evt_slew,
                          const uint8_t *evt_val, const uint32_t *ev_pin, const int32_t *pin_gate,
                          const uint8_t *pin_local, int64_t chunk_ticks, const uint32_t *first,
                          const uint32_t *pin_off, const uint8_t *st, const KeyFmt &kf, uint64_t *key_out,
                          float *slew_out, uint32_t *orig_out, hipStream_t s) {
  hipLaunchKernelGGL(k_scatter, dim3(grid_for(E)), dim3(kLT), 0, s, E, P, G, evt_t, evt_slew, evt_val, ev_pin,
                     pin_gate, pin_local, chunk_ticks, first, pin_off, st, kf, key_out, slew_out, orig_out);
  return hipGetLastError();
}

hipError_t launch_chunk_base(int32_t Q, int64_t P, int64_t E, const uint32_t *pin_off, uint32_t *cb,
                             hipStream_t s) {
  hipLaunchKernelGGL(k_chunk_base, dim3(grid_for(Q + 1)), dim3(kLT), 0, s, Q, P, E, pin_off, cb);
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
