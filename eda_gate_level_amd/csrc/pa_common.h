// pa_common.h -- internal types shared by the host side and the gfx950 kernels
// of the power-analysis library.  Not part of the public ABI (include/pa.h).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "pa.h"

namespace pa {

// ---------------------------------------------------------------------------
// Exact unsigned 32-bit division by a divisor fixed at load time, by a
// multiply-high and two shifts (Granlund & Montgomery, "Division by invariant
// integers using multiplication", PLDI 1994, Fig. 4.1):
//   l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1,
//   t = mulhi(m, n), q = (t + ((n - t) >> min(l,1))) >> max(l-1,0).
// Exact for every 1 <= d < 2^32 and 0 <= n < 2^32.  Cycle indices of events
// (t / T) are integer decisions and must match plain division bit for bit.
// ---------------------------------------------------------------------------
struct DivU32 {
  uint32_t m, sh1, sh2, d;
};

inline DivU32 make_divu32(uint32_t d) {
  uint32_t l = 0;
  while (l < 32 && (uint64_t(1) << l) < d) ++l;
  DivU32 D;
  D.m = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
  D.sh1 = l < 1 ? l : 1;
  D.sh2 = l > 0 ? l - 1 : 0;
  D.d = d;
  return D;
}

__host__ __device__ inline uint32_t divu32(uint32_t n, const DivU32 &D) {
  uint32_t t = uint32_t((uint64_t(n) * D.m) >> 32);
  return (t + ((n - t) >> D.sh1)) >> D.sh2;
}

// ---------------------------------------------------------------------------
// Packed 64-bit event key of the event layout, fixed fields:
//   bits [42, 64)  gate id (designs up to 2^22 - 1 gates)
//   bit  41        head: first event of its segment
//   bits [ 9, 41)  lk = (pin code << t_bits) | t_rel
//   bit   8        val: the pin's value after the event
//   bits [ 0,  8)  S0: input-pin state of the gate at the start of the segment
// A segment is one (time chunk, gate, time window) triple: chunks are Cc
// clock cycles long and every gate's chunk is cut into 2^s windows whose
// length follows the gate's event density, so that no segment holds more
// than a fixed number of events.  pin code = input pin index 0..k-1, or
// kOutCode(p_bits) for the output pin; t_rel = timestamp minus the start of
// the event's chunk.  Inside a segment the lk words increase strictly in
// (pin code, t_rel) order.
// ---------------------------------------------------------------------------
constexpr uint32_t kKeyGateShift = 42;
constexpr uint32_t kKeyHeadShift = 41;
constexpr uint32_t kKeyLkShift = 9;
constexpr uint32_t kKeyValShift = 8;
constexpr uint64_t kKeyMaxGates = uint64_t(1) << 22;
constexpr int kSegMax = 128;  // most events of one segment

__host__ __device__ inline uint32_t out_code(uint32_t p_bits) { return (1u << p_bits) - 1u; }

struct KeyFmt {
  uint32_t t_bits;  // width of t_rel
  uint32_t p_bits;  // width of the pin code
};

// Kernel arguments of one pass (passed by value).
struct PassArgs {
  // events, chunk-major layout
  const uint64_t *key;
  const float *slew;
  const uint32_t *orig;        // caller's CSR index of each laid-out event
  const uint32_t *chunk_base;  // [Q+1]
  const uint32_t *rstart;      // [n_ranges+1] nominal starts of the block ranges (inside one chunk each)
  const uint32_t *rchunk;      // [n_ranges] chunk of each range
  int32_t n_ranges;
  int64_t E;
  int32_t Q, Cc;
  int64_t C;
  uint32_t T;
  DivU32 divT;
  int64_t chunk_ticks;
  int64_t t_max;
  double tick_s;
  KeyFmt kf;
  // design
  int64_t G;
  const uint32_t *gate_info;  // cell | (cap segment << 24)
  const double *gate_capfrac;
  const double *gate_esw;     // 0.5 * c * Vdd^2
  const int64_t *pin_base;    // [G+1]
  const uint8_t *pin_init;    // [P]
  const int32_t *cell_k;
  const uint32_t *cell_lut_base;
  const uint32_t *cell_leak_base;
  const double *lut;
  const double *leak;
  const double *slew_axis;  // [n_cells][n_slew]
  const double *slew_invw;  // [n_cells][n_slew-1]
  int32_t n_slew, n_cap;
  int32_t n_cells;
  int64_t n_leak;             // entries of the leakage table
  // accumulators
  double *acc_wave;                  // [8][C]
  unsigned long long *acc_cnt;       // [8][C]  events | glitches << 32
  double *dP;                        // [Q]   leakage power change inside each chunk
  double *tot;                       // [8]   e_int, e_sw, e_gl, e_leak_changes, L0, -, -, -
  unsigned long long *tot_cnt;       // [2]   n_glitches, -
  // diagnostics (may be null)
  uint8_t *evt_glitch;
  uint8_t *evt_state;
};

struct FinalArgs {
  int64_t C;
  int32_t Cc, Q;
  uint32_t T;
  int64_t t_max;
  double tick_s;
  int64_t E;
  double *acc_wave;
  unsigned long long *acc_cnt;
  const double *dP;
  const double *tot;
  const unsigned long long *tot_cnt;
  double *dP_next;                   // other parity set, zeroed here
  double *tot_next;
  unsigned long long *tot_cnt_next;
  int32_t Q_next;
  double *wave_out;
  uint64_t *cyc_events;
  uint64_t *cyc_glitches;
  double *res;                       // [16] results for the host
};

// Launchers (defined in pa_pass.hip).
hipError_t launch_pass(const PassArgs &a, int grid_blocks, hipStream_t s);
hipError_t launch_finalize(const FinalArgs &a, hipStream_t s);
int pass_block_threads();
int pass_batch_events();
int pass_max_chunk_cycles();
bool pass_cells_fit_lds(int n_cells, int n_slew, int64_t n_leak);
int pass_wave_batch();

}  // namespace pa
