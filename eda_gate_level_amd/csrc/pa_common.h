// pa_common.h -- internal types shared by the host side and the gfx950 kernels
// of the power-analysis library.  Not part of the public ABI (include/pa.h).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa.h"

namespace pa {

constexpr int kMaxInputs = 8;  // inputs of a cell (pa_load_design rejects more)

// ---------------------------------------------------------------------------
// Event layout.  Time is cut into chunks of Cc clock cycles (a power of two);
// inside a chunk every gate's cycles are cut into 2^s equal windows, s chosen
// per gate from its event density (the paper's event-density-aware per-gate
// cycle partitioning); a gate's input-pin events and its output-pin events go
// to windows of their own.  Inside a window the events are in
//   (cycle, time, pin code)
// order: the events of one clock cycle form one run in time order, events of
// one timestamp ordered by pin code.  Every block of the pass owns a range of
// whole windows of one chunk; its windows go in phases of up to 64 windows of
// one kind to its waves, one window per lane, each lane's window padded to
// an even length and to the phase's longest.  A wave's 64 lane streams are
// interleaved in pairs: slot j of lane l sits at base + (j / 2) * 128 + 2 l +
// j % 2.  Empty slots hold the pad key (an output-pin 1->0 event in cycle Cc,
// or key 0 when the chunk leaves no spare cycle bit), which no event has.
//
// Packed 64-bit key of an event (gb = bits of the largest gate id, cs = pb + tb):
//   bits [42 + gb, 64)  the high bits of the cycle in the chunk (22 - gb of them)
//   bits [42, 42 + gb)  gate id (designs up to 2^22 - 1 gates)
//   bit  41             window head: first event of its (chunk, gate, window)
//   bit  40             val: the pin's value after the event
//   bits [32, 40)       S0: the gate's input-pin state at the window start (on
//                       window heads; zero elsewhere)
//   bits [ 0, 32)       (low bits of the cycle in the chunk << cs) | (tic << pb) | pin code
// so the cycle in the chunk, (key >> 32 >> (10 + gb)) << (32 - cs) | low word >> cs,
// has 32 - cs + 22 - gb bits.  tic = time minus the start of the event's clock
// cycle (tb bits); pin code = input pin index 0..k-1, or out_code(pb) for the
// output pin.
// ---------------------------------------------------------------------------
constexpr uint32_t kKeyGateShift = 42;
constexpr uint32_t kKeyHeadShift = 41;
constexpr uint32_t kKeyValShift = 40;
constexpr uint32_t kKeyS0Shift = 32;
constexpr uint64_t kKeyMaxGates = uint64_t(1) << 22;

__host__ __device__ inline uint32_t out_code(uint32_t pb) { return (1u << pb) - 1u; }

// Smallest float at or above x.  The slew-axis segment of an event is found
// by comparing its fp32 slew with the axis points; for every float s,
// s >= float_at_or_above(x) holds exactly when (double)s >= x, so comparing
// in fp32 against these thresholds picks the same segment as fp64 compares.
inline float float_at_or_above(double x) {
  float f = (float)x;
  if ((double)f < x) f = __builtin_nextafterf(f, __builtin_inff());
  return f;
}

// Kernel arguments of one pass (passed by value).
struct PassArgs {
  // events
  const uint64_t *key;
  const float *slew;
  const uint32_t *orig;    // caller's CSR index of each laid-out event (~0 in empty slots and headers)
  uint64_t pad_key;        // key of an empty slot (no event has it)
  const uint2 *wdesc;      // [n_ranges][waves] every wave's (first slot, events per lane)
  const uint32_t *rchunk;  // [n_ranges] chunk of each range
  int32_t n_ranges;
  int64_t E;
  int32_t Q, Cc;
  int64_t C;
  uint32_t T;
  uint32_t tb, pb;         // bit widths of tic and of the pin code in the key's low word
  uint32_t gb;             // bit width of the gate id
  uint32_t last_len;       // ticks of the last cycle bin
  int64_t chunk_ticks;
  int64_t t_max;
  double tick_s;
  // design
  int64_t G;
  const uint4 *gate_rec;      // (load c as fp64 bits lo, hi; cell | (cap segment << 24); 0)
  const int64_t *pin_base;    // [G+1]
  const uint8_t *pin_init;    // [P]
  const uint2 *cell_meta;     // x = k | leak base << 4, y = LUT base
  const float *cell_thr;      // [n_cells][n_thr] inner slew-axis points as float, rounded up
  const double2 *cell_axw;    // [n_cells][n_slew-1] (slew-axis point, 1 / segment width)
  const double2 *cell_caxw;   // [n_cells][n_cap-1] (cap-axis point, 1 / segment width)
  double hv2;                 // 0.5 Vdd^2
  const double *lut;
  const double *leak;
  int32_t n_slew, n_cap, n_cells, n_thr;
  int64_t n_leak;
  int32_t kmax;               // most inputs of a cell (pin slots per lane: kmax + 1)
  // cells whose LUTs every block copies into LDS (see launch_lut_plan)
  const uint2 *lut_plan;      // [n_ranges][pass_lut_plan_slots()] (cell, LDS offset in doubles), cell ~0 = none
  int32_t lut_lds;            // LDS reserved for them, doubles (0: none)
  // the walk kernel: every block's LUT range [x, x + y) in doubles, all of it in the block's LDS
  const uint2 *blk_lut;
  int32_t walk_lut;           // LDS doubles reserved for the largest range (0: the walk kernel is not used)
  // the walk kernel's stream, slot for slot with key/slew: 32-bit keys (cycle << (tbc + ck) | tic << ck |
  // pin code >> 1; ~0 = empty; an all-ones tic field = a phase's header pair) and slews whose sign bit
  // holds the pin code's low bit (input pins) or the new value (output pin)
  const uint32_t *ckey;
  const uint32_t *cslew;
  uint32_t tbc, ck;
  int32_t plain_bins;         // timing aid: 1 plain adds, 2 plain stores to the bins (results wrong)
  // the walk kernel's per-event outputs, in stream order: 16 bits a slot (state before | glitch << 8),
  // two slots per 32-bit word (null: none)
  uint32_t *evs;
  double *wrec;               // walk kernel: [pairs][4] every window's sums (internal, switching, glitch,
                              // leakage to t_max) at its header's pair of the lane streams
  // per-block results, reduced by the finalize kernel
  double *blk_wave;              // [grid][Cc] energy per cycle of the block's chunk
  unsigned long long *blk_cnt;   // [grid][Cc] events | glitches << 32
  double *blk_part;              // [grid][8] e_int, e_sw, e_gl, e_leak changes, L0 part, dP sum, n_gl, -
  // diagnostics (may be null)
  uint8_t *evt_glitch;
  uint8_t *evt_state;
  double *gate_J;             // [G][4] per-gate energies, caller's gate order (added to)
  const int32_t *gate_perm;   // internal gate -> caller gate
};

struct FinalArgs {
  int64_t C;
  int32_t Cc, Q;
  uint32_t T;
  uint32_t last_len;
  int64_t t_max;
  double tick_s;
  int32_t grid;
  const uint32_t *chunk_blk;  // [Q+1] first block of every chunk (blocks are in chunk order)
  uint32_t cblk[64];          // the same values when Q < 64, passed by value (no dependent load)
  const double *blk_wave;
  const unsigned long long *blk_cnt;
  const double *blk_part;
  double l0;                  // leakage power at t = 0, summed at load
  double *wave_out;
  uint64_t *cyc_events;
  uint64_t *cyc_glitches;
  double *res;                // [16] results for the host
};

// Launchers (defined in pa_pass.hip).  Given two events, they time the
// kernel's own execution (events attached to its dispatch).
hipError_t launch_pass(const PassArgs &a, int grid_blocks, hipStream_t s, hipEvent_t e0 = nullptr,
                       hipEvent_t e1 = nullptr);
hipError_t launch_finalize(const FinalArgs &a, hipStream_t s, hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);
// Per-event outputs of the walk kernel: every event's slot by its caller
// index (n slots of the caller-index array); the 16-bit slot values into
// the caller's order (either output may be null).
hipError_t launch_slot_of(int64_t n, const uint32_t *orig, uint32_t *slot_of, hipStream_t s);
hipError_t launch_event_out(int64_t E, const uint32_t *slot_of, const uint32_t *evs, uint8_t *glitch,
                            uint8_t *state, hipStream_t s);
// Per block, the cells whose LUTs it copies into the LDS left over by its bins,
// pin records and cell tables (lut_lds doubles, from pass_lut_lds_doubles): 64
// windows sampled evenly over the block's window range [bwin[b], bwin[b+1])
// (window w starts at sorted event ws[w], skey holds the sorted keys) give
// each cell present a weight, and the heaviest cells that still fit are
// taken, at most pass_lut_plan_slots() of them.  plan holds that many
// (cell, LDS offset) pairs per block; unused slots have cell ~0.
hipError_t launch_lut_plan(const uint64_t *skey, const uint32_t *ws, const uint32_t *bwin, int32_t n_ranges,
                           const uint4 *gate_rec, const uint2 *cell_meta, uint32_t gb, int n_slew, int n_cap,
                           int32_t lut_lds, uint2 *plan, hipStream_t s);
int pass_lut_plan_slots();
// The walk kernel (one template per supported axis size): every block's LUT
// range (first entry, entries) from its first and last window's gates; the
// LDS doubles left for a block's LUT range beside its bins, pin records and
// cell tables (0: none).
hipError_t launch_block_luts(int32_t nr, const uint64_t *skey, const uint32_t *ws, const uint32_t *bwin,
                             const uint4 *gate_rec, const uint2 *cell_meta, uint32_t gb, int n_slew, int n_cap,
                             uint2 *out, hipStream_t s);
bool walk_supported(int n_slew, int n_cap);
int32_t walk_lut_doubles(int Cc, int n_cells, int n_slew, int n_cap, int n_thr, int64_t n_leak, int kmax);
int32_t pass_lut_lds_doubles(int Cc, int n_cells, int n_slew, int n_cap, int n_thr, int64_t n_leak, int kmax);
int pass_block_threads();
int pass_blocks_per_cu();       // blocks of the pass resident on one compute unit
int pass_waves_per_block();
size_t pass_static_lds_bytes();  // static LDS of a block of the pass
int pass_wave_batch();
int pass_max_chunk_cycles();
// dynamic LDS bytes of the pass, and whether the cell tables fit in it
size_t pass_lds_bytes(int Cc, int n_cells, int n_slew, int n_cap, int n_thr, int64_t n_leak, int kmax, bool cells);
bool pass_cells_fit_lds(int Cc, int n_cells, int n_slew, int n_cap, int n_thr, int64_t n_leak, int kmax);

}  // namespace pa
