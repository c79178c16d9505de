// pa_load.h -- load-time kernel launchers and validation flags (internal).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa_common.h"

namespace pa {

// validation flags set by the load kernels
enum : uint32_t {
  ERR_CELL_ID = 1u << 0,     // gate_cell outside [0, n_cells)
  ERR_CAP = 1u << 1,         // non-finite gate load
  ERR_PIN_PTR = 1u << 2,     // pin_ptr decreases
  ERR_INIT = 1u << 3,        // pin_init not in {0, 1}
  ERR_TIME_RANGE = 1u << 4,  // t < 0 or t >= t_max
  ERR_TIME_ORDER = 1u << 5,  // timestamps not strictly increasing on a pin
  ERR_VALUE = 1u << 6,       // values do not alternate starting from !init
  ERR_SLEW = 1u << 7,        // slew not finite and > 0
  ERR_ENDS = 1u << 8,        // pin_ptr[0] != 0 or pin_ptr[P] != n_events
};

// bit widths of the event layout
struct LayoutFmt {
  int64_t T;     // clock period, ticks
  int32_t Cc;    // cycles per chunk (2^lc)
  uint32_t lc;   // log2 Cc
  uint32_t pb;   // pin-code bits
  uint32_t tb;   // tic bits
  uint32_t gb;   // gate-id bits of the sort key and of the packed key
};

hipError_t launch_gate_tables(int64_t G, const int32_t *perm, const int32_t *gate_cell, const double *gate_cap,
                              int32_t n_cells, const int32_t *cell_k, const double *cap_axis, int32_t n_cap, double vdd,
                              uint32_t *gate_info, uint4 *gate_rec, int32_t *gate_k, uint32_t *err, hipStream_t s);
// leakage power at t = 0 into *l0 (part: leak0_parts() doubles of scratch)
hipError_t launch_leak0(int64_t G, const uint32_t *gate_info, const uint2 *cell_meta, const double *leak,
                        const int64_t *pin_base, const uint8_t *pin_init, double *part, double *l0, hipStream_t s);
int leak0_parts();
// per-gate output rows (caller's gate order): zero dynamic parts, leakage at the initial state over the window
hipError_t launch_gate_rows(int64_t G, const uint32_t *gate_info, const uint2 *cell_meta, const double *leak,
                            const int64_t *pin_base, const uint8_t *pin_init, const int32_t *perm, double window,
                            double *gate_J, hipStream_t s);
// the windows ranked gate-major (internal gate order): every window's gate (key) and index (value); after a
// stable sort by key, every window's rank, every gate's first rank (goff[G + 1]) and its pieces for the
// row sums (npiece[G]; their exclusive prefix is pfirst[G + 1])
hipError_t launch_win_gates(uint32_t W, const uint32_t *ws, const uint64_t *skey, uint32_t gb, uint32_t *key,
                            uint32_t *val, hipStream_t s);
hipError_t launch_win_ranks(uint32_t W, int64_t G, const uint32_t *key, const uint32_t *val, uint32_t *rank,
                            uint32_t *goff, uint32_t *npiece, hipStream_t s);
// per-gate output rows (caller's gate order) from the walk kernel's window sums (rec[pairs][4], the window
// of rank r at pair wpos[r]): the gate's windows (or, for a larger gate, its pieces, part[n_pieces][4],
// summed first) added in a fixed order, plus the leakage at the initial state over the window (gleak[G])
hipError_t launch_gate_sums(int64_t G, uint32_t n_pieces, const uint32_t *goff, const uint32_t *pfirst,
                            const uint32_t *pgate, const double *gleak, const int32_t *perm, const uint32_t *wpos,
                            const double *rec, double *part, double *gate_J, hipStream_t s);
// once per event load, for the row sums: every gate's leakage at its initial state over the window
// (gleak[G], internal order) and every piece's gate (pgate[n_pieces])
hipError_t launch_gate_prep(int64_t G, const uint32_t *gate_info, const uint2 *cell_meta, const double *leak,
                            const int64_t *pin_base, const uint8_t *pin_init, double window, const uint32_t *pfirst,
                            double *gleak, uint32_t *pgate, hipStream_t s);
hipError_t launch_pin_owner(int64_t G, const int64_t *pin_base, const int32_t *gate_k, int32_t *pin_gate,
                            uint8_t *pin_local, hipStream_t s);
hipError_t launch_pin_check(int64_t P, int64_t E, const int64_t *pin_ptr, const uint8_t *pin_init, uint32_t *err,
                            hipStream_t s);
hipError_t launch_event_check(int64_t E, int64_t P, const int64_t *pin_ptr, const uint8_t *pin_init,
                              const int64_t *evt_t, const uint8_t *evt_val, const float *evt_slew, int64_t t_max,
                              uint32_t *mark, uint32_t *ev_pin, uint32_t *err, void *tmp, size_t *tmp_bytes,
                              hipStream_t s);
// per-gate window level: fixed_level >= 0 gives every gate that level, else density-aware
hipError_t launch_gate_levels(int64_t G, const int64_t *pin_base, const int32_t *gate_k, const int64_t *pin_ptr,
                              int64_t C, int32_t Cc, int32_t lc, double target, int32_t fixed_level,
                              uint8_t *level, hipStream_t s);
// chunk == nullptr: one 64-bit key (chunk, gate, lk); else key = (gate, lk) and chunk[e] apart
hipError_t launch_sort_keys(int64_t E, const int64_t *evt_t, const uint32_t *ev_pin, const int32_t *pin_gate,
                            const uint8_t *pin_local, const int32_t *gate_k, const LayoutFmt &f, uint64_t *key,
                            uint32_t *chunk, uint32_t *idx, hipStream_t s);
hipError_t launch_chunk_of(int64_t E, const uint32_t *perm, const uint32_t *chunk, uint32_t *chunk_sorted,
                           hipStream_t s);
hipError_t launch_layout(int64_t E, const uint32_t *perm, const uint64_t *skey, const int64_t *evt_t,
                         const float *evt_slew, const uint8_t *evt_val, const uint32_t *ev_pin,
                         const int32_t *pin_gate, const uint8_t *pin_local, const int32_t *gate_k,
                         const uint8_t *level, const LayoutFmt &f, uint64_t *key_out, float *slew_out,
                         uint32_t *orig_out, uint32_t *chunk_out, hipStream_t s);
// the start state of every input window into its first event's key (after the windows are known)
hipError_t launch_window_s0(uint32_t W, const uint32_t *ws, const uint32_t *chunk_sorted, const uint8_t *level,
                            const int32_t *gate_k, const int64_t *pin_base, const int64_t *pin_ptr,
                            const uint8_t *pin_init, const int64_t *evt_t, const LayoutFmt &f, uint64_t *skey,
                            hipStream_t s);
hipError_t launch_chunk_base(int64_t E, int32_t Q, const uint32_t *chunk_sorted, uint32_t *cb, hipStream_t s);
// lane streams of the pass (see pa_load.hip): head flags; window starts
// (ws[W] = E); every block's first window; window sort keys (block, kind,
// length), indices and lengths; the phase plan: every window's place in its
// lane's stream and every wave's stream length (ph: phase_plan_entries(W, nr)
// entries of scratch); the scatter of the sorted events into the streams
hipError_t launch_head_flags(int64_t E, const uint64_t *skey, uint32_t *flag, hipStream_t s);
hipError_t launch_win_starts(int64_t E, const uint64_t *skey, const uint32_t *winc, uint32_t *ws, hipStream_t s);
hipError_t launch_block_windows(int32_t nr, int64_t E, const uint32_t *rstart, const uint64_t *skey,
                                const uint32_t *winc, uint32_t W, uint32_t *bwin, hipStream_t s);
hipError_t launch_win_keys(uint32_t W, const uint32_t *ws, const uint32_t *bwin, int32_t nr, const uint64_t *skey,
                           uint32_t outc, uint64_t *wkey, uint32_t *widx, uint32_t *wlen, hipStream_t s);
size_t phase_plan_entries(uint32_t W, int32_t nr);
// hp: slots of a header pair in front of every phase (2) or none (0); w_in,
// w_out: relative cost of a slot of an input or an output phase
hipError_t launch_phase_plan(int32_t nr, const uint32_t *bwin, const uint32_t *worder, const uint64_t *wkey,
                             const uint32_t *wlen, uint32_t hp, uint32_t w_in, uint32_t w_out, uint2 *ph,
                             uint2 *wlane, uint32_t *wave_len, hipStream_t s);
// the walk kernel's 8-byte-slot stream from the 16-byte one, then every window's header pair (and,
// by the window's rank in gate order, the header's pair index: wpos[rank[w]])
hipError_t launch_compact(int64_t n, const uint64_t *key, const float *slew, uint64_t pad_key, uint32_t pb,
                          uint32_t tb, uint32_t gb, uint32_t tbc, uint32_t ck, uint32_t *ckey, uint32_t *cslew,
                          hipStream_t s);
hipError_t launch_headers(uint32_t W, const uint2 *wlane, const uint2 *wdesc, const uint32_t *ws, const uint64_t *skey,
                          const uint4 *gate_rec, const uint32_t *rank, uint32_t gb, uint32_t outc, uint32_t hdr,
                          uint32_t out_bit, uint32_t *ckey, uint32_t *cslew, uint32_t *wpos, hipStream_t s);
hipError_t launch_scatter(int64_t E, const uint64_t *skey, const float *sslew, const uint32_t *sorig,
                          const uint32_t *winc, const uint32_t *ws, const uint2 *wlane, const uint2 *wdesc,
                          uint64_t *key, float *slew, uint32_t *orig, hipStream_t s);
int lane_plan_lanes();  // lanes of a block of the pass
hipError_t launch_fill_u64(int64_t n, uint64_t v, uint64_t *out, hipStream_t s);
// the cost of every sorted event in the pass (kind weight plus a window head's
// weight); the first event past each cost target; the cost before given events
hipError_t launch_event_cost(int64_t E, const uint64_t *skey, uint32_t outc, uint32_t w_in, uint32_t w_out,
                             uint32_t w_head, const int32_t *gate_k, uint32_t gb, uint64_t *cost, hipStream_t s);
hipError_t launch_cost_cuts(int32_t n, const uint64_t *target, const uint64_t *pref, int64_t E, uint32_t *pos,
                            hipStream_t s);
hipError_t launch_gather_prefix(int32_t n, const uint32_t *at, const uint64_t *pref, uint64_t *out, hipStream_t s);
hipError_t scan_inclusive_u64(const uint64_t *in, uint64_t *out, int64_t n, void *tmp, size_t *tmp_bytes,
                              hipStream_t s);
hipError_t scan_inclusive_u32(const uint32_t *in, uint32_t *out, int64_t n, void *tmp, size_t *tmp_bytes,
                              hipStream_t s);
hipError_t sort_pairs_u64(uint64_t **k0, uint64_t **k1, uint32_t **v0, uint32_t **v1, int64_t n, int end_bit,
                          void *tmp, size_t *tmp_bytes, hipStream_t s);
hipError_t sort_pairs_u32(uint32_t **k0, uint32_t **k1, uint32_t **v0, uint32_t **v1, int64_t n, int end_bit,
                          void *tmp, size_t *tmp_bytes, hipStream_t s);

}  // namespace pa
