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
};

hipError_t launch_gate_tables(int64_t G, const int32_t *gate_cell, const double *gate_cap, int32_t n_cells,
                              const int32_t *cell_k, const double *cap_axis, int32_t n_cap, double vdd,
                              uint32_t *gate_info, double *capfrac, double *esw, int32_t *gate_k, uint32_t *err,
                              hipStream_t s);
hipError_t launch_pin_owner(int64_t G, const int64_t *pin_base, int32_t *pin_gate, uint8_t *pin_local,
                            hipStream_t s);
hipError_t launch_pin_check(int64_t P, const int64_t *pin_ptr, const uint8_t *pin_init, uint32_t *err,
                            hipStream_t s);
hipError_t launch_event_check(int64_t E, int64_t P, const int64_t *pin_ptr, const uint8_t *pin_init,
                              const int64_t *evt_t, const uint8_t *evt_val, const float *evt_slew, int64_t t_max,
                              uint32_t *ev_pin, uint32_t *err, hipStream_t s);
hipError_t launch_gate_levels(int64_t G, const int64_t *pin_base, const int64_t *pin_ptr, int64_t C, int32_t Cc,
                              int32_t lc, double target, uint8_t *level, hipStream_t s);
hipError_t launch_pw_len(int64_t G, const int32_t *gate_k, const uint8_t *level, int64_t *pw_len, hipStream_t s);
hipError_t launch_count_w(int64_t E, const int64_t *evt_t, const uint32_t *ev_pin, const int32_t *pin_gate,
                          const uint8_t *pin_local, const int32_t *gate_k, const uint8_t *level,
                          const int64_t *pwbase, int64_t PW, int64_t T, int32_t lc, uint32_t *cnt, hipStream_t s);
hipError_t launch_winmax(int64_t G, int32_t Q, const int32_t *gate_k, const uint8_t *level, const int64_t *pwbase,
                         int64_t PW, int32_t lc, const uint32_t *cnt, uint8_t *level_next, uint32_t *flags,
                         uint32_t *max_seg, hipStream_t s);
hipError_t launch_pin_windows(int64_t P, int32_t Q, const int64_t *pin_ptr, const uint8_t *pin_init,
                              const int32_t *pin_gate, const uint8_t *pin_local, const int32_t *gate_k,
                              const uint8_t *level, const int64_t *pwbase, int64_t PW, const uint32_t *cnt,
                              uint32_t *first, uint8_t *vstart, hipStream_t s);
hipError_t launch_scatter_w(int64_t E, const int64_t *evt_t, const float *evt_slew, const uint8_t *evt_val,
                            const uint32_t *ev_pin, const int32_t *pin_gate, const uint8_t *pin_local,
                            const int32_t *gate_k, const uint8_t *level, const int64_t *pwbase, int64_t PW, int64_t T,
                            int32_t lc, int64_t chunk_ticks, const uint32_t *first, const uint32_t *off,
                            const uint8_t *vstart, const KeyFmt &kf, uint64_t *key_out, float *slew_out,
                            uint32_t *orig_out, hipStream_t s);
hipError_t launch_chunk_base_w(int32_t Q, int64_t PW, const uint32_t *off, uint32_t *cb, hipStream_t s);
hipError_t scan_exclusive_u32(const uint32_t *in, uint32_t *out, int64_t n, void *tmp, size_t *tmp_bytes,
                              hipStream_t s);
hipError_t scan_exclusive_i64(const int64_t *in, int64_t *out, int64_t n, void *tmp, size_t *tmp_bytes,
                              hipStream_t s);

}  // namespace pa
