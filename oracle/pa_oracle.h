/*
 * pa_oracle.h -- interface of the CPU oracle (TEST INFRASTRUCTURE ONLY).
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use
 * this.  The product library neither includes nor links it.
 *
 * All pointers are host pointers.  Array layouts follow the power-analysis
 * method of "GPU-Accelerated Gate-Level Time-Based Power Analysis via
 * Event-Density-Aware Partitioning and Kernel Fusion" (arXiv 2609.05960):
 *   gate_cell[G], gate_cap_F[G]                per-gate cell id and output load
 *   cell_n_in[n_cells]                         k inputs (1..8) -> 2^k states
 *   slew_axis[n_cells][n_slew], cap_axis[n_cells][n_cap]  strictly increasing
 *   lut_J   per cell, concatenated: [2^k][k][n_slew][n_cap]   (state-indexed)
 *   leak_W  per cell, concatenated: [2^k]                     (state-indexed)
 *   pins are gate-major: gate g owns k_g input pins then 1 output pin
 *   pin_ptr[P+1] CSR offsets into evt_t / evt_val / evt_slew
 * Outputs: wave_J, cyc_events, cyc_glitches have ceil(t_max/t_clk) entries;
 * evt_glitch and evt_state_before have pin_ptr[P] entries or are NULL;
 * gate_J[G][4] (NULL = not wanted) receives every processed gate's internal,
 * switching, glitch and leakage energy in J.
 * Only gates [gate_lo, gate_hi) are processed; outputs hold their share.
 */
#ifndef PA_ORACLE_H
#define PA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ORACLE_EARG 1
#define PA_ORACLE_EDATA 2
#define PA_ORACLE_ENOMEM 3

typedef struct {
  double p_int_W, p_sw_W, p_gl_W, p_leak_W;
  double e_int_J, e_sw_J, e_gl_J, e_leak_J;
  uint64_t n_events, n_glitches;
  int64_t n_cycles;
} pa_oracle_totals;

double pa_oracle_bilerp(int n_slew, int n_cap, const double *slew_axis, const double *cap_axis,
                        const double *table, double x_slew, double x_cap);

int64_t pa_oracle_n_cycles(int64_t t_clk, int64_t t_max);

int pa_oracle_run(int64_t n_gates, const int32_t *gate_cell, const double *gate_cap_F, int32_t n_cells,
                  const int32_t *cell_n_in, int32_t n_slew, int32_t n_cap, const double *slew_axis,
                  const double *cap_axis, const double *lut_J, const double *leak_W, double vdd_V,
                  int64_t n_pins, const int64_t *pin_ptr, const uint8_t *pin_init, const int64_t *evt_t,
                  const uint8_t *evt_val, const float *evt_slew, int64_t t_clk, int64_t t_max, double tick_s,
                  int64_t gate_lo, int64_t gate_hi, pa_oracle_totals *out, double *wave_J,
                  uint64_t *cyc_events, uint64_t *cyc_glitches, uint8_t *evt_glitch,
                  uint8_t *evt_state_before, double *gate_J);

/* The same run on n_threads host threads (1..1024): gates [gate_lo, gate_hi)
 * are cut into contiguous ranges of about equal work, each walked by one
 * thread into private bins, totals and counts, merged in range order. */
int pa_oracle_run_mt(int64_t n_gates, const int32_t *gate_cell, const double *gate_cap_F, int32_t n_cells,
                     const int32_t *cell_n_in, int32_t n_slew, int32_t n_cap, const double *slew_axis,
                     const double *cap_axis, const double *lut_J, const double *leak_W, double vdd_V,
                     int64_t n_pins, const int64_t *pin_ptr, const uint8_t *pin_init, const int64_t *evt_t,
                     const uint8_t *evt_val, const float *evt_slew, int64_t t_clk, int64_t t_max, double tick_s,
                     int64_t gate_lo, int64_t gate_hi, int32_t n_threads, pa_oracle_totals *out, double *wave_J,
                     uint64_t *cyc_events, uint64_t *cyc_glitches, uint8_t *evt_glitch,
                     uint8_t *evt_state_before, double *gate_J);

#ifdef __cplusplus
}
#endif
#endif
