/*
 * pa.h -- C ABI of the MI355X (gfx950) gate-level time-based power analysis
 * library.
 *
 * The method is the one of "GPU-Accelerated Gate-Level Time-Based Power
 * Analysis via Event-Density-Aware Partitioning and Kernel Fusion" (arXiv
 * 2609.05960), called "the paper" below:
 *   - per event: reconstruct the gate state before the event (Sec. 2.4.1),
 *     pick the state's internal-power LUT and interpolate it on input slew
 *     and output load (Sec. 2.4.1, Fig. 2), add 1/2 c v^2 for a 0->1 event on
 *     the output pin (Eq. 1), detect glitches by counting a pin's events per
 *     clock cycle and scale their energy by r_gl (Sec. 2.4.1, Eq. 2, Fig. 7),
 *     and add the energy to the bin of its clock cycle;
 *   - per gate: merge the pin streams in time order, apply all events of a
 *     timestamp together, charge state-dependent leakage over every
 *     inter-event interval (Eq. 4) and spread it over the cycle bins it
 *     overlaps in proportion to the overlap (Sec. 2.4.2);
 *   - powers are energies over the analysis window (Eq. 3).
 * Readings of what the paper leaves open (its Eqs. 1-4 are not printed in the
 * available text) are fixed as follows and are part of this contract:
 *   E_sw = 0.5 * c * Vdd^2 per 0->1 output event (0 J for 1->0);
 *   r_gl = min(1, pw / ((rSlew + fSlew) / 2)), pw = time since the previous
 *     event on the same pin, rSlew/fSlew = slews of that event and this one;
 *   the m-th event (m >= 2) of a pin inside one clock cycle is a glitch and
 *     adds r_gl * E to the glitch component (only) and to the waveform;
 *   state S = sum_i v_i 2^i over the input pins (pin 0 = LSB);
 *   bins are [c T, (c+1) T), N_cyc = ceil(t_max / T), the last may be partial;
 *   bilinear interpolation extrapolates linearly outside the LUT axes;
 *   P = E / (t_max * tick_s), E_leak = p_leak * dt * tick_s.
 *
 * Conventions for every function:
 *   - returns PA_OK (0) or a negative PA_E* code; no exception crosses the ABI;
 *     pa_last_error() gives a message for the calling thread's last failure;
 *   - array arguments are DEVICE pointers on the context's device (torch
 *     tensors' data_ptr(), or hipMalloc'd memory), unless stated otherwise;
 *   - the load calls copy their inputs into library-owned device memory, so
 *     the caller may free or reuse its arrays once the call returns;
 *   - a failing load leaves the previously loaded data intact;
 *   - one context per device; a context is not thread-safe.
 */
#ifndef PA_H
#define PA_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_OK 0
#define PA_EINVAL (-1) /* bad argument (null pointer, size out of range, call-shape error) */
#define PA_EDATA (-2)  /* design or event data break the contract above */
#define PA_ENOMEM (-3) /* device or host allocation failed */
#define PA_EHIP (-4)   /* HIP runtime error */
#define PA_ESTATE (-5) /* wrong call order (e.g. pa_run before both loads) */

typedef struct pa_ctx pa_ctx;

/* Speed knobs.  They never change results beyond fp64 summation order; a
 * zero field means "choose automatically". */
typedef struct {
  int32_t chunk_cycles;   /* cycles per time chunk of the event layout; rounded down to a
                             power of two, at most 2048 and at most what the key's bits
                             allow for the clock period and gate count (0 = 2048) */
  int32_t grid_blocks;    /* target block count of the fused pass (0 = one 1024-thread block
                             per compute unit);
                             the pass cuts the events into about this many ranges */
  int32_t time_kernels;   /* 0: no timing; 1: device times of the fused kernel and of the
                             finalize kernel (events attached to each kernel's dispatch: the
                             kernel's own execution) and of the whole pass; 2: the whole pass
                             only (events recorded before the first kernel and after the last) */
  int32_t fixed_window_cycles; /* 0: density-aware windows (below); n > 0: every gate's
                             windows are n cycles (rounded down to a power of two, at most the
                             chunk) -- the fixed-window layout the paper compares against */
  int32_t lut_lds_kib;    /* LDS each block of the pass may fill with copies of the LUTs its
                             events use most: 0 = all the LDS its bins and cell tables leave;
                             n > 0 = at most n KiB; negative = none (every LUT read goes
                             through the caches) */
  int32_t device_mib_cap; /* debug: 0 = no cap; n > 0 = the context's device buffers may hold
                             at most n MiB together, and an allocation past that fails with
                             PA_ENOMEM as a real out-of-memory would (for testing the
                             out-of-memory paths; a failed load keeps the loaded data) */
  int32_t plain_bins;     /* timing aid for the paper's waveform-bin atomic stress test (its
                             high-activity synthetic waveforms with 1-8 toggles per cycle),
                             0, 1 or 2: 0 = atomic adds to the pass's per-cycle bins; 1 = plain
                             loads, adds and stores; 2 = plain stores of each contribution (the
                             no-atomic variant "regular writes" read literally).  With 1 or 2
                             the waveform, counts and leakage are wrong (updates are lost or
                             overwritten), so results are for timing only.  Used by the walk
                             kernel; the other kernels ignore it */
} pa_tunables;

/* Create a context on HIP device `hip_device`, launching on `hip_stream`
 * (a hipStream_t; NULL = the device's null stream).  `t` may be NULL. */
int pa_create(pa_ctx **out, int hip_device, void *hip_stream, const pa_tunables *t);
void pa_destroy(pa_ctx *ctx);
/* Change the stream later calls launch on (a hipStream_t). */
int pa_set_stream(pa_ctx *ctx, void *hip_stream);
const char *pa_last_error(void);
/* Change the timing mode of later pa_run calls (the time_kernels field:
 * 0, 1 or 2; PA_EINVAL otherwise). */
int pa_set_timing(pa_ctx *ctx, int32_t time_kernels);

/* Load the design (paper Sec. 2.4.1-2.4.2, Figs. 2-3: per-gate cell, state-
 * indexed internal-power LUTs per input pin, state-indexed leakage).
 *   gate_cell[G]   int32 cell id in [0, n_cells)
 *   gate_cap_F[G]  float64 total output load c (pin + wire), farads, finite
 *   cell_n_in[n_cells] int32 input count k in 1..8 (2^k states; the gate has k
 *                  input pins then one output pin)
 *   slew_axis[n_cells][n_slew]  float64 ticks, strictly increasing per cell
 *   cap_axis[n_cells][n_cap]    float64 farads, strictly increasing per cell
 *   lut_J   float64, per cell concatenated: [2^k][k][n_slew][n_cap] joules
 *   leak_W  float64, per cell concatenated: [2^k] watts
 *   2 <= n_slew, n_cap <= 16; the LUTs of all cells together hold fewer than
 *   2^31 entries and the leakage tables fewer than 2^28 (PA_EINVAL otherwise).
 *   Loading a design drops any loaded events. */
int pa_load_design(pa_ctx *ctx, int64_t n_gates, const int32_t *gate_cell, const double *gate_cap_F,
                   int32_t n_cells, const int32_t *cell_n_in, int32_t n_slew, int32_t n_cap,
                   const double *slew_axis, const double *cap_axis, const double *lut_J,
                   const double *leak_W, double vdd_V);

/* Load the activity (paper Sec. 2.4.1-2.4.2: per-pin sorted event streams).
 *   n_pins  must equal sum_g (k_g + 1); pins are gate-major, inputs 0..k-1,
 *           output k; the design may hold at most 2^22 - 1 gates here
 *   n_events must equal pin_ptr[n_pins]; 0 <= n_events < 2^31
 *   pin_ptr[P+1]  int64 CSR offsets, pin_ptr[0] = 0, nondecreasing
 *   pin_init[P]   uint8 value of the pin at t = 0, in {0, 1}
 *   evt_t[E]      int64 ticks, strictly increasing per pin, 0 <= t < t_max
 *   evt_val[E]    uint8 new value, alternating per pin starting from !init
 *   evt_slew[E]   float32 ticks, finite and > 0 (same unit as slew_axis)
 *   t_clk  clock period in ticks, 1 <= t_clk <= 2^(32 - b) where b is the
 *          bit count of the largest input count k of the design (b = 1 for
 *          k = 1, 2 for k = 2..3, 3 for k = 4..7, 4 for k = 8);
 *   t_max > 0 analysis end, at most 2^28 clock cycles; tick_s seconds per
 *   tick (> 0).
 * The events are validated (PA_EDATA for a broken rule above; the
 * previously loaded events stay usable) and re-laid out into library-owned
 * memory: time chunks of chunk_cycles cycles; every gate's part of a chunk
 * is cut into 2^s equal windows sized from the gate's event density (the
 * paper's event-density-aware per-gate cycle partitioning), a gate's input
 * events and its output events in windows of their own, the events of a
 * window in clock cycle, time and pin order.  The pass's blocks are cut so
 * that each carries about the same walk cost (events and window heads);
 * a block's windows go in phases of up to 64 windows of one pin kind, dealt
 * to its waves by cost, one window per lane, and every lane walks its window
 * event by event.  Besides the 16-byte event records the layout keeps an
 * 8-byte record per slot (cycle, tick and pin packed into 32 bits, the slew
 * as float32) that the pass streams when the sizes allow. */
int pa_load_events(pa_ctx *ctx, int64_t n_pins, int64_t n_events, const int64_t *pin_ptr,
                   const uint8_t *pin_init, const int64_t *evt_t, const uint8_t *evt_val,
                   const float *evt_slew, int64_t t_clk, int64_t t_max, double tick_s);

typedef struct {
  double p_int_W, p_sw_W, p_gl_W, p_leak_W; /* Eq. 3 powers */
  double e_int_J, e_sw_J, e_gl_J, e_leak_J; /* energies over [0, t_max) */
  uint64_t n_events, n_glitches;
  int64_t n_cycles;
} pa_totals;

/* One pass of the power analysis over the loaded design and events.
 *   out            HOST pointer, filled on return (pa_run synchronizes its stream)
 *   wave_J[C]      device: energy per cycle bin, J (power = wave_J[c] / (len_c * tick_s))
 *   cyc_events[C]  device: number of events whose cycle is c
 *   cyc_glitches[C] device: number of glitch events in cycle c
 *   evt_glitch[E]  device or NULL: 1 if the event is a glitch (caller's CSR order)
 *   evt_state_before[E] device or NULL: S(t-) of input-pin events, 0 for output
 *                  events (caller's CSR order)
 * C = n_cycles = ceil(t_max / t_clk).  The output arrays must not overlap.
 * With per-event outputs and the walk kernel (pa_info.walk_kernel), the kernel
 * writes them in its stream's order and a small kernel moves them into the
 * caller's order through every event's slot; the first such call builds that
 * map (4 bytes per event and 2 per stream slot of device memory, kept until
 * the next pa_load_events).  From run to run of one loaded layout, the
 * dynamic energies, every count and the per-event outputs repeat bit for bit;
 * the waveform bins and the leakage total, built with atomic adds in LDS
 * whose order between waves is free, repeat to rounding (about 1e-16
 * relative). */
int pa_run(pa_ctx *ctx, pa_totals *out, double *wave_J, uint64_t *cyc_events, uint64_t *cyc_glitches,
           uint8_t *evt_glitch, uint8_t *evt_state_before);

/* pa_run for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments, kernels and results, but the pass's own device scratch -- the
 * per-block cycle bins, cycle counts and block totals and the finalize's
 * result slots -- lives in one array of PA_NOALLOC_SCRATCH_BYTES that the
 * library holds per device for the life of the process, and the call
 * allocates nothing (no hipMalloc, no hipFree, no allocating library call).
 * The loaded events need 2 * blocks * chunk_cycles * 8 + blocks * 64 + 128
 * bytes of it (pieces rounded up to 256 bytes; blocks and chunk_cycles as
 * pa_get_info reports them); more is PA_EINVAL (pa_run has no such limit).
 * Every call on a device shares that device's array: calls that overlap in
 * time on one device (two contexts on two streams, or two threads) race and
 * give wrong results; calls that follow one another are safe (every call
 * rewrites all of the array it reads).  PA_EHIP if the array's device
 * address could not be looked up when the context was created.  Per-event
 * outputs take the walk kernel only when a pa_run with per-event outputs
 * has built its map for the loaded events; otherwise the general kernel. */
#define PA_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)
int pa_run_noalloc(pa_ctx *ctx, pa_totals *out, double *wave_J, uint64_t *cyc_events, uint64_t *cyc_glitches,
                   uint8_t *evt_glitch, uint8_t *evt_state_before);

/* pa_run plus every gate's own energies, the per-gate power the paper ranks
 * hotspots by (its spatial-accuracy evaluation, Fig. 10, Table 3):
 *   gate_J[G][4]   device: per gate (caller's order) the internal, switching,
 *                  glitch and leakage energy over [0, t_max), J; overwritten.
 * The gate rows add up to the totals (up to fp64 summation order).  With
 * the walk kernel (pa_info.walk_kernel) every window's energies and the
 * leakage of its power changes are stored at the window's header in the
 * lane streams, and kernels after the walk add each gate's windows in a
 * fixed order (the load ranks the windows gate-major): the rows repeat bit
 * for bit from run to run.  The first such call allocates room for the
 * window sums (16 bytes a slot of the lane streams, pa_info.n_slots; kept
 * until the next load).  Otherwise the diagnostic variant of the general
 * kernel adds them event by event with device atomics, so the rows may
 * differ between runs in the last bits.  The totals and the waveform
 * behave as in pa_run either way (dynamic energies and counts bit for bit,
 * the waveform bins and the leakage total to rounding). */
int pa_run_gates(pa_ctx *ctx, pa_totals *out, double *wave_J, uint64_t *cyc_events, uint64_t *cyc_glitches,
                 double *gate_J);

/* Events per window of the loaded layout (HOST struct): the windows are the
 * (chunk, gate, window) pieces whose first event carries the gate's state. */
typedef struct {
  int64_t n_windows;
  double mean;
  int64_t p50, p90, p99, max;
} pa_window_stats;
int pa_get_window_stats(pa_ctx *ctx, pa_window_stats *out);

/* Layout and launch facts of the loaded data (HOST struct). */
typedef struct {
  int64_t n_gates, n_pins, n_events, n_cycles;
  int32_t chunk_cycles, n_chunks;
  int32_t grid_blocks, block_threads;
  int32_t batch_events;       /* events one wave takes per step of the pass */
  int32_t max_segment_events; /* 0: no limit on the events of one gate in one clock cycle */
  int64_t device_bytes;       /* library-owned device memory: the loaded design and events, the
                                 per-pass scratch, and the staging of pa_run_text (the load's own
                                 scratch is freed when pa_load_events returns) */
  float kernel_ms[4];         /* last timed pa_run: fused, finalize, (unused), whole pass; mode 2 fills only the last */
  int64_t n_windows;          /* density-aware windows of the layout */
  int64_t n_slots;            /* slots of the pass's lane streams: the events, two header slots per
                                 window (walk kernel), and the empty slots that pad a phase's lanes to even
                                 lengths and to the phase's longest */
  int32_t wave_steps_max;     /* steps (event pairs) of the pass's longest wave */
  float wave_steps_mean;      /* steps of a wave, averaged over the waves with work */
  int32_t tables_in_lds;      /* 1: every block of the pass stages the per-cell tables (axes,
                                 slew thresholds, leakage) in LDS; 0: they are read through the
                                 caches (libraries too large for the LDS next to the bins) */
  int32_t walk_kernel;        /* 1: a pass over the loaded events without per-event or per-gate outputs
                                 (pa_run without them, pa_run_noalloc) runs the walk kernel (7- or
                                 8-point axes, every block's LUT range fits its LDS); 0: it runs the
                                 general pass kernel */
} pa_info;
int pa_get_info(pa_ctx *ctx, pa_info *info);

/* ---- Activity text: host-side event packing, overlapped with the GPU ----
 * The paper's GPU flow packs the events of its activity files on host
 * threads while the GPU computes, so that packing hides behind the power
 * computation (its end-to-end runtime breakdown, Fig. 13).  The text
 * read here is a subset of VCD with one slew per value change (the paper
 * does not print its input format; slews come from timing analysis there):
 *   - "$var <type> 1 <id> <name> [<more>] $end" declares one variable per
 *     pin, in the pin order of pa_load_events; other "$<keyword> ... $end"
 *     sections of the definitions are skipped; "$enddefinitions $end" ends
 *     them;
 *   - optionally "#0", then "$dumpvars <v><id> ... $end": the value of every
 *     pin at t = 0 (each pin at least once; the last entry counts);
 *   - then lines "#<t>" (a timestamp in ticks, nondecreasing, at most 18
 *     digits) and "<v><id> <slew>" (a value change at the current time; the
 *     slew in ticks as a decimal number, read as the nearest float32); the
 *     value changes before the first "#<t>" of the body are at t = 0; blank
 *     lines are allowed;
 *   <v> is 0 or 1; <id> is 1..8 characters in '!'..'~'.  Anything else
 *   (x/z values, vectors, unknown identifiers, other sections after
 *   $dumpvars, decreasing timestamps) is PA_EDATA, with the byte offset in
 *   pa_last_error().  The rules of pa_load_events (strictly increasing
 *   times per pin, values alternating from the initial value, slews finite
 *   and > 0) are checked where the events are loaded.
 *
 * pa_pack_text: the whole text as one CSR, in HOST memory (no device, no
 * context).  text[text_len] is host memory; n_pins must equal the declared
 * variables (PA_EDATA otherwise).  n_threads host threads (0 = min(16,
 * hardware threads), at most 256).  *n_events receives the number of value
 * changes.  With pin_ptr, pin_init, evt_t, evt_val and evt_slew all NULL
 * nothing else is written (a size query); otherwise all must be given,
 * pin_ptr[n_pins + 1], pin_init[n_pins], and the event arrays of max_events
 * entries (PA_EINVAL if fewer than *n_events).  At most 2^31 - 1 events. */
int pa_pack_text(const char *text, int64_t text_len, int64_t n_pins, int32_t n_threads, int64_t max_events,
                 int64_t *n_events, int64_t *pin_ptr, uint8_t *pin_init, int64_t *evt_t, uint8_t *evt_val,
                 float *evt_slew);

typedef struct {
  int32_t segment_cycles; /* clock cycles per segment (0 = 1024) */
  int32_t n_threads;      /* host threads that parse (0 = min(16, hardware threads)), at most 256 */
  int32_t serial;         /* 0: parse segment k + 1 while the GPU loads and computes segment k;
                             1: one after the other (to measure what the overlap hides) */
  int32_t reserved;       /* 0 */
} pa_text_opts;

typedef struct {
  int64_t n_segments, n_events, max_segment_events, text_bytes;
  double header_s; /* definitions and initial values (one thread) */
  double index_s;  /* cutting the value changes into segments (all threads) */
  double parse_s;  /* parsing and packing the segments, summed */
  double gpu_s;    /* copies, event loads and passes of the segments, summed */
  double wall_s;   /* the whole call */
} pa_text_stats;

/* The power analysis of an activity text: pa_load_events + pa_run over the
 * text's events, computed segment by segment.  Segment k holds clock cycles
 * [k S, (k + 1) S) (S = segment_cycles; the last may be shorter); host
 * threads parse and pack segment k + 1 into pinned host memory while a
 * second host thread copies segment k to the device, loads it (the load's
 * validation, layout and windows) and runs the pass into wave_J[k S ...],
 * cyc_events[k S ...] and cyc_glitches[k S ...].  Every quantity the paper
 * defines stays inside a clock cycle, given the pin values at the cycle
 * start, so the segments are independent: the waveform and counts equal
 * those of one pa_load_events + pa_run of the whole trace, and the totals
 * equal them up to fp64 summation order.
 *   text[text_len]  HOST memory (the format above)
 *   t_clk, t_max, tick_s  as for pa_load_events
 *   opts    may be NULL (all defaults); stats (HOST) may be NULL
 *   out     HOST totals over [0, t_max)
 *   wave_J, cyc_events, cyc_glitches  device, C = ceil(t_max / t_clk) entries
 * Needs a loaded design (PA_ESTATE).  The context holds no events afterwards
 * (pa_run then reports PA_ESTATE until the next pa_load_events). */
int pa_run_text(pa_ctx *ctx, const char *text, int64_t text_len, int64_t t_clk, int64_t t_max, double tick_s,
                const pa_text_opts *opts, pa_totals *out, double *wave_J, uint64_t *cyc_events,
                uint64_t *cyc_glitches, pa_text_stats *stats);

#ifdef __cplusplus
}
#endif
#endif
