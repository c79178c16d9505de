/*
 * pa_oracle.c -- plain, slow, single-threaded CPU oracle for gate-level
 * time-based power analysis.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the reference that the HIP path is
 * checked against.  Only tests/, __graft_entry__.smoke() and the cpu_baseline
 * leg of bench.py may load or call it.  The product library never links,
 * loads or calls it, and it shares no source, header, table or helper with
 * the product library.
 *
 * Source of the method: "GPU-Accelerated Gate-Level Time-Based Power
 * Analysis via Event-Density-Aware Partitioning and Kernel Fusion"
 * (arXiv 2609.05960), called "the paper" below.  Every step cites the
 * paper's section, equation or figure it follows.  The paper's display
 * equations (Eqs. 1-4) are not printed in the available text; where a form
 * had to be fixed, the reading is stated at the step and listed in the
 * design notes of the repository.
 *
 * What is computed (the plain definition; no blocking, no fusion, no
 * reordering of the sums beyond what the definition states):
 *   for every gate, walk the merged per-pin event streams in time order
 *   (paper, Sec. 2.4.2 and Fig. 3), and at each distinct timestamp
 *     1. charge the leakage of the interval that ends there at the state the
 *        gate held during it (Eq. 4), split over the clock-cycle bins it
 *        overlaps in proportion to the overlap (Sec. 2.4.2);
 *     2. for every pin with an event there (Fig. 7, the loop over pins with an
 *        event at t_cur): internal energy from the LUT that the state before
 *        the event selects, interpolated bilinearly on input slew and output
 *        load (Sec. 2.4.1, Fig. 2); switching energy 1/2 c v^2 for a 0->1
 *        event on the output pin (Eq. 1); clock-cycle glitch detection with a
 *        per-pin event counter (Sec. 2.4.1, Fig. 7 GlitchDetectUpdate) and
 *        scaling of a glitch's dynamic energy by r_gl (Eq. 2); the event's
 *        energy goes into the bin of its clock cycle (Sec. 2.4.1);
 *     3. apply every event at that timestamp to the gate state (Sec. 2.4.2).
 *   The interval after the last event runs to t_max.  Powers are energies
 *   over the analysis window (Eq. 3).
 *
 * Readings fixed here because the available text does not print them:
 *   - Eq. 1: E_sw = 0.5 * c * Vdd^2 for each 0->1 event on the output pin;
 *     a 1->0 output event carries no switching energy.
 *   - Eq. 2: r_gl = min(1, pw / ((rSlew + fSlew) / 2)) where pw is the time
 *     since the previous event on the same pin and rSlew, fSlew are the
 *     slews of that previous event and of the current one (the rise and the
 *     fall that bound the pulse).  Parity of this form against the paper is
 *     unpinned: the paper does not print it.
 *   - Glitch rule: per pin, the m-th event (m >= 2) of that pin inside one
 *     clock cycle is a glitch; the first event of a pin in a cycle is
 *     regular (Fig. 7, GlitchDetectUpdate).  A glitch adds r_gl * E to the
 *     glitch component and to the waveform, and nothing to the internal or
 *     switching component.
 *   - Eq. 3: P = E / (t_max * tick_s).  Eq. 4: E_leak = p_leak * dt * tick_s.
 *   - Gate state S = sum_i v_i 2^i over the input pins (pin 0 is the least
 *     significant bit); the output pin does not enter the state.
 *   - Bins are the half-open cycles [c T, (c+1) T); N_cyc = ceil(t_max / T);
 *     the last bin may be partial.
 *   - Bilinear interpolation: segment i = clamp(#{axis_j <= x} - 1, 0, n-2),
 *     fraction (x - x_i) / (x_{i+1} - x_i), extrapolating linearly outside.
 *   - Units: timestamps, T, t_max and slews in ticks; tick_s seconds per
 *     tick; cap in F, LUT in J, leakage in W, Vdd in V.  Slews arrive as
 *     fp32 and are widened to fp64 before any arithmetic.
 *
 * Every total and every bin is a Neumaier-compensated fp64 sum.
 *
 * pa_oracle_run_mt walks the same gates with the same per-gate code on host
 * threads: each thread takes a contiguous gate range with its own bins,
 * totals and counts, and the ranges are merged in order afterwards (again
 * with compensated sums).  Gates are independent apart from these shared
 * sums, so the result is the single-threaded one up to the order of fp64
 * additions; integer outputs are identical.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "pa_oracle.h"

/* ---------------------------------------------------------------- sums -- */

typedef struct {
  double s, c;
} nsum;

static void nadd(nsum *a, double x) {
  double t = a->s + x;
  if (fabs(a->s) >= fabs(x))
    a->c += (a->s - t) + x;
  else
    a->c += (x - t) + a->s;
  a->s = t;
}

static double nval(const nsum *a) { return a->s + a->c; }

/* ------------------------------------------------- bilinear LUT lookup -- */

/* Segment and fraction of x on a strictly increasing axis of n >= 2 points.
 * NLDM table lookup (paper, Sec. 2.4.1, Fig. 2) read as bilinear
 * interpolation that extrapolates linearly outside the axis range. */
static void axis_locate(const double *axis, int n, double x, int *seg, double *frac) {
  int m = 0;
  for (int j = 0; j < n; ++j)
    if (axis[j] <= x) m++;
  int i = m - 1;
  if (i < 0) i = 0;
  if (i > n - 2) i = n - 2;
  *seg = i;
  *frac = (x - axis[i]) / (axis[i + 1] - axis[i]);
}

double pa_oracle_bilerp(int n_slew, int n_cap, const double *slew_axis, const double *cap_axis,
                        const double *table, double x_slew, double x_cap) {
  int i, j;
  double a, b;
  axis_locate(slew_axis, n_slew, x_slew, &i, &a);
  axis_locate(cap_axis, n_cap, x_cap, &j, &b);
  double l00 = table[i * n_cap + j];
  double l01 = table[i * n_cap + j + 1];
  double l10 = table[(i + 1) * n_cap + j];
  double l11 = table[(i + 1) * n_cap + j + 1];
  return (1.0 - a) * (1.0 - b) * l00 + a * (1.0 - b) * l10 + (1.0 - a) * b * l01 + a * b * l11;
}

/* ------------------------------------------------------------ validation -- */

int64_t pa_oracle_n_cycles(int64_t t_clk, int64_t t_max) {
  if (t_clk <= 0 || t_max <= 0) return -1;
  return (t_max + t_clk - 1) / t_clk;
}

static int valid_design(int64_t n_gates, const int32_t *gate_cell, const double *gate_cap, int32_t n_cells,
                        const int32_t *cell_n_in, int32_t n_slew, int32_t n_cap, const double *slew_axis,
                        const double *cap_axis) {
  if (n_gates < 0 || n_cells < 1 || n_slew < 2 || n_cap < 2) return PA_ORACLE_EARG;
  for (int32_t c = 0; c < n_cells; ++c) {
    if (cell_n_in[c] < 1 || cell_n_in[c] > 8) return PA_ORACLE_EDATA;
    for (int j = 0; j + 1 < n_slew; ++j)
      if (!(slew_axis[(int64_t)c * n_slew + j] < slew_axis[(int64_t)c * n_slew + j + 1])) return PA_ORACLE_EDATA;
    for (int j = 0; j + 1 < n_cap; ++j)
      if (!(cap_axis[(int64_t)c * n_cap + j] < cap_axis[(int64_t)c * n_cap + j + 1])) return PA_ORACLE_EDATA;
  }
  for (int64_t g = 0; g < n_gates; ++g) {
    if (gate_cell[g] < 0 || gate_cell[g] >= n_cells) return PA_ORACLE_EDATA;
    if (!isfinite(gate_cap[g])) return PA_ORACLE_EDATA;
  }
  return 0;
}

static int valid_events(int64_t n_pins, const int64_t *pin_ptr, const uint8_t *pin_init, const int64_t *evt_t,
                        const uint8_t *evt_val, const float *evt_slew, int64_t t_clk, int64_t t_max,
                        double tick_s) {
  if (n_pins < 0 || t_clk <= 0 || t_max <= 0 || !(tick_s > 0.0)) return PA_ORACLE_EARG;
  if (pin_ptr[0] != 0) return PA_ORACLE_EDATA;
  for (int64_t p = 0; p < n_pins; ++p) {
    if (pin_ptr[p + 1] < pin_ptr[p]) return PA_ORACLE_EDATA;
    if (pin_init[p] > 1) return PA_ORACLE_EDATA;
    uint8_t v = pin_init[p];
    for (int64_t e = pin_ptr[p]; e < pin_ptr[p + 1]; ++e) {
      if (evt_t[e] < 0 || evt_t[e] >= t_max) return PA_ORACLE_EDATA;
      if (e > pin_ptr[p] && !(evt_t[e] > evt_t[e - 1])) return PA_ORACLE_EDATA;
      if (evt_val[e] != (uint8_t)(1 - v)) return PA_ORACLE_EDATA;
      v = evt_val[e];
      if (!(evt_slew[e] > 0.0f) || !isfinite(evt_slew[e])) return PA_ORACLE_EDATA;
    }
  }
  return 0;
}

/* ------------------------------------------------------------- the run -- */

/* What every gate walk reads (shared, read-only). */
typedef struct {
  int32_t n_slew, n_cap;
  const int32_t *gate_cell, *cell_n_in;
  const double *gate_cap, *slew_axis, *cap_axis, *lut, *leak;
  const int64_t *pin_base, *lut_base, *leak_base; /* per gate / per cell */
  const int64_t *pin_ptr, *evt_t;
  const uint8_t *pin_init, *evt_val;
  const float *evt_slew;
  double vdd, tick_s;
  int64_t T, t_max, n_cyc;
} run_in;

/* What a gate walk adds to: the waveform bins, the totals and the per-cycle
 * counts of the gates it walks (one set per thread), plus the current gate's
 * own share. */
typedef struct {
  nsum *wave;
  nsum e_int, e_sw, e_gl, e_leak;
  uint64_t *cyc_events, *cyc_glitches;
  uint64_t n_events, n_glitches;
  nsum g_int, g_sw, g_gl, g_leak;
} run_acc;

/* Leakage of the interval [a, b) at constant power p (paper, Sec. 2.4.2,
 * Eq. 4): energy p * (b - a) * tick_s, added to every overlapped cycle bin in
 * proportion to the overlap. */
static void leak_interval(const run_in *I, run_acc *R, double p, int64_t a, int64_t b) {
  if (b <= a) return;
  nadd(&R->e_leak, p * (double)(b - a) * I->tick_s);
  nadd(&R->g_leak, p * (double)(b - a) * I->tick_s);
  int64_t c_lo = a / I->T;
  int64_t c_hi = (b + I->T - 1) / I->T; /* exclusive */
  for (int64_t c = c_lo; c < c_hi; ++c) {
    int64_t lo = a > c * I->T ? a : c * I->T;
    int64_t hi = b < (c + 1) * I->T ? b : (c + 1) * I->T;
    if (hi > lo) nadd(&R->wave[c], p * (double)(hi - lo) * I->tick_s);
  }
}

/* Walk gates [g_lo, g_hi) one after the other, each in time order. */
static void walk_gates(const run_in *I, run_acc *R, int64_t g_lo, int64_t g_hi, uint8_t *evt_glitch,
                       uint8_t *evt_state_before, double *gate_J) {
  const int64_t *pin_ptr = I->pin_ptr, *evt_t = I->evt_t;
  const uint8_t *pin_init = I->pin_init, *evt_val = I->evt_val;
  const float *evt_slew = I->evt_slew;
  const int32_t n_slew = I->n_slew, n_cap = I->n_cap;
  const double vdd_V = I->vdd;
  for (int64_t g = g_lo; g < g_hi; ++g) {
    const int32_t cell = I->gate_cell[g];
    const int k = I->cell_n_in[cell];
    const double cap = I->gate_cap[g];
    const int64_t p0 = I->pin_base[g];
    int64_t cur[9], end[9], last_cyc[9], tprev[9];
    double sprev[9];
    uint8_t v[9];
    for (int i = 0; i <= k; ++i) {
      cur[i] = pin_ptr[p0 + i];
      end[i] = pin_ptr[p0 + i + 1];
      v[i] = pin_init[p0 + i];
      last_cyc[i] = -1;
      tprev[i] = 0;
      sprev[i] = 0.0;
    }
    unsigned S = 0; /* state over input pins, pin 0 = LSB */
    for (int i = 0; i < k; ++i) S |= (unsigned)v[i] << i;
    const double *cell_slew = I->slew_axis + (int64_t)cell * n_slew;
    const double *cell_cap = I->cap_axis + (int64_t)cell * n_cap;
    int64_t t_last = 0;
    memset(&R->g_int, 0, sizeof R->g_int);
    memset(&R->g_sw, 0, sizeof R->g_sw);
    memset(&R->g_gl, 0, sizeof R->g_gl);
    memset(&R->g_leak, 0, sizeof R->g_leak);

    for (;;) {
      /* next distinct timestamp of the k-way merge (Sec. 2.4.2, Fig. 3) */
      int64_t t = INT64_MAX;
      for (int i = 0; i <= k; ++i)
        if (cur[i] < end[i] && evt_t[cur[i]] < t) t = evt_t[cur[i]];
      if (t == INT64_MAX) break;

      /* leakage of the interval that ends here, at the state held in it */
      leak_interval(I, R, I->leak[I->leak_base[cell] + S], t_last, t);

      /* dynamic energy of every pin with an event at t (Fig. 7) */
      for (int i = 0; i <= k; ++i) {
        if (!(cur[i] < end[i] && evt_t[cur[i]] == t)) continue;
        const int64_t e = cur[i];
        const double slew = (double)evt_slew[e];
        const int64_t cyc = t / I->T;
        double E;
        int is_int;
        if (i < k) { /* input pin: state-selected internal-power LUT (Fig. 2) */
          const double *tab = I->lut + I->lut_base[cell] + ((int64_t)S * k + i) * n_slew * n_cap;
          E = pa_oracle_bilerp(n_slew, n_cap, cell_slew, cell_cap, tab, slew, cap);
          is_int = 1;
        } else { /* output pin: Eq. 1 for a 0->1 event */
          E = evt_val[e] == 1 ? 0.5 * cap * vdd_V * vdd_V : 0.0;
          is_int = 0;
        }
        R->cyc_events[cyc] += 1;
        R->n_events += 1;
        /* GlitchDetectUpdate: a second or later event of this pin in the
         * current clock cycle is a glitch (Sec. 2.4.1, Fig. 7) */
        const int glitch = (last_cyc[i] == cyc);
        if (glitch) {
          const double pw = (double)(t - tprev[i]);
          double r = pw / (0.5 * (slew + sprev[i])); /* Eq. 2 as read above */
          if (r > 1.0) r = 1.0;
          nadd(&R->e_gl, r * E);
          nadd(&R->g_gl, r * E);
          nadd(&R->wave[cyc], r * E);
          R->cyc_glitches[cyc] += 1;
          R->n_glitches += 1;
        } else {
          nadd(is_int ? &R->e_int : &R->e_sw, E);
          nadd(is_int ? &R->g_int : &R->g_sw, E);
          nadd(&R->wave[cyc], E);
        }
        if (evt_glitch) evt_glitch[e] = (uint8_t)glitch;
        if (evt_state_before) evt_state_before[e] = (uint8_t)(i < k ? S : 0);
        last_cyc[i] = cyc;
        tprev[i] = t;
        sprev[i] = slew;
      }

      /* apply every event at t, then rebuild the state (Sec. 2.4.2) */
      for (int i = 0; i <= k; ++i) {
        if (cur[i] < end[i] && evt_t[cur[i]] == t) {
          v[i] = evt_val[cur[i]];
          cur[i] += 1;
        }
      }
      S = 0;
      for (int i = 0; i < k; ++i) S |= (unsigned)v[i] << i;
      t_last = t;
    }
    /* leakage is always present: the last interval runs to t_max */
    leak_interval(I, R, I->leak[I->leak_base[cell] + S], t_last, I->t_max);
    /* the gate's own energies (the per-gate output the paper ranks hotspots by,
     * its spatial-accuracy evaluation: Table 3, Figs. 10-11) */
    if (gate_J) {
      gate_J[4 * g + 0] = nval(&R->g_int);
      gate_J[4 * g + 1] = nval(&R->g_sw);
      gate_J[4 * g + 2] = nval(&R->g_gl);
      gate_J[4 * g + 3] = nval(&R->g_leak);
    }
  }
}

/* Shared set-up of both entry points: validation and the per-gate / per-cell
 * bases.  On success the caller owns the three arrays in *I. */
static int set_up(run_in *I, int64_t n_gates, const int32_t *gate_cell, const double *gate_cap_F, int32_t n_cells,
                  const int32_t *cell_n_in, int32_t n_slew, int32_t n_cap, const double *slew_axis,
                  const double *cap_axis, const double *lut_J, const double *leak_W, double vdd_V, int64_t n_pins,
                  const int64_t *pin_ptr, const uint8_t *pin_init, const int64_t *evt_t, const uint8_t *evt_val,
                  const float *evt_slew, int64_t t_clk, int64_t t_max, double tick_s, int64_t gate_lo,
                  int64_t gate_hi) {
  int rc = valid_design(n_gates, gate_cell, gate_cap_F, n_cells, cell_n_in, n_slew, n_cap, slew_axis, cap_axis);
  if (rc) return rc;
  rc = valid_events(n_pins, pin_ptr, pin_init, evt_t, evt_val, evt_slew, t_clk, t_max, tick_s);
  if (rc) return rc;
  if (gate_lo < 0 || gate_hi > n_gates || gate_lo > gate_hi) return PA_ORACLE_EARG;
  memset(I, 0, sizeof *I);
  /* gate-major pins: gate g owns k_g input pins followed by one output pin */
  int64_t *pin_base = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_gates + 1));
  int64_t *lut_base = (int64_t *)malloc(sizeof(int64_t) * (size_t)n_cells);
  int64_t *leak_base = (int64_t *)malloc(sizeof(int64_t) * (size_t)n_cells);
  if (!pin_base || !lut_base || !leak_base) {
    free(pin_base); free(lut_base); free(leak_base);
    return PA_ORACLE_ENOMEM;
  }
  pin_base[0] = 0;
  for (int64_t g = 0; g < n_gates; ++g) pin_base[g + 1] = pin_base[g] + cell_n_in[gate_cell[g]] + 1;
  if (pin_base[n_gates] != n_pins) {
    free(pin_base); free(lut_base); free(leak_base);
    return PA_ORACLE_EDATA;
  }
  int64_t lb = 0, kb = 0;
  for (int32_t c = 0; c < n_cells; ++c) {
    int64_t k = cell_n_in[c];
    lut_base[c] = lb;
    leak_base[c] = kb;
    lb += ((int64_t)1 << k) * k * n_slew * n_cap;
    kb += (int64_t)1 << k;
  }
  I->n_slew = n_slew; I->n_cap = n_cap;
  I->gate_cell = gate_cell; I->cell_n_in = cell_n_in; I->gate_cap = gate_cap_F;
  I->slew_axis = slew_axis; I->cap_axis = cap_axis; I->lut = lut_J; I->leak = leak_W;
  I->pin_base = pin_base; I->lut_base = lut_base; I->leak_base = leak_base;
  I->pin_ptr = pin_ptr; I->evt_t = evt_t; I->pin_init = pin_init; I->evt_val = evt_val; I->evt_slew = evt_slew;
  I->vdd = vdd_V; I->tick_s = tick_s; I->T = t_clk; I->t_max = t_max;
  I->n_cyc = pa_oracle_n_cycles(t_clk, t_max);
  return 0;
}

static void free_in(run_in *I) {
  free((void *)I->pin_base);
  free((void *)I->lut_base);
  free((void *)I->leak_base);
}

static void write_totals(const run_in *I, const run_acc *R, pa_oracle_totals *out) {
  const double window_s = (double)I->t_max * I->tick_s;
  out->e_int_J = nval(&R->e_int);
  out->e_sw_J = nval(&R->e_sw);
  out->e_gl_J = nval(&R->e_gl);
  out->e_leak_J = nval(&R->e_leak);
  out->p_int_W = out->e_int_J / window_s; /* Eq. 3 */
  out->p_sw_W = out->e_sw_J / window_s;
  out->p_gl_W = out->e_gl_J / window_s;
  out->p_leak_W = out->e_leak_J / window_s;
  out->n_events = R->n_events;
  out->n_glitches = R->n_glitches;
  out->n_cycles = I->n_cyc;
}

int pa_oracle_run(int64_t n_gates, const int32_t *gate_cell, const double *gate_cap_F, int32_t n_cells,
                  const int32_t *cell_n_in, int32_t n_slew, int32_t n_cap, const double *slew_axis,
                  const double *cap_axis, const double *lut_J, const double *leak_W, double vdd_V,
                  int64_t n_pins, const int64_t *pin_ptr, const uint8_t *pin_init, const int64_t *evt_t,
                  const uint8_t *evt_val, const float *evt_slew, int64_t t_clk, int64_t t_max, double tick_s,
                  int64_t gate_lo, int64_t gate_hi, pa_oracle_totals *out, double *wave_J,
                  uint64_t *cyc_events, uint64_t *cyc_glitches, uint8_t *evt_glitch,
                  uint8_t *evt_state_before, double *gate_J) {
  if (!out || !wave_J || !cyc_events || !cyc_glitches) return PA_ORACLE_EARG;
  run_in I;
  int rc = set_up(&I, n_gates, gate_cell, gate_cap_F, n_cells, cell_n_in, n_slew, n_cap, slew_axis, cap_axis, lut_J,
                  leak_W, vdd_V, n_pins, pin_ptr, pin_init, evt_t, evt_val, evt_slew, t_clk, t_max, tick_s, gate_lo,
                  gate_hi);
  if (rc) return rc;
  run_acc R;
  memset(&R, 0, sizeof R);
  R.wave = (nsum *)calloc((size_t)I.n_cyc, sizeof(nsum));
  if (!R.wave) {
    free_in(&I);
    return PA_ORACLE_ENOMEM;
  }
  memset(cyc_events, 0, sizeof(uint64_t) * (size_t)I.n_cyc);
  memset(cyc_glitches, 0, sizeof(uint64_t) * (size_t)I.n_cyc);
  R.cyc_events = cyc_events;
  R.cyc_glitches = cyc_glitches;
  walk_gates(&I, &R, gate_lo, gate_hi, evt_glitch, evt_state_before, gate_J);
  for (int64_t c = 0; c < I.n_cyc; ++c) wave_J[c] = nval(&R.wave[c]);
  write_totals(&I, &R, out);
  free(R.wave);
  free_in(&I);
  return 0;
}

/* ------------------------------------------------ the run on host threads -- */

typedef struct {
  const run_in *I;
  run_acc R;
  int64_t g_lo, g_hi;
  uint8_t *evt_glitch, *evt_state_before;
  double *gate_J;
} shard;

static void *shard_main(void *arg) {
  shard *s = (shard *)arg;
  walk_gates(s->I, &s->R, s->g_lo, s->g_hi, s->evt_glitch, s->evt_state_before, s->gate_J);
  return NULL;
}

int pa_oracle_run_mt(int64_t n_gates, const int32_t *gate_cell, const double *gate_cap_F, int32_t n_cells,
                     const int32_t *cell_n_in, int32_t n_slew, int32_t n_cap, const double *slew_axis,
                     const double *cap_axis, const double *lut_J, const double *leak_W, double vdd_V,
                     int64_t n_pins, const int64_t *pin_ptr, const uint8_t *pin_init, const int64_t *evt_t,
                     const uint8_t *evt_val, const float *evt_slew, int64_t t_clk, int64_t t_max, double tick_s,
                     int64_t gate_lo, int64_t gate_hi, int32_t n_threads, pa_oracle_totals *out, double *wave_J,
                     uint64_t *cyc_events, uint64_t *cyc_glitches, uint8_t *evt_glitch,
                     uint8_t *evt_state_before, double *gate_J) {
  if (!out || !wave_J || !cyc_events || !cyc_glitches || n_threads < 1 || n_threads > 1024) return PA_ORACLE_EARG;
  run_in I;
  int rc = set_up(&I, n_gates, gate_cell, gate_cap_F, n_cells, cell_n_in, n_slew, n_cap, slew_axis, cap_axis, lut_J,
                  leak_W, vdd_V, n_pins, pin_ptr, pin_init, evt_t, evt_val, evt_slew, t_clk, t_max, tick_s, gate_lo,
                  gate_hi);
  if (rc) return rc;
  const int64_t n = gate_hi - gate_lo;
  if (n_threads > n) n_threads = n > 0 ? (int32_t)n : 1;
  shard *sh = (shard *)calloc((size_t)n_threads, sizeof(shard));
  pthread_t *th = (pthread_t *)calloc((size_t)n_threads, sizeof(pthread_t));
  int ok = sh && th;
  for (int32_t i = 0; ok && i < n_threads; ++i) {
    sh[i].R.wave = (nsum *)calloc((size_t)I.n_cyc, sizeof(nsum));
    sh[i].R.cyc_events = (uint64_t *)calloc((size_t)I.n_cyc, sizeof(uint64_t));
    sh[i].R.cyc_glitches = (uint64_t *)calloc((size_t)I.n_cyc, sizeof(uint64_t));
    ok = sh[i].R.wave && sh[i].R.cyc_events && sh[i].R.cyc_glitches;
  }
  if (ok) {
    /* contiguous gate ranges of about equal work: a gate costs its events
     * and, through its leakage intervals, every cycle of the window */
    const int64_t *pb = I.pin_base;
    double total = 0.0;
    for (int64_t g = gate_lo; g < gate_hi; ++g) total += 32.0 * (double)(pin_ptr[pb[g + 1]] - pin_ptr[pb[g]]) + (double)I.n_cyc;
    double acc = 0.0;
    int64_t g = gate_lo;
    for (int32_t i = 0; i < n_threads; ++i) {
      sh[i].I = &I;
      sh[i].evt_glitch = evt_glitch;
      sh[i].evt_state_before = evt_state_before;
      sh[i].gate_J = gate_J;
      sh[i].g_lo = g;
      const double goal = total * (double)(i + 1) / (double)n_threads;
      while (g < gate_hi && (i == n_threads - 1 || acc < goal)) {
        acc += 32.0 * (double)(pin_ptr[pb[g + 1]] - pin_ptr[pb[g]]) + (double)I.n_cyc;
        ++g;
      }
      sh[i].g_hi = g;
    }
    int32_t started = 0;
    for (; started < n_threads; ++started)
      if (pthread_create(&th[started], NULL, shard_main, &sh[started]) != 0) break;
    for (int32_t i = 0; i < started; ++i) pthread_join(th[i], NULL);
    /* a thread that could not start: its gates run here */
    for (int32_t i = started; i < n_threads; ++i) shard_main(&sh[i]);
    /* merge in shard order: compensated sums of the shards' bins and totals */
    run_acc M;
    memset(&M, 0, sizeof M);
    for (int64_t c = 0; c < I.n_cyc; ++c) {
      nsum w = {0.0, 0.0};
      uint64_t ne = 0, ng = 0;
      for (int32_t i = 0; i < n_threads; ++i) {
        nadd(&w, nval(&sh[i].R.wave[c]));
        ne += sh[i].R.cyc_events[c];
        ng += sh[i].R.cyc_glitches[c];
      }
      wave_J[c] = nval(&w);
      cyc_events[c] = ne;
      cyc_glitches[c] = ng;
    }
    for (int32_t i = 0; i < n_threads; ++i) {
      nadd(&M.e_int, nval(&sh[i].R.e_int));
      nadd(&M.e_sw, nval(&sh[i].R.e_sw));
      nadd(&M.e_gl, nval(&sh[i].R.e_gl));
      nadd(&M.e_leak, nval(&sh[i].R.e_leak));
      M.n_events += sh[i].R.n_events;
      M.n_glitches += sh[i].R.n_glitches;
    }
    write_totals(&I, &M, out);
  }
  for (int32_t i = 0; sh && i < n_threads; ++i) {
    free(sh[i].R.wave);
    free(sh[i].R.cyc_events);
    free(sh[i].R.cyc_glitches);
  }
  free(sh);
  free(th);
  free_in(&I);
  return ok ? 0 : PA_ORACLE_ENOMEM;
}
