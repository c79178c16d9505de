/* Sanitizer driver for the CPU oracle (oracle/pa_oracle.c): reads a design
 * and trace written by tests/test_sanitizers.py as raw little-endian arrays,
 * runs the single-threaded walk and the threaded driver, and prints their
 * totals.  Built with -fsanitize=address,undefined; any report fails the
 * test.  Usage: oracle_driver <dir> <threads> */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pa_oracle.h"

static void *slurp(const char *dir, const char *name, size_t *n) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "rb");
  if (!f) { fprintf(stderr, "missing %s\n", path); exit(2); }
  fseek(f, 0, SEEK_END);
  long len = ftell(f);
  fseek(f, 0, SEEK_SET);
  void *p = malloc(len > 0 ? (size_t)len : 1);
  if (len > 0 && fread(p, 1, (size_t)len, f) != (size_t)len) exit(2);
  fclose(f);
  *n = (size_t)len;
  return p;
}

int main(int argc, char **argv) {
  if (argc != 3) return 2;
  const char *dir = argv[1];
  const int threads = atoi(argv[2]);
  size_t n;
  int64_t *scal = (int64_t *)slurp(dir, "scalars.bin", &n); /* G, n_cells, n_slew, n_cap, P, E, t_clk, t_max */
  double *fsc = (double *)slurp(dir, "fscalars.bin", &n);   /* vdd, tick_s */
  int32_t *gate_cell = (int32_t *)slurp(dir, "gate_cell.bin", &n);
  double *gate_cap = (double *)slurp(dir, "gate_cap.bin", &n);
  int32_t *cell_k = (int32_t *)slurp(dir, "cell_k.bin", &n);
  double *sa = (double *)slurp(dir, "slew_axis.bin", &n);
  double *ca = (double *)slurp(dir, "cap_axis.bin", &n);
  double *lut = (double *)slurp(dir, "lut.bin", &n);
  double *leak = (double *)slurp(dir, "leak.bin", &n);
  int64_t *pin_ptr = (int64_t *)slurp(dir, "pin_ptr.bin", &n);
  uint8_t *pin_init = (uint8_t *)slurp(dir, "pin_init.bin", &n);
  int64_t *et = (int64_t *)slurp(dir, "evt_t.bin", &n);
  uint8_t *ev = (uint8_t *)slurp(dir, "evt_val.bin", &n);
  float *es = (float *)slurp(dir, "evt_slew.bin", &n);
  const int64_t G = scal[0], P = scal[4], E = scal[5], T = scal[6], tmax = scal[7];
  const int64_t C = pa_oracle_n_cycles(T, tmax);
  double *wave = (double *)malloc(sizeof(double) * (size_t)C);
  uint64_t *ce = (uint64_t *)malloc(sizeof(uint64_t) * (size_t)C);
  uint64_t *cg = (uint64_t *)malloc(sizeof(uint64_t) * (size_t)C);
  uint8_t *fl = (uint8_t *)malloc((size_t)(E > 0 ? E : 1));
  uint8_t *st = (uint8_t *)malloc((size_t)(E > 0 ? E : 1));
  double *gj = (double *)malloc(sizeof(double) * 4 * (size_t)(G > 0 ? G : 1));
  pa_oracle_totals a, b;
  int rc1 = pa_oracle_run(G, gate_cell, gate_cap, (int32_t)scal[1], cell_k, (int32_t)scal[2], (int32_t)scal[3], sa,
                          ca, lut, leak, fsc[0], P, pin_ptr, pin_init, et, ev, es, T, tmax, fsc[1], 0, G, &a, wave,
                          ce, cg, fl, st, gj);
  int rc2 = pa_oracle_run_mt(G, gate_cell, gate_cap, (int32_t)scal[1], cell_k, (int32_t)scal[2], (int32_t)scal[3],
                             sa, ca, lut, leak, fsc[0], P, pin_ptr, pin_init, et, ev, es, T, tmax, fsc[1], 0, G,
                             threads, &b, wave, ce, cg, fl, st, gj);
  printf("%d %d %.17g %.17g %.17g %.17g %llu %llu\n", rc1, rc2, a.e_int_J, a.e_sw_J, a.e_gl_J, a.e_leak_J,
         (unsigned long long)a.n_events, (unsigned long long)b.n_glitches);
  free(scal); free(fsc); free(gate_cell); free(gate_cap); free(cell_k); free(sa); free(ca); free(lut);
  free(leak); free(pin_ptr); free(pin_init); free(et); free(ev); free(es); free(wave); free(ce); free(cg);
  free(fl); free(st); free(gj);
  return 0;
}
