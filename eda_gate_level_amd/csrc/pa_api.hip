// pa_api.hip -- the C ABI of include/pa.h: context, design and event loads,
// and the pass.  Argument marshalling, validation and launches only; every
// step of the power analysis runs in the gfx950 kernels of pa_pass.hip and
// pa_load.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "pa.h"
#include "pa_common.h"
#include "pa_load.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

// owning device buffer
struct DBuf {
  void *p = nullptr;
  size_t bytes = 0;
  DBuf() = default;
  DBuf(const DBuf &) = delete;
  DBuf &operator=(const DBuf &) = delete;
  DBuf(DBuf &&o) noexcept : p(o.p), bytes(o.bytes) { o.p = nullptr; o.bytes = 0; }
  DBuf &operator=(DBuf &&o) noexcept {
    if (this != &o) { reset(); p = o.p; bytes = o.bytes; o.p = nullptr; o.bytes = 0; }
    return *this;
  }
  ~DBuf() { reset(); }
  void reset() {
    if (p) (void)hipFree(p);
    p = nullptr;
    bytes = 0;
  }
  hipError_t alloc(size_t n) {
    reset();
    if (n == 0) n = 16;
    hipError_t e = hipMalloc(&p, n);
    if (e != hipSuccess) { p = nullptr; return e; }
    bytes = n;
    return hipSuccess;
  }
  template <class T> T *as() const { return static_cast<T *>(p); }
};

uint32_t bits_for(uint64_t v) {  // bits needed to hold 0..v (at least 1)
  uint32_t b = 1;
  while (b < 64 && (v >> b) != 0) ++b;
  return b;
}

struct Design {
  int64_t G = 0, P = 0;
  int32_t n_cells = 0, n_slew = 0, n_cap = 0, kmax = 0;
  int64_t n_leak = 0;
  double vdd = 0;
  DBuf cell_k, cell_lut_base, cell_leak_base, lut, leak, slew_axis, slew_invw;
  DBuf gate_info, gate_capfrac, gate_esw, gate_k, pin_base, pin_gate, pin_local;
  int64_t bytes() const {
    return (int64_t)(cell_k.bytes + cell_lut_base.bytes + cell_leak_base.bytes + lut.bytes + leak.bytes +
                     slew_axis.bytes + slew_invw.bytes + gate_info.bytes + gate_capfrac.bytes + gate_esw.bytes +
                     gate_k.bytes + pin_base.bytes + pin_gate.bytes + pin_local.bytes);
  }
};

struct Events {
  int64_t E = 0, C = 0, T = 0, t_max = 0, chunk_ticks = 0;
  double tick_s = 0;
  int32_t Cc = 0, Q = 0;
  uint32_t max_seg = 0;
  pa::KeyFmt kf{};
  DBuf key, slew, orig, chunk_base, pin_init;
  std::vector<uint32_t> h_chunk_base;
  DBuf rstart, rchunk;  // block ranges of the pass
  int32_t n_ranges = 0;
  DBuf acc_wave, acc_cnt, dP[2], tot[2], tot_cnt[2], res;
  int64_t bytes() const {
    int64_t b = (int64_t)(key.bytes + slew.bytes + orig.bytes + chunk_base.bytes + pin_init.bytes + acc_wave.bytes +
                          acc_cnt.bytes + res.bytes + rstart.bytes + rchunk.bytes);
    for (int s = 0; s < 2; ++s) b += (int64_t)(dP[s].bytes + tot[s].bytes + tot_cnt[s].bytes);
    return b;
  }
};

}  // namespace

struct pa_ctx {
  int device = 0;
  hipStream_t stream = nullptr;
  pa_tunables tun{};
  int n_cu = 0;
  bool has_design = false, has_events = false;
  Design d;
  Events ev;
  int parity = 0;
  double *h_res = nullptr;
  hipEvent_t tev[3] = {nullptr, nullptr, nullptr};
  float kernel_ms[4] = {0, 0, 0, 0};
  int last_grid = 0;
};

#define HIPCHK(expr)                                                                             \
  do {                                                                                           \
    hipError_t e_ = (expr);                                                                      \
    if (e_ != hipSuccess) {                                                                      \
      if (e_ == hipErrorOutOfMemory || e_ == hipErrorMemoryAllocation)                           \
        return fail(PA_ENOMEM, "out of device memory in %s", #expr);                            \
      return fail(PA_EHIP, "HIP error %s in %s", hipGetErrorString(e_), #expr);                 \
    }                                                                                            \
  } while (0)

extern "C" {

const char *pa_last_error(void) { return g_err.c_str(); }

int pa_create(pa_ctx **out, int hip_device, void *hip_stream, const pa_tunables *t) {
  if (!out) return fail(PA_EINVAL, "pa_create: out is NULL");
  *out = nullptr;
  int ndev = 0;
  HIPCHK(hipGetDeviceCount(&ndev));
  if (hip_device < 0 || hip_device >= ndev) return fail(PA_EINVAL, "pa_create: device %d of %d", hip_device, ndev);
  HIPCHK(hipSetDevice(hip_device));
  hipDeviceProp_t prop;
  HIPCHK(hipGetDeviceProperties(&prop, hip_device));
  pa_ctx *c = new (std::nothrow) pa_ctx();
  if (!c) return fail(PA_ENOMEM, "pa_create: host allocation");
  c->device = hip_device;
  c->stream = (hipStream_t)hip_stream;
  if (t) c->tun = *t;
  c->n_cu = prop.multiProcessorCount;
  if (hipHostMalloc((void **)&c->h_res, 16 * sizeof(double), hipHostMallocDefault) != hipSuccess) {
    delete c;
    return fail(PA_ENOMEM, "pa_create: pinned host buffer");
  }
  for (auto &e : c->tev) {
    if (hipEventCreate(&e) != hipSuccess) {
      pa_destroy(c);
      return fail(PA_EHIP, "pa_create: hipEventCreate");
    }
  }
  *out = c;
  return PA_OK;
}

void pa_destroy(pa_ctx *c) {
  if (!c) return;
  (void)hipSetDevice(c->device);
  if (c->stream) (void)hipStreamSynchronize(c->stream); else (void)hipDeviceSynchronize();
  for (auto &e : c->tev)
    if (e) (void)hipEventDestroy(e);
  if (c->h_res) (void)hipHostFree(c->h_res);
  delete c;
}

int pa_set_stream(pa_ctx *c, void *hip_stream) {
  if (!c) return fail(PA_EINVAL, "pa_set_stream: NULL context");
  c->stream = (hipStream_t)hip_stream;
  return PA_OK;
}

int pa_load_design(pa_ctx *c, int64_t n_gates, const int32_t *gate_cell, const double *gate_cap_F,
                   int32_t n_cells, const int32_t *cell_n_in, int32_t n_slew, int32_t n_cap,
                   const double *slew_axis, const double *cap_axis, const double *lut_J, const double *leak_W,
                   double vdd_V) {
  if (!c) return fail(PA_EINVAL, "pa_load_design: NULL context");
  if (n_gates < 0 || n_gates >= (int64_t(1) << 31)) return fail(PA_EINVAL, "pa_load_design: n_gates out of range");
  if (n_cells < 1 || n_cells > (1 << 24)) return fail(PA_EINVAL, "pa_load_design: n_cells out of range");
  if (n_slew < 2 || n_slew > 16 || n_cap < 2 || n_cap > 16)
    return fail(PA_EINVAL, "pa_load_design: LUT axes need 2..16 points");
  if (!cell_n_in || !slew_axis || !cap_axis || !lut_J || !leak_W || (n_gates > 0 && (!gate_cell || !gate_cap_F)))
    return fail(PA_EINVAL, "pa_load_design: NULL array");
  if (!std::isfinite(vdd_V)) return fail(PA_EINVAL, "pa_load_design: Vdd not finite");
  HIPCHK(hipSetDevice(c->device));
  hipStream_t s = c->stream;

  std::vector<int32_t> hk(n_cells);
  std::vector<double> hsa((size_t)n_cells * n_slew), hca((size_t)n_cells * n_cap);
  HIPCHK(hipMemcpyAsync(hk.data(), cell_n_in, sizeof(int32_t) * n_cells, hipMemcpyDeviceToHost, s));
  HIPCHK(hipMemcpyAsync(hsa.data(), slew_axis, sizeof(double) * hsa.size(), hipMemcpyDeviceToHost, s));
  HIPCHK(hipMemcpyAsync(hca.data(), cap_axis, sizeof(double) * hca.size(), hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));
  std::vector<uint32_t> lut_base(n_cells), leak_base(n_cells);
  uint64_t lb = 0, kb = 0;
  int32_t kmax = 0;
  for (int32_t i = 0; i < n_cells; ++i) {
    const int32_t k = hk[i];
    if (k < 1 || k > 8) return fail(PA_EDATA, "pa_load_design: cell %d has %d inputs (1..8 allowed)", i, k);
    kmax = std::max(kmax, k);
    lut_base[i] = (uint32_t)lb;
    leak_base[i] = (uint32_t)kb;
    lb += (uint64_t(1) << k) * (uint64_t)k * n_slew * n_cap;
    kb += uint64_t(1) << k;
    if (lb >= (uint64_t(1) << 32) || kb >= (uint64_t(1) << 32))
      return fail(PA_EINVAL, "pa_load_design: LUT tables exceed 2^32 entries");
    for (int j = 0; j + 1 < n_slew; ++j)
      if (!(hsa[(size_t)i * n_slew + j] < hsa[(size_t)i * n_slew + j + 1]))
        return fail(PA_EDATA, "pa_load_design: slew axis of cell %d not strictly increasing", i);
    for (int j = 0; j + 1 < n_cap; ++j)
      if (!(hca[(size_t)i * n_cap + j] < hca[(size_t)i * n_cap + j + 1]))
        return fail(PA_EDATA, "pa_load_design: cap axis of cell %d not strictly increasing", i);
  }
  std::vector<double> invw((size_t)n_cells * (n_slew - 1));
  for (int32_t i = 0; i < n_cells; ++i)
    for (int j = 0; j + 1 < n_slew; ++j)
      invw[(size_t)i * (n_slew - 1) + j] = 1.0 / (hsa[(size_t)i * n_slew + j + 1] - hsa[(size_t)i * n_slew + j]);

  Design d;
  d.G = n_gates;
  d.n_cells = n_cells;
  d.n_slew = n_slew;
  d.n_cap = n_cap;
  d.kmax = kmax;
  d.n_leak = (int64_t)kb;
  d.vdd = vdd_V;
  const int64_t G = n_gates;
  DBuf cap_axis_d, err;
  HIPCHK(d.cell_k.alloc(sizeof(int32_t) * n_cells));
  HIPCHK(d.cell_lut_base.alloc(sizeof(uint32_t) * n_cells));
  HIPCHK(d.cell_leak_base.alloc(sizeof(uint32_t) * n_cells));
  HIPCHK(d.lut.alloc(sizeof(double) * lb));
  HIPCHK(d.leak.alloc(sizeof(double) * kb));
  HIPCHK(d.slew_axis.alloc(sizeof(double) * hsa.size()));
  HIPCHK(d.slew_invw.alloc(sizeof(double) * invw.size()));
  HIPCHK(cap_axis_d.alloc(sizeof(double) * hca.size()));
  HIPCHK(d.gate_info.alloc(sizeof(uint32_t) * G));
  HIPCHK(d.gate_capfrac.alloc(sizeof(double) * G));
  HIPCHK(d.gate_esw.alloc(sizeof(double) * G));
  HIPCHK(d.gate_k.alloc(sizeof(int32_t) * G));
  HIPCHK(d.pin_base.alloc(sizeof(int64_t) * (G + 1)));
  HIPCHK(err.alloc(sizeof(uint32_t)));
  HIPCHK(hipMemcpyAsync(d.cell_k.p, hk.data(), sizeof(int32_t) * n_cells, hipMemcpyHostToDevice, s));
  HIPCHK(hipMemcpyAsync(d.cell_lut_base.p, lut_base.data(), sizeof(uint32_t) * n_cells, hipMemcpyHostToDevice, s));
  HIPCHK(hipMemcpyAsync(d.cell_leak_base.p, leak_base.data(), sizeof(uint32_t) * n_cells, hipMemcpyHostToDevice, s));
  HIPCHK(hipMemcpyAsync(d.lut.p, lut_J, sizeof(double) * lb, hipMemcpyDeviceToDevice, s));
  HIPCHK(hipMemcpyAsync(d.leak.p, leak_W, sizeof(double) * kb, hipMemcpyDeviceToDevice, s));
  HIPCHK(hipMemcpyAsync(d.slew_axis.p, hsa.data(), sizeof(double) * hsa.size(), hipMemcpyHostToDevice, s));
  HIPCHK(hipMemcpyAsync(d.slew_invw.p, invw.data(), sizeof(double) * invw.size(), hipMemcpyHostToDevice, s));
  HIPCHK(hipMemcpyAsync(cap_axis_d.p, hca.data(), sizeof(double) * hca.size(), hipMemcpyHostToDevice, s));
  HIPCHK(hipMemsetAsync(err.p, 0, sizeof(uint32_t), s));
  if (G > 0)
    HIPCHK(pa::launch_gate_tables(G, gate_cell, gate_cap_F, n_cells, d.cell_k.as<int32_t>(), cap_axis_d.as<double>(),
                                  n_cap, vdd_V, d.gate_info.as<uint32_t>(), d.gate_capfrac.as<double>(),
                                  d.gate_esw.as<double>(), d.gate_k.as<int32_t>(), err.as<uint32_t>(), s));
  std::vector<int32_t> gk(G);
  uint32_t herr = 0;
  if (G > 0) HIPCHK(hipMemcpyAsync(gk.data(), d.gate_k.p, sizeof(int32_t) * G, hipMemcpyDeviceToHost, s));
  HIPCHK(hipMemcpyAsync(&herr, err.p, sizeof(uint32_t), hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));
  if (herr & pa::ERR_CELL_ID) return fail(PA_EDATA, "pa_load_design: gate cell id out of range");
  if (herr & pa::ERR_CAP) return fail(PA_EDATA, "pa_load_design: gate load not finite");
  std::vector<int64_t> pb(G + 1);
  pb[0] = 0;
  for (int64_t g = 0; g < G; ++g) pb[g + 1] = pb[g] + gk[g] + 1;
  d.P = pb[G];
  HIPCHK(hipMemcpyAsync(d.pin_base.p, pb.data(), sizeof(int64_t) * (G + 1), hipMemcpyHostToDevice, s));
  HIPCHK(d.pin_gate.alloc(sizeof(int32_t) * d.P));
  HIPCHK(d.pin_local.alloc(sizeof(uint8_t) * d.P));
  if (G > 0)
    HIPCHK(pa::launch_pin_owner(G, d.pin_base.as<int64_t>(), d.pin_gate.as<int32_t>(), d.pin_local.as<uint8_t>(), s));
  HIPCHK(hipStreamSynchronize(s));

  c->d = std::move(d);
  c->has_design = true;
  c->ev = Events();
  c->has_events = false;
  c->parity = 0;
  return PA_OK;
}

// Block ranges of the pass: every chunk's events are cut into pieces of about
// E / target events (never across a chunk, so a block's bins cover one chunk);
// the kernel moves each nominal cut forward to the next segment head.
static int build_ranges(pa_ctx *c) {
  Events &v = c->ev;
  const int64_t target_blocks = c->tun.grid_blocks > 0 ? c->tun.grid_blocks : 2 * (int64_t)c->n_cu;
  const int64_t min_events = 4 * (int64_t)pa::pass_wave_batch() * (pa::pass_block_threads() / 64);
  const int64_t per = std::max<int64_t>(min_events, (v.E + target_blocks - 1) / std::max<int64_t>(1, target_blocks));
  std::vector<uint32_t> rs, rq;
  for (int32_t q = 0; q < v.Q; ++q) {
    const int64_t a = v.h_chunk_base[q], b = v.h_chunk_base[q + 1];
    if (b <= a) continue;
    const int64_t n = std::max<int64_t>(1, (b - a + per / 2) / per);
    for (int64_t i = 0; i < n; ++i) {
      rs.push_back((uint32_t)(a + (b - a) * i / n));
      rq.push_back((uint32_t)q);
    }
  }
  v.n_ranges = (int32_t)rs.size();
  rs.push_back((uint32_t)v.E);
  rq.push_back(0);
  HIPCHK(v.rstart.alloc(sizeof(uint32_t) * rs.size()));
  HIPCHK(v.rchunk.alloc(sizeof(uint32_t) * rq.size()));
  HIPCHK(hipMemcpyAsync(v.rstart.p, rs.data(), sizeof(uint32_t) * rs.size(), hipMemcpyHostToDevice, c->stream));
  HIPCHK(hipMemcpyAsync(v.rchunk.p, rq.data(), sizeof(uint32_t) * rq.size(), hipMemcpyHostToDevice, c->stream));
  HIPCHK(hipStreamSynchronize(c->stream));
  return PA_OK;
}

static int zero_accumulators(pa_ctx *c) {
  Events &v = c->ev;
  hipStream_t s = c->stream;
  HIPCHK(hipMemsetAsync(v.acc_wave.p, 0, v.acc_wave.bytes, s));
  HIPCHK(hipMemsetAsync(v.acc_cnt.p, 0, v.acc_cnt.bytes, s));
  for (int k = 0; k < 2; ++k) {
    HIPCHK(hipMemsetAsync(v.dP[k].p, 0, v.dP[k].bytes, s));
    HIPCHK(hipMemsetAsync(v.tot[k].p, 0, v.tot[k].bytes, s));
    HIPCHK(hipMemsetAsync(v.tot_cnt[k].p, 0, v.tot_cnt[k].bytes, s));
  }
  c->parity = 0;
  return PA_OK;
}

int pa_load_events(pa_ctx *c, int64_t n_pins, int64_t n_events, const int64_t *pin_ptr, const uint8_t *pin_init,
                   const int64_t *evt_t, const uint8_t *evt_val, const float *evt_slew, int64_t t_clk,
                   int64_t t_max, double tick_s) {
  if (!c) return fail(PA_EINVAL, "pa_load_events: NULL context");
  if (!c->has_design) return fail(PA_ESTATE, "pa_load_events: no design loaded");
  const Design &d = c->d;
  if (n_pins != d.P) return fail(PA_EINVAL, "pa_load_events: n_pins %lld != %lld pins of the design",
                                 (long long)n_pins, (long long)d.P);
  if (n_events < 0 || n_events >= (int64_t(1) << 31)) return fail(PA_EINVAL, "pa_load_events: n_events out of range");
  if (t_clk < 1 || t_clk >= (int64_t(1) << 32)) return fail(PA_EINVAL, "pa_load_events: t_clk out of range");
  if (t_max < 1) return fail(PA_EINVAL, "pa_load_events: t_max must be > 0");
  if ((t_max + t_clk - 1) / t_clk > (int64_t(1) << 28)) return fail(PA_EINVAL, "pa_load_events: more than 2^28 clock cycles");
  if (!(tick_s > 0.0) || !std::isfinite(tick_s)) return fail(PA_EINVAL, "pa_load_events: tick_s must be > 0");
  if (!pin_ptr || (n_pins > 0 && !pin_init) || (n_events > 0 && (!evt_t || !evt_val || !evt_slew)))
    return fail(PA_EINVAL, "pa_load_events: NULL array");
  HIPCHK(hipSetDevice(c->device));
  hipStream_t s = c->stream;
  const int64_t P = n_pins, E = n_events, G = d.G;
  int64_t ends[2] = {0, 0};
  HIPCHK(hipMemcpyAsync(&ends[0], pin_ptr, sizeof(int64_t), hipMemcpyDeviceToHost, s));
  HIPCHK(hipMemcpyAsync(&ends[1], pin_ptr + P, sizeof(int64_t), hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));
  if (ends[0] != 0 || ends[1] != E) return fail(PA_EDATA, "pa_load_events: pin_ptr[0] must be 0 and pin_ptr[P] = n_events");

  // ---- validation
  DBuf err, ev_pin;
  HIPCHK(err.alloc(sizeof(uint32_t)));
  HIPCHK(ev_pin.alloc(sizeof(uint32_t) * E));
  HIPCHK(hipMemsetAsync(err.p, 0, sizeof(uint32_t), s));
  if (P > 0) HIPCHK(pa::launch_pin_check(P, pin_ptr, pin_init, err.as<uint32_t>(), s));
  uint32_t herr = 0;
  HIPCHK(hipMemcpyAsync(&herr, err.p, sizeof(uint32_t), hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));
  if (herr & pa::ERR_PIN_PTR) return fail(PA_EDATA, "pa_load_events: pin_ptr decreases");
  if (herr & pa::ERR_INIT) return fail(PA_EDATA, "pa_load_events: pin_init not in {0,1}");
  if (E > 0) HIPCHK(pa::launch_event_check(E, P, pin_ptr, pin_init, evt_t, evt_val, evt_slew, t_max,
                                           ev_pin.as<uint32_t>(), err.as<uint32_t>(), s));
  HIPCHK(hipMemcpyAsync(&herr, err.p, sizeof(uint32_t), hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));
  if (herr & pa::ERR_TIME_RANGE) return fail(PA_EDATA, "pa_load_events: event time outside [0, t_max)");
  if (herr & pa::ERR_TIME_ORDER) return fail(PA_EDATA, "pa_load_events: timestamps not strictly increasing on a pin");
  if (herr & pa::ERR_VALUE) return fail(PA_EDATA, "pa_load_events: values do not alternate starting from !init");
  if (herr & pa::ERR_SLEW) return fail(PA_EDATA, "pa_load_events: slew not finite and > 0");

  // ---- key packing and chunk length
  Events v;
  v.E = E;
  v.T = t_clk;
  v.t_max = t_max;
  v.tick_s = tick_s;
  v.C = (t_max + t_clk - 1) / t_clk;
  if ((uint64_t)G > pa::kKeyMaxGates - 1)
    return fail(PA_EINVAL, "pa_load_events: designs of more than 2^22 - 1 gates are not supported");
  const uint32_t pbits = bits_for((uint64_t)d.kmax);
  // the pass keeps (pin, t_rel) of an event in one 32-bit word
  const int tb_lim = 32 - (int)pbits;
  const uint64_t max_ticks = uint64_t(1) << tb_lim;
  const int64_t cc_cap = (int64_t)(max_ticks / (uint64_t)t_clk);
  if (cc_cap < 1) return fail(PA_EINVAL, "pa_load_events: clock period longer than 2^%d ticks", tb_lim);
  // chunk length: a power of two (window lengths halve it), at most the LDS bins
  int64_t Cc_want = c->tun.chunk_cycles > 0 ? c->tun.chunk_cycles : 256;
  Cc_want = std::min<int64_t>({Cc_want, (int64_t)pa::pass_max_chunk_cycles(), cc_cap});
  int64_t Cc = 1;
  while (Cc * 2 <= Cc_want) Cc *= 2;
  int32_t lc = 0;
  while ((int64_t(1) << lc) < Cc) ++lc;
  v.Cc = (int32_t)Cc;
  v.Q = (int32_t)((v.C + Cc - 1) / Cc);
  v.chunk_ticks = Cc * t_clk;
  v.kf.t_bits = bits_for((uint64_t)(v.chunk_ticks - 1));
  v.kf.p_bits = pbits;
  if (v.kf.t_bits + pbits > 32) return fail(PA_EINVAL, "pa_load_events: event key overflow");
  const int32_t Q = v.Q;

  // ---- density-aware windows: per-gate level s (2^s windows per chunk), refined
  //      until no (chunk, gate, window) segment holds more than kSegMax events
  DBuf level, level_next, pw_len, pwbase, cnt, tmp, flags;
  size_t tmp_bytes = 0;
  HIPCHK(level.alloc(G));
  HIPCHK(level_next.alloc(G));
  HIPCHK(pw_len.alloc(sizeof(int64_t) * (G + 1)));
  HIPCHK(pwbase.alloc(sizeof(int64_t) * (G + 1)));
  HIPCHK(flags.alloc(sizeof(uint32_t) * 2));
  if (G > 0)
    HIPCHK(pa::launch_gate_levels(G, d.pin_base.as<int64_t>(), pin_ptr, v.C, (int32_t)Cc, lc,
                                  (double)pa::kSegMax / 4.0, level.as<uint8_t>(), s));
  int64_t PW = 0;
  uint32_t hflags[2] = {0, 0};
  for (int iter = 0;; ++iter) {
    HIPCHK(hipMemsetAsync(pw_len.p, 0, pw_len.bytes, s));
    if (G > 0) HIPCHK(pa::launch_pw_len(G, d.gate_k.as<int32_t>(), level.as<uint8_t>(), pw_len.as<int64_t>(), s));
    tmp_bytes = 0;
    HIPCHK(pa::scan_exclusive_i64(pw_len.as<int64_t>(), pwbase.as<int64_t>(), G + 1, nullptr, &tmp_bytes, s));
    HIPCHK(tmp.alloc(tmp_bytes));
    HIPCHK(pa::scan_exclusive_i64(pw_len.as<int64_t>(), pwbase.as<int64_t>(), G + 1, tmp.p, &tmp_bytes, s));
    HIPCHK(hipMemcpyAsync(&PW, pwbase.as<int64_t>() + G, sizeof(int64_t), hipMemcpyDeviceToHost, s));
    HIPCHK(hipStreamSynchronize(s));
    if ((int64_t)Q * PW >= (int64_t(1) << 31)) return fail(PA_ENOMEM, "pa_load_events: too many (window, pin) pairs");
    HIPCHK(cnt.alloc(sizeof(uint32_t) * (size_t)(Q * PW + 1)));
    HIPCHK(hipMemsetAsync(cnt.p, 0, cnt.bytes, s));
    if (E > 0)
      HIPCHK(pa::launch_count_w(E, evt_t, ev_pin.as<uint32_t>(), d.pin_gate.as<int32_t>(), d.pin_local.as<uint8_t>(),
                                d.gate_k.as<int32_t>(), level.as<uint8_t>(), pwbase.as<int64_t>(), PW, t_clk, lc,
                                cnt.as<uint32_t>(), s));
    HIPCHK(hipMemsetAsync(flags.p, 0, flags.bytes, s));
    HIPCHK(hipMemcpyAsync(level_next.p, level.p, G, hipMemcpyDeviceToDevice, s));
    if (G > 0)
      HIPCHK(pa::launch_winmax(G, Q, d.gate_k.as<int32_t>(), level.as<uint8_t>(), pwbase.as<int64_t>(), PW, lc,
                               cnt.as<uint32_t>(), level_next.as<uint8_t>(), flags.as<uint32_t>(),
                               flags.as<uint32_t>() + 1, s));
    HIPCHK(hipMemcpyAsync(hflags, flags.p, sizeof hflags, hipMemcpyDeviceToHost, s));
    HIPCHK(hipStreamSynchronize(s));
    if (hflags[0] & 2u)
      return fail(PA_EDATA, "pa_load_events: a gate has more than %d events inside one clock cycle", pa::kSegMax);
    if (!(hflags[0] & 1u)) break;
    std::swap(level, level_next);
  }
  v.max_seg = hflags[1];

  // ---- layout: offsets of every (chunk, gate, window, pin) run, window-start values, scatter
  const int64_t QPW = (int64_t)Q * PW;
  DBuf off, first, vstart;
  HIPCHK(off.alloc(sizeof(uint32_t) * (size_t)(QPW + 1)));
  HIPCHK(first.alloc(sizeof(uint32_t) * (size_t)(QPW + 1)));
  HIPCHK(vstart.alloc((size_t)QPW + 1));
  tmp_bytes = 0;
  HIPCHK(pa::scan_exclusive_u32(cnt.as<uint32_t>(), off.as<uint32_t>(), QPW + 1, nullptr, &tmp_bytes, s));
  HIPCHK(tmp.alloc(tmp_bytes));
  HIPCHK(pa::scan_exclusive_u32(cnt.as<uint32_t>(), off.as<uint32_t>(), QPW + 1, tmp.p, &tmp_bytes, s));
  if (P > 0)
    HIPCHK(pa::launch_pin_windows(P, Q, pin_ptr, pin_init, d.pin_gate.as<int32_t>(), d.pin_local.as<uint8_t>(),
                                  d.gate_k.as<int32_t>(), level.as<uint8_t>(), pwbase.as<int64_t>(), PW,
                                  cnt.as<uint32_t>(), first.as<uint32_t>(), vstart.as<uint8_t>(), s));
  HIPCHK(v.key.alloc(sizeof(uint64_t) * E));
  HIPCHK(v.slew.alloc(sizeof(float) * E));
  HIPCHK(v.orig.alloc(sizeof(uint32_t) * E));
  HIPCHK(v.chunk_base.alloc(sizeof(uint32_t) * (Q + 1)));
  HIPCHK(v.pin_init.alloc(P));
  if (E > 0)
    HIPCHK(pa::launch_scatter_w(E, evt_t, evt_slew, evt_val, ev_pin.as<uint32_t>(), d.pin_gate.as<int32_t>(),
                                d.pin_local.as<uint8_t>(), d.gate_k.as<int32_t>(), level.as<uint8_t>(),
                                pwbase.as<int64_t>(), PW, t_clk, lc, v.chunk_ticks, first.as<uint32_t>(),
                                off.as<uint32_t>(), vstart.as<uint8_t>(), v.kf, v.key.as<uint64_t>(),
                                v.slew.as<float>(), v.orig.as<uint32_t>(), s));
  HIPCHK(pa::launch_chunk_base_w(Q, PW, off.as<uint32_t>(), v.chunk_base.as<uint32_t>(), s));
  if (P > 0) HIPCHK(hipMemcpyAsync(v.pin_init.p, pin_init, P, hipMemcpyDeviceToDevice, s));
  v.h_chunk_base.resize(Q + 1);
  HIPCHK(hipMemcpyAsync(v.h_chunk_base.data(), v.chunk_base.p, sizeof(uint32_t) * (Q + 1), hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));

  // ---- accumulators of the pass
  HIPCHK(v.acc_wave.alloc(sizeof(double) * 8 * v.C));
  HIPCHK(v.acc_cnt.alloc(sizeof(unsigned long long) * 8 * v.C));
  for (int k = 0; k < 2; ++k) {
    HIPCHK(v.dP[k].alloc(sizeof(double) * v.Q));
    HIPCHK(v.tot[k].alloc(sizeof(double) * 8));
    HIPCHK(v.tot_cnt[k].alloc(sizeof(unsigned long long) * 2));
  }
  HIPCHK(v.res.alloc(sizeof(double) * 16));
  HIPCHK(hipStreamSynchronize(s));

  c->ev = std::move(v);
  c->has_events = true;
  int rc = build_ranges(c);
  if (rc == PA_OK) rc = zero_accumulators(c);
  if (rc == PA_OK && hipStreamSynchronize(s) != hipSuccess) rc = fail(PA_EHIP, "pa_load_events: sync");
  if (rc != PA_OK) {
    c->ev = Events();
    c->has_events = false;
  }
  return rc;
}

int pa_run(pa_ctx *c, pa_totals *out, double *wave_J, uint64_t *cyc_events, uint64_t *cyc_glitches,
           uint8_t *evt_glitch, uint8_t *evt_state_before) {
  if (!c) return fail(PA_EINVAL, "pa_run: NULL context");
  if (!c->has_design || !c->has_events) return fail(PA_ESTATE, "pa_run: design and events must be loaded first");
  if (!out || !wave_J || !cyc_events || !cyc_glitches) return fail(PA_EINVAL, "pa_run: NULL output");
  HIPCHK(hipSetDevice(c->device));
  const Design &d = c->d;
  Events &v = c->ev;
  hipStream_t s = c->stream;
  const int cur = c->parity, nxt = cur ^ 1;

  pa::PassArgs a{};
  a.key = v.key.as<uint64_t>();
  a.slew = v.slew.as<float>();
  a.orig = v.orig.as<uint32_t>();
  a.chunk_base = v.chunk_base.as<uint32_t>();
  a.E = v.E;
  a.Q = v.Q;
  a.Cc = v.Cc;
  a.C = v.C;
  a.T = (uint32_t)v.T;
  a.divT = pa::make_divu32((uint32_t)v.T);
  a.chunk_ticks = v.chunk_ticks;
  a.t_max = v.t_max;
  a.tick_s = v.tick_s;
  a.kf = v.kf;
  a.G = d.G;
  a.gate_info = d.gate_info.as<uint32_t>();
  a.gate_capfrac = d.gate_capfrac.as<double>();
  a.gate_esw = d.gate_esw.as<double>();
  a.pin_base = d.pin_base.as<int64_t>();
  a.pin_init = v.pin_init.as<uint8_t>();
  a.cell_k = d.cell_k.as<int32_t>();
  a.cell_lut_base = d.cell_lut_base.as<uint32_t>();
  a.cell_leak_base = d.cell_leak_base.as<uint32_t>();
  a.lut = d.lut.as<double>();
  a.leak = d.leak.as<double>();
  a.slew_axis = d.slew_axis.as<double>();
  a.slew_invw = d.slew_invw.as<double>();
  a.n_slew = d.n_slew;
  a.n_cap = d.n_cap;
  a.n_cells = d.n_cells;
  a.n_leak = d.n_leak;
  a.acc_wave = v.acc_wave.as<double>();
  a.acc_cnt = v.acc_cnt.as<unsigned long long>();
  a.dP = v.dP[cur].as<double>();
  a.tot = v.tot[cur].as<double>();
  a.tot_cnt = v.tot_cnt[cur].as<unsigned long long>();
  a.evt_glitch = evt_glitch;
  a.evt_state = evt_state_before;

  a.rstart = v.rstart.as<uint32_t>();
  a.rchunk = v.rchunk.as<uint32_t>();
  a.n_ranges = v.n_ranges;
  const int grid = std::max(1, v.n_ranges);
  c->last_grid = grid;

  pa::FinalArgs f{};
  f.C = v.C;
  f.Cc = v.Cc;
  f.Q = v.Q;
  f.T = (uint32_t)v.T;
  f.t_max = v.t_max;
  f.tick_s = v.tick_s;
  f.E = v.E;
  f.acc_wave = a.acc_wave;
  f.acc_cnt = a.acc_cnt;
  f.dP = a.dP;
  f.tot = a.tot;
  f.tot_cnt = a.tot_cnt;
  f.dP_next = v.dP[nxt].as<double>();
  f.tot_next = v.tot[nxt].as<double>();
  f.tot_cnt_next = v.tot_cnt[nxt].as<unsigned long long>();
  f.Q_next = v.Q;
  f.wave_out = wave_J;
  f.cyc_events = cyc_events;
  f.cyc_glitches = cyc_glitches;
  f.res = v.res.as<double>();

  const bool timed = c->tun.time_kernels != 0;
  if (timed) HIPCHK(hipEventRecord(c->tev[0], s));
  hipError_t e1 = pa::launch_pass(a, grid, s);
  if (timed && e1 == hipSuccess) e1 = hipEventRecord(c->tev[1], s);
  if (e1 == hipSuccess) e1 = pa::launch_finalize(f, s);
  if (timed && e1 == hipSuccess) e1 = hipEventRecord(c->tev[2], s);
  if (e1 == hipSuccess) e1 = hipMemcpyAsync(c->h_res, f.res, sizeof(double) * 16, hipMemcpyDeviceToHost, s);
  if (e1 == hipSuccess) e1 = hipStreamSynchronize(s);
  if (e1 != hipSuccess) {
    zero_accumulators(c);
    (void)hipStreamSynchronize(s);
    return fail(PA_EHIP, "pa_run: HIP error %s", hipGetErrorString(e1));
  }
  c->parity = nxt;
  if (timed) {
    (void)hipEventElapsedTime(&c->kernel_ms[0], c->tev[0], c->tev[1]);
    (void)hipEventElapsedTime(&c->kernel_ms[1], c->tev[1], c->tev[2]);
    c->kernel_ms[3] = c->kernel_ms[0] + c->kernel_ms[1];
  }
  const double *r = c->h_res;
  out->e_int_J = r[0];
  out->e_sw_J = r[1];
  out->e_gl_J = r[2];
  out->e_leak_J = r[3];
  out->p_int_W = r[4];
  out->p_sw_W = r[5];
  out->p_gl_W = r[6];
  out->p_leak_W = r[7];
  out->n_glitches = (uint64_t)r[8];
  out->n_events = (uint64_t)v.E;
  out->n_cycles = v.C;
  return PA_OK;
}

int pa_get_info(pa_ctx *c, pa_info *info) {
  if (!c || !info) return fail(PA_EINVAL, "pa_get_info: NULL argument");
  std::memset(info, 0, sizeof *info);
  info->n_gates = c->d.G;
  info->n_pins = c->d.P;
  info->n_events = c->ev.E;
  info->n_cycles = c->ev.C;
  info->chunk_cycles = c->ev.Cc;
  info->n_chunks = c->ev.Q;
  info->grid_blocks = c->last_grid;
  info->block_threads = pa::pass_block_threads();
  info->batch_events = pa::pass_wave_batch();
  info->max_segment_events = (int32_t)c->ev.max_seg;
  info->device_bytes = c->d.bytes() + c->ev.bytes();
  for (int k = 0; k < 4; ++k) info->kernel_ms[k] = c->kernel_ms[k];
  return PA_OK;
}

}  // extern "C"
