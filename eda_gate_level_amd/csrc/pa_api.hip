// pa_api.hip -- the C ABI of include/pa.h: context, design and event loads,
// and the pass.  Argument marshalling, validation and launches only; every
// step of the power analysis runs in the gfx950 kernels of pa_pass.hip and
// pa_load.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <condition_variable>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <functional>
#include <limits>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "pa.h"
#include "pa_common.h"
#include "pa_load.h"
#include "pa_text.h"

// Device memory of pa_run_noalloc: the pass's per-block partial results (cycle
// bins, cycle counts, block totals) and the finalize's result slots, in one
// array of fixed size instead of buffers the library allocates.  Every device
// the library runs on holds its own copy until the process ends.  Host code
// never uses the name below as an address: each device's address is looked up
// once (scratch_address) and passed to the kernels.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;

// Device-memory accounting of the context whose call this thread is serving:
// every library buffer adds its bytes while it lives; with a cap set
// (pa_tunables.device_mib_cap, a debug knob), an allocation that would take
// the live total past it fails as if the device were out of memory.
struct MemBudget {
  int64_t live = 0;
  int64_t cap = 0;  // 0 = none
};
thread_local MemBudget *g_budget = nullptr;

struct BudgetScope {  // RAII: the calls of one API entry are charged to its context
  MemBudget *prev;
  explicit BudgetScope(MemBudget *b) : prev(g_budget) { g_budget = b; }
  ~BudgetScope() { g_budget = prev; }
};

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

// The address of `scratch` on every device, looked up once per device (with
// that device current) by the first pa_create on it.
struct ScratchAddr {
  bool looked_up = false;
  hipError_t err = hipSuccess;
  void *p = nullptr;
};
std::mutex g_scratch_mu;
std::vector<ScratchAddr> g_scratch_addr;

// called with `device` current
ScratchAddr scratch_address(int device) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((int)g_scratch_addr.size() <= device) g_scratch_addr.resize((size_t)device + 1);
  ScratchAddr &a = g_scratch_addr[(size_t)device];
  if (!a.looked_up) {
    a.err = hipGetSymbolAddress(&a.p, HIP_SYMBOL(scratch));
    if (a.err != hipSuccess) a.p = nullptr;
    a.looked_up = true;
  }
  return a;
}

// owning device buffer
struct DBuf {
  void *p = nullptr;
  size_t bytes = 0;
  MemBudget *budget = nullptr;  // the context charged for this buffer
  DBuf() = default;
  DBuf(const DBuf &) = delete;
  DBuf &operator=(const DBuf &) = delete;
  DBuf(DBuf &&o) noexcept : p(o.p), bytes(o.bytes), budget(o.budget) {
    o.p = nullptr;
    o.bytes = 0;
    o.budget = nullptr;
  }
  DBuf &operator=(DBuf &&o) noexcept {
    if (this != &o) {
      reset();
      p = o.p;
      bytes = o.bytes;
      budget = o.budget;
      o.p = nullptr;
      o.bytes = 0;
      o.budget = nullptr;
    }
    return *this;
  }
  ~DBuf() { reset(); }
  void reset() {
    if (p) (void)hipFree(p);
    if (budget) budget->live -= (int64_t)bytes;
    p = nullptr;
    bytes = 0;
    budget = nullptr;
  }
  hipError_t alloc(size_t n) {
    reset();
    if (n == 0) n = 16;
    MemBudget *b = g_budget;
    if (b && b->cap > 0 && b->live + (int64_t)n > b->cap) return hipErrorOutOfMemory;
    hipError_t e = hipMalloc(&p, n);
    if (e != hipSuccess) { p = nullptr; return e; }
    bytes = n;
    budget = b;
    if (b) b->live += (int64_t)n;
    return hipSuccess;
  }
  // at least n bytes, keeping the allocation when it is large enough
  hipError_t ensure(size_t n) { return (p && bytes >= n) ? hipSuccess : alloc(n); }
  template <class T> T *as() const { return static_cast<T *>(p); }
};

uint32_t bits_for(uint64_t v) {  // bits needed to hold 0..v (at least 1)
  uint32_t b = 1;
  while (b < 64 && (v >> b) != 0) ++b;
  return b;
}

struct Design {
  int64_t G = 0, P = 0;
  int32_t n_cells = 0, n_slew = 0, n_cap = 0, kmax = 0, n_thr = 0;
  int64_t n_leak = 0;
  double vdd = 0;
  DBuf cell_k, cell_meta, cell_thr, cell_axw, cell_caxw, lut, leak;
  DBuf gate_info, gate_rec, gate_k, pin_base, pin_gate, pin_local;
  DBuf perm;  // internal gate -> caller gate
  int64_t bytes() const {
    return (int64_t)(cell_k.bytes + cell_meta.bytes + cell_thr.bytes + cell_axw.bytes + cell_caxw.bytes + lut.bytes +
                     leak.bytes + gate_info.bytes + gate_rec.bytes + gate_k.bytes + pin_base.bytes + pin_gate.bytes +
                     pin_local.bytes + perm.bytes);
  }
};

struct Events {
  int64_t E = 0, C = 0, T = 0, t_max = 0, chunk_ticks = 0;
  double tick_s = 0;
  int32_t Cc = 0, Q = 0;
  uint32_t tb = 0, pb = 0, gb = 1, last_len = 0;
  DBuf key, slew, orig, pin_init;
  std::vector<uint32_t> h_chunk_base;
  int64_t n_windows = 0, slots = 0;  // windows; slots of the lane streams (events and empty slots)
  int32_t wave_steps_max = 0;       // steps of the longest wave, and the mean over waves with work
  float wave_steps_mean = 0.f;
  DBuf rstart, rchunk, chunk_blk;  // block ranges of the pass, first block of every chunk
  std::vector<uint32_t> chunk_blk_host;
  double l0_host = 0.0;            // the leakage power at t = 0 (the value in l0)
  DBuf wdesc, wlen, l0;            // every wave's (first slot, events per lane); events per window; leakage at t = 0
  DBuf lplan;                      // per block, the cells whose LUTs it copies into LDS
  int32_t lut_lds = 0;             // LDS doubles of a block for those copies (0: none)
  uint64_t pad_key = 0;            // key of an empty slot of the lane streams
  DBuf blk_lut;                    // walk kernel: every block's LUT range (first entry, entries)
  int32_t walk_lut = 0;            // walk kernel: LDS doubles for the largest range (0: not used)
  // walk kernel: the 8-byte-slot stream (keys, slews with a code or value bit) with a
  // header pair in front of every phase; tbc = tic bits, ck = pin-code bits in the key
  bool compact_ok = false;         // the chunk leaves the compact key its bits
  DBuf ckey, cslew;
  uint32_t tbc = 0, ck = 0;
  // per-event outputs from the walk kernel: every event's slot by its caller
  // index, and the kernel's 16-bit values in stream order; built by the first
  // pa_run that asks for per-event outputs, dropped by the next load
  DBuf slot_of, evs;
  bool ev_map = false;
  // per-gate rows from the walk kernel: the windows ranked gate-major, every
  // gate's first rank and first piece (G + 1 entries each; a gate of many
  // windows is summed in pieces by whole blocks first), every window's
  // header pair by rank; made by the first pa_run_gates: room for four sums
  // at every pair of the lane streams (the walk kernel stores a window's at
  // its header pair), every piece's sums and gate, every gate's leakage at
  // its initial state over the window
  DBuf goff, pfirst, wpos, wrec, wpart, pgate, gleak;
  uint32_t n_pieces = 0;
  bool gate_prep = false;
  int32_t n_ranges = 0, grid = 1;
  DBuf blk_wave, blk_cnt, blk_part, res;
  int64_t bytes() const {
    return (int64_t)(key.bytes + slew.bytes + orig.bytes + pin_init.bytes + rstart.bytes + rchunk.bytes +
                     chunk_blk.bytes + wdesc.bytes + wlen.bytes + l0.bytes + lplan.bytes + blk_wave.bytes + blk_cnt.bytes + blk_part.bytes +
                     res.bytes + blk_lut.bytes + ckey.bytes + cslew.bytes + slot_of.bytes + evs.bytes +
                     goff.bytes + pfirst.bytes + wpos.bytes + wrec.bytes + wpart.bytes + pgate.bytes +
                     gleak.bytes);
  }
};

// owning pinned host buffer (grow-only)
struct PinnedBuf {
  void *p = nullptr;
  size_t bytes = 0;
  PinnedBuf() = default;
  PinnedBuf(const PinnedBuf &) = delete;
  PinnedBuf &operator=(const PinnedBuf &) = delete;
  ~PinnedBuf() {
    if (p) (void)hipHostFree(p);
  }
  hipError_t ensure(size_t n) {
    if (p && bytes >= n) return hipSuccess;
    if (p) (void)hipHostFree(p);
    p = nullptr;
    bytes = 0;
    const hipError_t e = hipHostMalloc(&p, n, hipHostMallocDefault);
    if (e != hipSuccess) {
      p = nullptr;
      return e;
    }
    bytes = n;
    return hipSuccess;
  }
};

// device buffers of the event load that live only during it; kept (grow-only)
// so that repeated loads, e.g. the segments of an activity text, allocate
// and free nothing
struct LoadScratch {
  DBuf err, ev_pin, chunk_sorted, cbase, level, k0, k1, idx, perm, chunk, tmp, part;
  DBuf skey, sslew, sorig;            // the events in window order
  DBuf winc, ws, bwin, wkey0, wkey1, widx, worder, wlane, phase, wave_len;  // lane streams
};

}  // namespace

struct pa_ctx {
  MemBudget mem;  // declared first: destroyed after every buffer below
  int device = 0;
  hipStream_t stream = nullptr;
  pa_tunables tun{};
  int n_cu = 0;
  bool has_design = false, has_events = false;
  Design d;
  Events ev;
  Events ev_spare;  // the events before the current ones: their buffers serve the next load
  LoadScratch ls;
  bool keep_load_buffers = false;  // pa_run_text: ev_spare and ls live until the text is done
  PinnedBuf text_host[2];  // pa_run_text: packed segments on the host, and their device copy
  PinnedBuf readback;      // the load's small device-to-host reads, gathered for one synchronisation
  DBuf text_dev;
  double *h_res = nullptr;
  ScratchAddr scratch;  // this device's copy of the fixed scratch of pa_run_noalloc
  hipEvent_t tev[6] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};  // pass start, end; walk, finalize
  float kernel_ms[4] = {0, 0, 0, 0};
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
  if (t && (t->time_kernels < 0 || t->time_kernels > 2))
    return fail(PA_EINVAL, "pa_create: time_kernels must be 0, 1 or 2");
  if (t && t->device_mib_cap < 0) return fail(PA_EINVAL, "pa_create: device_mib_cap must be >= 0");
  if (t && (t->plain_bins < 0 || t->plain_bins > 2))
    return fail(PA_EINVAL, "pa_create: plain_bins must be 0, 1 or 2");
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
  c->mem.cap = (int64_t)c->tun.device_mib_cap << 20;
  c->n_cu = prop.multiProcessorCount;
  c->scratch = scratch_address(hip_device);  // checked by pa_run_noalloc, the only user
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

int pa_set_timing(pa_ctx *c, int32_t time_kernels) {
  if (!c) return fail(PA_EINVAL, "pa_set_timing: NULL context");
  if (time_kernels < 0 || time_kernels > 2) return fail(PA_EINVAL, "pa_set_timing: mode must be 0, 1 or 2");
  c->tun.time_kernels = time_kernels;
  return PA_OK;
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
  BudgetScope bs(&c->mem);
  HIPCHK(hipSetDevice(c->device));
  hipStream_t s = c->stream;

  std::vector<int32_t> hk(n_cells);
  std::vector<double> hsa((size_t)n_cells * n_slew), hca((size_t)n_cells * n_cap);
  HIPCHK(hipMemcpyAsync(hk.data(), cell_n_in, sizeof(int32_t) * n_cells, hipMemcpyDeviceToHost, s));
  HIPCHK(hipMemcpyAsync(hsa.data(), slew_axis, sizeof(double) * hsa.size(), hipMemcpyDeviceToHost, s));
  HIPCHK(hipMemcpyAsync(hca.data(), cap_axis, sizeof(double) * hca.size(), hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));
  // per-cell tables of the pass: (k | leakage base << 4, LUT base), the inner
  // slew-axis points as floats rounded up (segment search on the fp32 slew),
  // and (axis point, 1 / segment width) pairs
  const int32_t n_thr = ((n_slew - 2) + 3) / 4 * 4;
  std::vector<uint32_t> meta(2 * (size_t)n_cells);
  std::vector<float> thr((size_t)n_cells * n_thr, INFINITY);
  std::vector<double> axw(2 * (size_t)n_cells * (n_slew - 1)), caxw(2 * (size_t)n_cells * (n_cap - 1));
  uint64_t lb = 0, kb = 0;
  int32_t kmax = 0;
  for (int32_t i = 0; i < n_cells; ++i) {
    const int32_t k = hk[i];
    if (k < 1 || k > pa::kMaxInputs)
      return fail(PA_EDATA, "pa_load_design: cell %d has %d inputs (1..%d allowed)", i, k, pa::kMaxInputs);
    kmax = std::max(kmax, k);
    meta[2 * i] = (uint32_t)k | (uint32_t)(kb << 4);
    meta[2 * i + 1] = (uint32_t)lb;
    lb += (uint64_t(1) << k) * (uint64_t)k * n_slew * n_cap;
    kb += uint64_t(1) << k;
    if (lb >= (uint64_t(1) << 31) || kb >= (uint64_t(1) << 28))
      return fail(PA_EINVAL, "pa_load_design: LUT tables reach 2^31 entries or leakage tables 2^28");
    const double *sa = &hsa[(size_t)i * n_slew];
    for (int j = 0; j + 1 < n_slew; ++j)
      if (!(sa[j] < sa[j + 1]))
        return fail(PA_EDATA, "pa_load_design: slew axis of cell %d not strictly increasing", i);
    for (int j = 0; j + 1 < n_cap; ++j)
      if (!(hca[(size_t)i * n_cap + j] < hca[(size_t)i * n_cap + j + 1]))
        return fail(PA_EDATA, "pa_load_design: cap axis of cell %d not strictly increasing", i);
    for (int j = 1; j + 1 < n_slew; ++j) thr[(size_t)i * n_thr + j - 1] = pa::float_at_or_above(sa[j]);
    for (int j = 0; j + 1 < n_slew; ++j) {
      axw[2 * ((size_t)i * (n_slew - 1) + j)] = sa[j];
      axw[2 * ((size_t)i * (n_slew - 1) + j) + 1] = 1.0 / (sa[j + 1] - sa[j]);
    }
    const double *ca = &hca[(size_t)i * n_cap];
    for (int j = 0; j + 1 < n_cap; ++j) {
      caxw[2 * ((size_t)i * (n_cap - 1) + j)] = ca[j];
      caxw[2 * ((size_t)i * (n_cap - 1) + j) + 1] = 1.0 / (ca[j + 1] - ca[j]);
    }
  }

  Design d;
  d.G = n_gates;
  d.n_cells = n_cells;
  d.n_slew = n_slew;
  d.n_cap = n_cap;
  d.kmax = kmax;
  d.n_thr = n_thr;
  d.n_leak = (int64_t)kb;
  d.vdd = vdd_V;
  const int64_t G = n_gates;
  DBuf cap_axis_d, err;
  HIPCHK(d.cell_k.alloc(sizeof(int32_t) * n_cells));
  HIPCHK(d.cell_meta.alloc(sizeof(uint32_t) * meta.size()));
  HIPCHK(d.cell_thr.alloc(sizeof(float) * thr.size()));
  HIPCHK(d.cell_axw.alloc(sizeof(double) * axw.size()));
  HIPCHK(d.cell_caxw.alloc(sizeof(double) * caxw.size()));
  HIPCHK(d.lut.alloc(sizeof(double) * lb));
  HIPCHK(d.leak.alloc(sizeof(double) * kb));
  HIPCHK(cap_axis_d.alloc(sizeof(double) * hca.size()));
  HIPCHK(d.gate_info.alloc(sizeof(uint32_t) * G));
  HIPCHK(d.gate_rec.alloc(4 * sizeof(uint32_t) * G));
  HIPCHK(d.gate_k.alloc(sizeof(int32_t) * G));
  HIPCHK(d.pin_base.alloc(sizeof(int64_t) * (G + 1)));
  HIPCHK(err.alloc(sizeof(uint32_t)));
  HIPCHK(hipMemcpyAsync(d.cell_k.p, hk.data(), sizeof(int32_t) * n_cells, hipMemcpyHostToDevice, s));
  HIPCHK(hipMemcpyAsync(d.cell_meta.p, meta.data(), sizeof(uint32_t) * meta.size(), hipMemcpyHostToDevice, s));
  if (!thr.empty())
    HIPCHK(hipMemcpyAsync(d.cell_thr.p, thr.data(), sizeof(float) * thr.size(), hipMemcpyHostToDevice, s));
  HIPCHK(hipMemcpyAsync(d.cell_axw.p, axw.data(), sizeof(double) * axw.size(), hipMemcpyHostToDevice, s));
  HIPCHK(hipMemcpyAsync(d.cell_caxw.p, caxw.data(), sizeof(double) * caxw.size(), hipMemcpyHostToDevice, s));
  HIPCHK(hipMemcpyAsync(d.lut.p, lut_J, sizeof(double) * lb, hipMemcpyDeviceToDevice, s));
  HIPCHK(hipMemcpyAsync(d.leak.p, leak_W, sizeof(double) * kb, hipMemcpyDeviceToDevice, s));
  HIPCHK(hipMemcpyAsync(cap_axis_d.p, hca.data(), sizeof(double) * hca.size(), hipMemcpyHostToDevice, s));
  // internal gate order: sorted by cell (stable), so that the gates of a
  // wave's events mostly share a cell and their LUT rows share cache lines;
  // pins keep the caller's numbering
  std::vector<int32_t> gcell(G);
  if (G > 0) HIPCHK(hipMemcpyAsync(gcell.data(), gate_cell, sizeof(int32_t) * G, hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));
  std::vector<int64_t> cstart(n_cells + 1, 0);
  for (int64_t g = 0; g < G; ++g) {
    if (gcell[g] < 0 || gcell[g] >= n_cells) return fail(PA_EDATA, "pa_load_design: gate cell id out of range");
    ++cstart[gcell[g] + 1];
  }
  for (int32_t i = 0; i < n_cells; ++i) cstart[i + 1] += cstart[i];
  std::vector<int32_t> perm(G);  // internal gate -> caller gate
  for (int64_t g = 0; g < G; ++g) perm[cstart[gcell[g]]++] = (int32_t)g;
  std::vector<int64_t> pbc(G + 1), pb(G + 1);  // first caller pin of every caller / internal gate
  pbc[0] = 0;
  for (int64_t g = 0; g < G; ++g) pbc[g + 1] = pbc[g] + hk[gcell[g]] + 1;
  for (int64_t i = 0; i < G; ++i) pb[i] = pbc[perm[i]];
  pb[G] = pbc[G];
  d.P = pbc[G];
  DBuf &perm_d = d.perm;
  HIPCHK(perm_d.alloc(sizeof(int32_t) * G));
  if (G > 0) HIPCHK(hipMemcpyAsync(perm_d.p, perm.data(), sizeof(int32_t) * G, hipMemcpyHostToDevice, s));
  HIPCHK(hipMemsetAsync(err.p, 0, sizeof(uint32_t), s));
  if (G > 0)
    HIPCHK(pa::launch_gate_tables(G, perm_d.as<int32_t>(), gate_cell, gate_cap_F, n_cells, d.cell_k.as<int32_t>(),
                                  cap_axis_d.as<double>(), n_cap, vdd_V, d.gate_info.as<uint32_t>(),
                                  d.gate_rec.as<uint4>(), d.gate_k.as<int32_t>(), err.as<uint32_t>(), s));
  uint32_t herr = 0;
  HIPCHK(hipMemcpyAsync(&herr, err.p, sizeof(uint32_t), hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));
  if (herr & pa::ERR_CELL_ID) return fail(PA_EDATA, "pa_load_design: gate cell id out of range");
  if (herr & pa::ERR_CAP) return fail(PA_EDATA, "pa_load_design: gate load not finite");
  HIPCHK(hipMemcpyAsync(d.pin_base.p, pb.data(), sizeof(int64_t) * (G + 1), hipMemcpyHostToDevice, s));
  HIPCHK(d.pin_gate.alloc(sizeof(int32_t) * d.P));
  HIPCHK(d.pin_local.alloc(sizeof(uint8_t) * d.P));
  if (G > 0)
    HIPCHK(pa::launch_pin_owner(G, d.pin_base.as<int64_t>(), d.gate_k.as<int32_t>(), d.pin_gate.as<int32_t>(),
                                d.pin_local.as<uint8_t>(), s));
  HIPCHK(hipStreamSynchronize(s));

  c->d = std::move(d);
  c->has_design = true;
  c->ev = Events();
  c->has_events = false;
  return PA_OK;
}

// Density-aware windows: a gate's windows are the longest power-of-two parts
// of a chunk whose expected event count is at most this.  A lane walks whole
// windows, so the longest window bounds the longest lane.
#ifndef PA_WINDOW_EVENTS
#define PA_WINDOW_EVENTS 32.0
#endif
static constexpr double kWindowEvents = PA_WINDOW_EVENTS;
#ifndef PA_WALK_COST_IN
#define PA_WALK_COST_IN 10
#endif
#ifndef PA_WALK_COST_OUT
#define PA_WALK_COST_OUT 4
#endif
#ifndef PA_WALK_COST_HEAD
#define PA_WALK_COST_HEAD 4
#endif
// The walk kernel's relative costs of an input-pin event (three LDS atomics,
// four LUT reads and the table reads; a gate with one or two inputs costs 2
// or 1 less, one with five or more 1 more), an output-pin event (two
// atomics) and a window's set-up: a least-squares fit of the blocks' walk
// times to their event and window counts on the 10M-event, skewed,
// glitch-heavy and 200M-event workloads, then the output and window weights
// moved from 3 and 5 to 4 and 4 by timing weight variants on the same
// workloads (the skewed one 1.9% faster, the others unchanged)
static constexpr uint32_t kWalkCostIn = PA_WALK_COST_IN, kWalkCostOut = PA_WALK_COST_OUT,
                          kWalkCostHead = PA_WALK_COST_HEAD;

static void swap_bufs(DBuf &a, DBuf &b) {
  std::swap(a.p, b.p);
  std::swap(a.bytes, b.bytes);
}

// Radix sort of (k_in, v_in) pairs by the key's low end_bit bits, stable;
// the sorted pairs end in (k_out, v_out), the inputs are overwritten.
static hipError_t sort_pairs64(DBuf &k_in, DBuf &k_out, DBuf &v_in, DBuf &v_out, int64_t n, int end_bit, DBuf &tmp,
                               hipStream_t s) {
  uint64_t *ka = k_in.as<uint64_t>(), *kb = k_out.as<uint64_t>();
  uint32_t *va = v_in.as<uint32_t>(), *vb = v_out.as<uint32_t>();
  size_t tb = 0;
  hipError_t e = pa::sort_pairs_u64(&ka, &kb, &va, &vb, n, end_bit, nullptr, &tb, s);
  if (e == hipSuccess) e = tmp.ensure(tb);
  if (e == hipSuccess) e = pa::sort_pairs_u64(&ka, &kb, &va, &vb, n, end_bit, tmp.p, &tb, s);
  if (e != hipSuccess) return e;
  // the result is in (ka, va): k_in's buffer unless the passes ended in k_out's
  if (ka == k_in.p) {
    swap_bufs(k_in, k_out);
    swap_bufs(v_in, v_out);
  }
  return hipSuccess;
}

// Block ranges of the pass and the lane streams.  Every chunk's events are cut
// into pieces of about 1 / target of the total cost of the pass (the walk
// kernel's relative costs of its events and window set-ups; never across a
// chunk, so a block's bins cover one chunk), each cut moved to the next
// window start; a block's
// windows are then dealt to its lanes (pa_load.hip) and scattered into the
// interleaved streams.  Also the first block of every chunk, for the
// finalize kernel.  The sorted events are in c->ls.skey / sslew / sorig.
// When the walk kernel can run but some block's LUT range does not fit in
// its LDS, the target doubles (smaller blocks span fewer cells), a few times
// at most.
static int build_ranges(pa_ctx *c, Events &v, const int64_t *pin_ptr, const uint8_t *pin_init, const int64_t *evt_t) {
  const Design &d = c->d;
  hipStream_t s = c->stream;
  LoadScratch &ls = c->ls;
  if (pa::pass_block_threads() != pa::lane_plan_lanes())
    return fail(PA_EINVAL, "pa_load_events: lane plan and pass disagree on the block size");
  const int NW = pa::pass_waves_per_block();
  int64_t target_blocks =
      c->tun.grid_blocks > 0 ? c->tun.grid_blocks : (int64_t)pa::pass_blocks_per_cu() * c->n_cu;
  const int64_t min_events = 4 * (int64_t)pa::pass_wave_batch() * NW;

  // ---- device work that needs no host decision, read back in one go: the
  // window count (a scan of the head flags), every sorted event's cost in
  // the pass (the walk kernel's relative costs of input-pin and output-pin
  // events and of a window's set-up, else one per event) and the cost before
  // every chunk, the chunks' first events, and the leakage power at t = 0
  const int64_t E = v.E;
  const bool try_walk = E > 0 && v.compact_ok;  // with events there is a window
  const int32_t room =
      try_walk ? pa::walk_lut_doubles(v.Cc, d.n_cells, d.n_slew, d.n_cap, d.n_thr, d.n_leak, d.kmax) : 0;
  const size_t nq = (size_t)v.Q + 1;
  HIPCHK(ls.wkey0.ensure(sizeof(uint64_t) * nq));
  if (E > 0) {
    HIPCHK(ls.winc.ensure(sizeof(uint32_t) * E));
    HIPCHK(ls.widx.ensure(sizeof(uint32_t) * E));  // head flags first, window indices later
    HIPCHK(pa::launch_head_flags(E, ls.skey.as<uint64_t>(), ls.widx.as<uint32_t>(), s));
    size_t tb = 0;
    HIPCHK(pa::scan_inclusive_u32(ls.widx.as<uint32_t>(), ls.winc.as<uint32_t>(), E, nullptr, &tb, s));
    HIPCHK(ls.tmp.ensure(tb));
    HIPCHK(pa::scan_inclusive_u32(ls.widx.as<uint32_t>(), ls.winc.as<uint32_t>(), E, ls.tmp.p, &tb, s));
    HIPCHK(ls.k0.ensure(sizeof(uint64_t) * E));  // the sort's buffers, free again here
    HIPCHK(ls.k1.ensure(sizeof(uint64_t) * E));
    HIPCHK(pa::launch_event_cost(E, ls.skey.as<uint64_t>(), pa::out_code(v.pb), try_walk ? kWalkCostIn : 1u,
                                 try_walk ? kWalkCostOut : 1u, try_walk ? kWalkCostHead : 0u,
                                 try_walk ? d.gate_k.as<int32_t>() : nullptr, v.gb, ls.k0.as<uint64_t>(),
                                 s));
    tb = 0;
    HIPCHK(pa::scan_inclusive_u64(ls.k0.as<uint64_t>(), ls.k1.as<uint64_t>(), E, nullptr, &tb, s));
    HIPCHK(ls.tmp.ensure(tb));
    HIPCHK(pa::scan_inclusive_u64(ls.k0.as<uint64_t>(), ls.k1.as<uint64_t>(), E, ls.tmp.p, &tb, s));
    HIPCHK(pa::launch_gather_prefix(v.Q + 1, ls.cbase.as<uint32_t>(), ls.k1.as<uint64_t>(), ls.wkey0.as<uint64_t>(),
                                    s));
  } else {
    HIPCHK(hipMemsetAsync(ls.wkey0.p, 0, sizeof(uint64_t) * nq, s));
  }
  DBuf &part = ls.part;
  HIPCHK(part.ensure(sizeof(double) * pa::leak0_parts()));
  HIPCHK(v.l0.ensure(sizeof(double)));
  HIPCHK(pa::launch_leak0(d.G, d.gate_info.as<uint32_t>(), d.cell_meta.as<uint2>(), d.leak.as<double>(),
                          d.pin_base.as<int64_t>(), v.pin_init.as<uint8_t>(), part.as<double>(), v.l0.as<double>(), s));
  // pinned: [l0][cpre Q+1][W][chunk bases Q+1]
  const size_t rb_bytes = sizeof(double) + sizeof(uint64_t) * nq + sizeof(uint32_t) * (1 + nq);
  HIPCHK(c->readback.ensure(rb_bytes));
  unsigned char *rb = static_cast<unsigned char *>(c->readback.p);
  double *rb_l0 = reinterpret_cast<double *>(rb);
  uint64_t *rb_cpre = reinterpret_cast<uint64_t *>(rb + sizeof(double));
  uint32_t *rb_w = reinterpret_cast<uint32_t *>(rb_cpre + nq);
  uint32_t *rb_cb = rb_w + 1;
  *rb_w = 0;
  HIPCHK(hipMemcpyAsync(rb_l0, v.l0.p, sizeof(double), hipMemcpyDeviceToHost, s));
  HIPCHK(hipMemcpyAsync(rb_cpre, ls.wkey0.p, sizeof(uint64_t) * nq, hipMemcpyDeviceToHost, s));
  if (E > 0) HIPCHK(hipMemcpyAsync(rb_w, ls.winc.as<uint32_t>() + (E - 1), sizeof(uint32_t), hipMemcpyDeviceToHost, s));
  HIPCHK(hipMemcpyAsync(rb_cb, ls.cbase.p, sizeof(uint32_t) * nq, hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));
  v.l0_host = *rb_l0;
  std::vector<uint64_t> cpre(rb_cpre, rb_cpre + nq);
  const uint32_t W = *rb_w;
  v.h_chunk_base.assign(rb_cb, rb_cb + nq);

  // ---- windows: starts and lengths
  v.n_windows = W;
  HIPCHK(ls.ws.ensure(sizeof(uint32_t) * ((size_t)W + 1)));
  HIPCHK(v.wlen.ensure(sizeof(uint32_t) * std::max<size_t>(W, 1)));
  if (W > 0) {
    HIPCHK(pa::launch_win_starts(E, ls.skey.as<uint64_t>(), ls.winc.as<uint32_t>(), ls.ws.as<uint32_t>(), s));
    // the input windows' start states, into their first events' keys
    pa::LayoutFmt f{};
    f.T = v.T;
    f.Cc = v.Cc;
    f.lc = bits_for((uint64_t)v.Cc) - 1;
    f.pb = v.pb;
    f.tb = v.tb;
    f.gb = v.gb;
    HIPCHK(pa::launch_window_s0(W, ls.ws.as<uint32_t>(), ls.chunk_sorted.as<uint32_t>(), ls.level.as<uint8_t>(),
                                d.gate_k.as<int32_t>(), d.pin_base.as<int64_t>(), pin_ptr, pin_init, evt_t, f,
                                ls.skey.as<uint64_t>(), s));
  }
  const uint64_t total = cpre[v.Q];

  // ---- block ranges; with windows, every block's first window and LUT range
  int32_t nr = 0;
  std::vector<uint32_t> rs, rq, cb(v.Q + 1);
  std::vector<uint64_t> tgt;
  std::vector<size_t> tgt_at;
  v.walk_lut = 0;
  for (int attempt = 0;; ++attempt) {
    const uint64_t per_cost = std::max<uint64_t>(1, (total + target_blocks - 1) / std::max<int64_t>(1, target_blocks));
    rs.clear();
    rq.clear();
    tgt.clear();
    tgt_at.clear();
    for (int32_t q = 0; q < v.Q; ++q) {
      cb[q] = (uint32_t)rs.size();
      const int64_t a = v.h_chunk_base[q], b = v.h_chunk_base[q + 1];
      if (b <= a) continue;
      // never more blocks than the target, nor blocks of fewer than min_events events
      const uint64_t cq = cpre[q + 1] - cpre[q];
      const int64_t n = std::max<int64_t>(1, std::min<int64_t>((int64_t)(cq / per_cost), (b - a) / min_events));
      for (int64_t i = 0; i < n; ++i) {
        if (i > 0) {
          tgt.push_back(cpre[q] + cq * (uint64_t)i / (uint64_t)n);
          tgt_at.push_back(rs.size());
        }
        rs.push_back((uint32_t)a);
        rq.push_back((uint32_t)q);
      }
    }
    if (!tgt.empty()) {
      // every inner cut: the first event past its share of the chunk's cost
      HIPCHK(ls.wkey1.ensure(sizeof(uint64_t) * tgt.size()));
      HIPCHK(ls.worder.ensure(sizeof(uint32_t) * tgt.size()));
      HIPCHK(hipMemcpyAsync(ls.wkey1.p, tgt.data(), sizeof(uint64_t) * tgt.size(), hipMemcpyHostToDevice, s));
      HIPCHK(pa::launch_cost_cuts((int32_t)tgt.size(), ls.wkey1.as<uint64_t>(), ls.k1.as<uint64_t>(), E,
                                  ls.worder.as<uint32_t>(), s));
      std::vector<uint32_t> pos(tgt.size());
      HIPCHK(hipMemcpyAsync(pos.data(), ls.worder.p, sizeof(uint32_t) * pos.size(), hipMemcpyDeviceToHost, s));
      HIPCHK(hipStreamSynchronize(s));
      for (size_t i = 0; i < pos.size(); ++i) rs[tgt_at[i]] = pos[i];
    }
    cb[v.Q] = (uint32_t)rs.size();
    nr = (int32_t)rs.size();
    rs.push_back((uint32_t)v.E);
    rq.push_back(0);
    HIPCHK(v.rstart.ensure(sizeof(uint32_t) * rs.size()));
    HIPCHK(hipMemcpyAsync(v.rstart.p, rs.data(), sizeof(uint32_t) * rs.size(), hipMemcpyHostToDevice, s));
    if (W == 0) break;
    HIPCHK(ls.bwin.ensure(sizeof(uint32_t) * ((size_t)nr + 1)));
    HIPCHK(pa::launch_block_windows(nr, E, v.rstart.as<uint32_t>(), ls.skey.as<uint64_t>(), ls.winc.as<uint32_t>(), W,
                                    ls.bwin.as<uint32_t>(), s));
    if (!try_walk) break;
    // the walk kernel: every block's LUT range, used when each fits in a block's LDS
    HIPCHK(v.blk_lut.ensure(sizeof(uint2) * (size_t)nr));
    HIPCHK(pa::launch_block_luts(nr, ls.skey.as<uint64_t>(), ls.ws.as<uint32_t>(), ls.bwin.as<uint32_t>(),
                                 d.gate_rec.as<uint4>(), d.cell_meta.as<uint2>(), v.gb, d.n_slew, d.n_cap,
                                 v.blk_lut.as<uint2>(), s));
    std::vector<uint2> hl((size_t)nr);
    HIPCHK(hipMemcpyAsync(hl.data(), v.blk_lut.p, sizeof(uint2) * hl.size(), hipMemcpyDeviceToHost, s));
    HIPCHK(hipStreamSynchronize(s));
    uint32_t most = 0;
    for (const uint2 &r : hl) most = std::max(most, r.y);
    // at least the entries a lane without a window reads (its row 0, segment n, cap segment 0)
    most = std::max<uint32_t>(most, 2u * (uint32_t)(d.n_slew * d.n_cap));
    if ((int64_t)most <= (int64_t)room) {
      v.walk_lut = (int32_t)most;
      break;
    }
    if (c->tun.grid_blocks > 0 || attempt >= 3) break;
    target_blocks *= 2;
  }
  v.n_ranges = nr;
  v.grid = std::max(1, nr);
  HIPCHK(v.rchunk.ensure(sizeof(uint32_t) * rq.size()));
  HIPCHK(v.chunk_blk.ensure(sizeof(uint32_t) * cb.size()));
  HIPCHK(v.blk_wave.ensure(sizeof(double) * (size_t)v.grid * v.Cc));
  HIPCHK(v.blk_cnt.ensure(sizeof(unsigned long long) * (size_t)v.grid * v.Cc));
  HIPCHK(v.blk_part.ensure(sizeof(double) * 8 * (size_t)v.grid));
  HIPCHK(v.res.ensure(sizeof(double) * 16));
  HIPCHK(hipMemcpyAsync(v.rchunk.p, rq.data(), sizeof(uint32_t) * rq.size(), hipMemcpyHostToDevice, s));
  HIPCHK(hipMemcpyAsync(v.chunk_blk.p, cb.data(), sizeof(uint32_t) * cb.size(), hipMemcpyHostToDevice, s));
  v.chunk_blk_host = cb;
  HIPCHK(v.wdesc.ensure(sizeof(uint2) * (size_t)v.grid * NW));
  HIPCHK(hipMemsetAsync(v.wdesc.p, 0, sizeof(uint2) * (size_t)v.grid * NW, s));
  std::vector<uint32_t> wave_len((size_t)nr * NW, 0);
  if (W > 0) {
    // ---- every block's windows, longest first (a stable sort keeps gate order among equals)
    HIPCHK(ls.wkey0.ensure(sizeof(uint64_t) * W));
    HIPCHK(ls.wkey1.ensure(sizeof(uint64_t) * W));
    HIPCHK(ls.worder.ensure(sizeof(uint32_t) * W));
    HIPCHK(pa::launch_win_keys(W, ls.ws.as<uint32_t>(), ls.bwin.as<uint32_t>(), nr, ls.skey.as<uint64_t>(),
                               pa::out_code(v.pb), ls.wkey0.as<uint64_t>(), ls.widx.as<uint32_t>(),
                               v.wlen.as<uint32_t>(), s));
    const int end_bit = 32 + (int)bits_for((uint64_t)std::max(nr - 1, 0));
    HIPCHK(sort_pairs64(ls.wkey0, ls.wkey1, ls.widx, ls.worder, W, end_bit, ls.tmp, s));
    // ---- phases: every window's place in its lane's stream, every wave's stream length
    HIPCHK(ls.wlane.ensure(sizeof(uint2) * W));
    HIPCHK(ls.phase.ensure(sizeof(uint2) * pa::phase_plan_entries(W, nr)));
    HIPCHK(ls.wave_len.ensure(sizeof(uint32_t) * (size_t)nr * NW));
    // the walk kernel's slots of an input phase cost about 2.5 times those of
    // an output phase (no table reads, leakage or pin records there)
    const bool walk = v.walk_lut > 0;
    HIPCHK(pa::launch_phase_plan(nr, ls.bwin.as<uint32_t>(), ls.worder.as<uint32_t>(), ls.wkey1.as<uint64_t>(),
                                 v.wlen.as<uint32_t>(), walk ? 2u : 0u, walk ? kWalkCostIn : 1u,
                                 walk ? kWalkCostOut : 1u, ls.phase.as<uint2>(), ls.wlane.as<uint2>(),
                                 ls.wave_len.as<uint32_t>(), s));
    HIPCHK(hipMemcpyAsync(wave_len.data(), ls.wave_len.p, sizeof(uint32_t) * wave_len.size(), hipMemcpyDeviceToHost,
                          s));
    HIPCHK(hipStreamSynchronize(s));
  }
  // ---- every wave's first slot: 64 lane streams of its longest stream's length each
  std::vector<uint2> wd((size_t)v.grid * NW, make_uint2(0u, 0u));
  uint64_t slots = 0, busy = 0;
  uint32_t longest = 0;
  for (size_t w = 0; w < wave_len.size(); ++w) {
    wd[w] = make_uint2((uint32_t)slots, wave_len[w]);
    slots += 64 * (uint64_t)wave_len[w];
    longest = std::max(longest, wave_len[w]);
    busy += wave_len[w] > 0 ? 1 : 0;
  }
  v.wave_steps_max = (int32_t)(longest / 2);
  v.wave_steps_mean = busy ? (float)((double)slots / 128.0 / (double)busy) : 0.f;
  if (slots >= (uint64_t(1) << 31))
    return fail(PA_EINVAL, "pa_load_events: the lane streams need %llu slots (2^31 allowed)",
                (unsigned long long)slots);
  v.slots = (int64_t)slots;
  v.ev_map = false;  // the slots moved: the per-event map is built again when asked for
  HIPCHK(hipMemcpyAsync(v.wdesc.p, wd.data(), sizeof(uint2) * wd.size(), hipMemcpyHostToDevice, s));
  // ---- the streams: keys and slews, the caller's index of every event; empty slots hold the pad key
  const int64_t Sa = (int64_t)slots + 2;  // two zeroed entries past the streams
  HIPCHK(v.key.ensure(sizeof(uint64_t) * Sa));
  HIPCHK(v.slew.ensure(sizeof(float) * Sa));
  HIPCHK(v.orig.ensure(sizeof(uint32_t) * Sa));
  HIPCHK(pa::launch_fill_u64(Sa, v.pad_key, v.key.as<uint64_t>(), s));
  HIPCHK(hipMemsetD32Async((hipDeviceptr_t)v.slew.p, 0x3F800000, Sa, s));  // 1.0f: a pad slot's slew
  HIPCHK(hipMemsetAsync(v.orig.p, 0xFF, sizeof(uint32_t) * Sa, s));
  if (W > 0)
    HIPCHK(pa::launch_scatter(E, ls.skey.as<uint64_t>(), ls.sslew.as<float>(), ls.sorig.as<uint32_t>(),
                              ls.winc.as<uint32_t>(), ls.ws.as<uint32_t>(), ls.wlane.as<uint2>(), v.wdesc.as<uint2>(),
                              v.key.as<uint64_t>(), v.slew.as<float>(), v.orig.as<uint32_t>(), s));
  // the walk kernel's compact stream and the phases' header pairs
  if (v.walk_lut > 0) {
    HIPCHK(v.ckey.ensure(sizeof(uint32_t) * Sa));
    HIPCHK(v.cslew.ensure(sizeof(uint32_t) * Sa));
    HIPCHK(pa::launch_compact(Sa, v.key.as<uint64_t>(), v.slew.as<float>(), v.pad_key, v.pb, v.tb, v.gb, v.tbc, v.ck,
                              v.ckey.as<uint32_t>(), v.cslew.as<uint32_t>(), s));
    // the windows ranked gate-major (a stable sort keeps a gate's windows in
    // time order), every gate's first rank and its pieces for the row sums
    HIPCHK(v.goff.ensure(sizeof(uint32_t) * (size_t)(d.G + 1)));
    HIPCHK(v.pfirst.ensure(sizeof(uint32_t) * (size_t)(d.G + 1)));
    HIPCHK(v.wpos.ensure(sizeof(uint32_t) * (size_t)std::max<int64_t>(W, 1)));
    HIPCHK(hipMemsetAsync(v.pfirst.p, 0, sizeof(uint32_t) * (size_t)(d.G + 1), s));
    v.n_pieces = 0;
    v.gate_prep = false;
    if (W > 0) {
      HIPCHK(ls.wkey0.ensure(sizeof(uint32_t) * 2 * (size_t)W));
      // the values' two buffers: either ends up free after the sort, and holds the gates' pieces
      HIPCHK(ls.widx.ensure(sizeof(uint32_t) * (size_t)std::max<int64_t>(W, d.G)));
      HIPCHK(ls.worder.ensure(sizeof(uint32_t) * (size_t)std::max<int64_t>(W, d.G)));
      HIPCHK(ls.wkey1.ensure(sizeof(uint32_t) * (size_t)W));
      uint32_t *qk = ls.wkey0.as<uint32_t>(), *qs = qk + W, *qv = ls.widx.as<uint32_t>(),
               *qw = ls.worder.as<uint32_t>();
      HIPCHK(pa::launch_win_gates(W, ls.ws.as<uint32_t>(), ls.skey.as<uint64_t>(), v.gb, qk, qv, s));
      const int gbits = (int)bits_for((uint64_t)std::max<int64_t>(d.G - 1, 0));
      size_t tb = 0;
      HIPCHK(pa::sort_pairs_u32(&qk, &qs, &qv, &qw, W, gbits, nullptr, &tb, s));
      HIPCHK(ls.tmp.ensure(tb));
      HIPCHK(pa::sort_pairs_u32(&qk, &qs, &qv, &qw, W, gbits, ls.tmp.p, &tb, s));
      // the pieces per gate, their prefix after pfirst[0] = 0
      uint32_t *npiece = qw;
      HIPCHK(pa::launch_win_ranks(W, d.G, qk, qv, ls.wkey1.as<uint32_t>(), v.goff.as<uint32_t>(), npiece, s));
      tb = 0;
      HIPCHK(pa::scan_inclusive_u32(npiece, v.pfirst.as<uint32_t>() + 1, d.G, nullptr, &tb, s));
      HIPCHK(ls.tmp.ensure(tb));
      HIPCHK(pa::scan_inclusive_u32(npiece, v.pfirst.as<uint32_t>() + 1, d.G, ls.tmp.p, &tb, s));
      HIPCHK(hipMemcpyAsync(&v.n_pieces, v.pfirst.as<uint32_t>() + d.G, sizeof(uint32_t), hipMemcpyDeviceToHost, s));
    }
    const uint32_t hdr = ((1u << v.tbc) - 1u) << v.ck;
    HIPCHK(pa::launch_headers(W, ls.wlane.as<uint2>(), v.wdesc.as<uint2>(), ls.ws.as<uint32_t>(),
                              ls.skey.as<uint64_t>(), d.gate_rec.as<uint4>(), ls.wkey1.as<uint32_t>(), v.gb,
                              pa::out_code(v.pb), hdr, 1u << (v.tbc + v.ck), v.ckey.as<uint32_t>(),
                              v.cslew.as<uint32_t>(), v.wpos.as<uint32_t>(), s));
  }
  // the cells whose LUTs every block copies into its spare LDS
  v.lut_lds = pa::pass_lut_lds_doubles(v.Cc, d.n_cells, d.n_slew, d.n_cap, d.n_thr, d.n_leak, d.kmax);
  if (c->tun.lut_lds_kib < 0) v.lut_lds = 0;
  else if (c->tun.lut_lds_kib > 0) v.lut_lds = std::min<int32_t>(v.lut_lds, c->tun.lut_lds_kib * 128);
  if (v.lut_lds > 0 && nr > 0 && W > 0) {
    HIPCHK(v.lplan.ensure(sizeof(uint2) * (size_t)nr * pa::pass_lut_plan_slots()));
    HIPCHK(pa::launch_lut_plan(ls.skey.as<uint64_t>(), ls.ws.as<uint32_t>(), ls.bwin.as<uint32_t>(), nr,
                               d.gate_rec.as<uint4>(), d.cell_meta.as<uint2>(), v.gb, d.n_slew, d.n_cap, v.lut_lds,
                               v.lplan.as<uint2>(), s));
  } else {
    v.lut_lds = 0;
  }
  HIPCHK(hipStreamSynchronize(s));
  return PA_OK;
}

// the buffers of the previous event load and the load's scratch: kept across
// the many loads of one activity text, dropped after a load of the caller's own
static void release_load_buffers(pa_ctx *c) {
  c->ls = LoadScratch();
  c->ev_spare = Events();
}

static int load_events(pa_ctx *c, int64_t n_pins, int64_t n_events, const int64_t *pin_ptr, const uint8_t *pin_init,
                       const int64_t *evt_t, const uint8_t *evt_val, const float *evt_slew, int64_t t_clk,
                       int64_t t_max, double tick_s);

int pa_load_events(pa_ctx *c, int64_t n_pins, int64_t n_events, const int64_t *pin_ptr, const uint8_t *pin_init,
                   const int64_t *evt_t, const uint8_t *evt_val, const float *evt_slew, int64_t t_clk,
                   int64_t t_max, double tick_s) {
  BudgetScope bs(c ? &c->mem : nullptr);
  const int rc = load_events(c, n_pins, n_events, pin_ptr, pin_init, evt_t, evt_val, evt_slew, t_clk, t_max, tick_s);
  if (c && !c->keep_load_buffers) {
    (void)hipSetDevice(c->device);
    if (c->stream) (void)hipStreamSynchronize(c->stream);
    release_load_buffers(c);
  }
  return rc;
}

static int load_events(pa_ctx *c, int64_t n_pins, int64_t n_events, const int64_t *pin_ptr, const uint8_t *pin_init,
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
  // ---- validation: the pin checks and the event checks run back to back
  // (the event kernels stay in bounds whatever pin_ptr holds) and are read
  // back once, reported in order
  DBuf &err = c->ls.err, &ev_pin = c->ls.ev_pin;
  HIPCHK(err.ensure(sizeof(uint32_t)));
  HIPCHK(ev_pin.ensure(sizeof(uint32_t) * std::max<int64_t>(E, 1)));
  HIPCHK(hipMemsetAsync(err.p, 0, sizeof(uint32_t), s));
  HIPCHK(pa::launch_pin_check(P, E, pin_ptr, pin_init, err.as<uint32_t>(), s));
  if (E > 0) {
    // owning pins (a scatter of every pin's index at its first event and a
    // running maximum), then the checks
    DBuf &mark = c->ls.idx, &tmp = c->ls.tmp;
    HIPCHK(mark.ensure(sizeof(uint32_t) * E));
    size_t tb = 0;
    HIPCHK(pa::launch_event_check(E, P, pin_ptr, pin_init, evt_t, evt_val, evt_slew, t_max, mark.as<uint32_t>(),
                                  ev_pin.as<uint32_t>(), err.as<uint32_t>(), nullptr, &tb, s));
    HIPCHK(tmp.ensure(tb));
    HIPCHK(pa::launch_event_check(E, P, pin_ptr, pin_init, evt_t, evt_val, evt_slew, t_max, mark.as<uint32_t>(),
                                  ev_pin.as<uint32_t>(), err.as<uint32_t>(), tmp.p, &tb, s));
  }
  uint32_t herr = 0;
  HIPCHK(hipMemcpyAsync(&herr, err.p, sizeof(uint32_t), hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));
  if (herr & pa::ERR_ENDS) return fail(PA_EDATA, "pa_load_events: pin_ptr[0] must be 0 and pin_ptr[P] = n_events");
  if (herr & pa::ERR_PIN_PTR) return fail(PA_EDATA, "pa_load_events: pin_ptr decreases");
  if (herr & pa::ERR_INIT) return fail(PA_EDATA, "pa_load_events: pin_init not in {0,1}");
  if (herr & pa::ERR_TIME_RANGE) return fail(PA_EDATA, "pa_load_events: event time outside [0, t_max)");
  if (herr & pa::ERR_TIME_ORDER) return fail(PA_EDATA, "pa_load_events: timestamps not strictly increasing on a pin");
  if (herr & pa::ERR_VALUE) return fail(PA_EDATA, "pa_load_events: values do not alternate starting from !init");
  if (herr & pa::ERR_SLEW) return fail(PA_EDATA, "pa_load_events: slew not finite and > 0");

  // ---- bit widths of the layout: lk = (cycle in chunk | pin code | time in cycle) in 32 bits
  // the new layout goes into the buffers of the events before the current
  // ones; the current events stay usable until the load succeeds
  Events v = std::move(c->ev_spare);
  c->ev_spare = Events();
  v.E = E;
  v.T = t_clk;
  v.t_max = t_max;
  v.tick_s = tick_s;
  v.C = (t_max + t_clk - 1) / t_clk;
  v.last_len = (uint32_t)(t_max - (v.C - 1) * t_clk);
  if ((uint64_t)G > pa::kKeyMaxGates - 1)
    return fail(PA_EINVAL, "pa_load_events: designs of more than 2^22 - 1 gates are not supported");
  v.pb = bits_for((uint64_t)d.kmax);  // the output pin's code 2^pb - 1 is above every input pin index
  v.tb = t_clk > 1 ? bits_for((uint64_t)(t_clk - 1)) : 0;
  if (v.pb + v.tb > 32)
    return fail(PA_EINVAL, "pa_load_events: clock period longer than 2^%d ticks", 32 - (int)v.pb);
  // chunk length: a power of two (window lengths halve it), at most the LDS bins
  // the cycle in the chunk has the low word's bits above pin code and tic, and
  // the bits the gate id leaves free in the high word
  const uint32_t gb = bits_for((uint64_t)std::max<int64_t>(G - 1, 0));
  const uint32_t lc_max = (32 - v.pb - v.tb) + (22 - gb);
  int64_t Cc_want = c->tun.chunk_cycles > 0 ? c->tun.chunk_cycles : pa::pass_max_chunk_cycles();
  Cc_want = std::min<int64_t>(Cc_want, (int64_t)pa::pass_max_chunk_cycles());
  if (lc_max < 31) Cc_want = std::min<int64_t>(Cc_want, int64_t(1) << lc_max);
  // the walk kernel's 32-bit key: cycle, tic (bits of t_clk itself, so the
  // tic field is never all ones in an event) and the pin code's high bits;
  // unless the caller fixed the chunk, it is cut to what that key holds
  v.tbc = bits_for((uint64_t)t_clk);
  v.ck = d.kmax > 2 ? bits_for((uint64_t)((d.kmax - 1) >> 1)) : 0;
  const bool compact_want = pa::walk_supported(d.n_slew, d.n_cap) && c->tun.lut_lds_kib == 0 &&
                            d.n_cells < (1 << 20) && v.tbc + v.ck + 6 <= 32;
  if (compact_want && c->tun.chunk_cycles == 0)
    Cc_want = std::min<int64_t>(Cc_want, int64_t(1) << (32 - v.tbc - v.ck));
  int64_t Cc = 1;
  while (Cc * 2 <= Cc_want) Cc *= 2;
  uint32_t lc = 0;
  while ((int64_t(1) << lc) < Cc) ++lc;
  v.compact_ok = compact_want && lc + v.tbc + v.ck <= 32;
  v.Cc = (int32_t)Cc;
  v.Q = (int32_t)((v.C + Cc - 1) / Cc);
  // the pad key: an output-pin 1->0 event at time 0 of cycle Cc (no event's
  // cycle in its chunk reaches Cc); without a spare cycle bit empty slots are
  // key 0 (no event has it: an event at a window start is a head)
  v.pad_key = 0;
  if (lc + 1 <= lc_max) {
    const uint64_t lk = ((uint64_t)Cc << (v.pb + v.tb)) | pa::out_code(v.pb);
    v.pad_key = ((lk >> 32) << (pa::kKeyGateShift + gb)) | (lk & 0xFFFFFFFFull);
  }
  v.chunk_ticks = Cc * t_clk;
  pa::LayoutFmt f{};
  f.T = t_clk;
  f.Cc = (int32_t)Cc;
  f.lc = lc;
  f.pb = v.pb;
  f.tb = v.tb;
  f.gb = gb;
  v.gb = gb;
  const uint32_t lkb = lc + v.pb + v.tb + 1;  // (kind, cycle, time, pin): kind 1 = the output pin
  const uint32_t qbits = bits_for((uint64_t)std::max<int32_t>(v.Q - 1, 0));
  const int32_t Q = v.Q;

  // the events in window order (scratch); build_ranges lays them out for the pass
  DBuf &skey = c->ls.skey, &sslew = c->ls.sslew, &sorig = c->ls.sorig;
  HIPCHK(skey.ensure(sizeof(uint64_t) * std::max<int64_t>(E, 1)));
  HIPCHK(sslew.ensure(sizeof(float) * std::max<int64_t>(E, 1)));
  HIPCHK(sorig.ensure(sizeof(uint32_t) * std::max<int64_t>(E, 1)));
  HIPCHK(v.pin_init.ensure(P));
  DBuf &chunk_sorted = c->ls.chunk_sorted, &cbase = c->ls.cbase;
  HIPCHK(chunk_sorted.ensure(sizeof(uint32_t) * E));
  HIPCHK(cbase.ensure(sizeof(uint32_t) * (Q + 1)));
  if (E > 0) {
    // ---- density-aware window level per gate
    DBuf &level = c->ls.level;
    HIPCHK(level.ensure(G));
    int32_t fixed_level = -1;
    if (c->tun.fixed_window_cycles > 0) {
      int64_t n = 1;
      while (n * 2 <= c->tun.fixed_window_cycles && n * 2 <= Cc) n *= 2;
      fixed_level = 0;
      while ((Cc >> fixed_level) > n) ++fixed_level;
    }
    HIPCHK(pa::launch_gate_levels(G, d.pin_base.as<int64_t>(), d.gate_k.as<int32_t>(), pin_ptr, v.C, (int32_t)Cc,
                                  (int32_t)lc, kWindowEvents, fixed_level, level.as<uint8_t>(), s));
    // ---- order (chunk, gate, kind, cycle, time, pin) by radix sort
    DBuf &k0 = c->ls.k0, &k1 = c->ls.k1, &idx = c->ls.idx, &perm = c->ls.perm, &tmp = c->ls.tmp;
    size_t tmp_bytes = 0;
    HIPCHK(k0.ensure(sizeof(uint64_t) * E));
    HIPCHK(k1.ensure(sizeof(uint64_t) * E));
    HIPCHK(idx.ensure(sizeof(uint32_t) * E));
    HIPCHK(perm.ensure(sizeof(uint32_t) * E));
    const bool one_key = qbits + f.gb + lkb <= 64;
    DBuf &chunk = c->ls.chunk;
    if (!one_key) HIPCHK(chunk.ensure(sizeof(uint32_t) * E));
    HIPCHK(pa::launch_sort_keys(E, evt_t, ev_pin.as<uint32_t>(), d.pin_gate.as<int32_t>(), d.pin_local.as<uint8_t>(),
                                d.gate_k.as<int32_t>(), f, k0.as<uint64_t>(),
                                one_key ? nullptr : chunk.as<uint32_t>(), idx.as<uint32_t>(), s));
    const int end_bit = (int)(one_key ? qbits + f.gb + lkb : f.gb + lkb);
    HIPCHK(sort_pairs64(k0, k1, idx, perm, E, end_bit, tmp, s));  // sorted keys in k1, permutation in perm
    if (!one_key) {
      // stable second pass by chunk (the keys in k0's buffer as 32-bit words)
      uint32_t *qk = reinterpret_cast<uint32_t *>(k0.p), *qs = qk + E;
      HIPCHK(pa::launch_chunk_of(E, perm.as<uint32_t>(), chunk.as<uint32_t>(), qk, s));
      uint32_t *pa_ = perm.as<uint32_t>(), *pb_ = idx.as<uint32_t>();
      tmp_bytes = 0;
      HIPCHK(pa::sort_pairs_u32(&qk, &qs, &pa_, &pb_, E, (int)qbits, nullptr, &tmp_bytes, s));
      HIPCHK(tmp.ensure(tmp_bytes));
      HIPCHK(pa::sort_pairs_u32(&qk, &qs, &pa_, &pb_, E, (int)qbits, tmp.p, &tmp_bytes, s));
      if (pa_ != perm.p) swap_bufs(perm, idx);  // the permutation ended in idx's buffer
    }
    // ---- packed keys and window heads (the start states come with the windows)
    HIPCHK(pa::launch_layout(E, perm.as<uint32_t>(), one_key ? k1.as<uint64_t>() : nullptr, evt_t, evt_slew, evt_val,
                             ev_pin.as<uint32_t>(), d.pin_gate.as<int32_t>(), d.pin_local.as<uint8_t>(),
                             d.gate_k.as<int32_t>(), level.as<uint8_t>(), f, skey.as<uint64_t>(), sslew.as<float>(),
                             sorig.as<uint32_t>(), chunk_sorted.as<uint32_t>(), s));
  }
  HIPCHK(pa::launch_chunk_base(E, Q, chunk_sorted.as<uint32_t>(), cbase.as<uint32_t>(), s));
  if (P > 0) HIPCHK(hipMemcpyAsync(v.pin_init.p, pin_init, P, hipMemcpyDeviceToDevice, s));
  int rc = build_ranges(c, v, pin_ptr, pin_init, evt_t);
  if (rc != PA_OK) return rc;
  c->ev_spare = std::move(c->ev);
  c->ev = std::move(v);
  c->has_events = true;
  return PA_OK;
}

// Where the pass puts its per-block partial results and the finalize its
// result slots: [grid][Cc] bins, [grid][Cc] counts, [grid][8] totals, [16].
struct PassScratch {
  double *blk_wave = nullptr;
  unsigned long long *blk_cnt = nullptr;
  double *blk_part = nullptr;
  double *res = nullptr;
};

static PassScratch loaded_scratch(Events &v) {
  return PassScratch{v.blk_wave.as<double>(), v.blk_cnt.as<unsigned long long>(), v.blk_part.as<double>(),
                     v.res.as<double>()};
}

// the same four pieces carved from one block at base (256-byte aligned pieces);
// returns the bytes they take
static size_t carve_scratch(const Events &v, void *base, PassScratch *out) {
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t n = (size_t)v.grid * (size_t)v.Cc;
  const size_t o_cnt = al(sizeof(double) * n), o_part = o_cnt + al(sizeof(unsigned long long) * n),
               o_res = o_part + al(sizeof(double) * 8 * (size_t)v.grid), end = o_res + al(sizeof(double) * 16);
  if (out) {
    char *b = static_cast<char *>(base);
    *out = PassScratch{reinterpret_cast<double *>(b), reinterpret_cast<unsigned long long *>(b + o_cnt),
                       reinterpret_cast<double *>(b + o_part), reinterpret_cast<double *>(b + o_res)};
  }
  return end;
}

static int run_pass(pa_ctx *c, const PassScratch &sc, pa_totals *out, double *wave_J, uint64_t *cyc_events,
                    uint64_t *cyc_glitches, uint8_t *evt_glitch, uint8_t *evt_state_before, double *gate_J) {
  const Design &d = c->d;
  Events &v = c->ev;
  hipStream_t s = c->stream;
  // per-gate rows from the walk kernel: every window's sums stored at its
  // rank, the rows made from them after the pass; else the general kernel,
  // which adds to rows set up before it
  const bool gate_walk = gate_J && !evt_glitch && !evt_state_before && v.walk_lut > 0 && c->tun.plain_bins == 0 &&
                         v.n_windows > 0;
  if (gate_walk && !v.gate_prep) {
    HIPCHK(v.wrec.ensure(sizeof(double) * 4 * (size_t)((v.slots + 3) / 2)));
    HIPCHK(v.wpart.ensure(sizeof(double) * 4 * (size_t)std::max<uint32_t>(v.n_pieces, 1)));
    HIPCHK(v.pgate.ensure(sizeof(uint32_t) * (size_t)std::max<uint32_t>(v.n_pieces, 1)));
    HIPCHK(v.gleak.ensure(sizeof(double) * (size_t)d.G));
    HIPCHK(pa::launch_gate_prep(d.G, d.gate_info.as<uint32_t>(), d.cell_meta.as<uint2>(), d.leak.as<double>(),
                                d.pin_base.as<int64_t>(), v.pin_init.as<uint8_t>(), (double)v.t_max * v.tick_s,
                                v.pfirst.as<uint32_t>(), v.gleak.as<double>(), v.pgate.as<uint32_t>(), s));
    v.gate_prep = true;
  }
  if (gate_J && !gate_walk)
    HIPCHK(pa::launch_gate_rows(d.G, d.gate_info.as<uint32_t>(), d.cell_meta.as<uint2>(), d.leak.as<double>(),
                                d.pin_base.as<int64_t>(), v.pin_init.as<uint8_t>(), d.perm.as<int32_t>(),
                                (double)v.t_max * v.tick_s, gate_J, s));

  pa::PassArgs a{};
  a.key = v.key.as<uint64_t>();
  a.slew = v.slew.as<float>();
  a.orig = v.orig.as<uint32_t>();
  a.wdesc = v.wdesc.as<uint2>();
  a.rchunk = v.rchunk.as<uint32_t>();
  a.n_ranges = v.n_ranges;
  a.E = v.E;
  a.Q = v.Q;
  a.Cc = v.Cc;
  a.C = v.C;
  a.T = (uint32_t)v.T;
  a.tb = v.tb;
  a.pb = v.pb;
  a.gb = v.gb;
  a.last_len = v.last_len;
  a.chunk_ticks = v.chunk_ticks;
  a.t_max = v.t_max;
  a.tick_s = v.tick_s;
  a.G = d.G;
  a.gate_rec = d.gate_rec.as<uint4>();
  a.hv2 = 0.5 * d.vdd * d.vdd;
  a.pin_base = d.pin_base.as<int64_t>();
  a.pin_init = v.pin_init.as<uint8_t>();
  a.cell_meta = d.cell_meta.as<uint2>();
  a.cell_thr = d.cell_thr.as<float>();
  a.cell_axw = d.cell_axw.as<double2>();
  a.cell_caxw = d.cell_caxw.as<double2>();
  a.lut = d.lut.as<double>();
  a.leak = d.leak.as<double>();
  a.n_slew = d.n_slew;
  a.n_cap = d.n_cap;
  a.n_cells = d.n_cells;
  a.n_thr = d.n_thr;
  a.n_leak = d.n_leak;
  a.kmax = d.kmax;
  a.lut_plan = v.lut_lds > 0 ? v.lplan.as<uint2>() : nullptr;
  a.lut_lds = v.lut_lds;
  a.pad_key = v.pad_key;
  a.blk_lut = v.walk_lut > 0 ? v.blk_lut.as<uint2>() : nullptr;
  a.walk_lut = v.walk_lut;
  a.ckey = v.walk_lut > 0 ? v.ckey.as<uint32_t>() : nullptr;
  a.cslew = v.walk_lut > 0 ? v.cslew.as<uint32_t>() : nullptr;
  a.tbc = v.tbc;
  a.ck = v.ck;
  a.plain_bins = c->tun.plain_bins;
  a.blk_wave = sc.blk_wave;
  a.blk_cnt = sc.blk_cnt;
  a.blk_part = sc.blk_part;
  a.evt_glitch = evt_glitch;
  a.gate_J = gate_walk ? nullptr : gate_J;
  a.wrec = gate_walk ? v.wrec.as<double>() : nullptr;
  a.gate_perm = d.perm.as<int32_t>();
  a.evt_state = evt_state_before;
  // per-event outputs from the walk kernel (in stream order, then into the
  // caller's order) once the slot map is built; else the general kernel
  const bool ev_walk = (evt_glitch || evt_state_before) && !gate_J && v.walk_lut > 0 && c->tun.plain_bins == 0 &&
                       v.ev_map;
  if (ev_walk) {
    a.evt_glitch = nullptr;
    a.evt_state = nullptr;
    a.evs = v.evs.as<uint32_t>();
  }

  pa::FinalArgs f{};
  f.C = v.C;
  f.Cc = v.Cc;
  f.Q = v.Q;
  f.T = (uint32_t)v.T;
  f.last_len = v.last_len;
  f.t_max = v.t_max;
  f.tick_s = v.tick_s;
  f.grid = v.grid;
  f.chunk_blk = v.chunk_blk.as<uint32_t>();
  if (v.Q < 64)
    for (int i = 0; i <= v.Q; ++i) f.cblk[i] = v.chunk_blk_host[i];
  f.l0 = v.l0_host;
  f.blk_wave = a.blk_wave;
  f.blk_cnt = a.blk_cnt;
  f.blk_part = a.blk_part;
  f.wave_out = wave_J;
  f.cyc_events = cyc_events;
  f.cyc_glitches = cyc_glitches;
  f.res = sc.res;

  const bool timed = c->tun.time_kernels != 0, per_kernel = c->tun.time_kernels == 1;
  // mode 1 times each kernel by events attached to its dispatch, mode 2 the
  // whole pass by events recorded before the first and after the last
  if (timed) HIPCHK(hipEventRecord(c->tev[0], s));
  hipError_t e1 = per_kernel ? pa::launch_pass(a, v.grid, s, c->tev[2], c->tev[3]) : pa::launch_pass(a, v.grid, s);
  if (e1 == hipSuccess && ev_walk)
    e1 = pa::launch_event_out(v.E, v.slot_of.as<uint32_t>(), v.evs.as<uint32_t>(), evt_glitch, evt_state_before, s);
  if (e1 == hipSuccess && gate_walk)
    e1 = pa::launch_gate_sums(d.G, v.n_pieces, v.goff.as<uint32_t>(), v.pfirst.as<uint32_t>(),
                              v.pgate.as<uint32_t>(), v.gleak.as<double>(), d.perm.as<int32_t>(),
                              v.wpos.as<uint32_t>(), v.wrec.as<double>(), v.wpart.as<double>(), gate_J, s);
  if (e1 == hipSuccess)
    e1 = per_kernel ? pa::launch_finalize(f, s, c->tev[4], c->tev[5]) : pa::launch_finalize(f, s);
  if (timed && e1 == hipSuccess) e1 = hipEventRecord(c->tev[1], s);
  if (e1 == hipSuccess) e1 = hipMemcpyAsync(c->h_res, f.res, sizeof(double) * 16, hipMemcpyDeviceToHost, s);
  if (e1 == hipSuccess) e1 = hipStreamSynchronize(s);
  if (e1 != hipSuccess) {
    (void)hipStreamSynchronize(s);
    return fail(PA_EHIP, "pa_run: HIP error %s", hipGetErrorString(e1));
  }
  if (per_kernel) {
    (void)hipEventElapsedTime(&c->kernel_ms[0], c->tev[2], c->tev[3]);
    (void)hipEventElapsedTime(&c->kernel_ms[1], c->tev[4], c->tev[5]);
  } else if (timed) {
    c->kernel_ms[0] = c->kernel_ms[1] = 0.0f;
  }
  if (timed) (void)hipEventElapsedTime(&c->kernel_ms[3], c->tev[0], c->tev[1]);
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

int pa_run(pa_ctx *c, pa_totals *out, double *wave_J, uint64_t *cyc_events, uint64_t *cyc_glitches,
           uint8_t *evt_glitch, uint8_t *evt_state_before) {
  if (!c) return fail(PA_EINVAL, "pa_run: NULL context");
  if (!c->has_design || !c->has_events) return fail(PA_ESTATE, "pa_run: design and events must be loaded first");
  if (!out || !wave_J || !cyc_events || !cyc_glitches) return fail(PA_EINVAL, "pa_run: NULL output");
  BudgetScope bs(&c->mem);
  HIPCHK(hipSetDevice(c->device));
  Events &v = c->ev;
  if ((evt_glitch || evt_state_before) && v.walk_lut > 0 && c->tun.plain_bins == 0 && v.E > 0 && !v.ev_map) {
    // the walk kernel's per-event outputs: every event's slot (the inverse of the
    // stream's caller-index array), and room for the values in stream order
    const int64_t Sa = v.slots + 2;
    HIPCHK(v.slot_of.ensure(sizeof(uint32_t) * (size_t)v.E));
    HIPCHK(v.evs.ensure(sizeof(uint32_t) * (size_t)((Sa + 1) / 2)));
    HIPCHK(pa::launch_slot_of(Sa, v.orig.as<uint32_t>(), v.slot_of.as<uint32_t>(), c->stream));
    v.ev_map = true;
  }
  return run_pass(c, loaded_scratch(c->ev), out, wave_J, cyc_events, cyc_glitches, evt_glitch, evt_state_before,
                  nullptr);
}

int pa_run_noalloc(pa_ctx *c, pa_totals *out, double *wave_J, uint64_t *cyc_events, uint64_t *cyc_glitches,
                   uint8_t *evt_glitch, uint8_t *evt_state_before) {
  if (!c) return fail(PA_EINVAL, "pa_run_noalloc: NULL context");
  if (!c->has_design || !c->has_events)
    return fail(PA_ESTATE, "pa_run_noalloc: design and events must be loaded first");
  if (!out || !wave_J || !cyc_events || !cyc_glitches) return fail(PA_EINVAL, "pa_run_noalloc: NULL output");
  if (!c->scratch.p)
    return fail(PA_EHIP, "pa_run_noalloc: no address for the fixed scratch on device %d (%s)", c->device,
                hipGetErrorString(c->scratch.err));
  const size_t need = carve_scratch(c->ev, nullptr, nullptr);
  if (need > (size_t)PA_NOALLOC_SCRATCH_BYTES)
    return fail(PA_EINVAL,
                "pa_run_noalloc: the loaded events need %zu bytes of pass scratch (%d blocks x %d cycles), "
                "more than the fixed %zu; use pa_run",
                need, c->ev.grid, c->ev.Cc, (size_t)PA_NOALLOC_SCRATCH_BYTES);
  HIPCHK(hipSetDevice(c->device));
  PassScratch sc;
  carve_scratch(c->ev, c->scratch.p, &sc);
  return run_pass(c, sc, out, wave_J, cyc_events, cyc_glitches, evt_glitch, evt_state_before, nullptr);
}

int pa_run_gates(pa_ctx *c, pa_totals *out, double *wave_J, uint64_t *cyc_events, uint64_t *cyc_glitches,
                 double *gate_J) {
  if (!c) return fail(PA_EINVAL, "pa_run_gates: NULL context");
  if (!c->has_design || !c->has_events)
    return fail(PA_ESTATE, "pa_run_gates: design and events must be loaded first");
  if (!out || !wave_J || !cyc_events || !cyc_glitches || (!gate_J && c->d.G > 0))
    return fail(PA_EINVAL, "pa_run_gates: NULL output");
  BudgetScope bs(&c->mem);
  HIPCHK(hipSetDevice(c->device));
  return run_pass(c, loaded_scratch(c->ev), out, wave_J, cyc_events, cyc_glitches, nullptr, nullptr, gate_J);
}

int pa_get_window_stats(pa_ctx *c, pa_window_stats *out) {
  if (!c || !out) return fail(PA_EINVAL, "pa_get_window_stats: NULL argument");
  if (!c->has_events) return fail(PA_ESTATE, "pa_get_window_stats: no events loaded");
  HIPCHK(hipSetDevice(c->device));
  const Events &v = c->ev;
  hipStream_t s = c->stream;
  *out = pa_window_stats{};
  if (v.E == 0) return PA_OK;
  const uint64_t hn = (uint64_t)v.n_windows;
  std::vector<uint32_t> h(hn);
  if (hn) HIPCHK(hipMemcpyAsync(h.data(), v.wlen.p, sizeof(uint32_t) * hn, hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));
  std::sort(h.begin(), h.end());
  out->n_windows = (int64_t)hn;
  if (hn) {
    double sum = 0.0;
    for (uint32_t x : h) sum += x;
    out->mean = sum / (double)hn;
    auto pct = [&](double q) { return (int64_t)h[std::min<size_t>(hn - 1, (size_t)(q * (double)(hn - 1) + 0.5))]; };
    out->p50 = pct(0.50);
    out->p90 = pct(0.90);
    out->p99 = pct(0.99);
    out->max = (int64_t)h.back();
  }
  return PA_OK;
}

int pa_get_info(pa_ctx *c, pa_info *info) {
  if (!c || !info) return fail(PA_EINVAL, "pa_get_info: NULL argument");
  std::memset(info, 0, sizeof *info);
  info->n_gates = c->d.G;
  info->n_pins = c->d.P;
  info->n_events = c->has_events ? c->ev.E : 0;  // nothing loaded: nothing for a pass
  info->n_cycles = c->has_events ? c->ev.C : 0;
  info->chunk_cycles = c->ev.Cc;
  info->n_chunks = c->ev.Q;
  info->grid_blocks = c->has_events ? c->ev.grid : 0;
  info->block_threads = pa::pass_block_threads();
  info->batch_events = pa::pass_wave_batch();
  info->max_segment_events = 0;  // no limit
  const LoadScratch &ls = c->ls;
  info->device_bytes = c->d.bytes() + c->ev.bytes() + c->ev_spare.bytes() + (int64_t)c->text_dev.bytes +
                       (int64_t)(ls.err.bytes + ls.ev_pin.bytes + ls.chunk_sorted.bytes + ls.cbase.bytes +
                                 ls.level.bytes + ls.k0.bytes + ls.k1.bytes + ls.idx.bytes + ls.perm.bytes +
                                 ls.chunk.bytes + ls.tmp.bytes + ls.part.bytes + ls.skey.bytes + ls.sslew.bytes +
                                 ls.sorig.bytes + ls.winc.bytes + ls.ws.bytes + ls.bwin.bytes + ls.wkey0.bytes +
                                 ls.wkey1.bytes + ls.widx.bytes + ls.worder.bytes + ls.wlane.bytes +
                                 ls.phase.bytes + ls.wave_len.bytes);
  for (int k = 0; k < 4; ++k) info->kernel_ms[k] = c->kernel_ms[k];
  info->n_windows = c->has_events ? c->ev.n_windows : 0;
  info->n_slots = c->has_events ? c->ev.slots : 0;
  info->wave_steps_max = c->has_events ? c->ev.wave_steps_max : 0;
  info->wave_steps_mean = c->has_events ? c->ev.wave_steps_mean : 0.f;
  info->tables_in_lds = (c->has_design && c->has_events &&
                         pa::pass_cells_fit_lds(c->ev.Cc, c->d.n_cells, c->d.n_slew, c->d.n_cap, c->d.n_thr,
                                                c->d.n_leak, c->d.kmax))
                            ? 1
                            : 0;
  info->walk_kernel = c->has_events && c->ev.walk_lut > 0 ? 1 : 0;
  return PA_OK;
}


}  // extern "C"

// ------------------------------------------------------------ activity text --

namespace {

double now_s() {
  return std::chrono::duration<double>(std::chrono::steady_clock::now().time_since_epoch()).count();
}

int text_threads(int32_t n) {
  if (n > 0) return std::min<int32_t>(n, 256);
  const unsigned h = std::thread::hardware_concurrency();
  return (int)std::max(1u, std::min(16u, h ? h : 1u));
}

// one packed segment: pin_ptr, pin_init and the three event arrays in one block
struct SegLayout {
  size_t o_ptr = 0, o_init = 0, o_t = 0, o_val = 0, o_slew = 0, bytes = 0;
};

SegLayout seg_layout(int64_t P, int64_t E) {
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  SegLayout L;
  size_t o = 0;
  L.o_ptr = o;
  o += al(sizeof(int64_t) * (size_t)(P + 1));
  L.o_init = o;
  o += al((size_t)P);
  L.o_t = o;
  o += al(sizeof(int64_t) * (size_t)E);
  L.o_val = o;
  o += al((size_t)E);
  L.o_slew = o;
  o += al(sizeof(float) * (size_t)E);
  L.bytes = std::max<size_t>(o, 256);
  return L;
}

pa::text::Csr carve(void *base, const SegLayout &L) {
  char *b = static_cast<char *>(base);
  return pa::text::Csr{reinterpret_cast<int64_t *>(b + L.o_ptr), reinterpret_cast<uint8_t *>(b + L.o_init),
                       reinterpret_cast<int64_t *>(b + L.o_t), reinterpret_cast<uint8_t *>(b + L.o_val),
                       reinterpret_cast<float *>(b + L.o_slew)};
}

}  // namespace

extern "C" {

int pa_pack_text(const char *text, int64_t text_len, int64_t n_pins, int32_t n_threads, int64_t max_events,
                 int64_t *n_events, int64_t *pin_ptr, uint8_t *pin_init, int64_t *evt_t, uint8_t *evt_val,
                 float *evt_slew) {
  if (text_len < 0 || (!text && text_len > 0)) return fail(PA_EINVAL, "pa_pack_text: bad text");
  if (!n_events) return fail(PA_EINVAL, "pa_pack_text: n_events is NULL");
  if (n_threads < 0) return fail(PA_EINVAL, "pa_pack_text: n_threads < 0");
  const bool query = !pin_ptr && !pin_init && !evt_t && !evt_val && !evt_slew;
  if (!query && (!pin_ptr || !pin_init || !evt_t || !evt_val || !evt_slew))
    return fail(PA_EINVAL, "pa_pack_text: give all output arrays or none");
  *n_events = 0;
  std::string err;
  pa::text::Header h;
  if (pa::text::parse_header(text, (size_t)text_len, h, err) != 0) return fail(PA_EDATA, "pa_pack_text: %s", err.c_str());
  if (h.n_pins != n_pins)
    return fail(PA_EDATA, "pa_pack_text: the text declares %lld variables, n_pins is %lld", (long long)h.n_pins,
                (long long)n_pins);
  pa::text::Pool pool(text_threads(n_threads));
  pa::text::SegmentIndex ix;
  const int64_t big = std::numeric_limits<int64_t>::max();
  if (pa::text::index_segments(text, (size_t)text_len, h, big, 1, big, pool, ix, err) != 0)
    return fail(PA_EDATA, "pa_pack_text: %s", err.c_str());
  *n_events = ix.events[0];
  if (query) return PA_OK;
  if (max_events < ix.events[0])
    return fail(PA_EINVAL, "pa_pack_text: %lld value changes, max_events is %lld", (long long)ix.events[0],
                (long long)max_events);
  pa::text::Packer pk(pool);
  std::vector<uint8_t> init_end((size_t)n_pins);
  const pa::text::Csr out{pin_ptr, pin_init, evt_t, evt_val, evt_slew};
  if (pk.pack(text, ix.begin[0], ix.begin[1], h, ix.events[0], 0, h.init.data(), out, init_end.data(), err) != 0)
    return fail(PA_EDATA, "pa_pack_text: %s", err.c_str());
  return PA_OK;
}

int pa_run_text(pa_ctx *c, const char *text, int64_t text_len, int64_t t_clk, int64_t t_max, double tick_s,
                const pa_text_opts *o, pa_totals *out, double *wave_J, uint64_t *cyc_events, uint64_t *cyc_glitches,
                pa_text_stats *st) {
  const double w0 = now_s();
  if (!c) return fail(PA_EINVAL, "pa_run_text: NULL context");
  if (!c->has_design) return fail(PA_ESTATE, "pa_run_text: no design loaded");
  if (text_len < 0 || (!text && text_len > 0)) return fail(PA_EINVAL, "pa_run_text: bad text");
  if (!out || !wave_J || !cyc_events || !cyc_glitches) return fail(PA_EINVAL, "pa_run_text: NULL output");
  if (t_clk < 1 || t_clk >= (int64_t(1) << 32)) return fail(PA_EINVAL, "pa_run_text: t_clk out of range");
  if (t_max < 1) return fail(PA_EINVAL, "pa_run_text: t_max must be > 0");
  const int64_t C = (t_max + t_clk - 1) / t_clk;
  if (C > (int64_t(1) << 28)) return fail(PA_EINVAL, "pa_run_text: more than 2^28 clock cycles");
  if (!(tick_s > 0.0) || !std::isfinite(tick_s)) return fail(PA_EINVAL, "pa_run_text: tick_s must be > 0");
  if (o && (o->segment_cycles < 0 || o->n_threads < 0 || o->serial < 0 || o->serial > 1 || o->reserved != 0))
    return fail(PA_EINVAL, "pa_run_text: bad options");
  const int64_t S = o && o->segment_cycles > 0 ? o->segment_cycles : 1024;
  const bool serial = o && o->serial == 1;
  BudgetScope bs(&c->mem);
  HIPCHK(hipSetDevice(c->device));
  // the segments' loads reuse one another's buffers; they go when the text is done
  struct HoldLoadBuffers {
    pa_ctx *c;
    explicit HoldLoadBuffers(pa_ctx *x) : c(x) { c->keep_load_buffers = true; }
    ~HoldLoadBuffers() {
      c->keep_load_buffers = false;
      if (c->stream) (void)hipStreamSynchronize(c->stream);
      release_load_buffers(c);
    }
  } hold(c);
  const int64_t P = c->d.P;
  hipStream_t s = c->stream;

  std::string err;
  double t0 = now_s();
  pa::text::Header h;
  if (pa::text::parse_header(text, (size_t)text_len, h, err) != 0) return fail(PA_EDATA, "pa_run_text: %s", err.c_str());
  if (h.n_pins != P)
    return fail(PA_EDATA, "pa_run_text: the text declares %lld variables, the design has %lld pins",
                (long long)h.n_pins, (long long)P);
  const double header_s = now_s() - t0;
  pa::text::Pool pool(text_threads(o ? o->n_threads : 0));
  const int64_t n_seg = (C + S - 1) / S, seg_ticks = S * t_clk;
  t0 = now_s();
  pa::text::SegmentIndex ix;
  if (pa::text::index_segments(text, (size_t)text_len, h, seg_ticks, n_seg, t_max, pool, ix, err) != 0)
    return fail(PA_EDATA, "pa_run_text: %s", err.c_str());
  const double index_s = now_s() - t0;
  int64_t e_max = 0, e_all = 0;
  for (int64_t k = 0; k < n_seg; ++k) {
    e_max = std::max(e_max, ix.events[(size_t)k]);
    e_all += ix.events[(size_t)k];
  }

  const SegLayout L = seg_layout(P, e_max);
  // pinned host slots and the device staging area, kept by the context for later calls
  pa::text::Csr hcsr[2];
  for (int i = 0; i < (serial ? 1 : 2); ++i) {
    HIPCHK(c->text_host[i].ensure(L.bytes));
    hcsr[i] = carve(c->text_host[i].p, L);
  }
  HIPCHK(c->text_dev.ensure(L.bytes));
  const pa::text::Csr dcsr = carve(c->text_dev.p, L);
  std::vector<uint8_t> cur(h.init), nxt((size_t)P);
  pa::text::Packer pk(pool);

  // every segment's load replaces the context's events; none stay loaded
  struct DropEvents {
    pa_ctx *c;
    ~DropEvents() { c->has_events = false; }
  } drop{c};
  double acc[4] = {0, 0, 0, 0}, parse_s = 0.0, gpu_s = 0.0;
  uint64_t n_gl = 0;

  // copy, load and run segment k from host slot `slot`; release() once the slot's copies are done
  auto gpu_segment = [&](int slot, int64_t k, const std::function<void()> &release) -> int {
    const int64_t c0 = k * S, ts = c0 * t_clk, te = std::min(t_max, ts + seg_ticks);
    const int64_t E = ix.events[(size_t)k];
    const pa::text::Csr &hc = hcsr[slot];
    HIPCHK(hipMemcpyAsync(dcsr.pin_ptr, hc.pin_ptr, sizeof(int64_t) * (size_t)(P + 1), hipMemcpyHostToDevice, s));
    if (P > 0) HIPCHK(hipMemcpyAsync(dcsr.pin_init, hc.pin_init, (size_t)P, hipMemcpyHostToDevice, s));
    if (E > 0) {
      HIPCHK(hipMemcpyAsync(dcsr.t, hc.t, sizeof(int64_t) * (size_t)E, hipMemcpyHostToDevice, s));
      HIPCHK(hipMemcpyAsync(dcsr.val, hc.val, (size_t)E, hipMemcpyHostToDevice, s));
      HIPCHK(hipMemcpyAsync(dcsr.slew, hc.slew, sizeof(float) * (size_t)E, hipMemcpyHostToDevice, s));
    }
    int rc = pa_load_events(c, P, E, dcsr.pin_ptr, dcsr.pin_init, dcsr.t, dcsr.val, dcsr.slew, t_clk, te - ts, tick_s);
    const hipError_t se = hipStreamSynchronize(s);
    release();
    if (rc != PA_OK) return rc;
    if (se != hipSuccess) return fail(PA_EHIP, "pa_run_text: HIP error %s", hipGetErrorString(se));
    pa_totals t{};
    rc = run_pass(c, loaded_scratch(c->ev), &t, wave_J + c0, cyc_events + c0, cyc_glitches + c0, nullptr, nullptr,
                  nullptr);
    if (rc != PA_OK) return rc;
    acc[0] += t.e_int_J;
    acc[1] += t.e_sw_J;
    acc[2] += t.e_gl_J;
    acc[3] += t.e_leak_J;
    n_gl += t.n_glitches;
    return PA_OK;
  };
  auto pack = [&](int slot, int64_t k) -> int {
    const double p0 = now_s();
    const int rc = pk.pack(text, ix.begin[(size_t)k], ix.begin[(size_t)k + 1], h, ix.events[(size_t)k],
                           k * seg_ticks, cur.data(), hcsr[slot], nxt.data(), err);
    parse_s += now_s() - p0;
    if (rc == 0) cur.swap(nxt);
    return rc;
  };

  if (serial) {
    for (int64_t k = 0; k < n_seg; ++k) {
      if (pack(0, k) != 0) return fail(PA_EDATA, "pa_run_text: %s", err.c_str());
      const double g0 = now_s();
      const int rc = gpu_segment(0, k, [] {});
      gpu_s += now_s() - g0;
      if (rc != PA_OK) return rc;
    }
  } else {
    std::mutex mu;
    std::condition_variable cv;
    int64_t packed = -1;
    bool slot_free[2] = {true, true}, stop = false;
    int grc = PA_OK;
    std::string gmsg;
    std::thread gpu([&] {
      BudgetScope gbs(&c->mem);
      if (hipSetDevice(c->device) != hipSuccess) {
        std::lock_guard<std::mutex> g(mu);
        stop = true;
        grc = PA_EHIP;
        gmsg = "pa_run_text: hipSetDevice failed on the copy thread";
        cv.notify_all();
        return;
      }
      for (int64_t k = 0; k < n_seg; ++k) {
        {
          std::unique_lock<std::mutex> lk(mu);
          cv.wait(lk, [&] { return stop || packed >= k; });
          if (stop) return;
        }
        const int slot = (int)(k & 1);
        const double g0 = now_s();
        const int rc = gpu_segment(slot, k, [&] {
          std::lock_guard<std::mutex> g(mu);
          slot_free[slot] = true;
          cv.notify_all();
        });
        gpu_s += now_s() - g0;
        if (rc != PA_OK) {
          std::lock_guard<std::mutex> g(mu);
          stop = true;
          grc = rc;
          gmsg = g_err;
          cv.notify_all();
          return;
        }
      }
    });
    int prc = 0;
    for (int64_t k = 0; k < n_seg; ++k) {
      const int slot = (int)(k & 1);
      {
        std::unique_lock<std::mutex> lk(mu);
        cv.wait(lk, [&] { return stop || slot_free[slot]; });
        if (stop) break;
        slot_free[slot] = false;
      }
      prc = pack(slot, k);
      std::lock_guard<std::mutex> g(mu);
      if (prc != 0) {
        stop = true;
        cv.notify_all();
        break;
      }
      packed = k;
      cv.notify_all();
    }
    gpu.join();
    // the copy thread works on earlier segments than the parser: its error comes first
    if (grc != PA_OK) return fail(grc, "%s", gmsg.c_str());
    if (prc != 0) return fail(PA_EDATA, "pa_run_text: %s", err.c_str());
  }

  const double window = (double)t_max * tick_s;
  out->e_int_J = acc[0];
  out->e_sw_J = acc[1];
  out->e_gl_J = acc[2];
  out->e_leak_J = acc[3];
  out->p_int_W = acc[0] / window;
  out->p_sw_W = acc[1] / window;
  out->p_gl_W = acc[2] / window;
  out->p_leak_W = acc[3] / window;
  out->n_events = (uint64_t)e_all;
  out->n_glitches = n_gl;
  out->n_cycles = C;
  if (st) {
    st->n_segments = n_seg;
    st->n_events = e_all;
    st->max_segment_events = e_max;
    st->text_bytes = text_len;
    st->header_s = header_s;
    st->index_s = index_s;
    st->parse_s = parse_s;
    st->gpu_s = gpu_s;
    st->wall_s = now_s() - w0;
  }
  return PA_OK;
}

}  // extern "C"
