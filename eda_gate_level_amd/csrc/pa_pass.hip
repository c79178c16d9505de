// pa_pass.hip -- the hot path of gate-level time-based power analysis on
// gfx950: one fused pass over the chunk-major event layout plus a finalize.
//
// Method: "GPU-Accelerated Gate-Level Time-Based Power Analysis via
// Event-Density-Aware Partitioning and Kernel Fusion" (arXiv 2609.05960).
// Per event (Sec. 2.4.1, Fig. 2, Eqs. 1-3): the gate state before the event
// selects the internal-power LUT, bilinear on input slew and output load; a
// 0->1 output event draws 1/2 c v^2; the m-th event (m >= 2) of a pin in a
// clock cycle is a glitch scaled by r_gl; the energy lands in the event's
// cycle bin.  Per gate (Sec. 2.4.2, Fig. 3, Eq. 4): state-dependent leakage
// over every inter-event interval, spread over the cycle bins it overlaps.
// The paper fuses both parts into one thread per (gate, cycle window)
// (Fig. 7); this pass instead gives each lane one event and lets a block
// share its events through LDS:
//   * events are laid out chunk-major (time chunks of Cc cycles), then by
//     gate, pin, time; each 64-bit key also carries the gate's input state at
//     the chunk start, so a (chunk, gate) segment is self-contained;
//   * a block streams a contiguous range of segments through LDS in batches
//     (coalesced key/slew loads, next batch prefetched into registers while
//     the current one is computed);
//   * the state before an event comes from one binary search per other input
//     pin inside the segment (value of that pin's last event before t, or the
//     chunk-start state), which is the k-way merge of Sec. 2.4.2 done by
//     search instead of by a sequential walk;
//   * leakage is charged as power changes: at every distinct input timestamp
//     one event (the lowest input pin switching there) adds
//     dP = leak[S+] - leak[S-]; its partial bin gets dP * (bin end - t) and
//     all later bins get dP * their length through an in-LDS prefix sum per
//     chunk and a per-chunk carry; the leakage at t = 0 is the sum over gates
//     of leak[S0].  This is the same sum as the paper's per-interval,
//     per-overlapped-bin split (Sec. 2.4.2), reordered;
//   * per-cycle bins live in LDS and are flushed once per (block, chunk) with
//     fp64/u64 atomics into one of 8 copies (one per XCD), which the
//     finalize kernel adds up.
#include <hip/hip_runtime.h>

#include "pa_common.h"

namespace pa {

namespace {

#ifndef PA_NT
#define PA_NT 1024
#endif
#ifndef PA_R
#define PA_R 2
#endif
#ifndef PA_CCMAX
#define PA_CCMAX 512
#endif
#ifndef PA_GATE_LDS
#define PA_GATE_LDS 2048
#endif
constexpr int kNT = PA_NT;        // threads per block
constexpr int kR = PA_R;          // events per thread per batch
constexpr int kECAP = kNT * kR;
constexpr int kCCMAX = PA_CCMAX;  // max cycles per chunk (LDS bins)
constexpr int kNW = kNT / 64;
constexpr int kXCD = 8;

__device__ __forceinline__ uint32_t key_gate(uint64_t k) { return uint32_t(k >> kKeyGateShift); }
__device__ __forceinline__ uint32_t key_lk(uint64_t k) { return uint32_t(k >> kKeyLkShift); }
__device__ __forceinline__ uint32_t key_val(uint64_t k) { return uint32_t(k >> kKeyValShift) & 1u; }

// first segment head at or after position x (a head starts a (chunk, gate)
// segment); executed by one whole wave
__device__ int find_head(const PassArgs &a, int64_t x) {
  if (x >= a.E) return int(a.E);
  if (x <= 0) return 0;
  // chunk of x: last q with chunk_base[q] <= x
  int lo = 0, hi = a.Q;  // answer in [0, Q-1]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (int64_t(a.chunk_base[mid]) <= x) lo = mid; else hi = mid;
  }
  const int64_t cb0 = a.chunk_base[lo], cb1 = a.chunk_base[lo + 1];
  if (x == cb0) return int(x);
  const int lane = threadIdx.x & 63;
  for (;;) {
    int64_t y = x + lane;
    bool h;
    if (y >= cb1 || y >= a.E) {
      h = true;
    } else {
      h = key_gate(a.key[y]) != key_gate(a.key[y - 1]);
    }
    unsigned long long m = __ballot(h);
    if (m) return int(x + __ffsll((long long)m) - 1);
    x += 64;
  }
}

__device__ __forceinline__ double wave_sum(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// per-cell tables staged in LDS when the library is small enough
constexpr int kMaxCellsLds = 256;
constexpr int kCellDoubles = 2048;
constexpr int kGateLds = PA_GATE_LDS;             // most distinct gate ids in one batch
constexpr int kGPT = (kGateLds + kNT - 1) / kNT;
constexpr int kSeqMax = 64;                       // longest segment merged by one thread
constexpr int kSeqPins = 4;                       // most input pins merged by one thread
constexpr uint32_t kInf = 0xFFFFFFFFu;
static_assert(kR * kNW <= 64, "segment counts of one batch must fit one wave");

// first position in [lo, hi) whose value is >= target (hi if none)
__device__ __forceinline__ int lower_bound_u32(const uint32_t *s, int lo, int hi, uint32_t target) {
  int n = hi - lo;
  while (n > 0) {
    const int half = n >> 1;
    const int mid = lo + half;
    const bool lt = s[mid] < target;
    lo = lt ? mid + 1 : lo;
    n = lt ? n - half - 1 : half;
  }
  return lo;
}

template <bool CELL_LDS, bool DIAG>
__global__ __launch_bounds__(kNT) void k_fused(PassArgs a) {
  // batch staging, decoded from the packed keys
  __shared__ uint32_t sgl[kECAP];        // gate id
  __shared__ uint32_t slk[kECAP];        // (pin << t_bits) | t_rel
  __shared__ uint16_t saux[kECAP];       // S0 | val << 8
  __shared__ uint16_t scyc[kECAP];       // cycle inside the chunk
  __shared__ float sslew[kECAP];
  __shared__ uint32_t ssmo[kECAP];       // state before | switching-pin mask << 8 | owner << 16
  __shared__ uint16_t sseg[kECAP];       // segment index of each event
  __shared__ uint16_t ssegst[kECAP + 1]; // segment starts
  // per-cycle bins of the current chunk
  __shared__ double bw[kCCMAX];               // energy: dynamic + partial-bin leakage
  __shared__ double bb[kCCMAX];               // leakage power change
  __shared__ unsigned long long bc[kCCMAX];   // events | glitches << 32
  // gate data of the batch's gate-id span, cell library
  __shared__ uint32_t s_ginfo[kGateLds];
  __shared__ double s_gcf[kGateLds];
  __shared__ double s_gesw[kGateLds];
  __shared__ double s_cell[CELL_LDS ? kCellDoubles : 1];     // slew axes, inverse widths, leakage
  __shared__ uint32_t s_meta[CELL_LDS ? kMaxCellsLds : 1];   // k | leak base << 4
  __shared__ uint32_t s_lutb[CELL_LDS ? kMaxCellsLds : 1];
  __shared__ int s_hcnt[kR * kNW];
  __shared__ int s_hlast[kR * kNW];
  __shared__ int s_flag;
  __shared__ int s_range[2];
  __shared__ double s_red[kNW * 6];
  __shared__ double s_scan[kNW];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const uint32_t tbits = a.kf.t_bits;
  const uint32_t tmask = (1u << tbits) - 1u;
  const int nb = gridDim.x, b = blockIdx.x;
  const int xcd = b % kXCD;
  const int ns = a.n_slew, nc = a.n_cap;
  const int sa_off = 0, iw_off = a.n_cells * ns, lk_off = iw_off + a.n_cells * (ns - 1);

  // ---- this block's range of whole segments
  if (wid < 2) {
    int64_t nominal = (a.E * (int64_t)(b + wid)) / nb;
    int h = find_head(a, nominal);
    if (lane == 0) s_range[wid] = h;
  }
  for (int c = tid; c < kCCMAX; c += kNT) {
    bw[c] = 0.0;
    bb[c] = 0.0;
    bc[c] = 0ull;
  }
  if constexpr (CELL_LDS) {
    for (int c = tid; c < a.n_cells; c += kNT) {
      s_meta[c] = (uint32_t)a.cell_k[c] | (a.cell_leak_base[c] << 4);
      s_lutb[c] = a.cell_lut_base[c];
    }
    for (int j = tid; j < a.n_cells * ns; j += kNT) s_cell[sa_off + j] = a.slew_axis[j];
    for (int j = tid; j < a.n_cells * (ns - 1); j += kNT) s_cell[iw_off + j] = a.slew_invw[j];
    for (int j = tid; j < a.n_leak; j += kNT) s_cell[lk_off + j] = a.leak[j];
  }
  __syncthreads();
  const int s0 = s_range[0], s1 = s_range[1];

  auto cell_k = [&](uint32_t c) -> uint32_t {
    if constexpr (CELL_LDS) return s_meta[c] & 15u; else return (uint32_t)a.cell_k[c];
  };
  auto leak_base = [&](uint32_t c) -> uint32_t {
    if constexpr (CELL_LDS) return s_meta[c] >> 4; else return a.cell_leak_base[c];
  };
  auto lut_base = [&](uint32_t c) -> uint32_t {
    if constexpr (CELL_LDS) return s_lutb[c]; else return a.cell_lut_base[c];
  };
  auto slew_ax = [&](uint32_t c, int j) -> double {
    if constexpr (CELL_LDS) return s_cell[sa_off + c * ns + j]; else return a.slew_axis[(size_t)c * ns + j];
  };
  auto slew_iw = [&](uint32_t c, int j) -> double {
    if constexpr (CELL_LDS) return s_cell[iw_off + c * (ns - 1) + j]; else return a.slew_invw[(size_t)c * (ns - 1) + j];
  };
  auto leak_of = [&](uint32_t j) -> double {
    if constexpr (CELL_LDS) return s_cell[lk_off + j]; else return a.leak[j];
  };

  double e_int = 0.0, e_sw = 0.0, e_gl = 0.0, e_lk = 0.0, l0 = 0.0;
  unsigned n_gl = 0;

  // ---- leakage at t = 0: sum over gates of leak[S0] (Sec. 2.4.2, Fig. 3)
  for (int64_t g = (int64_t)b * kNT + tid; g < a.G; g += (int64_t)nb * kNT) {
    const uint32_t cell = a.gate_info[g] & 0xFFFFFFu;
    const int kk = (int)cell_k(cell);
    const int64_t p0 = a.pin_base[g];
    uint32_t S = 0;
    for (int j = 0; j < kk; ++j) S |= uint32_t(a.pin_init[p0 + j]) << j;
    l0 += leak_of(leak_base(cell) + S);
  }

  // ---- walk the chunks this block's range touches
  int q = 0;
  if (s0 < s1) {
    int lo = 0, hi = a.Q;
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if ((int)a.chunk_base[mid] <= s0) lo = mid; else hi = mid;
    }
    q = lo;
  }
  int pos = s0;
  uint64_t pk[kR];
  float ps[kR];
  int pf_pos = -1, pf_n = 0;

  while (pos < s1) {
    const int qend = min(s1, (int)a.chunk_base[q + 1]);
    if (pos >= qend) { ++q; continue; }
    const int64_t cstart = (int64_t)q * a.chunk_ticks;
    const int64_t clen = min(a.chunk_ticks, a.t_max - cstart);
    const uint32_t clen32 = (uint32_t)clen;
    const int ncyc = (int)((clen + a.T - 1) / a.T);
    const int64_t tail_from_chunk = a.t_max - cstart;  // t_max - t = tail_from_chunk - t_rel

    while (pos < qend) {
      const int n = min(kECAP, qend - pos);
      // ---- stage and decode the batch (from the prefetch registers when they hold it)
      if (!(pf_pos == pos && pf_n >= n)) {
#pragma unroll
        for (int r = 0; r < kR; ++r) {
          const int x = r * kNT + tid;
          if (x < n) { pk[r] = a.key[pos + x]; ps[r] = a.slew[pos + x]; }
        }
      }
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int x = r * kNT + tid;
        if (x < n) {
          const uint64_t k = pk[r];
          const uint32_t lk = key_lk(k);
          sgl[x] = key_gate(k);
          slk[x] = lk;
          saux[x] = (uint16_t)(uint32_t(k) & 0x1FFu);  // S0 | val << 8
          scyc[x] = (uint16_t)divu32(lk & tmask, a.divT);
          sslew[x] = ps[r];
        }
      }
      if (tid == 0) s_flag = 0;
      __syncthreads();

      // ---- cut the batch so that its gate ids span at most kGateLds, then load their data
      const uint32_t g_lo = sgl[0];
      int n_eff = n;
      if (sgl[n - 1] - g_lo >= (uint32_t)kGateLds) n_eff = lower_bound_u32(sgl, 0, n, g_lo + kGateLds);
      const uint32_t g_span = sgl[n_eff - 1] - g_lo + 1;
      uint32_t pgi[kGPT];
      double pgc[kGPT], pge[kGPT];
#pragma unroll
      for (int u = 0; u < kGPT; ++u) {
        const uint32_t j = u * kNT + tid;
        if (j < g_span) {
          pgi[u] = a.gate_info[g_lo + j];
          pgc[u] = a.gate_capfrac[g_lo + j];
          pge[u] = a.gate_esw[g_lo + j];
        }
      }

      // ---- number the (chunk, gate) segments of the batch
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int x = r * kNT + tid;
        const bool h = (x < n_eff) && (x == 0 || sgl[x] != sgl[x - 1]);
        const unsigned long long hm = __ballot(h);
        if (lane == 0) {
          s_hcnt[r * kNW + wid] = __popcll(hm);
          s_hlast[r * kNW + wid] = hm ? (r * kNT + wid * 64 + 63 - __clzll((long long)hm)) : -1;
        }
      }
      __syncthreads();
      // prefix of the per-(round, wave) head counts, one lane per entry
      const int hc = lane < kR * kNW ? s_hcnt[lane] : 0;
      int hincl = hc;
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(hincl, o, 64);
        if (lane >= o) hincl += v;
      }
      int hl = lane < kR * kNW ? s_hlast[lane] : -1;
      for (int o = 32; o > 0; o >>= 1) hl = max(hl, __shfl_xor(hl, o, 64));
      const int nseg_all = __shfl(hincl, 63, 64);
      const int last_head = hl;
      const bool defer = (n_eff == n) && (pos + n < qend) && last_head > 0;
      const int nproc = defer ? last_head : n_eff;
      const int nseg = defer ? nseg_all - 1 : nseg_all;
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int x = r * kNT + tid;
        const int ent = r * kNW + wid;
        const int sbase = __shfl(hincl, ent, 64) - __shfl(hc, ent, 64);
        const bool h = (x < n_eff) && (x == 0 || sgl[x] != sgl[x - 1]);
        const unsigned long long hm = __ballot(h);
        if (x < nproc) {
          const unsigned long long upto = (lane == 63) ? hm : (hm & ((2ull << lane) - 1ull));
          const int sidx = sbase + __popcll(upto) - 1;
          sseg[x] = (uint16_t)sidx;
          if (h) ssegst[sidx] = (uint16_t)x;
        }
      }
      if (tid == 0) ssegst[nseg] = (uint16_t)nproc;

      // ---- prefetch the next batch while this one is computed
      {
        const int npos = pos + nproc;
        int nend = qend;
        if (npos >= qend) nend = min(s1, (int)a.chunk_base[min(q + 2, a.Q)]);
        const int nn = min(kECAP, nend - npos);
        pf_pos = npos;
        pf_n = nn > 0 ? nn : 0;
#pragma unroll
        for (int r = 0; r < kR; ++r) {
          const int x = r * kNT + tid;
          if (x < pf_n) { pk[r] = a.key[npos + x]; ps[r] = a.slew[npos + x]; }
        }
      }
#pragma unroll
      for (int u = 0; u < kGPT; ++u) {
        const uint32_t j = u * kNT + tid;
        if (j < g_span) {
          s_ginfo[j] = pgi[u];
          s_gcf[j] = pgc[u];
          s_gesw[j] = pge[u];
        }
      }
      __syncthreads();

      // ---- k-way merge of each segment's input-pin streams in time order
      //      (Sec. 2.4.2, Fig. 3): one thread per (chunk, gate) segment walks the
      //      distinct timestamps; every input event gets the state before it, the
      //      set of input pins switching at its timestamp, and whether it is the
      //      lowest of them (that one charges the leakage change).
      for (int sg = tid; sg < nseg; sg += kNT) {
        const int st = ssegst[sg], en = ssegst[sg + 1];
        const uint32_t kk = cell_k(s_ginfo[sgl[st] - g_lo] & 0xFFFFFFu);
        if (kk > (uint32_t)kSeqPins || en - st > kSeqMax) {
          s_flag = 1;
          continue;
        }
        int n0 = 0, n1 = 0, n2 = 0, n3 = 0;
        for (int m = st; m < en; ++m) {
          const uint32_t p = slk[m] >> tbits;
          n0 += p == 0u;
          n1 += p == 1u;
          n2 += p == 2u;
          n3 += p == 3u;
        }
        // pins at or above kk are the output pin: no state, not merged
        if (kk < 4u) n3 = 0;
        if (kk < 3u) n2 = 0;
        if (kk < 2u) n1 = 0;
        int c0 = st, c1 = st + n0, c2 = c1 + n1, c3 = c2 + n2;
        const int e0 = c1, e1 = c2, e2 = c3, e3 = c3 + n3;
        uint32_t S = saux[st] & 0xFFu;
        uint32_t h0 = c0 < e0 ? (slk[c0] & tmask) : kInf;
        uint32_t h1 = c1 < e1 ? (slk[c1] & tmask) : kInf;
        uint32_t h2 = c2 < e2 ? (slk[c2] & tmask) : kInf;
        uint32_t h3 = c3 < e3 ? (slk[c3] & tmask) : kInf;
        for (;;) {
          const uint32_t t = min(min(h0, h1), min(h2, h3));
          if (t == kInf) break;
          const uint32_t mask = (h0 == t ? 1u : 0u) | (h1 == t ? 2u : 0u) | (h2 == t ? 4u : 0u) | (h3 == t ? 8u : 0u);
          const uint32_t own = __ffs((int)mask) - 1;
          const uint32_t w = S | (mask << 8);
          if (h0 == t) { ssmo[c0] = w | ((own == 0u) << 16); ++c0; h0 = c0 < e0 ? (slk[c0] & tmask) : kInf; }
          if (h1 == t) { ssmo[c1] = w | ((own == 1u) << 16); ++c1; h1 = c1 < e1 ? (slk[c1] & tmask) : kInf; }
          if (h2 == t) { ssmo[c2] = w | ((own == 2u) << 16); ++c2; h2 = c2 < e2 ? (slk[c2] & tmask) : kInf; }
          if (h3 == t) { ssmo[c3] = w | ((own == 3u) << 16); ++c3; h3 = c3 < e3 ? (slk[c3] & tmask) : kInf; }
          S ^= mask;
        }
      }
      __syncthreads();

      // ---- long or wide segments: each other input pin's value just before t by
      //      binary search inside the segment (run only when a batch has one)
      if (s_flag) {
#pragma unroll
        for (int r = 0; r < kR; ++r) {
          const int x = r * kNT + tid;
          if (x >= nproc) continue;
          const uint32_t lk = slk[x];
          const uint32_t i = lk >> tbits;
          const uint32_t kk = cell_k(s_ginfo[sgl[x] - g_lo] & 0xFFFFFFu);
          const int sg = sseg[x];
          const int st = ssegst[sg], en = ssegst[sg + 1];
          if (i >= kk || (kk <= (uint32_t)kSeqPins && en - st <= kSeqMax)) continue;
          const uint32_t trel = lk & tmask;
          const uint32_t au = saux[x];
          uint32_t Sm = ((au & 0xFFu) & ~(1u << i)) | ((((au >> 8) & 1u) ^ 1u) << i);
          uint32_t mask = 1u << i;
          uint32_t owner = 1u;
          for (uint32_t j = 0; j < kk; ++j) {
            if (j == i) continue;
            const uint32_t target = (j << tbits) | trel;
            const int lo = j < i ? st : x + 1;
            const int hi = j < i ? x : en;
            const int p = lower_bound_u32(slk, lo, hi, target);
            if (p > st && (slk[p - 1] >> tbits) == j) Sm = (Sm & ~(1u << j)) | (((saux[p - 1] >> 8) & 1u) << j);
            if (p < en && slk[p] == target) {
              mask |= 1u << j;
              if (j < i) owner = 0u;
            }
          }
          ssmo[x] = Sm | (mask << 8) | (owner << 16);
        }
        __syncthreads();
      }

      // ---- one event per lane: energies, glitches, leakage changes, bins
      double L[kR][4];  // input event: 2x2 LUT corners; output event: L[r][0] = 0.5 c Vdd^2
      double fa[kR], fb[kR];
      uint32_t smo[kR];  // state before | mask << 8 | owner << 16 | input << 17
      uint32_t gi_r[kR];
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int x = r * kNT + tid;
        smo[r] = 0;
        gi_r[r] = 0;
        if (x >= nproc) continue;
        const uint32_t i = slk[x] >> tbits;
        const uint32_t gl = sgl[x] - g_lo;
        const uint32_t ginfo = s_ginfo[gl];
        gi_r[r] = ginfo;
        const uint32_t cell = ginfo & 0xFFFFFFu;
        const uint32_t kk = cell_k(cell);
        if (i >= kk) {  // output pin: no LUT, no state
          L[r][0] = s_gesw[gl];
          continue;
        }
        fb[r] = s_gcf[gl];
        const uint32_t so = ssmo[x];
        smo[r] = so | (1u << 17);
        const uint32_t Sm = so & 0xFFu;
        // slew segment on the cell's axis (Sec. 2.4.1, Fig. 2)
        const double sl = (double)sslew[x];
        int si = 0;
        for (int j = 1; j < ns - 1; ++j) si += (sl >= slew_ax(cell, j)) ? 1 : 0;
        fa[r] = (sl - slew_ax(cell, si)) * slew_iw(cell, si);
        const double *Lp = a.lut + lut_base(cell) + ((Sm * kk + i) * (uint32_t)ns + si) * (uint32_t)nc + (ginfo >> 24);
        L[r][0] = Lp[0];
        L[r][1] = Lp[1];
        L[r][2] = Lp[nc];
        L[r][3] = Lp[nc + 1];
      }
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int x = r * kNT + tid;
        if (x >= nproc) continue;
        const uint32_t lk = slk[x];
        const uint32_t i = lk >> tbits;
        const uint32_t trel = lk & tmask;
        const uint32_t cyc = scyc[x];
        const uint32_t val = (saux[x] >> 8) & 1u;
        const int sst = ssegst[sseg[x]];
        // glitch: previous event of the same pin inside the same cycle (Fig. 7)
        bool glitch = false;
        double r_gl = 0.0;
        if (x > sst && (slk[x - 1] >> tbits) == i && scyc[x - 1] == cyc) {
          glitch = true;
          const double pw = (double)(trel - (slk[x - 1] & tmask));
          const double rr = pw / (0.5 * ((double)sslew[x] + (double)sslew[x - 1]));  // Eq. 2 (reading)
          r_gl = rr > 1.0 ? 1.0 : rr;
        }
        const uint32_t so = smo[r];
        double E, extra = 0.0;
        if (so & (1u << 17)) {
          // bilinear internal energy
          const double v0 = L[r][0] + fb[r] * (L[r][1] - L[r][0]);
          const double v1 = L[r][2] + fb[r] * (L[r][3] - L[r][2]);
          E = v0 + fa[r] * (v1 - v0);
          if (so & (1u << 16)) {
            // leakage power change at this timestamp (owner = lowest switching input pin)
            const uint32_t Sm = so & 0xFFu, mask = (so >> 8) & 0xFFu;
            const uint32_t lb = leak_base(gi_r[r] & 0xFFFFFFu);
            const double dp = leak_of(lb + (Sm ^ mask)) - leak_of(lb + Sm);
            if (dp != 0.0) {
              const uint32_t bend = min((cyc + 1u) * a.T, clen32);
              extra = dp * (double)(bend - trel) * a.tick_s;
              atomicAdd(&bb[cyc], dp);
              e_lk += dp * (double)(tail_from_chunk - (int64_t)trel) * a.tick_s;
            }
          }
          if (!glitch) e_int += E;
        } else {
          // switching energy of a 0->1 output event (Eq. 1)
          E = val ? L[r][0] : 0.0;
          if (!glitch) e_sw += E;
        }
        double contrib = E;
        if (glitch) {
          contrib = r_gl * E;
          e_gl += contrib;
          ++n_gl;
        }
        contrib += extra;
        if (contrib != 0.0) atomicAdd(&bw[cyc], contrib);
        atomicAdd(&bc[cyc], 1ull | ((unsigned long long)glitch << 32));
        if constexpr (DIAG) {
          const uint32_t o = a.orig[pos + x];
          if (a.evt_glitch) a.evt_glitch[o] = glitch ? 1 : 0;
          if (a.evt_state) a.evt_state[o] = (uint8_t)(so & 0xFFu);
        }
      }
      pos += nproc;
      __syncthreads();
    }

    // ---- flush this chunk's bins: in-chunk prefix of leakage changes, then atomics
    {
      constexpr int PER = kCCMAX / kNT > 0 ? kCCMAX / kNT : 1;
      double loc[PER];
      double s = 0.0;
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int c = tid * PER + u;
        loc[u] = (c < ncyc) ? bb[c] : 0.0;
        s += loc[u];
      }
      // exclusive scan of per-thread sums across the block
      double incl = s;
      for (int o = 1; o < 64; o <<= 1) {
        const double v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
      }
      if (lane == 63) s_scan[wid] = incl;
      __syncthreads();
      double wbase = 0.0, total = 0.0;
      for (int w = 0; w < kNW; ++w) {
        const double v = s_scan[w];
        if (w < wid) wbase += v;
        total += v;
      }
      double run = wbase + incl - s;
      const int64_t cg0 = (int64_t)q * a.Cc;
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int c = tid * PER + u;
        if (c < ncyc) {
          const int64_t cg = cg0 + c;
          const double len = (cg == a.C - 1) ? (double)(a.t_max - cg * (int64_t)a.T) : (double)a.T;
          const double v = bw[c] + run * len * a.tick_s;
          if (v != 0.0) atomicAdd(&a.acc_wave[(size_t)xcd * a.C + cg], v);
          const unsigned long long cn = bc[c];
          if (cn) atomicAdd(&a.acc_cnt[(size_t)xcd * a.C + cg], cn);
          run += loc[u];
        }
      }
      if (tid == 0 && total != 0.0) atomicAdd(&a.dP[q], total);
      __syncthreads();
      for (int c = tid; c < kCCMAX; c += kNT) {
        bw[c] = 0.0;
        bb[c] = 0.0;
        bc[c] = 0ull;
      }
      __syncthreads();
    }
    ++q;
  }

  // ---- block totals
  {
    double v[5] = {e_int, e_sw, e_gl, e_lk, l0};
#pragma unroll
    for (int u = 0; u < 5; ++u) v[u] = wave_sum(v[u]);
    unsigned long long ng = n_gl;
    for (int o = 32; o > 0; o >>= 1) ng += __shfl_xor(ng, o, 64);
    if (lane == 0) {
#pragma unroll
      for (int u = 0; u < 5; ++u) s_red[wid * 6 + u] = v[u];
      s_red[wid * 6 + 5] = (double)ng;
    }
    __syncthreads();
    if (tid < 6) {
      double t = 0.0;
      for (int w = 0; w < kNW; ++w) t += s_red[w * 6 + tid];
      if (tid < 5) {
        if (t != 0.0) atomicAdd(&a.tot[tid], t);
      } else {
        if (t != 0.0) atomicAdd(&a.tot_cnt[0], (unsigned long long)t);
      }
    }
  }
}

constexpr int kFT = 256;

__global__ __launch_bounds__(kFT) void k_finalize(FinalArgs f) {
  __shared__ double s_base[kFT / 64];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * kFT;
  const int qa = (int)(c0 / f.Cc);
  // leakage power at the start of chunk qa: L0 + sum of earlier chunks' changes
  double part = 0.0;
  for (int j = tid; j < qa; j += kFT) part += f.dP[j];
  part = wave_sum(part);
  if (lane == 0) s_base[wid] = part;
  __syncthreads();
  double base = f.tot[4];
  for (int w = 0; w < kFT / 64; ++w) base += s_base[w];
  const int64_t c = c0 + tid;
  if (c < f.C) {
    const int qc = (int)(c / f.Cc);
    double P = base;
    for (int j = qa; j < qc; ++j) P += f.dP[j];
    const double len = (c == f.C - 1) ? (double)(f.t_max - c * (int64_t)f.T) : (double)f.T;
    double w = P * len * f.tick_s;
    unsigned long long cnt = 0;
#pragma unroll
    for (int x = 0; x < kXCD; ++x) {
      w += f.acc_wave[(size_t)x * f.C + c];
      cnt += f.acc_cnt[(size_t)x * f.C + c];
      f.acc_wave[(size_t)x * f.C + c] = 0.0;
      f.acc_cnt[(size_t)x * f.C + c] = 0ull;
    }
    f.wave_out[c] = w;
    f.cyc_events[c] = cnt & 0xFFFFFFFFull;
    f.cyc_glitches[c] = cnt >> 32;
  }
  if (blockIdx.x == 0) {
    for (int j = tid; j < f.Q_next; j += kFT) f.dP_next[j] = 0.0;
    if (tid < 8) f.tot_next[tid] = 0.0;
    if (tid < 2) f.tot_cnt_next[tid] = 0ull;
    if (tid == 0) {
      const double window = (double)f.t_max * f.tick_s;
      const double e_leak = f.tot[4] * window + f.tot[3];
      f.res[0] = f.tot[0];
      f.res[1] = f.tot[1];
      f.res[2] = f.tot[2];
      f.res[3] = e_leak;
      f.res[4] = f.tot[0] / window;  // Eq. 3
      f.res[5] = f.tot[1] / window;
      f.res[6] = f.tot[2] / window;
      f.res[7] = e_leak / window;
      f.res[8] = (double)f.tot_cnt[0];
    }
  }
}

}  // namespace

int pass_block_threads() { return kNT; }
int pass_batch_events() { return kECAP; }
int pass_max_chunk_cycles() { return kCCMAX; }

bool pass_cells_fit_lds(int n_cells, int n_slew, int64_t n_leak) {
  return n_cells <= kMaxCellsLds && (int64_t)n_cells * (2 * n_slew - 1) + n_leak <= kCellDoubles;
}

hipError_t launch_pass(const PassArgs &a, int grid_blocks, hipStream_t s) {
  const bool cells = pass_cells_fit_lds(a.n_cells, a.n_slew, a.n_leak);
  const bool diag = a.evt_glitch || a.evt_state;
  if (cells && !diag)
    hipLaunchKernelGGL((k_fused<true, false>), dim3(grid_blocks), dim3(kNT), 0, s, a);
  else if (cells)
    hipLaunchKernelGGL((k_fused<true, true>), dim3(grid_blocks), dim3(kNT), 0, s, a);
  else if (!diag)
    hipLaunchKernelGGL((k_fused<false, false>), dim3(grid_blocks), dim3(kNT), 0, s, a);
  else
    hipLaunchKernelGGL((k_fused<false, true>), dim3(grid_blocks), dim3(kNT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_finalize(const FinalArgs &f, hipStream_t s) {
  const int grid = (int)((f.C + kFT - 1) / kFT);
  hipLaunchKernelGGL(k_finalize, dim3(grid), dim3(kFT), 0, s, f);
  return hipGetLastError();
}

}  // namespace pa
