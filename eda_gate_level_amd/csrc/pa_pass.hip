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
// (Fig. 7).  This pass keeps the fusion and maps it onto 64-lane waves:
//   * events are laid out chunk-major (time chunks of Cc cycles); inside a
//     chunk, gate-major segments of one gate and one time window (a power-
//     of-two part of the chunk picked per gate from its event density when
//     the events are loaded, so that no segment holds more than 128 events:
//     the event-density-aware per-gate partitioning of the paper), each
//     segment pin-major and time-sorted per pin.  Every 64-bit key carries
//     gate, segment-head bit, pin code, time in the chunk, value and the
//     gate's input state at the segment start, so a segment is
//     self-contained;
//   * a block owns a range of whole segments inside one chunk; each of its
//     waves streams a share of them in batches of 128 events (two per lane)
//     with coalesced nontemporal key/slew loads, the next batch prefetched
//     into registers, and no block barrier inside the loop;
//   * per batch one lane per segment walks its input-pin streams in time
//     order (the k-way merge of Sec. 2.4.2, Fig. 3), giving every input
//     event the state before it, the set of input pins switching at its
//     timestamp and whether it is the lowest of them;
//   * then one lane per event: state-selected LUT, bilinear on slew and load
//     (Sec. 2.4.1, Fig. 2), switching energy (Eq. 1), glitch test against the
//     previous event of the same pin (Fig. 7, Eq. 2), energies added to
//     per-cycle bins in LDS;
//   * leakage is charged as power changes: at every distinct input timestamp
//     the lowest switching input pin adds dP = leak[S+] - leak[S-]; its
//     partial bin gets dP * (bin end - t) and all later bins get dP * their
//     length through an in-LDS prefix sum per chunk and a per-chunk carry;
//     the leakage at t = 0 is the sum over gates of leak[S0].  This is the
//     paper's per-interval, per-overlapped-bin split (Sec. 2.4.2, Eq. 4)
//     summed in another order;
//   * the bins are flushed once per block with fp64/u64 atomics into one of 8
//     copies (one per XCD), which the finalize kernel adds up.
#include <hip/hip_runtime.h>

#include "pa_common.h"

namespace pa {

namespace {

#ifndef PA_NT
#define PA_NT 512
#endif
#ifndef PA_CCMAX
#define PA_CCMAX 512
#endif
constexpr int kNT = PA_NT;         // threads per block
constexpr int kNW = kNT / 64;      // waves per block, each working on its own batches
constexpr int kRW = kSegMax / 64;  // events per lane per wave batch
constexpr int kWB = 64 * kRW;      // events per wave batch (= the longest segment)
constexpr int kCCMAX = PA_CCMAX;   // max cycles per chunk (LDS bins)
constexpr int kXCD = 8;
constexpr int kMaxCellsLds = 256;
constexpr int kCellBytesMax = 24 * 1024;
constexpr uint32_t kInf = 0xFFFFFFFFu;
static_assert(kWB == kSegMax, "a wave batch holds the longest segment");

__device__ __forceinline__ uint32_t key_gate(uint64_t k) { return uint32_t(k >> kKeyGateShift); }
__device__ __forceinline__ uint32_t key_head(uint64_t k) { return uint32_t(k >> kKeyHeadShift) & 1u; }
__device__ __forceinline__ uint32_t key_lk(uint64_t k) { return uint32_t(k >> kKeyLkShift); }

// first segment head at or after position x (E if none); one whole wave
__device__ int find_head(const uint64_t *key, int64_t E, int64_t x) {
  const int lane = threadIdx.x & 63;
  for (;;) {
    if (x >= E) return (int)E;
    const int64_t y = x + lane;
    const bool h = (y >= E) || key_head(key[y]);
    const unsigned long long m = __ballot(h);
    if (m) return (int)(x + __ffsll((long long)m) - 1);
    x += 64;
  }
}

__device__ __forceinline__ double wave_sum(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// LDS ordering between the lanes of one wave (no block barrier)
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// bytes of the cell tables staged in dynamic LDS
__host__ __device__ inline int64_t cell_lds_bytes(int n_cells, int n_slew, int64_t n_leak) {
  return 8 * ((int64_t)n_cells * (2 * n_slew - 1) + n_leak) + 8 * (int64_t)n_cells;
}

template <bool CELL_LDS, bool DIAG>
__global__ __launch_bounds__(kNT) void k_fused(PassArgs a) {
  extern __shared__ double s_dyn[];  // cell tables: slew axes | inverse widths | leakage | meta | LUT bases
  // per-wave batch staging
  __shared__ uint32_t w_lk[kNW][kWB];   // (pin code << t_bits) | t_rel
  __shared__ uint32_t w_g[kNW][kWB];    // gate id
  __shared__ uint32_t w_smo[kNW][kWB];  // state before | switching-pin mask << 8 | owner << 16
  __shared__ float w_slew[kNW][kWB];
  __shared__ uint16_t w_aux[kNW][kWB];  // S0 | val << 8
  __shared__ uint16_t w_cyc[kNW][kWB];  // cycle inside the chunk
  __shared__ uint16_t w_segst[kNW][kWB + 2];
  __shared__ uint8_t w_seg[kNW][kWB];
  // per-cycle bins of the block's chunk
  __shared__ double bw[kCCMAX];               // energy: dynamic + partial-bin leakage
  __shared__ double bb[kCCMAX];               // leakage power change
  __shared__ unsigned long long bc[kCCMAX];   // events | glitches << 32
  __shared__ int s_bounds[kNW + 1];
  __shared__ double s_red[kNW * 6];
  __shared__ double s_scan[kNW];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const uint32_t tbits = a.kf.t_bits;
  const uint32_t tmask = (1u << tbits) - 1u;
  const uint32_t outc = out_code(a.kf.p_bits);
  const int nb = gridDim.x, b = blockIdx.x;
  const int xcd = b % kXCD;
  const int ns = a.n_slew, nc = a.n_cap;
  const bool has_range = b < a.n_ranges;

  // cell tables in dynamic LDS
  double *c_sa = s_dyn;
  double *c_iw = c_sa + a.n_cells * ns;
  double *c_lk = c_iw + a.n_cells * (ns - 1);
  uint32_t *c_meta = reinterpret_cast<uint32_t *>(c_lk + a.n_leak);  // k | leak base << 4
  uint32_t *c_lutb = c_meta + a.n_cells;
  auto cell_k = [&](uint32_t c) -> uint32_t {
    if constexpr (CELL_LDS) return c_meta[c] & 15u; else return (uint32_t)a.cell_k[c];
  };
  auto leak_base = [&](uint32_t c) -> uint32_t {
    if constexpr (CELL_LDS) return c_meta[c] >> 4; else return a.cell_leak_base[c];
  };
  auto lut_base = [&](uint32_t c) -> uint32_t {
    if constexpr (CELL_LDS) return c_lutb[c]; else return a.cell_lut_base[c];
  };
  auto slew_ax = [&](uint32_t c, int j) -> double {
    if constexpr (CELL_LDS) return c_sa[c * ns + j]; else return a.slew_axis[(size_t)c * ns + j];
  };
  auto slew_iw = [&](uint32_t c, int j) -> double {
    if constexpr (CELL_LDS) return c_iw[c * (ns - 1) + j]; else return a.slew_invw[(size_t)c * (ns - 1) + j];
  };
  auto leak_of = [&](uint32_t j) -> double {
    if constexpr (CELL_LDS) return c_lk[j]; else return a.leak[j];
  };

  // ---- the block's range (inside one chunk) and its waves' sub-ranges, all cut at segment heads
  int q = 0;
  if (has_range) {
    q = (int)a.rchunk[b];
    const int64_t r0 = a.rstart[b], r1 = a.rstart[b + 1];
    for (int w = wid; w <= kNW; w += kNW) {
      const int h = find_head(a.key, a.E, r0 + (r1 - r0) * w / kNW);
      if (lane == 0) s_bounds[w] = h;
    }
  } else if (tid == 0) {
    s_bounds[0] = 0;
  }
  for (int c = tid; c < kCCMAX; c += kNT) {
    bw[c] = 0.0;
    bb[c] = 0.0;
    bc[c] = 0ull;
  }
  if constexpr (CELL_LDS) {
    for (int c = tid; c < a.n_cells; c += kNT) {
      c_meta[c] = (uint32_t)a.cell_k[c] | (a.cell_leak_base[c] << 4);
      c_lutb[c] = a.cell_lut_base[c];
    }
    for (int j = tid; j < a.n_cells * ns; j += kNT) c_sa[j] = a.slew_axis[j];
    for (int j = tid; j < a.n_cells * (ns - 1); j += kNT) c_iw[j] = a.slew_invw[j];
    for (int j = tid; j < a.n_leak; j += kNT) c_lk[j] = a.leak[j];
  }
  __syncthreads();

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

  const int64_t cstart = (int64_t)q * a.chunk_ticks;
  const int64_t clen = min(a.chunk_ticks, a.t_max - cstart);
  const uint32_t clen32 = (uint32_t)clen;
  const int ncyc = (int)((clen + a.T - 1) / a.T);
  const int64_t tail_from_chunk = a.t_max - cstart;  // t_max - t = tail_from_chunk - t_rel

  if (has_range) {
    uint32_t *lk_w = w_lk[wid];
    uint32_t *g_w = w_g[wid];
    uint32_t *smo_w = w_smo[wid];
    float *sl_w = w_slew[wid];
    uint16_t *aux_w = w_aux[wid];
    uint16_t *cyc_w = w_cyc[wid];
    uint16_t *segst_w = w_segst[wid];
    uint8_t *seg_w = w_seg[wid];
    const int wb = s_bounds[wid + 1];
    int pos = s_bounds[wid];
    uint64_t pk[kRW];
    float ps[kRW];
    {
      const int n0 = min(kWB, wb - pos);
#pragma unroll
      for (int r = 0; r < kRW; ++r) {
        const int x = r * 64 + lane;
        if (x < n0) {
          pk[r] = __builtin_nontemporal_load(a.key + pos + x);
          ps[r] = __builtin_nontemporal_load(a.slew + pos + x);
        }
      }
    }
    while (pos < wb) {
      const int n = min(kWB, wb - pos);
      // ---- segments of the batch: head bits, the last (maybe incomplete) one deferred
      unsigned long long hm[kRW];
      int last = -1;
#pragma unroll
      for (int r = 0; r < kRW; ++r) {
        const int x = r * 64 + lane;
        hm[r] = __ballot(x < n && key_head(pk[r]));
        if (hm[r]) last = r * 64 + 63 - __clzll((long long)hm[r]);
      }
      const int nproc = (pos + n < wb && last > 0) ? last : n;
      int nseg = 0;
      int sidx[kRW];
#pragma unroll
      for (int r = 0; r < kRW; ++r) {
        const int lim = nproc - r * 64;  // lanes below lim are in [0, nproc)
        const unsigned long long valid = lim >= 64 ? ~0ull : (lim <= 0 ? 0ull : ((1ull << lim) - 1ull));
        const unsigned long long upto = (lane == 63) ? hm[r] : (hm[r] & ((2ull << lane) - 1ull));
        sidx[r] = nseg + __popcll(upto) - 1;
        nseg += __popcll(hm[r] & valid);
      }
      // ---- decode into the wave's LDS region; issue the gate-data loads
      uint32_t gi[kRW];
      double gcf[kRW], gesw[kRW];
#pragma unroll
      for (int r = 0; r < kRW; ++r) {
        const int x = r * 64 + lane;
        gi[r] = 0;
        if (x < nproc) {
          const uint64_t k = pk[r];
          const uint32_t lk = key_lk(k);
          const uint32_t g = key_gate(k);
          lk_w[x] = lk;
          g_w[x] = g;
          aux_w[x] = (uint16_t)(uint32_t(k) & 0x1FFu);  // S0 | val << 8
          cyc_w[x] = (uint16_t)divu32(lk & tmask, a.divT);
          sl_w[x] = ps[r];
          seg_w[x] = (uint8_t)sidx[r];
          if ((hm[r] >> lane) & 1ull) segst_w[sidx[r]] = (uint16_t)x;
          gi[r] = a.gate_info[g];
          gcf[r] = a.gate_capfrac[g];
          gesw[r] = a.gate_esw[g];
        }
      }
      if (lane == 0) segst_w[nseg] = (uint16_t)nproc;
      // ---- prefetch the next batch
      const int npos = pos + nproc;
      {
        const int nn = min(kWB, wb - npos);
#pragma unroll
        for (int r = 0; r < kRW; ++r) {
          const int x = r * 64 + lane;
          if (x < nn) {
            pk[r] = __builtin_nontemporal_load(a.key + npos + x);
            ps[r] = __builtin_nontemporal_load(a.slew + npos + x);
          }
        }
      }
      wave_sync();

      // ---- k-way merge of each segment's input-pin streams in time order
      //      (Sec. 2.4.2, Fig. 3): one lane per segment walks the distinct
      //      timestamps; every input event gets the state before it, the set of
      //      input pins switching at its timestamp, and whether it is the lowest
      //      of them (that one charges the leakage change).
      for (int sg = lane; sg < nseg; sg += 64) {
        const int st = segst_w[sg], en = segst_w[sg + 1];
        int n0 = 0, n1 = 0, n2 = 0, n3 = 0, nhi = 0;
        for (int m = st; m < en; ++m) {
          const uint32_t p = lk_w[m] >> tbits;
          // the output pin's code is not an input pin (it may equal 1 or 3)
          n0 += p == 0u;
          n1 += (p == 1u && p != outc);
          n2 += p == 2u;
          n3 += (p == 3u && p != outc);
          nhi += (p >= 4u && p != outc);
        }
        const uint32_t S0 = aux_w[st] & 0xFFu;
        if (nhi == 0) {
          int c0 = st, c1 = st + n0, c2 = c1 + n1, c3 = c2 + n2;
          const int e0 = c1, e1 = c2, e2 = c3, e3 = c3 + n3;
          uint32_t S = S0;
          uint32_t h0 = c0 < e0 ? (lk_w[c0] & tmask) : kInf;
          uint32_t h1 = c1 < e1 ? (lk_w[c1] & tmask) : kInf;
          uint32_t h2 = c2 < e2 ? (lk_w[c2] & tmask) : kInf;
          uint32_t h3 = c3 < e3 ? (lk_w[c3] & tmask) : kInf;
          for (;;) {
            const uint32_t t = min(min(h0, h1), min(h2, h3));
            if (t == kInf) break;
            const uint32_t mask = (h0 == t ? 1u : 0u) | (h1 == t ? 2u : 0u) | (h2 == t ? 4u : 0u) | (h3 == t ? 8u : 0u);
            const uint32_t own = __ffs((int)mask) - 1;
            const uint32_t wv = S | (mask << 8);
            if (h0 == t) { smo_w[c0] = wv | ((own == 0u) << 16); ++c0; h0 = c0 < e0 ? (lk_w[c0] & tmask) : kInf; }
            if (h1 == t) { smo_w[c1] = wv | ((own == 1u) << 16); ++c1; h1 = c1 < e1 ? (lk_w[c1] & tmask) : kInf; }
            if (h2 == t) { smo_w[c2] = wv | ((own == 2u) << 16); ++c2; h2 = c2 < e2 ? (lk_w[c2] & tmask) : kInf; }
            if (h3 == t) { smo_w[c3] = wv | ((own == 3u) << 16); ++c3; h3 = c3 < e3 ? (lk_w[c3] & tmask) : kInf; }
            S ^= mask;
          }
        } else {
          // gates with more than four inputs: every input event scans its segment
          for (int x = st; x < en; ++x) {
            const uint32_t lx = lk_w[x];
            const uint32_t ix = lx >> tbits;
            if (ix == outc) continue;
            const uint32_t tx = lx & tmask;
            uint32_t Sm = (S0 & ~(1u << ix)) | ((((aux_w[x] >> 8) & 1u) ^ 1u) << ix);
            uint32_t mask = 1u << ix, owner = 1u;
            for (int m = st; m < en; ++m) {
              const uint32_t lm = lk_w[m];
              const uint32_t im = lm >> tbits;
              if (im == outc || im == ix) continue;
              const uint32_t tm = lm & tmask;
              if (tm < tx) Sm = (Sm & ~(1u << im)) | (((aux_w[m] >> 8) & 1u) << im);
              else if (tm == tx) {
                mask |= 1u << im;
                if (im < ix) owner = 0u;
              }
            }
            smo_w[x] = Sm | (mask << 8) | (owner << 16);
          }
        }
      }
      wave_sync();

      // ---- one event per lane: energies, glitches, leakage changes, bins
      double L[kRW][4];  // input event: 2x2 LUT corners; output event: L[r][0] = 0.5 c Vdd^2
      double fa[kRW];
      uint32_t smo[kRW];  // state before | mask << 8 | owner << 16 | input << 17
#pragma unroll
      for (int r = 0; r < kRW; ++r) {
        const int x = r * 64 + lane;
        smo[r] = 0;
        if (x >= nproc) continue;
        const uint32_t code = lk_w[x] >> tbits;
        if (code == outc) {  // output pin: no LUT, no state
          L[r][0] = gesw[r];
          continue;
        }
        const uint32_t cell = gi[r] & 0xFFFFFFu;
        const uint32_t kk = cell_k(cell);
        const uint32_t so = smo_w[x];
        smo[r] = so | (1u << 17);
        const uint32_t Sm = so & ((1u << kk) - 1u);  // no-op for valid states; keeps the LUT row inside the cell
        // slew segment on the cell's axis (Sec. 2.4.1, Fig. 2)
        const double sl = (double)sl_w[x];
        int si = 0;
        for (int j = 1; j < ns - 1; ++j) si += (sl >= slew_ax(cell, j)) ? 1 : 0;
        fa[r] = (sl - slew_ax(cell, si)) * slew_iw(cell, si);
        const double *Lp = a.lut + lut_base(cell) + ((Sm * kk + code) * (uint32_t)ns + si) * (uint32_t)nc + (gi[r] >> 24);
        L[r][0] = Lp[0];
        L[r][1] = Lp[1];
        L[r][2] = Lp[nc];
        L[r][3] = Lp[nc + 1];
      }
#pragma unroll
      for (int r = 0; r < kRW; ++r) {
        const int x = r * 64 + lane;
        if (x >= nproc) continue;
        const uint32_t lk = lk_w[x];
        const uint32_t code = lk >> tbits;
        const uint32_t trel = lk & tmask;
        const uint32_t cyc = cyc_w[x];
        const uint32_t val = (aux_w[x] >> 8) & 1u;
        const int sst = segst_w[seg_w[x]];
        // glitch: previous event of the same pin inside the same cycle (Fig. 7)
        bool glitch = false;
        double r_gl = 0.0;
        if (x > sst && (lk_w[x - 1] >> tbits) == code && cyc_w[x - 1] == cyc) {
          glitch = true;
          const double pw = (double)(trel - (lk_w[x - 1] & tmask));
          const double rr = pw / (0.5 * ((double)sl_w[x] + (double)sl_w[x - 1]));  // Eq. 2 (reading)
          r_gl = rr > 1.0 ? 1.0 : rr;
        }
        const uint32_t so = smo[r];
        double E, extra = 0.0;
        if (so & (1u << 17)) {
          // bilinear internal energy
          const double v0 = L[r][0] + gcf[r] * (L[r][1] - L[r][0]);
          const double v1 = L[r][2] + gcf[r] * (L[r][3] - L[r][2]);
          E = v0 + fa[r] * (v1 - v0);
          if (so & (1u << 16)) {
            // leakage power change at this timestamp (owner = lowest switching input pin)
            const uint32_t Sm = so & 0xFFu, mask = (so >> 8) & 0xFFu;
            const uint32_t lb = leak_base(gi[r] & 0xFFFFFFu);
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
      wave_sync();
      pos = npos;
    }
  }
  __syncthreads();

  // ---- flush the chunk's bins: in-chunk prefix of leakage changes, then atomics
  if (has_range) {
    constexpr int PER = kCCMAX / kNT > 0 ? kCCMAX / kNT : 1;
    double loc[PER];
    double s = 0.0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid * PER + u;
      loc[u] = (c < ncyc) ? bb[c] : 0.0;
      s += loc[u];
    }
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
int pass_batch_events() { return kWB; }
int pass_wave_batch() { return kWB; }
int pass_max_chunk_cycles() { return kCCMAX; }

bool pass_cells_fit_lds(int n_cells, int n_slew, int64_t n_leak) {
  return n_cells <= kMaxCellsLds && cell_lds_bytes(n_cells, n_slew, n_leak) <= kCellBytesMax;
}

hipError_t launch_pass(const PassArgs &a, int grid_blocks, hipStream_t s) {
  const bool cells = pass_cells_fit_lds(a.n_cells, a.n_slew, a.n_leak);
  const bool diag = a.evt_glitch || a.evt_state;
  const size_t dyn = cells ? (size_t)cell_lds_bytes(a.n_cells, a.n_slew, a.n_leak) : 0;
  if (cells && !diag)
    hipLaunchKernelGGL((k_fused<true, false>), dim3(grid_blocks), dim3(kNT), dyn, s, a);
  else if (cells)
    hipLaunchKernelGGL((k_fused<true, true>), dim3(grid_blocks), dim3(kNT), dyn, s, a);
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
