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

constexpr int kNT = 1024;     // threads per block
constexpr int kR = 4;         // events per thread per batch
constexpr int kECAP = kNT * kR;
constexpr int kCCMAX = 1024;  // max cycles per chunk (LDS bins)
constexpr int kNW = kNT / 64;
constexpr int kXCD = 8;

struct Keys {
  uint32_t g_sh, p_sh, t_sh, v_sh;
  uint32_t p_mask, s_mask;
  uint64_t t_mask;
};

__device__ __forceinline__ uint32_t key_gate(uint64_t k, const Keys &K) { return uint32_t(k >> K.g_sh); }
__device__ __forceinline__ uint32_t key_pin(uint64_t k, const Keys &K) { return uint32_t(k >> K.p_sh) & K.p_mask; }
__device__ __forceinline__ uint32_t key_trel(uint64_t k, const Keys &K) { return uint32_t((k >> K.t_sh) & K.t_mask); }
__device__ __forceinline__ uint32_t key_val(uint64_t k, const Keys &K) { return uint32_t(k >> K.v_sh) & 1u; }

// first position in [lo, hi) whose key is >= target (hi if none)
__device__ __forceinline__ int lower_bound_lds(const uint64_t *s, int lo, int hi, uint64_t target) {
  int n = hi - lo;
  while (n > 0) {
    int half = n >> 1;
    int mid = lo + half;
    bool lt = s[mid] < target;
    lo = lt ? mid + 1 : lo;
    n = lt ? n - half - 1 : half;
  }
  return lo;
}

// first segment head at or after position x (a head starts a (chunk, gate)
// segment); executed by one whole wave
__device__ int find_head(const PassArgs &a, const Keys &K, int64_t x) {
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
      h = key_gate(a.key[y], K) != key_gate(a.key[y - 1], K);
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

__global__ __launch_bounds__(kNT) void k_fused(PassArgs a) {
  __shared__ uint64_t skey[kECAP];
  __shared__ float sslew[kECAP];
  __shared__ uint16_t send[kECAP];
  __shared__ double bw[kCCMAX];               // per-cycle energy (dynamic + partial leakage)
  __shared__ double bb[kCCMAX];               // per-cycle leakage power change
  __shared__ unsigned long long bc[kCCMAX];   // events | glitches << 32
  __shared__ int sws[2][kNW];
  __shared__ int s_range[2];
  __shared__ double s_red[kNW * 6];
  __shared__ double s_scan[kNW];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const Keys K{a.kf.g_sh, a.kf.p_sh, a.kf.t_sh, a.kf.v_sh, a.kf.p_mask, (1u << a.kf.s_bits) - 1u, a.kf.t_mask};
  const int nb = gridDim.x, b = blockIdx.x;
  const int xcd = b % kXCD;
  const uint64_t gate_field_mask = ~((uint64_t(1) << K.g_sh) - 1);

  // ---- this block's range of whole segments
  if (wid < 2) {
    int64_t nominal = (a.E * (int64_t)(b + wid)) / nb;
    int h = find_head(a, K, nominal);
    if (lane == 0) s_range[wid] = h;
  }
  for (int c = tid; c < kCCMAX; c += kNT) {
    bw[c] = 0.0;
    bb[c] = 0.0;
    bc[c] = 0ull;
  }
  __syncthreads();
  const int s0 = s_range[0], s1 = s_range[1];

  double e_int = 0.0, e_sw = 0.0, e_gl = 0.0, e_lk = 0.0, l0 = 0.0;
  unsigned n_gl = 0;

  // ---- leakage at t = 0: sum over gates of leak[S0] (Sec. 2.4.2, Fig. 3)
  for (int64_t g = (int64_t)b * kNT + tid; g < a.G; g += (int64_t)nb * kNT) {
    const uint32_t cell = a.gate_info[g] & 0xFFFFFFu;
    const int kk = a.cell_k[cell];
    const int64_t p0 = a.pin_base[g];
    uint32_t S = 0;
    for (int j = 0; j < kk; ++j) S |= uint32_t(a.pin_init[p0 + j]) << j;
    l0 += a.leak[a.cell_leak_base[cell] + S];
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
  // prefetch registers
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
      // ---- stage the batch: from the prefetch registers or directly
      if (pf_pos == pos && pf_n >= n) {
#pragma unroll
        for (int r = 0; r < kR; ++r) {
          const int x = r * kNT + tid;
          if (x < n) { skey[x] = pk[r]; sslew[x] = ps[r]; }
        }
      } else {
#pragma unroll
        for (int r = 0; r < kR; ++r) {
          const int x = r * kNT + tid;
          if (x < n) { pk[r] = a.key[pos + x]; ps[r] = a.slew[pos + x]; }
        }
#pragma unroll
        for (int r = 0; r < kR; ++r) {
          const int x = r * kNT + tid;
          if (x < n) { skey[x] = pk[r]; sslew[x] = ps[r]; }
        }
      }
      __syncthreads();

      // ---- segment starts: running max of head positions (round-major scan)
      int ss[kR];
      int carry = -1;
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int x = r * kNT + tid;
        bool h = false;
        if (x < n) h = (x == 0) || (key_gate(skey[x], K) != key_gate(skey[x - 1], K));
        const unsigned long long m = __ballot(h);
        const unsigned long long below = (lane == 63) ? m : (m & ((2ull << lane) - 1ull));
        const int lstart = below ? 63 - __clzll((long long)below) : -1;
        if (lane == 0) sws[r & 1][wid] = m ? (r * kNT + wid * 64 + 63 - __clzll((long long)m)) : -1;
        __syncthreads();
        int cin = carry, rmax = carry;
#pragma unroll
        for (int w = 0; w < kNW; ++w) {
          const int v = sws[r & 1][w];
          if (w < wid) cin = max(cin, v);
          rmax = max(rmax, v);
        }
        ss[r] = lstart >= 0 ? r * kNT + wid * 64 + lstart : cin;
        carry = rmax;
      }
      const int last_head = carry;
      const int nproc = (pos + n < qend && last_head > 0) ? last_head : n;

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

      // ---- segment ends
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int x = r * kNT + tid;
        if (x < nproc) {
          const bool tail = (x + 1 == nproc) || (key_gate(skey[x + 1], K) != key_gate(skey[x], K));
          if (tail) send[ss[r]] = (uint16_t)(x + 1 - ss[r]);
        }
      }
      __syncthreads();

      // ---- one event per lane
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int x = r * kNT + tid;
        if (x >= nproc) continue;
        const int sst = ss[r];
        const int sen = sst + send[sst];
        const uint64_t k = skey[x];
        const uint32_t g = key_gate(k, K);
        const uint32_t i = key_pin(k, K);
        const uint32_t trel = key_trel(k, K);
        const uint32_t val = key_val(k, K);
        const uint32_t S0 = uint32_t(k) & K.s_mask;
        const uint32_t ginfo = a.gate_info[g];
        const uint32_t cell = ginfo & 0xFFFFFFu;
        const uint32_t kk = (uint32_t)a.cell_k[cell];
        const uint32_t cyc = divu32(trel, a.divT);
        const double sl = (double)sslew[x];

        // glitch: previous event of the same pin inside the same cycle (Fig. 7)
        bool glitch = false;
        double r_gl = 0.0;
        if (x > sst) {
          const uint64_t kp = skey[x - 1];
          if (key_pin(kp, K) == i) {
            const uint32_t tp = key_trel(kp, K);
            if (divu32(tp, a.divT) == cyc) {
              glitch = true;
              const double pw = (double)(trel - tp);
              const double rr = pw / (0.5 * (sl + (double)sslew[x - 1]));  // Eq. 2 (reading)
              r_gl = rr > 1.0 ? 1.0 : rr;
            }
          }
        }

        double E, extra = 0.0;
        uint32_t Sm = 0;
        if (i < kk) {
          // state before t: each other input pin's value just before t
          uint32_t mask = 1u << i;
          bool owner = true;
          Sm = (val ^ 1u) << i;
          const uint64_t base_t = (k & gate_field_mask) | (uint64_t(trel) << K.t_sh);
          for (uint32_t j = 0; j < kk; ++j) {
            if (j == i) continue;
            const uint64_t target = base_t | (uint64_t(j) << K.p_sh);
            const int lo = j < i ? sst : x + 1;
            const int hi = j < i ? x : sen;
            const int p = lower_bound_lds(skey, lo, hi, target);
            uint32_t vj = (S0 >> j) & 1u;
            if (p > sst) {
              const uint64_t kb = skey[p - 1];
              if (key_pin(kb, K) == j) vj = key_val(kb, K);
            }
            if (p < sen) {
              const uint64_t kn = skey[p];
              if ((kn >> K.t_sh) == (target >> K.t_sh)) {
                mask |= 1u << j;
                if (j < i) owner = false;
              }
            }
            Sm |= vj << j;
          }
          // internal energy: state-selected LUT, bilinear (Sec. 2.4.1, Fig. 2)
          const int ns = a.n_slew, nc = a.n_cap;
          const double *sa = a.slew_axis + (size_t)cell * ns;
          int si = 0;
          for (int j = 1; j < ns - 1; ++j) si += (sl >= sa[j]) ? 1 : 0;
          const double fa = (sl - sa[si]) * a.slew_invw[(size_t)cell * (ns - 1) + si];
          const uint32_t cseg = ginfo >> 24;
          const double fb = a.gate_capfrac[g];
          const double *L = a.lut + a.cell_lut_base[cell] + ((size_t)(Sm * kk + i) * ns + si) * nc + cseg;
          const double l00 = L[0], l01 = L[1], l10 = L[nc], l11 = L[nc + 1];
          const double v0 = l00 + fb * (l01 - l00);
          const double v1 = l10 + fb * (l11 - l10);
          E = v0 + fa * (v1 - v0);
          // leakage power change at this timestamp (owner = lowest switching input pin)
          if (owner) {
            const uint32_t lb = a.cell_leak_base[cell];
            const double dp = a.leak[lb + (Sm ^ mask)] - a.leak[lb + Sm];
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
          E = val ? a.gate_esw[g] : 0.0;
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
        if (a.evt_glitch || a.evt_state) {
          const uint32_t o = a.orig[pos + x];
          if (a.evt_glitch) a.evt_glitch[o] = glitch ? 1 : 0;
          if (a.evt_state) a.evt_state[o] = (uint8_t)Sm;
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

hipError_t launch_pass(const PassArgs &a, int grid_blocks, hipStream_t s) {
  hipLaunchKernelGGL(k_fused, dim3(grid_blocks), dim3(kNT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_finalize(const FinalArgs &f, hipStream_t s) {
  const int grid = (int)((f.C + kFT - 1) / kFT);
  hipLaunchKernelGGL(k_finalize, dim3(grid), dim3(kFT), 0, s, f);
  return hipGetLastError();
}

}  // namespace pa
