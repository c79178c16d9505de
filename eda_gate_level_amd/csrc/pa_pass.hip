// pa_pass.hip -- the hot path of gate-level time-based power analysis on
// gfx950: one fused pass over the event layout plus a finalize.
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
// (Fig. 7).  This pass keeps that mapping and lays the data out for 64-lane
// waves:
//   * every gate's part of a time chunk is cut into density-aware windows
//     whose first event (the head) carries the gate's input state at the
//     window start; a lane walks whole windows, one event after the other,
//     in time order: the k-way merge of Sec. 2.4.2 is the layout's order;
//   * at load, a block's windows are dealt to its 1024 lanes longest first,
//     each to a lane whose stream is shortest so far, so the lanes' event
//     counts come out nearly equal;
//     a wave's 64 lane streams are interleaved two events at a time, so that
//     step i of the wave reads events 2i and 2i+1 of every lane with one
//     coalesced 16-byte load per lane (the next step's pair prefetched);
//   * per lane, in registers: the input state, the state at the start of the
//     current timestamp (all events of one timestamp see it), the pins that
//     already switched in the current cycle (the per-pin counter of Fig. 7:
//     an event whose pin is in that set is a glitch), and the gate's leakage
//     power; the gate record, cell entry, cap position and slew thresholds
//     are read once per window, at its head.  Every pin's last time and slew
//     in the current cycle sit in LDS for the pulse width of Eq. 2;
//   * per event: state-selected LUT, bilinear on slew and load (Sec. 2.4.1,
//     Fig. 2), switching energy (Eq. 1), energies added to per-cycle bins in
//     LDS.  The LUTs of the cells most of a block's events use are copied into
//     the block's spare LDS at its start (chosen at load from a sample of its
//     windows); the other cells are read through the caches;
//   * leakage is charged as power changes: every input event adds
//     dP = leak[S after] - leak[S before] (the events of one timestamp add up
//     to the change of the whole set); its partial bin gets dP * (bin end - t)
//     and all later bins get dP * their length through an in-LDS prefix sum
//     per chunk and a per-chunk carry; the leakage at t = 0 is the sum over
//     gates of leak[S0].  This is the paper's per-interval, per-overlapped-bin
//     split (Sec. 2.4.2, Eq. 4) summed in another order;
//   * every block writes its bins and totals to its own slots; the finalize
//     kernel adds them up in a fixed order (no global atomics).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "pa_common.h"

namespace pa {

namespace {

#ifndef PA_NT
#define PA_NT 1024
#endif
#ifndef PA_FUSED_ATTR
#define PA_FUSED_ATTR
#endif
constexpr int kNT = PA_NT;           // threads per block
constexpr int kNW = kNT / 64;        // waves per block, each walking its own 64 lane streams
constexpr int kBPC = 1024 / kNT;     // blocks per compute unit (16 waves each)
constexpr int kB = 128;              // events per wave step, two consecutive ones per lane
constexpr int kCCMAX = 2048;         // max cycles per chunk (LDS bins)
constexpr int kPlan = 8;             // cells per block whose LUTs may sit in LDS
constexpr uint32_t kLutLds = 0x80000000u;  // LUT base flag in a block's cell table: offset into its LDS copy
typedef __attribute__((address_space(3))) double lds_f64;
constexpr size_t kLdsMax = 160 * 1024 / kBPC;  // LDS of a block (gfx950: 160 KB per compute unit)

typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// r_gl (Eq. 2 as read): the pulse width over the mean of the two slews, at
// most 1.  The reciprocal of the mean is the hardware estimate refined by
// two Newton steps (each doubles its correct bits), a few ulp from the
// quotient instead of the exact division's dozen instructions.
__device__ __forceinline__ double glitch_ratio(double pw, double s0, double s1) {
  const double m = 0.5 * (s0 + s1);
  double x = __builtin_amdgcn_rcp(m);
  x = fma(fma(-m, x, 1.0), x, x);
  x = fma(fma(-m, x, 1.0), x, x);
  return fmin(pw * x, 1.0);
}

__device__ __forceinline__ double wave_sum(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// A double moved between lanes by a DPP control (both halves; lanes whose
// source is out of range or whose row is masked off get 0).
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, ROWS, 0xf, true);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, ROWS, 0xf, true);
  return __hiloint2double(hi, lo);
}

// Inclusive sum over the lanes of a wave up to this one, in a fixed order,
// with DPP lane moves (no LDS): a scan within every row of 16 lanes (shifts
// by 1, 2, 4, 8), then the rows' totals carried on by the row broadcasts of
// lane 15 and lane 31.  Lane 63 holds the wave's total.
__device__ __forceinline__ double wave_incl_scan(double v) {
  v += dpp_f64<0x111, 0xf>(v);  // row_shr:1
  v += dpp_f64<0x112, 0xf>(v);  // row_shr:2
  v += dpp_f64<0x114, 0xf>(v);  // row_shr:4
  v += dpp_f64<0x118, 0xf>(v);  // row_shr:8
  v += dpp_f64<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_f64<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Inclusive sum within every row of 16 lanes, in a fixed order.
__device__ __forceinline__ double row_incl_scan(double v) {
  v += dpp_f64<0x111, 0xf>(v);  // row_shr:1
  v += dpp_f64<0x112, 0xf>(v);  // row_shr:2
  v += dpp_f64<0x114, 0xf>(v);  // row_shr:4
  v += dpp_f64<0x118, 0xf>(v);  // row_shr:8
  return v;
}

// The same two scans of 32-bit integers.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xf, true);
}
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  v += dpp_u32<0x111, 0xf>(v);
  v += dpp_u32<0x112, 0xf>(v);
  v += dpp_u32<0x114, 0xf>(v);
  v += dpp_u32<0x118, 0xf>(v);
  v += dpp_u32<0x142, 0xa>(v);
  v += dpp_u32<0x143, 0xc>(v);
  return v;
}
__device__ __forceinline__ uint32_t row_incl_scan_u32(uint32_t v) {
  v += dpp_u32<0x111, 0xf>(v);
  v += dpp_u32<0x112, 0xf>(v);
  v += dpp_u32<0x114, 0xf>(v);
  v += dpp_u32<0x118, 0xf>(v);
  return v;
}

// lane l's double, l wave-uniform
__device__ __forceinline__ double lane_f64(double v, int l) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l),
                          __builtin_amdgcn_readlane(__double2loint(v), l));
}

struct CellLds {
  double2 *axw, *caxw;
  float *thr;
  double *bw, *bb;
  unsigned long long *bc;
  uint2 *prec;  // [waves][pin slots][64]: a pin's last (time in cycle, slew) per lane
  double *leak;
  uint2 *meta;
  double *lut;  // the block's LUT copies, 16-byte aligned after the cell meta
};

__host__ __device__ inline size_t cell_bytes(int n_cells, int n_slew, int n_cap, int n_thr, int64_t n_leak) {
  return 16 * (size_t)n_cells * (n_slew - 1 + n_cap - 1) + 4 * (size_t)n_cells * n_thr + 8 * (size_t)n_leak +
         8 * (size_t)n_cells;
}

// pin slots of a lane: the input pins 0..kmax-1 and the output pin (slot kmax)
__host__ __device__ inline size_t prec_bytes(int kmax) { return (size_t)kNW * (kmax + 1) * 64 * 8; }

// dynamic LDS: [slew (axis, 1/width) pairs][cap (axis, 1/width) pairs][slew thresholds][bins: wave,
// leakage change, counts][pin records][leakage][cell meta][LUT copies]
__device__ __forceinline__ CellLds carve(unsigned char *s, int Cc, int n_cells, int n_slew, int n_cap, int n_thr,
                                         int64_t n_leak, int kmax, bool cells) {
  CellLds L;
  L.axw = reinterpret_cast<double2 *>(s);
  L.caxw = L.axw + (cells ? n_cells * (n_slew - 1) : 0);
  L.thr = reinterpret_cast<float *>(L.caxw + (cells ? n_cells * (n_cap - 1) : 0));
  L.bw = reinterpret_cast<double *>(L.thr + (cells ? n_cells * n_thr : 0));
  L.bb = L.bw + Cc;
  L.bc = reinterpret_cast<unsigned long long *>(L.bb + Cc);
  L.prec = reinterpret_cast<uint2 *>(L.bc + Cc);
  L.leak = reinterpret_cast<double *>(L.prec + (size_t)kNW * (kmax + 1) * 64);
  L.meta = reinterpret_cast<uint2 *>(L.leak + (cells ? n_leak : 0));
  const size_t end = (size_t)(reinterpret_cast<unsigned char *>(L.meta + (cells ? n_cells : 0)) - s);
  L.lut = reinterpret_cast<double *>(s + ((end + 15) & ~size_t(15)));
  return L;
}

// NIN: number of inner slew-axis points when fixed at compile time (-1: any)
template <bool CELL_LDS, bool DIAG, int NIN>
__global__ __launch_bounds__(kNT) PA_FUSED_ATTR void k_fused(PassArgs a) {
  extern __shared__ __align__(16) unsigned char s_dyn[];
  __shared__ double s_red[kNW][8];
  __shared__ double s_scan[kNW];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int b = blockIdx.x;
  const int Cc = a.Cc, ns = a.n_slew, nc = a.n_cap, nthr = a.n_thr;
  const CellLds L = carve(s_dyn, Cc, a.n_cells, ns, nc, nthr, a.n_leak, a.kmax, CELL_LDS);
  const bool has_range = b < a.n_ranges;

  auto meta_of = [&](uint32_t c) -> uint2 {
    if constexpr (CELL_LDS) return L.meta[c]; else return a.cell_meta[c];
  };
  auto thr_of = [&](uint32_t c, int j) -> float4 {
    // cells < 2^24 and short axes: every offset here is a full-rate 24-bit product
    if constexpr (CELL_LDS) return *reinterpret_cast<const float4 *>(L.thr + __umul24(c, nthr) + j);
    else return *reinterpret_cast<const float4 *>(a.cell_thr + __umul24(c, nthr) + j);
  };
  auto axw_of = [&](uint32_t c, uint32_t j) -> double2 {
    if constexpr (CELL_LDS) return L.axw[__umul24(c, ns - 1) + j]; else return a.cell_axw[__umul24(c, ns - 1) + j];
  };
  auto caxw_of = [&](uint32_t c, uint32_t j) -> double2 {
    if constexpr (CELL_LDS) return L.caxw[__umul24(c, nc - 1) + j]; else return a.cell_caxw[__umul24(c, nc - 1) + j];
  };
  auto leak_of = [&](uint32_t j) -> double {
    if constexpr (CELL_LDS) return L.leak[j]; else return a.leak[j];
  };

  // ---- this wave's 64 lane streams: slots [base, base + 64 len), lane l's
  // event j at base + (j / 2) * 128 + 2 l + j % 2; the first pair is fetched
  // before the tables are staged
  int base = 0, len = 0, q = 0;
  if (has_range) {
    q = (int)a.rchunk[b];
    const uint2 d = a.wdesc[b * kNW + wid];
    // wave-uniform, so the step loop is steered by scalar branches
    base = __builtin_amdgcn_readfirstlane((int)d.x);
    len = __builtin_amdgcn_readfirstlane((int)d.y);
  }
  u64x2 kp = {0ull, 0ull};
  f32x2 sp = {0.f, 0.f};
  auto load_pair = [&](int j) {
    const int x = base + j * 64 + 2 * lane;
    kp = __builtin_nontemporal_load(reinterpret_cast<const u64x2 *>(a.key + x));
    sp = __builtin_nontemporal_load(reinterpret_cast<const f32x2 *>(a.slew + x));
  };
  if (len > 0) load_pair(0);
  for (int c = tid; c < Cc; c += kNT) {
    L.bw[c] = 0.0;
    L.bb[c] = 0.0;
    L.bc[c] = 0ull;
  }
  if constexpr (CELL_LDS) {
    for (int j = tid; j < a.n_cells * (ns - 1); j += kNT) L.axw[j] = a.cell_axw[j];
    for (int j = tid; j < a.n_cells * (nc - 1); j += kNT) L.caxw[j] = a.cell_caxw[j];
    for (int j = tid; j < a.n_cells * nthr; j += kNT) L.thr[j] = a.cell_thr[j];
    for (int j = tid; j < a.n_leak; j += kNT) L.leak[j] = a.leak[j];
    // the cells whose LUTs this block reads from LDS: their table entries
    // point into the copy instead of the global LUT
    uint32_t pc[kPlan], po[kPlan];
#pragma unroll
    for (int e = 0; e < kPlan; ++e) {
      const uint2 v = (has_range && a.lut_lds > 0) ? a.lut_plan[(size_t)b * kPlan + e] : make_uint2(~0u, 0u);
      pc[e] = v.x;
      po[e] = v.y;
    }
    for (int j = tid; j < a.n_cells; j += kNT) {
      uint2 mv = a.cell_meta[j];
#pragma unroll
      for (int e = 0; e < kPlan; ++e)
        if (pc[e] == (uint32_t)j) mv.y = kLutLds | po[e];
      L.meta[j] = mv;
    }
    // LUT sizes 2^k k ns nc are even, so every table starts 16-byte aligned
#pragma unroll 1
    for (int e = 0; e < kPlan; ++e) {
      if (pc[e] == ~0u) break;
      const uint2 gm = a.cell_meta[pc[e]];
      const uint32_t k = gm.x & 15u;
      const int n2 = (int)((((1u << k) * k) * (uint32_t)(ns * nc)) >> 1);
      const double2 *src = reinterpret_cast<const double2 *>(a.lut + gm.y);
      double2 *dst = reinterpret_cast<double2 *>(L.lut + po[e]);
#pragma unroll 4
      for (int j = tid; j < n2; j += kNT) dst[j] = src[j];
    }
  }
  __syncthreads();

  double e_int = 0.0, e_sw = 0.0, e_gl = 0.0, e_lk = 0.0;
  unsigned n_gl = 0;

  const int64_t cstart = (int64_t)q * a.chunk_ticks;
  const int64_t clen = min(a.chunk_ticks, a.t_max - cstart);
  const int ncyc = (int)((clen + a.T - 1) / a.T);
  const bool last_chunk = (q == a.Q - 1);
  const uint32_t lastc = (uint32_t)(ncyc - 1);
  const uint32_t T = a.T;
  const double Td = (double)T;
  const double tail = (double)(a.t_max - cstart);  // t_max - t = tail - (cyc T + tic)
  const double tick = a.tick_s;
  const uint32_t tb = a.tb, pb = a.pb, cs = tb + pb;
  const uint32_t gmask = (1u << a.gb) - 1u, ysh = 10u + a.gb;  // gate id and high cycle bits in the key's high word
  const uint32_t tmask = (1u << tb) - 1u;
  const uint32_t outc = (1u << pb) - 1u;
  const uint32_t kmax = (uint32_t)a.kmax;

  if (len > 0) {
    // the lane's window: its gate and cell entry, the load's position on
    // the cell's cap segment, the switching energy, the slew thresholds
    uint32_t gate = 0, cell = 0, kk = 0, lb = 0, lutb = 0, cseg = 0;
    double fc = 0.0, esw = 0.0;
    constexpr int NTH = NIN > 0 ? NIN : 1;
    float th[NTH];
#pragma unroll
    for (int j = 0; j < NTH; ++j) th[j] = __builtin_inff();
    // the lane's running state: input pins after the last event, at the start
    // of the current timestamp, pins switched in the current cycle, the time
    // of the last event, the leakage power of the current state
    uint32_t S = 0, St = 0, seen = 0, pcyc = ~0u, ptic = 0;
    double lkS = 0.0;
    uint2 *prec = L.prec + (size_t)wid * (kmax + 1) * 64 + lane;

#pragma unroll 1
    for (int j = 0; j < len; j += 2) {
      const uint64_t K0 = kp.x, K1 = kp.y;
      const float s0 = sp.x, s1 = sp.y;
      if (j + 2 < len) load_pair(j + 2);
      const uint32_t h0 = (uint32_t)(K0 >> 32);
      // a window head: windows have even lengths in the lane's stream, so a
      // head is always the first of a pair (an empty slot holds the pad key)
      if (K0 != a.pad_key && ((h0 >> 9) & 1u)) {
        gate = (h0 >> 10) & gmask;
        const uint4 rec = a.gate_rec[gate];
        const double cap = __hiloint2double((int)rec.y, (int)rec.x);
        cell = rec.z & 0xFFFFFFu;
        cseg = rec.z >> 24;
        const uint2 m = meta_of(cell);
        kk = m.x & 15u;
        lb = m.x >> 4;
        lutb = m.y;
        const double2 cx = caxw_of(cell, cseg);
        fc = (cap - cx.x) * cx.y;  // position on the gate's cap segment (Sec. 2.4.1, Fig. 2)
        esw = a.hv2 * cap;         // Eq. 1
        if constexpr (NIN > 0) {
#pragma unroll
          for (int i = 0; i < NIN; i += 4) {
            const float4 t4 = thr_of(cell, i);
            th[i] = t4.x;
            if (i + 1 < NIN) th[i + 1] = t4.y;
            if (i + 2 < NIN) th[i + 2] = t4.z;
            if (i + 3 < NIN) th[i + 3] = t4.w;
          }
        }
        S = h0 & 0xFFu;  // input state at the window start
        St = S;
        seen = 0;
        pcyc = ~0u;
        lkS = leak_of(lb + S);
      }

      // ---- the pair's two events, in phases so that both events' LDS reads
      // are in flight together.  Phase 1, integer and branch-free: the fields,
      // the state before each event (all events of one timestamp see the
      // state before the first of them, Sec. 2.4.2), the glitch flags (the pin
      // already switched in this clock cycle, Sec. 2.4.1, Fig. 7), the slew
      // segment and the LUT row.  An empty slot (the pad key: a short lane
      // stream or an odd window) changes no state and adds nothing.
      uint32_t code[2], tic[2], cyc[2], Sm[2], Sa[2], si[2], lo[2];
      bool act[2], input[2], glitch[2], rise[2];
      float sl[2] = {s0, s1};
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const uint64_t K = r ? K1 : K0;
        act[r] = K != a.pad_key;
        const uint32_t lk = (uint32_t)K, hw = (uint32_t)(K >> 32);
        code[r] = lk & outc;                   // pin code
        tic[r] = (lk >> pb) & tmask;           // time inside the cycle
        cyc[r] = (uint32_t)((((uint64_t)hw >> ysh) << 32 | lk) >> cs);  // cycle in the chunk
        rise[r] = (hw >> 8) & 1u;              // the pin's value after the event
        input[r] = act[r] && code[r] != outc;
        const bool newcyc = cyc[r] != pcyc;
        if (act[r] && (newcyc || tic[r] != ptic)) St = S;
        Sm[r] = St;
        if (act[r] && newcyc) seen = 0;
        const uint32_t bit = 1u << code[r];
        glitch[r] = act[r] && ((seen & bit) != 0u);
        if (act[r]) {
          seen |= bit;
          pcyc = cyc[r];
          ptic = tic[r];
        }
        if (input[r]) S ^= bit;
        Sa[r] = S;  // state after the event (leakage)
        // slew segment on the cell's axis: inner points at or below the slew (Sec. 2.4.1, Fig. 2)
        uint32_t n = 0;
        if constexpr (NIN > 0) {
#pragma unroll
          for (int i = 0; i < NIN; ++i) n += sl[r] >= th[i] ? 1u : 0u;
        } else {
          // padding points are +inf and never counted
          for (int i = 0; i < nthr; i += 4) {
            const float4 t4 = thr_of(cell, i);
            n += (sl[r] >= t4.x ? 1u : 0u) + (sl[r] >= t4.y ? 1u : 0u) + (sl[r] >= t4.z ? 1u : 0u) +
                 (sl[r] >= t4.w ? 1u : 0u);
          }
        }
        si[r] = n;
        const uint32_t cl = input[r] ? code[r] : 0u;
        lo[r] = __umul24(__umul24(__umul24(Sm[r], kk) + cl, ns) + n, nc) + cseg;
      }
      // ---- phase 2: every table read of both events
      double2 aw[2];
      double L00[2], L01[2], L10[2], L11[2], lkn[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        aw[r] = axw_of(cell, si[r]);
        lkn[r] = leak_of(lb + Sa[r]);
      }
      if (CELL_LDS && (lutb & kLutLds) != 0u) {
        // an LDS-typed pointer, so the two branches' loads stay ds reads and
        // global loads instead of merging into flat loads
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const lds_f64 *Lp = (const lds_f64 *)(L.lut) + ((lutb & ~kLutLds) + lo[r]);
          L00[r] = Lp[0], L01[r] = Lp[1], L10[r] = Lp[nc], L11[r] = Lp[nc + 1];
        }
      } else {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const double *Lp = a.lut + (lutb + lo[r]);
          L00[r] = Lp[0], L01[r] = Lp[1], L10[r] = Lp[nc], L11[r] = Lp[nc + 1];
        }
      }
      // ---- phase 3: energies (Sec. 2.4.1, Fig. 2; Eq. 1) and leakage changes (Sec. 2.4.2, Eq. 4)
      double E[2], dp[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const double fa = ((double)sl[r] - aw[r].x) * aw[r].y;
        const double v0 = L00[r] + fc * (L01[r] - L00[r]);
        const double v1 = L10[r] + fc * (L11[r] - L10[r]);
        const double Eint = v0 + fa * (v1 - v0);
        E[r] = input[r] ? Eint : ((act[r] && rise[r]) ? esw : 0.0);  // Eq. 1: 0->1 output events only
        // the toggle of an input moves the gate's leakage power from lkS to lkn
        const double lprev = r ? (input[0] ? lkn[0] : lkS) : lkS;
        dp[r] = input[r] ? lkn[r] - lprev : 0.0;
      }
      if (input[0]) lkS = lkn[0];
      if (input[1]) lkS = lkn[1];
      // ---- phase 4 (rare): a glitch's energy scaled by r_gl, from the pulse
      // width and the slews of the pin's previous event in the cycle and this one (Eq. 2)
      double scale[2] = {1.0, 1.0};
      if (glitch[0] || glitch[1]) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          uint2 *pr = prec + (size_t)min(code[r], kmax) * 64;
          if (glitch[r]) {
            const uint2 prev = *pr;  // the pin's previous event in this cycle
            scale[r] = glitch_ratio((double)(tic[r] - prev.x), (double)sl[r], (double)__uint_as_float(prev.y));
          }
          if (act[r]) *pr = make_uint2(tic[r], __float_as_uint(sl[r]));
        }
      } else {
#pragma unroll
        for (int r = 0; r < 2; ++r)
          if (act[r]) prec[(size_t)min(code[r], kmax) * 64] = make_uint2(tic[r], __float_as_uint(sl[r]));
      }
      // ---- phase 5: totals and bins
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        if (!act[r]) continue;
        double contrib = E[r];
        if (glitch[r]) {
          contrib = scale[r] * E[r];
          e_gl += contrib;
          ++n_gl;
        } else if (input[r]) {
          e_int += E[r];
        } else {
          e_sw += E[r];
        }
        const double dyn = contrib;  // this event's dynamic energy after the glitch scale
        if (dp[r] != 0.0) {
          // rest of the event's bin (the flush corrects a partial last bin)
          const double part = dp[r] * tick * (double)(T - tic[r]);
          if constexpr (DIAG) {
            if (a.gate_J)
              atomicAdd(a.gate_J + 4 * (size_t)a.gate_perm[gate] + 3,
                        dp[r] * tick * (double)(a.t_max - cstart - ((int64_t)cyc[r] * T + tic[r])));
          }
          contrib += part;
          e_lk += part;
          atomicAdd(&L.bb[cyc[r]], dp[r]);
        }
        if (contrib != 0.0) atomicAdd(&L.bw[cyc[r]], contrib);
        atomicAdd(&L.bc[cyc[r]], 1ull | ((unsigned long long)glitch[r] << 32));
        if constexpr (DIAG) {
          const uint32_t o = a.orig[base + j * 64 + 2 * lane + r];
          if (a.evt_glitch) a.evt_glitch[o] = glitch[r] ? 1 : 0;
          if (a.evt_state) a.evt_state[o] = (uint8_t)(input[r] ? Sm[r] : 0u);
          // the gate's own energy: internal, switching or glitch (device atomics)
          if (a.gate_J && dyn != 0.0)
            atomicAdd(a.gate_J + 4 * (size_t)a.gate_perm[gate] + (glitch[r] ? 2 : (input[r] ? 0 : 1)), dyn);
        }
      }
    }
  }
  __syncthreads();
  // ---- the block's bins: in-chunk prefix of the leakage changes, then its own slots
  double dsum = 0.0;
  {
    constexpr int PER = (kCCMAX + kNT - 1) / kNT;
    double loc[PER];
    double s = 0.0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid * PER + u;
      loc[u] = (has_range && c < ncyc) ? L.bb[c] : 0.0;
      s += loc[u];
    }
    double incl = s;
    for (int o = 1; o < 64; o <<= 1) {
      const double v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    if (lane == 63) s_scan[wid] = incl;
    __syncthreads();
    double wbase = 0.0;
    for (int w = 0; w < kNW; ++w) {
      const double v = s_scan[w];
      if (w < wid) wbase += v;
      dsum += v;
    }
    double run = wbase + incl - s;
    double *ow = a.blk_wave + (size_t)b * Cc;
    unsigned long long *oc = a.blk_cnt + (size_t)b * Cc;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid * PER + u;
      if (c < Cc) {
        double v = 0.0;
        unsigned long long cn = 0ull;
        if (has_range && c < ncyc) {
          // leakage changes of earlier bins of the chunk; the changes of this
          // bin reach t_max from the bin end on (its own part is in bw)
          const bool partial = last_chunk && c == (int)lastc;
          const double len = partial ? (double)a.last_len : Td;
          v = L.bw[c] + run * len * tick;
          if (partial) {
            const double fix = loc[u] * tick * (Td - (double)a.last_len);
            v -= fix;
            e_lk -= fix;
          } else {
            e_lk += loc[u] * tick * (tail - Td * (double)(c + 1));
          }
          cn = L.bc[c];
          run += loc[u];
        }
        ow[c] = v;
        oc[c] = cn;
      }
    }
  }

  // ---- block totals
  {
    double v[6] = {e_int, e_sw, e_gl, e_lk, 0.0, (double)n_gl};
#pragma unroll
    for (int u = 0; u < 6; ++u) v[u] = wave_sum(v[u]);
    if (lane == 0) {
#pragma unroll
      for (int u = 0; u < 6; ++u) s_red[wid][u] = v[u];
    }
    __syncthreads();
    if (tid < 8) {
      double t = 0.0;
      if (tid < 5) {
        for (int w = 0; w < kNW; ++w) t += s_red[w][tid];
      } else if (tid == 5) {
        t = dsum;
      } else if (tid == 6) {
        for (int w = 0; w < kNW; ++w) t += s_red[w][5];
      }
      a.blk_part[(size_t)b * 8 + tid] = t;
    }
  }
}


// ---------------------------------------------------------------------------
// The walk kernel: the same pass for the common case -- the cell tables and
// every LUT the block's gates use fit in its LDS, the slew and cap axes have
// NS and NC points, no per-event or per-gate outputs -- written for latency
// hiding and few instructions per event:
//   * the compact stream, 8 bytes a slot: a 32-bit key (cycle, tic, the pin
//     code's high bits) and the slew with the code's low bit (input pins) or
//     the new value (output pin) in its sign bit;
//   * windows start only at phase starts, all lanes of a wave together, each
//     phase behind a header pair that carries every lane's gate data (cell,
//     cap segment, start state, load), so the walk reads nothing but its
//     stream: one ring of stream pairs in registers, loaded a fixed number of
//     steps ahead, and no load depends on another;
//   * a phase walks the input-pin path or the output-pin path, never both;
//   * all LUT reads from the block's LDS copy of the contiguous LUT range of
//     its cells (gates are numbered in cell order, so a block's gates use a
//     contiguous range of cells);
//   * leakage changes are binned as (change at the bin start, minus the
//     change times its time in the bin), which needs no partial-bin fix-up.

// the walk kernel keeps the pin records of gates with at most this many
// inputs in registers
constexpr int kWalkRegPins = 4;

struct WalkBin {
  double w;    // energy: dynamic, minus leakage change x time in the bin
  double d;    // leakage power changes in the bin
  uint32_t n;  // events
  uint32_t g;  // glitches
};

typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) f64x2 lds_f64x2;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) WalkBin lds_bin;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;

// LDS pointers (32-bit addresses)
struct WalkLds {
  lds_f64x2 *axw, *caxw;
  lds_f32 *thr;
  lds_bin *bins;      // [Cc + 1]: bin Cc takes the pad slots
  lds_u32 *prec;      // [waves][input pins][64][2]: a pin's last (time in cycle, slew bits) per lane
  lds_f64 *leak;
  lds_u32x2 *meta;
  lds_f64 *lut;       // the block's LUT range, 16-byte aligned
};

__host__ __device__ inline size_t walk_fixed_bytes(int Cc, int n_cells, int n_slew, int n_cap, int n_thr,
                                                   int64_t n_leak, int kmax) {
  // pin records for the input pins only: output events walk windows of their own
  const size_t b = 16 * (size_t)n_cells * (n_slew - 1 + n_cap - 1) + 4 * (size_t)n_cells * n_thr +
                   24 * ((size_t)Cc + 1) + (size_t)kNW * kmax * 64 * 8 + 8 * (size_t)n_leak + 8 * (size_t)n_cells;
  return (b + 15) & ~size_t(15);
}

__device__ __forceinline__ WalkLds walk_carve(unsigned char *s, int Cc, int n_cells, int n_slew, int n_cap,
                                              int n_thr, int64_t n_leak, int kmax) {
  typedef __attribute__((address_space(3))) unsigned char lds_u8;
  lds_u8 *b = (lds_u8 *)s;
  WalkLds L;
  L.axw = (lds_f64x2 *)b;
  L.caxw = L.axw + n_cells * (n_slew - 1);
  L.thr = (lds_f32 *)(L.caxw + n_cells * (n_cap - 1));
  L.bins = (lds_bin *)(L.thr + n_cells * n_thr);
  L.prec = (lds_u32 *)(L.bins + Cc + 1);
  L.leak = (lds_f64 *)(L.prec + kNW * kmax * 64 * 2);
  L.meta = (lds_u32x2 *)(L.leak + (int)n_leak);
  L.lut = (lds_f64 *)(b + walk_fixed_bytes(Cc, n_cells, n_slew, n_cap, n_thr, n_leak, kmax));
  return L;
}

// 24-bit multiply-add (full rate; every operand here is far below 2^24)
__device__ __forceinline__ uint32_t mad24(uint32_t x, uint32_t y, uint32_t z) {
  return (x & 0xFFFFFFu) * (y & 0xFFFFFFu) + z;
}

// Add to a bin: an LDS atomic (PLAIN 0), or, as timing aids whose results
// are wrong, a plain load, add and store that loses an update meeting another
// on the same address (1), or a plain store of the contribution alone (2).
template <int PLAIN, class T, class P>
__device__ __forceinline__ void bin_add(P *p, T v) {
  if constexpr (PLAIN == 1) *p += v;
  else if constexpr (PLAIN == 2) *p = v;
  else __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

template <int NS, int NC, int PLAIN, int KREG, int MODE>
__global__ __launch_bounds__(kNT) PA_FUSED_ATTR void k_walk(PassArgs a) {
  constexpr int NIN = NS - 2;  // inner slew-axis points: the segment is the count at or below the slew
#ifndef PA_WALK_GROUP
#define PA_WALK_GROUP 2
#endif
#ifndef PA_WALK_LEAD
#define PA_WALK_LEAD 2
#endif
  constexpr int GP = PA_WALK_GROUP;  // pairs per group of the stream
  constexpr int LD = PA_WALK_LEAD;   // groups a load runs ahead of its use
  extern __shared__ __align__(16) unsigned char s_dyn[];
  __shared__ double s_red[kNW][8];
  __shared__ double s_scan[kNW];
  __shared__ uint32_t s_redu[kNW];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int b = blockIdx.x;
  const int Cc = a.Cc, nthr = a.n_thr;
  const WalkLds L = walk_carve(s_dyn, Cc, a.n_cells, NS, NC, nthr, a.n_leak, a.kmax);
  const bool has_range = b < a.n_ranges;

  int base = 0, len = 0, q = 0;
  uint2 lut_range = make_uint2(0u, 0u);  // the block's LUT range (first entry, entries)
  if (has_range) {
    q = (int)a.rchunk[b];
    const uint2 d = a.wdesc[b * kNW + wid];
    lut_range = a.blk_lut[b];
    base = __builtin_amdgcn_readfirstlane((int)d.x);
    len = __builtin_amdgcn_readfirstlane((int)d.y);
  }
  const int npair = len >> 1;  // lane streams have even lengths
  // the ring: R = LD + 1 groups of GP pairs; before group g is walked, the
  // loads of group g + LD go into the slots group g - 1 has freed.  The walk
  // loop is unrolled R times, so every slot keeps its registers and no load
  // in flight is ever copied (a copy would have to wait for it).
  constexpr int R = LD + 1;
  u32x2 kr[R][GP], sr[R][GP];
  auto load_pair = [&](int p, u32x2 &k, u32x2 &sl) {
    const int x = base + p * 128 + 2 * lane;
    k = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(a.ckey + x));
    sl = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(a.cslew + x));
  };

  // block set-up: bins, cell tables and the LUT range.
  // The first element of every table per thread and up to KU LUT pairs per
  // thread are loaded before the first store, so the set-up waits for
  // memory once (larger tables and ranges loop on).
  constexpr int KU = 6;
  const uint32_t lut_lo = lut_range.x;
  const int n2 = (int)(lut_range.y >> 1);  // cell LUT sizes 2^k k NS NC are even: the range is 16-byte aligned
  const f64x2 *lsrc = reinterpret_cast<const f64x2 *>(a.lut + lut_lo);
  lds_f64x2 *ldst = (lds_f64x2 *)L.lut;
  f64x2 lv[KU];
#pragma unroll
  for (int u = 0; u < KU; ++u)
    if (u * kNT < n2) lv[u] = lsrc[min(u * kNT + tid, n2 - 1)];
  const f64x2 *ax = reinterpret_cast<const f64x2 *>(a.cell_axw), *cx = reinterpret_cast<const f64x2 *>(a.cell_caxw);
  const u32x2 *me = reinterpret_cast<const u32x2 *>(a.cell_meta);
  const int nax = a.n_cells * (NS - 1), ncx = a.n_cells * (NC - 1), nth = a.n_cells * nthr, nlk = (int)a.n_leak,
            nme = a.n_cells;
  const f64x2 vax = ax[min(tid, nax - 1)], vcx = cx[min(tid, ncx - 1)];
  const float vth = a.cell_thr[min(tid, nth - 1)];
  const double vlk = a.leak[min(tid, nlk - 1)];
  const u32x2 vme = me[min(tid, nme - 1)];
  // the ring's first group, issued after the tables so that waiting for the
  // tables does not wait for it (loads complete in order); the next groups
  // after the set-up barrier: every wave of the chip asks for its first
  // stream bytes at once, and asking for one group instead of LD halves that
  // burst, so the first group arrives sooner
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < GP; ++i) {
      kr[r][i] = u32x2{~0u, ~0u};
      sr[r][i] = u32x2{0x3F800000u, 0x3F800000u};
      if (r == 0 && npair > 0) load_pair(min(i, npair - 1), kr[r][i], sr[r][i]);
    }
  for (int c = tid; c <= Cc; c += kNT) {
    L.bins[c].w = 0.0;
    L.bins[c].d = 0.0;
    L.bins[c].n = 0u;
    L.bins[c].g = 0u;
  }
  if (tid < nax) L.axw[tid] = vax;
  if (tid < ncx) L.caxw[tid] = vcx;
  if (tid < nth) L.thr[tid] = vth;
  if (tid < nlk) L.leak[tid] = vlk;
  if (tid < nme) L.meta[tid] = vme;
#pragma unroll
  for (int u = 0; u < KU; ++u)
    if (u * kNT + tid < n2) ldst[u * kNT + tid] = lv[u];
  for (int j = tid + kNT; j < nax; j += kNT) L.axw[j] = ax[j];
  for (int j = tid + kNT; j < ncx; j += kNT) L.caxw[j] = cx[j];
  for (int j = tid + kNT; j < nth; j += kNT) L.thr[j] = a.cell_thr[j];
  for (int j = tid + kNT; j < nlk; j += kNT) L.leak[j] = a.leak[j];
  for (int j = tid + kNT; j < nme; j += kNT) L.meta[j] = me[j];
  for (int j = KU * kNT + tid; j < n2; j += kNT) ldst[j] = lsrc[j];
  __syncthreads();
#pragma unroll
  for (int r = 1; r < LD; ++r)
#pragma unroll
    for (int i = 0; i < GP; ++i)
      if (npair > 0) load_pair(min(r * GP + i, npair - 1), kr[r][i], sr[r][i]);

  // the leakage changes' times in their bins are not summed here: the bins
  // hold the energies minus them, so the flush gets their sum from the bins
  double e_int = 0.0, e_sw = 0.0, e_gl = 0.0;
  const int64_t cstart = (int64_t)q * a.chunk_ticks;
  const int64_t clen = min(a.chunk_ticks, a.t_max - cstart);
  const int ncyc = (int)((clen + a.T - 1) / a.T);
  const bool last_chunk = (q == a.Q - 1);
  const uint32_t lastc = (uint32_t)(ncyc - 1);
  const double Td = (double)a.T;
  const double tail = (double)(a.t_max - cstart);
  const double tick = a.tick_s;
  const uint32_t ck = a.ck, tsh = a.tbc + a.ck;
  const uint32_t tmask = (1u << a.tbc) - 1u, ckmask = (1u << ck) - 1u;
  const uint32_t hdr = tmask << ck, out_bit = 1u << tsh;
  const uint32_t cmask = (uint32_t)Cc - 1u;
  constexpr uint32_t kPad = ~0u;
  constexpr uint32_t PSZ = NS * NC;  // LUT entries per (state, pin)
  // a bin by cycle: a full-rate 24-bit offset (a bin is 24 bytes)
  auto bin_at = [&](uint32_t cyc) -> lds_bin * {
    return (lds_bin *)((__attribute__((address_space(3))) unsigned char *)L.bins + mad24(cyc & cmask, 24u, 0u));
  };

  if (npair > 0) {
    // the lane's window: LUT row base in the LDS copy, state stride, axis-table
    // and leakage bases, load position on the cap segment, switching energy,
    // slew thresholds
    uint32_t wbase = 0, kpsz = 0, axb = 0, lb = 0;
    double fc = 0.0, esw = 0.0;
    float th[NIN];
#pragma unroll
    for (int j = 0; j < NIN; ++j) th[j] = __builtin_inff();
    // running state: inputs after the last event, at the start of the current
    // timestamp, pins switched in the current cycle, last cycle, time and
    // slew, leakage power of the current state
    uint32_t S = 0, St = 0, seen = 0, pcyc = ~0u, ptic = 0;
    float pslew = 1.f;
    bool out_phase = false;  // the kind of the current phase's windows (wave-uniform)
    // per-gate rows (MODE 2): the window's header pair, the lane's energy
    // sums at the window start, the window's leakage to t_max
    uint32_t gid = ~0u;
    double g_int0 = 0.0, g_sw0 = 0.0, g_gl0 = 0.0, g_lk = 0.0;
    // the window's four sums, stored at its header pair (every window once a
    // pass): the wave's lanes store 2 KB in one piece
    auto flush_gate = [&]() {
      if (gid != ~0u) {
        double2 *r = reinterpret_cast<double2 *>(a.wrec) + 2 * (size_t)gid;
        r[0] = make_double2(e_int - g_int0, e_sw - g_sw0);
        r[1] = make_double2(e_gl - g_gl0, g_lk * tick);
      }
    };
    lds_u32 *prec = L.prec + (wid * a.kmax * 64 + lane) * 2;
    // with at most KREG = 4 input pins per gate, the pin records (last time
    // in the cycle, slew bits) live in registers instead: two 4-vectors whose
    // elements a per-lane pin selects (selects, not an indexed array, which
    // would go to scratch memory)
    static_assert(KREG == 0 || KREG == 4, "register pin records hold four pins");
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 rtic = {0u, 0u, 0u, 0u}, rslw = {0u, 0u, 0u, 0u};

    // a header pair: every lane with a window in the new phase sets it up (a
    // lane without one sets up cell 0 with load 0, and walks empty slots)
    auto header = [&](const u32x2 &k, const u32x2 &sw, bool own) {
      const double cap = own ? __hiloint2double((int)sw.y, (int)sw.x) : 0.0;
      if (out_phase) {
        esw = a.hv2 * cap;  // Eq. 1
        pcyc = ~0u;
        return;
      }
      // a lane without a window reads the first entries of the LDS range
      const uint32_t cell = own ? (k.y & 0xFFFFFu) : 0u, cseg = own ? ((k.y >> 20) & 15u) : 0u;
      const u32x2 m = L.meta[cell];
      lb = m.x >> 4;
      kpsz = own ? (m.x & 15u) * PSZ : 0u;
      wbase = own ? m.y - lut_lo + cseg : 0u;
      axb = mad24(cell, NS - 1, 0u);
      const f64x2 cx = L.caxw[mad24(cell, NC - 1, cseg)];
      fc = (cap - cx.x) * cx.y;  // position on the gate's cap segment (Sec. 2.4.1, Fig. 2)
#pragma unroll
      for (int i = 0; i < NIN; i += 4) {
        const f32x4 t4 = *(const lds_f32x4 *)(L.thr + mad24(cell, nthr, i));
        th[i] = t4.x;
        if (i + 1 < NIN) th[i + 1] = t4.y;
        if (i + 2 < NIN) th[i + 2] = t4.z;
        if (i + 3 < NIN) th[i + 3] = t4.w;
      }
      S = own ? k.y >> 24 : 0u;  // input state at the window start
      St = S;
      seen = 0;
      pcyc = ~0u;
    };

    // the two input-pin events of a pair (Sec. 2.4.1-2.4.2, Fig. 7), in
    // phases so that both events' table reads are in flight together and
    // their arithmetic interleaves; an empty slot toggles nothing, so its
    // leakage change is zero, and adds nothing
    auto pair_in = [&](const u32x2 &K, const u32x2 &SW, uint32_t &ev) {
      bool real[2], glitch[2];
      uint32_t tic[2], cyc[2], cl[2], lo[2], li[2], nseg[2];
      float sl[2];
      // the leakage power before the pair is read again rather than carried
      // from the previous pair, so no LDS result lives across the loop's joins
      const uint32_t l0 = lb + S;
      // integer work: fields, the state before each event (all events of one
      // timestamp see the state before the first of them, Sec. 2.4.2), the
      // glitch flags (the pin already switched in this cycle, Fig. 7), the
      // slew segment (inner axis points at or below the slew, Fig. 2), the
      // LUT row and the leakage entry of the state after the event
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const uint32_t k = r ? K.y : K.x, sw = r ? SW.y : SW.x;
        real[r] = k != kPad;
        const uint32_t code = ((k & ckmask) << 1) | (sw >> 31);
        sl[r] = __uint_as_float(sw & 0x7FFFFFFFu);
        tic[r] = (k >> ck) & tmask;
        cyc[r] = k >> tsh;
        const bool newcyc = cyc[r] != pcyc;
        if (newcyc || tic[r] != ptic) St = S;
        if (newcyc) seen = 0u;
        cl[r] = real[r] ? code : 0u;
        const uint32_t bit = real[r] ? 1u << code : 0u;
        glitch[r] = (seen & bit) != 0u;
        seen |= bit;
        pcyc = cyc[r];
        ptic = tic[r];
        const uint32_t Sm = St;
        S ^= bit;
        if constexpr (MODE == 1) ev |= (Sm | (glitch[r] ? 256u : 0u)) << (16 * r);
        uint32_t n = 0;
#pragma unroll
        for (int i = 0; i < NIN; ++i) n += sl[r] >= th[i] ? 1u : 0u;
        nseg[r] = n;
        // every factor is small; kpsz is a loop-carried value whose small
        // range the instruction selector cannot see: an empty asm hides it
        // from the optimizer too, so the multiply is a full-rate mad24
        uint32_t kp = kpsz;
        asm volatile("" : "+v"(kp));
        lo[r] = mad24(Sm, kp, mad24(cl[r], PSZ, mad24(n, NC, wbase)));
        li[r] = lb + S;
      }
      // every table read of both events
      double L00[2], L01[2], L10[2], L11[2], lkn[2];
      f64x2 aw[2];
      const double lkS = L.leak[l0];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const lds_f64 *Lp = L.lut + lo[r];
        L00[r] = Lp[0];
        L01[r] = Lp[1];
        L10[r] = Lp[NC];
        L11[r] = Lp[NC + 1];
        aw[r] = L.axw[axb + nseg[r]];
        lkn[r] = L.leak[li[r]];
      }
      // energies (bilinear on slew and load, Fig. 2) and leakage changes (Eq. 4)
      double E[2], dp[2], ct[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const double fa = ((double)sl[r] - aw[r].x) * aw[r].y;
        const double v0 = L00[r] + fc * (L01[r] - L00[r]);
        const double v1 = L10[r] + fc * (L11[r] - L10[r]);
        E[r] = v0 + fa * (v1 - v0);
      }
      dp[0] = lkn[0] - lkS;
      dp[1] = lkn[1] - lkn[0];
      if constexpr (MODE == 2)  // each power change's leakage up to t_max (an empty slot changes nothing)
        g_lk += dp[0] * (tail - Td * (double)cyc[0] - (double)tic[0]) +
                dp[1] * (tail - Td * (double)cyc[1] - (double)tic[1]);
#pragma unroll
      for (int r = 0; r < 2; ++r) ct[r] = dp[r] * (double)tic[r];
      // rarely, a glitch: Eq. 2 (reading), the pulse width and the slews of
      // the pin's previous event in the cycle and this one; the pin records
      // are read and written in event order (both events may be one pin's)
      if constexpr (KREG > 0) {
        if (glitch[0] || glitch[1]) {
          // the second event's pin record is the first event itself when both are one pin's
          const bool same = cl[1] == cl[0];
          const uint32_t pt0 = rtic[cl[0] & 3u], ps0 = rslw[cl[0] & 3u];
          const uint32_t pt1 = same ? tic[0] : rtic[cl[1] & 3u];
          const uint32_t ps1 = same ? __float_as_uint(sl[0]) : rslw[cl[1] & 3u];
          if (glitch[0]) {
            E[0] *= glitch_ratio((double)(tic[0] - pt0), (double)sl[0], (double)__uint_as_float(ps0));
            e_gl += E[0];
          }
          if (glitch[1]) {
            E[1] *= glitch_ratio((double)(tic[1] - pt1), (double)sl[1], (double)__uint_as_float(ps1));
            e_gl += E[1];
          }
        }
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          rtic[cl[r] & 3u] = tic[r];
          rslw[cl[r] & 3u] = __float_as_uint(sl[r]);
        }
      } else {
        lds_u32 *pr0 = prec + cl[0] * 128, *pr1 = prec + cl[1] * 128;
        if (glitch[0] || glitch[1]) {
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            lds_u32 *pr = r ? pr1 : pr0;
            if (glitch[r]) {
              const uint32_t ptic_pin = pr[0], pslew_pin = pr[1];
              E[r] *= glitch_ratio((double)(tic[r] - ptic_pin), (double)sl[r], (double)__uint_as_float(pslew_pin));
              e_gl += E[r];
            }
            pr[0] = tic[r];
            pr[1] = __float_as_uint(sl[r]);
          }
        } else {
          pr0[0] = tic[0];
          pr0[1] = __float_as_uint(sl[0]);
          pr1[0] = tic[1];
          pr1[1] = __float_as_uint(sl[1]);
        }
      }
      // the components and the bins; an empty slot adds nothing
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        if (real[r]) {
          e_int += glitch[r] ? 0.0 : E[r];
          lds_bin *bp = bin_at(cyc[r]);
          bin_add<PLAIN>(&bp->w, fma(ct[r], -tick, E[r]));
          bin_add<PLAIN>(&bp->d, dp[r]);
          bin_add<PLAIN>(&bp->n, 1u);
          if (glitch[r]) bin_add<PLAIN>(&bp->g, 1u);
        }
      }
    };

    // the two output-pin events of a pair: 1/2 c Vdd^2 for 0->1 (Eq. 1),
    // scaled by r_gl when the pin already switched in this cycle (Eq. 2,
    // Fig. 7); the window's only pin is the output, so its previous event is
    // the lane's previous event.  An empty slot (value bit 0) adds nothing.
    auto pair_out = [&](const u32x2 &K, const u32x2 &SW, uint32_t &ev) {
      bool real[2], glitch[2];
      uint32_t tic[2], cyc[2];
      float sl[2];
      double E[2];
      uint32_t pt = ptic;
      float ps = pslew;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const uint32_t k = r ? K.y : K.x, sw = r ? SW.y : SW.x;
        real[r] = k != kPad;
        sl[r] = __uint_as_float(sw & 0x7FFFFFFFu);
        tic[r] = (k >> ck) & tmask;
        cyc[r] = k >> tsh;
        glitch[r] = real[r] && cyc[r] == pcyc;
        if constexpr (MODE == 1) ev |= (glitch[r] ? 256u : 0u) << (16 * r);  // an output event's state is 0
        E[r] = (sw >> 31) ? esw : 0.0;
        pcyc = cyc[r];
      }
      if (glitch[0] || glitch[1]) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          if (glitch[r]) {
            E[r] *= glitch_ratio((double)(tic[r] - (r ? tic[0] : pt)), (double)sl[r], (double)(r ? sl[0] : ps));
            e_gl += E[r];
          }
        }
      }
      ptic = tic[1];
      pslew = sl[1];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        if (real[r]) {
          e_sw += glitch[r] ? 0.0 : E[r];
          lds_bin *bp = bin_at(cyc[r]);
          bin_add<PLAIN>(&bp->w, E[r]);
          bin_add<PLAIN>(&bp->n, 1u);
          if (glitch[r]) bin_add<PLAIN>(&bp->g, 1u);
        }
      }
    };

#pragma unroll 1
    for (int p0 = 0; p0 < npair; p0 += GP * R) {
      // issue priority by the share of the wave's stream still to walk (the
      // quarter: 3 for the first, 0 for the last): a SIMD issues oldest wave
      // first among equals, and a wave that falls behind the others of its
      // block catches up instead of finishing last
      {
        const int quarter = (4 * (npair - p0) - 1) / npair;
        if (quarter >= 3) __builtin_amdgcn_s_setprio(3);
        else if (quarter == 2) __builtin_amdgcn_s_setprio(2);
        else if (quarter == 1) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
      }
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int pg = p0 + u * GP;  // the group's first pair
        if (pg >= npair) break;
        // group g + LD's loads (past the end: the last pair again)
#pragma unroll
        for (int i = 0; i < GP; ++i)
          load_pair(min(pg + LD * GP + i, npair - 1), kr[(u + LD) % R][i], sr[(u + LD) % R][i]);
#pragma unroll
        for (int i = 0; i < GP; ++i) {
          if (pg + i >= npair) break;
          const u32x2 k = kr[u][i], sw = sr[u][i];
          // a header pair starts a phase in every lane at once: one wave-uniform
          // test, the phase's kind from the headers
          const bool own = (k.x & ~out_bit) == hdr;
          if (__ballot(own) != 0ull) {
            out_phase = __ballot(own && (k.x & out_bit)) != 0ull;
            if constexpr (MODE == 2) {
              // the previous window's sums; the new window's header pair
              flush_gate();
              gid = own ? ((uint32_t)base >> 1) + (uint32_t)(pg + i) * 64u + lane : ~0u;
              g_int0 = e_int;
              g_sw0 = e_sw;
              g_gl0 = e_gl;
              g_lk = 0.0;
            }
            header(k, sw, own);
            continue;
          }
          uint32_t ev = 0;  // the pair's per-event outputs: state before | glitch << 8, per slot
          if (out_phase) pair_out(k, sw, ev);
          else pair_in(k, sw, ev);
          // in stream order: the wave's 64 lanes store 256 contiguous bytes
          if constexpr (MODE == 1) a.evs[((uint32_t)base >> 1) + (uint32_t)(pg + i) * 64u + lane] = ev;
        }
      }
    }
    if constexpr (MODE == 2) flush_gate();
    __builtin_amdgcn_s_setprio(0);
  }
  // the walk's energies, summed within the wave as soon as it ends its walk
  // (a wave that ends early does it while the others still walk)
  {
    const double t0 = wave_incl_scan(e_int), t1 = wave_incl_scan(e_sw), t2 = wave_incl_scan(e_gl);
    if (lane == 63) {
      s_red[wid][0] = t0;
      s_red[wid][1] = t1;
      s_red[wid][2] = t2;
    }
  }
  __syncthreads();

  // ---- the block's bins: thread t owns bins 2t and 2t + 1.  The leakage
  // changes' in-chunk prefix: a DPP scan of the threads' pairs within every
  // wave, then the waves' totals over one row of 16 lanes; every thread
  // stores its two bins with one 16-byte store per array.
  static_assert(kCCMAX <= 2 * kNT && kNW == 16, "two bins per thread; one row of lanes for the waves");
  double xs = 0.0;   // the thread's share of the leakage part: changes' energy to t_max plus its bins' sum
  uint32_t ngl = 0;  // glitches in the thread's bins
  double dsum = 0.0;
  {
    const int c0 = 2 * tid;
    const bool in0 = has_range && c0 < ncyc, in1 = has_range && c0 + 1 < ncyc;
    const double d0 = in0 ? L.bins[c0].d : 0.0, d1 = in1 ? L.bins[c0 + 1].d : 0.0;
    const double incl = wave_incl_scan(d0 + d1);  // the wave's changes up to bin 2t + 1
    if (lane == 63) s_scan[wid] = incl;
    const double excl = dpp_f64<0x138, 0xf>(incl);  // wave_shr:1, lane 0 gets 0: up to bin 2t - 1
    __syncthreads();
    const double tw = row_incl_scan(lane < kNW ? s_scan[lane] : 0.0);
    const double wb = wid > 0 ? lane_f64(tw, wid - 1) : 0.0;  // changes of the earlier waves' bins
    dsum = lane_f64(tw, kNW - 1);
    // the bins' own changes count from the bin start; the bin corrects for their times
    const double r0 = (wb + excl) + d0, r1 = r0 + d1;
    double v0 = 0.0, v1 = 0.0;
    unsigned long long n0 = 0ull, n1 = 0ull;
    if (in0) {
      const double blen = (last_chunk && c0 == (int)lastc) ? (double)a.last_len : Td;
      const double w = L.bins[c0].w;
      const uint32_t g = L.bins[c0].g;
      v0 = w + r0 * blen * tick;
      xs += w + d0 * (tail - Td * (double)c0) * tick;
      n0 = (unsigned long long)L.bins[c0].n | ((unsigned long long)g << 32);
      ngl += g;
    }
    if (in1) {
      const double blen = (last_chunk && c0 + 1 == (int)lastc) ? (double)a.last_len : Td;
      const double w = L.bins[c0 + 1].w;
      const uint32_t g = L.bins[c0 + 1].g;
      v1 = w + r1 * blen * tick;
      xs += w + d1 * (tail - Td * (double)(c0 + 1)) * tick;
      n1 = (unsigned long long)L.bins[c0 + 1].n | ((unsigned long long)g << 32);
      ngl += g;
    }
    double *ow = a.blk_wave + (size_t)b * Cc;
    unsigned long long *oc = a.blk_cnt + (size_t)b * Cc;
    if (c0 + 1 < Cc) {  // Cc is a power of two, so here Cc is even and both stores are 16-byte aligned
      *reinterpret_cast<double2 *>(ow + c0) = make_double2(v0, v1);
      *reinterpret_cast<ulonglong2 *>(oc + c0) = make_ulonglong2(n0, n1);
    } else if (c0 < Cc) {
      ow[c0] = v0;
      oc[c0] = n0;
    }
  }

  // ---- block totals: the leakage part and the glitches within the waves,
  // then every quantity over the waves with one row scan
  {
    const double xw = wave_incl_scan(xs);
    const uint32_t gw = wave_incl_scan_u32(ngl);
    if (lane == 63) {
      s_red[wid][3] = xw;
      s_redu[wid] = gw;
    }
    __syncthreads();
    if (wid == 0) {
      // row q of the wave's lanes holds the waves' totals of quantity q: e_int, e_sw, e_gl, leakage part
      const double t = row_incl_scan(s_red[lane & 15][lane >> 4]);
      const uint32_t gt = row_incl_scan_u32(lane < kNW ? s_redu[lane] : 0u);
      const double T0 = lane_f64(t, 15), T1 = lane_f64(t, 31), T2 = lane_f64(t, 47), X = lane_f64(t, 63);
      const uint32_t G = __builtin_amdgcn_readlane(gt, 15);
      // the leakage: the changes' energy to t_max from their bins' starts, minus their times
      // in their bins (the bins' sum less the dynamic energies)
      if (lane < 8) {
        const double val = lane == 0 ? T0 : lane == 1 ? T1 : lane == 2 ? T2 : lane == 3 ? X - ((T0 + T1) + T2)
                         : lane == 5 ? dsum : lane == 6 ? (double)G : 0.0;
        a.blk_part[(size_t)b * 8 + lane] = val;
      }
    }
  }
}

// One wave per block: 64 windows sampled at the midpoints of 64 equal slices
// of the block's window range (windows in gate order, gates numbered in cell
// order, so the cells come out nondecreasing) give the cells present and each
// cell's share; the heaviest cells whose LUTs still fit in `budget` doubles
// are taken, heaviest first.
__global__ __launch_bounds__(64) void k_lut_plan(const uint64_t *skey, const uint32_t *ws, const uint32_t *bwin,
                                                 const uint4 *gate_rec, const uint2 *cell_meta, uint32_t gb, int ns,
                                                 int nc, uint32_t budget, uint2 *plan) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const uint32_t w0 = bwin[b], w1 = bwin[b + 1];
  const uint32_t gmask = (1u << gb) - 1u;
  uint32_t cell = ~0u;
  if (w1 > w0) {
    const uint32_t w = w0 + (uint32_t)((uint64_t)(w1 - w0) * (2 * lane + 1) / 128);
    const uint32_t g = (uint32_t)(skey[ws[w]] >> (32 + 10)) & gmask;
    cell = gate_rec[g].z & 0xFFFFFFu;
  }
  const uint32_t prev = __shfl_up(cell, 1);
  const bool start = cell != ~0u && (lane == 0 || prev != cell);
  const unsigned long long st = __ballot(start);
  uint32_t len = 0, sz = 0;
  if (start) {
    const unsigned long long after = lane < 63 ? (st >> (lane + 1)) << (lane + 1) : 0ull;
    len = (after ? (uint32_t)(__ffsll((long long)after) - 1) : 64u) - (uint32_t)lane;
    const uint32_t k = cell_meta[cell].x & 15u;
    sz = ((1u << k) * k) * (uint32_t)(ns * nc);
  }
  bool cand = start && sz <= budget;
  uint32_t used = 0;
  int ne = 0;
  while (ne < kPlan) {
    uint32_t v = cand ? (len << 6 | (63u - (uint32_t)lane)) : 0u;
    for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
    if (v == 0u) break;
    const int bl = 63 - (int)(v & 63u);
    const uint32_t bsz = (uint32_t)__shfl((int)sz, bl), bcell = (uint32_t)__shfl((int)cell, bl);
    if (lane == bl) cand = false;
    if (used + bsz <= budget) {
      if (lane == 0) plan[(size_t)b * kPlan + ne] = make_uint2(bcell, used);
      used += bsz;
      ++ne;
    }
  }
  if (lane >= ne && lane < kPlan) plan[(size_t)b * kPlan + lane] = make_uint2(~0u, 0u);
}

constexpr int kFC = 64;             // finalize: cycles per block (one per lane)
constexpr int kFP = 8;              // finalize: waves per block, each adding up a share of the blocks
constexpr int kFT = kFC * kFP;

// Lane l of wave p < 7 adds up, for cycle l of the block's 64, the bins of
// the p-th seventh of the cycle's chunk's blocks; wave 7 adds up the blocks'
// totals (so no wave waits for two rounds of loads).  Wave 0 then adds the
// shares in order after the leakage carried into the chunk (L0 plus the
// changes of earlier chunks); block 0 also writes the totals (Eq. 3).  Every
// sum runs in a fixed order.  L0 and the chunks' first blocks (fewer than 64
// chunks) come by value, and the loads of a loop step are issued
// unconditionally (an index past the end is clamped and its value dropped),
// so they go out together and wait once.
__global__ __launch_bounds__(kFT) void k_finalize(FinalArgs f) {
  __shared__ double s_w[kFP][kFC];
  __shared__ unsigned long long s_n[kFP][kFC];
  __shared__ double s_t[8];
  const int lane = threadIdx.x & 63, wp = threadIdx.x >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * kFC;
  const int64_t chi = min(c0 + kFC, f.C) - 1;
  const int64_t c = c0 + lane;
  const int qa = (int)(c0 / f.Cc), qb = (int)(chi / f.Cc);
  const int q = (int)(min(c, chi) / f.Cc);
  const bool inl = f.Q < 64;
  auto cblk = [&](int i) -> uint32_t { return inl ? f.cblk[i] : f.chunk_blk[i]; };
  const bool totals = blockIdx.x == 0;
  constexpr int kBW = kFP - 1;  // waves adding up bins
  if (wp < kBW) {
    // this wave's share of the cycle's chunk's blocks
    const uint32_t b0 = cblk(q), b1 = cblk(q + 1);
    const uint32_t n = b1 - b0, s0 = b0 + n * wp / kBW, s1 = b0 + n * (wp + 1) / kBW;
    const int cin = (int)(min(c, chi) - (int64_t)q * f.Cc);
    double w = 0.0;
    unsigned long long cnt = 0;
    for (uint32_t bb = s0; bb < s1; bb += 8) {
      double v[8];
      unsigned long long m[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t bi = min(bb + u, s1 - 1);
        v[u] = f.blk_wave[(size_t)bi * f.Cc + cin];
        m[u] = f.blk_cnt[(size_t)bi * f.Cc + cin];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool ok = bb + u < s1;
        w += ok ? v[u] : 0.0;
        cnt += ok ? m[u] : 0ull;
      }
    }
    s_w[wp][lane] = w;
    s_n[wp][lane] = cnt;
  } else {
    // the blocks' totals: the changes before chunk qa, and (block 0) the energies
    const uint32_t ba = cblk(qa);
    double t[7] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    for (int b8 = 0; b8 < f.grid; b8 += 64 * 8) {
      double d5[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) d5[u] = f.blk_part[(size_t)min(b8 + u * 64 + lane, f.grid - 1) * 8 + 5];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int bb = b8 + u * 64 + lane;
        t[1] += (bb < f.grid && (uint32_t)bb < ba) ? d5[u] : 0.0;
      }
      if (totals) {
        double pp[8][5];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const double *p = f.blk_part + (size_t)min(b8 + u * 64 + lane, f.grid - 1) * 8;
          pp[u][0] = p[0], pp[u][1] = p[1], pp[u][2] = p[2], pp[u][3] = p[3], pp[u][4] = p[6];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const bool ok = b8 + u * 64 + lane < f.grid;
#pragma unroll
          for (int x = 0; x < 5; ++x) t[2 + x] += ok ? pp[u][x] : 0.0;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 7; ++u) t[u] = wave_sum(t[u]);
    if (lane == 0) {
#pragma unroll
      for (int u = 0; u < 7; ++u) s_t[u] = t[u];
    }
    s_w[wp][lane] = 0.0;
    s_n[wp][lane] = 0ull;
  }
  __syncthreads();
  if (wp != 0) return;
  const double l0 = f.l0;
  const double pre = s_t[1];
  // the changes inside chunks qa .. qb-1 (qb - qa < 64), then their exclusive prefix
  double dq = 0.0;
  if (lane < qb - qa) {
    const uint32_t b0 = cblk(qa + lane), b1 = cblk(qa + lane + 1);
    for (uint32_t bb = b0; bb < b1; ++bb) dq += f.blk_part[(size_t)bb * 8 + 5];
  }
  double incl = dq;
  for (int o = 1; o < 64; o <<= 1) {
    const double v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  const double Pj = l0 + pre + (incl - dq);  // power carried into chunk qa + lane
  const double Pq = __shfl(Pj, q - qa, 64);
  if (c < f.C) {
    const double len = (c == f.C - 1) ? (double)f.last_len : (double)f.T;
    double w = Pq * len * f.tick_s;
    unsigned long long cnt = 0;
#pragma unroll
    for (int p = 0; p < kFP; ++p) {
      w += s_w[p][lane];
      cnt += s_n[p][lane];
    }
    f.wave_out[c] = w;
    f.cyc_events[c] = cnt & 0xFFFFFFFFull;
    f.cyc_glitches[c] = cnt >> 32;
  }
  if (totals && lane == 0) {
    double t[5];
    for (int u = 0; u < 5; ++u) t[u] = s_t[2 + u];
    const double window = (double)f.t_max * f.tick_s;
    const double e_leak = l0 * window + t[3];
    f.res[0] = t[0];
    f.res[1] = t[1];
    f.res[2] = t[2];
    f.res[3] = e_leak;
    f.res[4] = t[0] / window;  // Eq. 3
    f.res[5] = t[1] / window;
    f.res[6] = t[2] / window;
    f.res[7] = e_leak / window;
    f.res[8] = t[4];
  }
}

}  // namespace

int pass_block_threads() { return kNT; }
int pass_blocks_per_cu() { return kBPC; }
int pass_waves_per_block() { return kNW; }
// static LDS of the pass kernels: s_red [kNW][8] and s_scan (the walk kernel's
// holds a row of wave totals for every kNT bins of a chunk)
size_t pass_static_lds_bytes() {
  return (size_t)kNW * 8 * sizeof(double) + (size_t)((kCCMAX + kNT - 1) / kNT) * kNW * sizeof(double);
}

hipError_t launch_lut_plan(const uint64_t *skey, const uint32_t *ws, const uint32_t *bwin, int32_t n_ranges,
                           const uint4 *gate_rec, const uint2 *cell_meta, uint32_t gb, int n_slew, int n_cap,
                           int32_t lut_lds, uint2 *plan, hipStream_t s) {
  if (n_ranges <= 0 || lut_lds <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_lut_plan, dim3(n_ranges), dim3(64), 0, s, skey, ws, bwin, gate_rec, cell_meta, gb, n_slew,
                     n_cap, (uint32_t)lut_lds, plan);
  return hipGetLastError();
}
int pass_lut_plan_slots() { return kPlan; }
int pass_wave_batch() { return kB; }
int pass_max_chunk_cycles() { return kCCMAX; }

size_t pass_lds_bytes(int Cc, int n_cells, int n_slew, int n_cap, int n_thr, int64_t n_leak, int kmax, bool cells) {
  return 24 * (size_t)Cc + prec_bytes(kmax) + (cells ? cell_bytes(n_cells, n_slew, n_cap, n_thr, n_leak) : 0);
}

bool pass_cells_fit_lds(int Cc, int n_cells, int n_slew, int n_cap, int n_thr, int64_t n_leak, int kmax) {
  return pass_lds_bytes(Cc, n_cells, n_slew, n_cap, n_thr, n_leak, kmax, true) + pass_static_lds_bytes() <= kLdsMax;
}

static size_t lut_lds_offset(int Cc, int n_cells, int n_slew, int n_cap, int n_thr, int64_t n_leak, int kmax) {
  return (pass_lds_bytes(Cc, n_cells, n_slew, n_cap, n_thr, n_leak, kmax, true) + 15) & ~size_t(15);
}

int32_t pass_lut_lds_doubles(int Cc, int n_cells, int n_slew, int n_cap, int n_thr, int64_t n_leak, int kmax) {
  if (!pass_cells_fit_lds(Cc, n_cells, n_slew, n_cap, n_thr, n_leak, kmax)) return 0;
  const size_t used = lut_lds_offset(Cc, n_cells, n_slew, n_cap, n_thr, n_leak, kmax) + pass_static_lds_bytes();
  return used < kLdsMax ? (int32_t)((kLdsMax - used) / 16 * 2) : 0;
}

namespace {

// Every block's LUT range: the LUTs of the cells from its first window's gate's
// cell to its last window's (gates are numbered in cell order, and a block's
// windows are in gate order), as (first entry, entries).
__global__ void k_block_luts(int32_t nr, const uint64_t *skey, const uint32_t *ws, const uint32_t *bwin,
                             const uint4 *gate_rec, const uint2 *cell_meta, uint32_t gb, uint32_t psz, uint2 *out) {
  for (int b = blockIdx.x * blockDim.x + threadIdx.x; b < nr; b += gridDim.x * blockDim.x) {
    const uint32_t w0 = bwin[b], w1 = bwin[b + 1];
    uint2 r = make_uint2(0u, 0u);
    if (w1 > w0) {
      const uint32_t gmask = (1u << gb) - 1u;
      const uint32_t g0 = (uint32_t)(skey[ws[w0]] >> 42) & gmask, g1 = (uint32_t)(skey[ws[w1 - 1]] >> 42) & gmask;
      const uint32_t c0 = gate_rec[g0].z & 0xFFFFFFu, c1 = gate_rec[g1].z & 0xFFFFFFu;
      const uint2 m0 = cell_meta[c0], m1 = cell_meta[c1];
      const uint32_t k1 = m1.x & 15u;
      r = make_uint2(m0.y, m1.y + ((1u << k1) * k1) * psz - m0.y);
    }
    out[b] = r;
  }
}

}  // namespace

hipError_t launch_block_luts(int32_t nr, const uint64_t *skey, const uint32_t *ws, const uint32_t *bwin,
                             const uint4 *gate_rec, const uint2 *cell_meta, uint32_t gb, int n_slew, int n_cap,
                             uint2 *out, hipStream_t s) {
  if (nr <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_block_luts, dim3((nr + 255) / 256), dim3(256), 0, s, nr, skey, ws, bwin, gate_rec, cell_meta,
                     gb, (uint32_t)(n_slew * n_cap), out);
  return hipGetLastError();
}

bool walk_supported(int n_slew, int n_cap) { return (n_slew == 7 && n_cap == 7) || (n_slew == 8 && n_cap == 8); }

int32_t walk_lut_doubles(int Cc, int n_cells, int n_slew, int n_cap, int n_thr, int64_t n_leak, int kmax) {
  const size_t fixed = walk_fixed_bytes(Cc, n_cells, n_slew, n_cap, n_thr, n_leak, kmax) + pass_static_lds_bytes();
  return fixed < kLdsMax ? (int32_t)((kLdsMax - fixed) / 16 * 2) : 0;
}

// A launch; with events, they are attached to the kernel's dispatch and
// time the kernel's own execution (not the dispatch and completion around it).
template <class K, class A>
static void launch_timed(K kernel, dim3 g, dim3 t, size_t dyn, hipStream_t s, hipEvent_t e0, hipEvent_t e1,
                         const A &a) {
  if (e0 && e1) hipExtLaunchKernelGGL(kernel, g, t, (uint32_t)dyn, s, e0, e1, 0, a);
  else hipLaunchKernelGGL(kernel, g, t, dyn, s, a);
}

hipError_t launch_pass(const PassArgs &a, int grid_blocks, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const bool cells = pass_cells_fit_lds(a.Cc, a.n_cells, a.n_slew, a.n_cap, a.n_thr, a.n_leak, a.kmax);
  const bool diag = a.evt_glitch || a.evt_state || a.gate_J;
  if (a.walk_lut > 0 && !diag) {
    // the walk kernel: every block's LUT range in its LDS (at least the entries a lane without a window reads)
    const size_t dyn = walk_fixed_bytes(a.Cc, a.n_cells, a.n_slew, a.n_cap, a.n_thr, a.n_leak, a.kmax) +
                       8 * (size_t)max(a.walk_lut, 2 * a.n_slew * a.n_cap);
    if (!a.blk_lut || !a.ckey || !a.cslew || dyn + pass_static_lds_bytes() > kLdsMax) return hipErrorInvalidValue;
    const dim3 g(grid_blocks), t(kNT);
    const bool kreg = a.kmax <= kWalkRegPins;
    if (a.n_slew == 7 && a.n_cap == 7) {
      if (a.plain_bins == 1) launch_timed(k_walk<7, 7, 1, 0, 0>, g, t, dyn, s, e0, e1, a);
      else if (a.plain_bins == 2) launch_timed(k_walk<7, 7, 2, 0, 0>, g, t, dyn, s, e0, e1, a);
      else if (a.wrec && kreg) launch_timed(k_walk<7, 7, 0, kWalkRegPins, 2>, g, t, dyn, s, e0, e1, a);
      else if (a.wrec) launch_timed(k_walk<7, 7, 0, 0, 2>, g, t, dyn, s, e0, e1, a);
      else if (a.evs && kreg) launch_timed(k_walk<7, 7, 0, kWalkRegPins, 1>, g, t, dyn, s, e0, e1, a);
      else if (a.evs) launch_timed(k_walk<7, 7, 0, 0, 1>, g, t, dyn, s, e0, e1, a);
      else if (kreg) launch_timed(k_walk<7, 7, 0, kWalkRegPins, 0>, g, t, dyn, s, e0, e1, a);
      else launch_timed(k_walk<7, 7, 0, 0, 0>, g, t, dyn, s, e0, e1, a);
    } else if (a.n_slew == 8 && a.n_cap == 8) {
      if (a.plain_bins == 1) launch_timed(k_walk<8, 8, 1, 0, 0>, g, t, dyn, s, e0, e1, a);
      else if (a.plain_bins == 2) launch_timed(k_walk<8, 8, 2, 0, 0>, g, t, dyn, s, e0, e1, a);
      else if (a.wrec && kreg) launch_timed(k_walk<8, 8, 0, kWalkRegPins, 2>, g, t, dyn, s, e0, e1, a);
      else if (a.wrec) launch_timed(k_walk<8, 8, 0, 0, 2>, g, t, dyn, s, e0, e1, a);
      else if (a.evs && kreg) launch_timed(k_walk<8, 8, 0, kWalkRegPins, 1>, g, t, dyn, s, e0, e1, a);
      else if (a.evs) launch_timed(k_walk<8, 8, 0, 0, 1>, g, t, dyn, s, e0, e1, a);
      else if (kreg) launch_timed(k_walk<8, 8, 0, kWalkRegPins, 0>, g, t, dyn, s, e0, e1, a);
      else launch_timed(k_walk<8, 8, 0, 0, 0>, g, t, dyn, s, e0, e1, a);
    }
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  size_t dyn = pass_lds_bytes(a.Cc, a.n_cells, a.n_slew, a.n_cap, a.n_thr, a.n_leak, a.kmax, cells);
  if (cells && a.lut_lds > 0) {
    if (!a.lut_plan) return hipErrorInvalidValue;
    dyn = lut_lds_offset(a.Cc, a.n_cells, a.n_slew, a.n_cap, a.n_thr, a.n_leak, a.kmax) + 8 * (size_t)a.lut_lds;
  }
  if (dyn + pass_static_lds_bytes() > kLdsMax) return hipErrorInvalidValue;
  const dim3 g(grid_blocks), t(kNT);
  if (cells && !diag) {
    if (a.n_slew == 7) launch_timed(k_fused<true, false, 5>, g, t, dyn, s, e0, e1, a);
    else if (a.n_slew == 8) launch_timed(k_fused<true, false, 6>, g, t, dyn, s, e0, e1, a);
    else launch_timed(k_fused<true, false, -1>, g, t, dyn, s, e0, e1, a);
  } else if (cells) {
    launch_timed(k_fused<true, true, -1>, g, t, dyn, s, e0, e1, a);
  } else if (!diag) {
    launch_timed(k_fused<false, false, -1>, g, t, dyn, s, e0, e1, a);
  } else {
    launch_timed(k_fused<false, true, -1>, g, t, dyn, s, e0, e1, a);
  }
  return hipGetLastError();
}

// Every laid-out event's slot, by the caller's event index (the inverse of
// the stream's caller-index array; empty slots hold ~0 there).
__global__ void k_slot_of(int64_t n, const uint32_t *orig, uint32_t *slot_of) {
  const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (x >= n) return;
  const uint32_t o = orig[x];
  if (o < 0x80000000u) slot_of[o] = (uint32_t)x;  // ~0: an empty slot or a header
}

// The walk's per-event outputs (state before | glitch << 8, 16 bits a slot,
// in stream order) into the caller's event order.
__global__ void k_event_out(int64_t E, const uint32_t *slot_of, const uint16_t *evs, uint8_t *glitch,
                            uint8_t *state) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const uint32_t v = evs[slot_of[e]];
  if (glitch) glitch[e] = (uint8_t)(v >> 8);
  if (state) state[e] = (uint8_t)(v & 0xFFu);
}

hipError_t launch_slot_of(int64_t n, const uint32_t *orig, uint32_t *slot_of, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_slot_of, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, n, orig, slot_of);
  return hipGetLastError();
}

hipError_t launch_event_out(int64_t E, const uint32_t *slot_of, const uint32_t *evs, uint8_t *glitch,
                            uint8_t *state, hipStream_t s) {
  if (E <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_event_out, dim3((unsigned)((E + 255) / 256)), dim3(256), 0, s, E, slot_of,
                     reinterpret_cast<const uint16_t *>(evs), glitch, state);
  return hipGetLastError();
}

hipError_t launch_finalize(const FinalArgs &f, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int grid = (int)((f.C + kFC - 1) / kFC);
  launch_timed(k_finalize, dim3(grid), dim3(kFT), 0, s, e0, e1, f);
  return hipGetLastError();
}

}  // namespace pa
