// The single-workgroup prefix schedule for CDNA4 (gfx950), shared by the
// scheduler's own launches (schedule.hip) and the last step of the fused draft
// step (markov_kernels.h), which runs it on a workgroup that has no step work.
//
// [P1] section 二 design 2: candidates sorted globally by survival (a stable
// LSD radix sort, 4 passes of 8 bits, ballot-based peer ranking, per-wave
// digit counters in LDS), exact fixed-point prefix sums of the survivals in
// sorted order, Theta = tau * SPS(B) at every budget, the first argmax, and
// l_r = #{j : rank(r, j) < m*}.  Also the fused step's confidences, STS and
// survivals from the two parts of each confidence logit.
#pragma once

#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "dspark_internal.h"
#include "packed_words.h"

namespace dspark {
namespace {

constexpr int kT = 1024;          // threads
constexpr int kW = kT / 64;       // wavefronts
constexpr int kDig = 256;         // radix digits per pass
constexpr double kTauScale = 1099511627776.0;       // 2^40
constexpr double kTauInv = 1.0 / 1099511627776.0;   // 2^-40


// Shared state of a single-workgroup schedule with NW wavefronts.
template <int NW>
struct SchedSharedT {
  int cnt[NW * kDig];        // per-wave digit counters, then offsets
  int base[kDig];            // running global digit offsets
  int tot[kDig];             // digit totals
  unsigned long long wsum[NW];
  unsigned long long wpre[NW];   // exclusive prefix of the wave totals
  double bval[NW + 1];       // per-wave results, then the block's (slot NW)
  int bidx[NW + 1];
  unsigned long long bsum[NW + 1];
  unsigned long long carry;
  unsigned long long cin;    // carry before the current chunk
};
using SchedShared = SchedSharedT<kW>;

// ---- wavefront scans through DPP ----
// One step of a 64-lane inclusive scan: lanes read the value `CTRL` names (row
// shifts inside each 16-lane row, then the broadcasts of lane 15 and lane 31
// into the following rows, restricted to rows ROWS); a lane with no source, or
// outside ROWS, reads `ident`.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_read(uint32_t v, uint32_t ident) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, CTRL, ROWS, 0xf, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ unsigned long long dpp_read(unsigned long long v,
                                                       unsigned long long ident) {
  const uint32_t lo = dpp_read<CTRL, ROWS>((uint32_t)v, (uint32_t)ident);
  const uint32_t hi = dpp_read<CTRL, ROWS>((uint32_t)(v >> 32), (uint32_t)(ident >> 32));
  return ((unsigned long long)hi << 32) | lo;
}

// Inclusive scan of v over the wavefront under an associative op with
// identity ident (Hillis-Steele inside rows, then two row broadcasts).  All 64
// lanes must be active.
template <typename T, typename Op>
__device__ __forceinline__ T wave_iscan(T v, T ident, Op op) {
  v = op(v, dpp_read<0x111, 0xf>(v, ident));   // row_shr:1
  v = op(v, dpp_read<0x112, 0xf>(v, ident));   // row_shr:2
  v = op(v, dpp_read<0x114, 0xf>(v, ident));   // row_shr:4
  v = op(v, dpp_read<0x118, 0xf>(v, ident));   // row_shr:8
  v = op(v, dpp_read<0x142, 0xa>(v, ident));   // row_bcast:15 into rows 1 and 3
  v = op(v, dpp_read<0x143, 0xc>(v, ident));   // row_bcast:31 into rows 2 and 3
  return v;
}

__device__ __forceinline__ uint32_t lane_u32(uint32_t v, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}
__device__ __forceinline__ unsigned long long lane_u64(unsigned long long v, int lane) {
  return ((unsigned long long)lane_u32((uint32_t)(v >> 32), lane) << 32) | lane_u32((uint32_t)v, lane);
}

struct AddU32 { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; } };
struct AddU64 {
  __device__ unsigned long long operator()(unsigned long long a, unsigned long long b) const {
    return a + b;
  }
};
struct AddF32 {   // fp32 sums on the bit patterns (the scans move 32-bit words)
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }
};
struct MaxU64 {
  __device__ unsigned long long operator()(unsigned long long a, unsigned long long b) const {
    return a > b ? a : b;
  }
};
struct MinI32 {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const {
    return (uint32_t)min((int)a, (int)b);
  }
};

// Survivals are probabilities: a value outside [0, 1] is clamped into it and
// NaN is taken as 0 (so the fixed-point tau sum stays below R (1 + gamma) 2^40).
__device__ __forceinline__ float clamp_survival(float a) {
  return a > 0.0f ? (a < 1.0f ? a : 1.0f) : 0.0f;
}

__device__ __forceinline__ uint32_t key_of(float a) {
  // non-negative bits of the clamped value (-0 -> +0), complemented:
  // ascending = descending a
  return ~__float_as_uint(clamp_survival(a));
}

__device__ __forceinline__ float value_of(uint32_t ck) { return __uint_as_float(~ck); }

// Exclusive scan of the 256 digit totals tot[] into base[] (wave 0 does the work).
template <class SH>
__device__ void scan_digits(SH& sh, const int* tot) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int v[4];
    int s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = s;
      s += tot[lane * 4 + j];
    }
    // inclusive scan of s across the wave
    const int inc = (int)wave_iscan((uint32_t)s, 0u, AddU32{});
    const int ex = inc - s;
#pragma unroll
    for (int j = 0; j < 4; ++j) sh.base[lane * 4 + j] = ex + v[j];
  }
}

// Rank this wave's ITEMS elements by digit; rk[i] = rank among equal digits of
// this wave in (item, lane) order.  cnt row of this wave must be zero on entry.
template <int ITEMS, class SH>
__device__ __forceinline__ void rank_items(SH& sh, const uint32_t (&ck)[ITEMS],
                                           const bool (&ok)[ITEMS], int shift, int (&rk)[ITEMS]) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const unsigned long long lt = (1ull << lane) - 1ull;
  int* cnt = sh.cnt + w * kDig;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int d = (ck[i] >> shift) & 0xff;
    unsigned long long peers = __ballot(ok[i]);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (d >> b) & 1;
      const unsigned long long bal = __ballot(ok[i] && bit);
      peers &= bit ? bal : ~bal;
    }
    if (ok[i]) {
      const int before = cnt[d];
      rk[i] = before + __popcll(peers & lt);
      if ((peers & lt) == 0ull) cnt[d] = before + __popcll(peers);
    }
  }
}

// Single tile: per digit d (one thread each), cnt[w][d] becomes the count of
// digit d in waves before w, and tot[d] the digit's total.
template <int NW>
__device__ __forceinline__ void wave_prefix_and_totals(SchedSharedT<NW>& sh) {
  // One digit per thread (digits past 64 NW: a second round).
  for (int d = threadIdx.x; d < kDig; d += 64 * NW) {
    int c[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) c[w] = sh.cnt[w * kDig + d];
    int run = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      sh.cnt[w * kDig + d] = run;
      run += c[w];
    }
    sh.tot[d] = run;
  }
}

template <class SH>
__device__ __forceinline__ void zero_my_counters(SH& sh) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < kDig / 64; ++j) sh.cnt[w * kDig + lane + 64 * j] = 0;
}

// Block-wide exclusive scan of one uint64 per thread; returns the exclusive
// prefix and adds the block total to sh.carry (after the call, all threads see
// the old carry in `carry_in`).
template <int NW>
__device__ __forceinline__ unsigned long long block_exscan_u64(SchedSharedT<NW>& sh,
                                                               unsigned long long v,
                                                               unsigned long long& carry_in) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const unsigned long long inc = wave_iscan(v, 0ull, AddU64{});
  if (lane == 63) sh.wsum[w] = inc;
  __syncthreads();
  // Wave 0 scans the wave totals and moves the carry on.
  if (w == 0) {
    const unsigned long long t = lane < NW ? sh.wsum[lane] : 0ull;
    const unsigned long long ti = wave_iscan(t, 0ull, AddU64{});
    if (lane < NW) sh.wpre[lane] = ti - t;
    const unsigned long long total = lane_u64(ti, 63);
    if (lane == 0) {
      const unsigned long long c = sh.carry;
      sh.cin = c;
      sh.carry = c + total;
    }
  }
  __syncthreads();
  carry_in = sh.cin;
  return sh.wpre[w] + inc - v;
}

struct Best {
  double theta;
  int m;
  unsigned long long S;   // fixed-point prefix sum at m
};

__device__ __forceinline__ void better(Best& b, const Best& o) {
  if (o.theta > b.theta || (o.theta == b.theta && o.m < b.m)) b = o;
}

// Order-preserving 64-bit key of a double (larger value, larger key; -0 and
// +0 share one key, as they compare equal).
__device__ __forceinline__ unsigned long long theta_key(double x) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(x == 0.0 ? 0.0 : x);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// Argmax over the wavefront: the largest Theta, then the smallest m among the
// lanes holding it; every lane gets the winner.
__device__ __forceinline__ Best wave_best(const Best& b) {
  const unsigned long long key = theta_key(b.theta);
  const unsigned long long kmax = lane_u64(wave_iscan(key, 0ull, MaxU64{}), 63);
  const uint32_t mine = key == kmax ? (uint32_t)b.m : 0x7fffffffu;
  const int mmin = (int)lane_u32(wave_iscan(mine, 0x7fffffffu, MinI32{}), 63);
  const unsigned long long sel = __ballot(key == kmax && b.m == mmin);
  const int src = (int)__builtin_ctzll(sel);
  Best r;
  r.theta = __longlong_as_double((long long)lane_u64((unsigned long long)__double_as_longlong(b.theta), src));
  r.m = mmin;
  r.S = lane_u64(b.S, src);
  return r;
}

// Block argmax of Theta (largest Theta, smallest m); every thread gets the
// result.  Each wave reduces its lanes, wave 0 the per-wave winners.
template <int NW>
__device__ __forceinline__ void block_best(SchedSharedT<NW>& sh, Best& best) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const Best wb = wave_best(best);
  if (lane == 0) {
    sh.bval[w] = wb.theta;
    sh.bidx[w] = wb.m;
    sh.bsum[w] = wb.S;
  }
  __syncthreads();
  if (w == 0) {
    Best e{-1.0, 0x7fffffff, 0ull};
    if (lane < NW) e = Best{sh.bval[lane], sh.bidx[lane], sh.bsum[lane]};
    const Best bb = wave_best(e);
    if (lane == 0) {
      sh.bval[NW] = bb.theta;
      sh.bidx[NW] = bb.m;
      sh.bsum[NW] = bb.S;
    }
  }
  __syncthreads();
  best = Best{sh.bval[NW], sh.bidx[NW], sh.bsum[NW]};
}

// Block minimum / sum (every thread gets the result; sh's per-wave slots are
// free again on return).
template <int NW>
__device__ __forceinline__ int block_min_int(SchedSharedT<NW>& sh, int v) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  v = (int)lane_u32(wave_iscan((uint32_t)v, 0x7fffffffu, MinI32{}), 63);
  if (lane == 0) sh.bidx[w] = v;
  __syncthreads();
  if (w == 0) {
    const uint32_t t = lane < NW ? (uint32_t)sh.bidx[lane] : 0x7fffffffu;
    const int r = (int)lane_u32(wave_iscan(t, 0x7fffffffu, MinI32{}), 63);
    if (lane == 0) sh.bidx[NW] = r;
  }
  __syncthreads();
  const int r = sh.bidx[NW];
  __syncthreads();
  return r;
}

template <int NW>
__device__ __forceinline__ unsigned long long block_sum_sh(SchedSharedT<NW>& sh,
                                                           unsigned long long v) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  v = lane_u64(wave_iscan(v, 0ull, AddU64{}), 63);
  if (lane == 0) sh.wsum[w] = v;
  __syncthreads();
  if (w == 0) {
    const unsigned long long t = lane < NW ? sh.wsum[lane] : 0ull;
    const unsigned long long r = lane_u64(wave_iscan(t, 0ull, AddU64{}), 63);
    if (lane == 0) sh.bsum[NW] = r;
  }
  __syncthreads();
  const unsigned long long r = sh.bsum[NW];
  __syncthreads();
  return r;
}

// Theta_m with tau from the fixed-point prefix sum S_m (the single definition
// every mode uses).
__device__ __forceinline__ double theta_at(int R, unsigned long long S, float sps_b) {
  return __ull2double_rn(((unsigned long long)R << 40) + S) * kTauInv * (double)sps_b;
}

// Phase 3 + 4 for a sorted array (keys ck, ids) given in blocked chunks.
// load(p, ck, id) fetches the element at sorted position p.
//   mode 0 (global search): first argmax of Theta over every m;
//   mode 1 (early stop): the first m with Theta_{m+1} <= Theta_m, each element
//     comparing its Theta with the one before it (tau from S - q, exactly the
//     value the previous position has); N if Theta keeps rising;
//   mode 2 (capacity): m = m_cap.
// Modes 1 and 2 then sum the survivals below m* (tau*) from the sorted keys.
template <int ITEMS, int NW, typename Load, typename SetRank, typename SpsAt>
__device__ void scan_theta(SchedSharedT<NW>& sh, int N, int R, const float* __restrict__ sps,
                           float sps0, int mode, int m_cap, int32_t* __restrict__ order,
                           Load load, SetRank set_rank, SpsAt sps_at, Best& best) {
  const int tid = threadIdx.x;
  if (tid == 0) sh.carry = 0ull;
  best.theta = -1.0;
  best.m = 0x7fffffff;
  best.S = 0ull;
  if (tid == 0 && mode == 0) {
    best.theta = (double)R * (double)sps0;  // m = 0: tau = R, sps0 = sps[R - 1]
    best.m = 0;
  }
  int brk = 0x7fffffff;
  __syncthreads();
  const unsigned long long rfx = (unsigned long long)R << 40;
  constexpr int NT = 64 * NW;
  for (int c0 = 0; c0 < N; c0 += NT * ITEMS) {
    uint32_t ck[ITEMS];
    int id[ITEMS];
    unsigned long long q[ITEMS];
    unsigned long long tsum = 0;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int p = c0 + tid * ITEMS + i;
      if (p < N) {
        load(p, ck[i], id[i]);
        q[i] = __double2ull_rn((double)value_of(ck[i]) * kTauScale);
      } else {
        ck[i] = 0xffffffffu;
        id[i] = -1;
        q[i] = 0ull;
      }
      tsum += q[i];
    }
    unsigned long long carry_in;
    const unsigned long long ex = block_exscan_u64(sh, tsum, carry_in);
    unsigned long long S = carry_in + ex;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int p = c0 + tid * ITEMS + i;
      if (p < N) {
        S += q[i];
        if (mode == 0) {
          const double tau = __ull2double_rn(rfx + S) * kTauInv;
          const double th = tau * (double)sps_at(p, i);   // sps[R + p]: budget B = R + p + 1
          if (th > best.theta) {
            best.theta = th;
            best.m = p + 1;
            best.S = S;
          }
        } else if (mode == 1) {
          const double th = theta_at(R, S, sps_at(p, i));
          const double th_prev = theta_at(R, S - q[i], sps[R + p - 1]);
          if (!(th > th_prev)) brk = min(brk, p);
        }
        if (order) order[p] = id[i];
      }
    }
    __syncthreads();   // every element of this chunk is read before ranks overwrite storage
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int p = c0 + tid * ITEMS + i;
      if (p < N) set_rank(id[i], p);
    }
    __syncthreads();
  }
  if (mode == 0) {
    block_best(sh, best);
    return;
  }
  int m_star = m_cap;
  if (mode == 1) {
    m_star = block_min_int(sh, brk);
    if (m_star > N) m_star = N;
  }
  unsigned long long part = 0;
  for (int p = tid; p < m_star; p += NT) {
    uint32_t k;
    int i;
    load(p, k, i);
    part += __double2ull_rn((double)value_of(k) * kTauScale);
  }
  const unsigned long long Sm = block_sum_sh(sh, part);
  best.m = m_star;
  best.S = Sm;
  best.theta = theta_at(R, Sm, mode == 1 ? sps[R + m_star - 1] : 1.0f);
}

template <int NT>
__device__ void write_results(int R, int gamma, const Best& best, const int* rank,
                              int32_t* __restrict__ lengths, dspark_schedule_info* info) {
  const int m_star = best.m;
  for (int r = threadIdx.x; r < R; r += NT) {
    int l = 0;
    for (int j = 0; j < gamma; ++j) l += rank[r * gamma + j] < m_star ? 1 : 0;
    lengths[r] = l;
  }
  if (info && threadIdx.x == 0) {
    const unsigned long long tau_fx = ((unsigned long long)R << 40) + best.S;
    info->B_star = R + m_star;
    info->m_star = m_star;
    info->tau_fx = tau_fx;
    info->tau = __ull2double_rn(tau_fx) * kTauInv;
    info->theta = best.theta;
  }
}

// ---------------------------------------------------------------------------
// Single-tile path: N <= kT * ITEMS, everything in LDS.
// ---------------------------------------------------------------------------
// Inputs of the fused draft step's finishing work: packed words and the two
// parts of every confidence logit.  It runs in one of two places:
//   a launch after the last step (kFinAfter): `words` are the last step's, it
//     writes the last token, and every position's embedding term comes from se;
//   inside the last step's launch (kFinInStep), on a workgroup that has no
//     step work: `words` are those of the step before (NULL when gamma = 1:
//     the anchors), and it computes the last position's embedding term
//     w_e . W1[x_{gamma-2}] itself, since the last step's own is not there yet;
//     the step workgroups write the last token.
constexpr int kFinNone = 0, kFinAfter = 1, kFinInStep = 2;

struct FinishArgs {
  const unsigned long long* words;   // packed words [R][S] (see above)
  int S;
  int V;
  const float* sh;                   // w_h . h, [R * gamma]
  const float* se;                   // w_e . W1[x_{k-1}] in two K halves, [R * gamma][2]
  const float* sts;                  // [gamma] or NULL
  int32_t* tokens;                   // [R][gamma]: column gamma - 1 (kFinAfter)
  float* conf;                       // [R][gamma]
  float* surv;                       // [R][gamma]
  const int32_t* anchors;            // kFinInStep: x_{-1} when gamma = 1
  const uint16_t* W1;                // kFinInStep: embedding rows [V][r]
  const float* w_e;                  // kFinInStep: the embedding weights [r]
  int r;                             // kFinInStep: r % 8 == 0, r <= 512
};

// Confidence, STS and survival of request m ([P1] section 二 design 2):
// c_{m,k} = sigmoid((sh + (se_0 + se_1)) / T_k), a_{m,k} = a_{m,k-1} c_{m,k} in
// fp32; also the last token.  The survivals go to `sv` (by candidate id) too.
// The loads of up to kFinBatch positions are issued before any of them is
// used, so a request costs one memory round trip per kFinBatch positions.
constexpr int kFinBatch = 8;

// `el` (kFinInStep): the last position's embedding terms, by request.
template <int FIN>
__device__ __forceinline__ void finish_request(const FinishArgs& fa, int m, int gamma,
                                               float* __restrict__ sv, const float* el) {
  int32_t last = 0;
  if constexpr (FIN == kFinAfter) last = read_token(fa.words, m, fa.S, fa.V);
  float a = 1.0f;
  for (int k0 = 0; k0 < gamma; k0 += kFinBatch) {
    float s[kFinBatch], t[kFinBatch];
#pragma unroll
    for (int j = 0; j < kFinBatch; ++j) {
      const int k = k0 + j;
      s[j] = 0.0f;
      t[j] = 1.0f;
      if (k < gamma) {
        const size_t e = (size_t)m * gamma + k;
        if (FIN == kFinInStep && k == gamma - 1)
          s[j] = fa.sh[e] + el[m];
        else
          s[j] = fa.sh[e] + (fa.se[2 * e] + fa.se[2 * e + 1]);
        if (fa.sts) t[j] = fa.sts[k];
      }
    }
#pragma unroll
    for (int j = 0; j < kFinBatch; ++j) {
      const int k = k0 + j;
      if (k < gamma) {
        const size_t e = (size_t)m * gamma + k;
        const float c = 1.0f / (1.0f + expf(-(s[j] / t[j])));
        fa.conf[e] = c;
        a = k == 0 ? c : a * c;
        fa.surv[e] = a;
        if (sv) sv[e] = a;
      }
    }
  }
  if constexpr (FIN == kFinAfter) fa.tokens[(size_t)m * gamma + gamma - 1] = last;
}

// kFinInStep: the last position's embedding term of every request,
// w_e . W1[x_{gamma-2}] (x_{-1} = the anchor), NaN for an invalid id.  First
// every token into xs (one thread per request), then per wavefront eight
// requests at a time: lane l multiplies piece l (8 entries) of the row, one
// 16-byte load, and the wavefront sums in a fixed order.  Every load reads a
// valid address (row 0 and piece 0 stand in for an invalid id and for lanes
// past r / 8) and is replaced by zeros after all eight are issued, so the
// eight are in flight together.  el may share xs's storage: a wavefront reads
// the ids of its eight requests before it writes their terms, and no other
// wavefront touches them.
template <int NW>
__device__ void last_embedding(const FinishArgs& fa, int R, int gamma, int* xs, float* el) {
  constexpr int NT = 64 * NW;
  constexpr int kB = 8;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int m = threadIdx.x; m < R; m += NT) {
    int x;
    if (gamma == 1) {
      const int a = fa.anchors[m];
      x = (a >= 0 && a < fa.V) ? a : -1;
    } else {
      x = read_token(fa.words, m, fa.S, fa.V);
    }
    xs[m] = x;
  }
  __syncthreads();
  const bool lok = lane < fa.r / 8;
  const int pl = lok ? lane : 0;
  const float4 e0 = reinterpret_cast<const float4*>(fa.w_e)[2 * pl];
  const float4 e1 = reinterpret_cast<const float4*>(fa.w_e)[2 * pl + 1];
  const float we[8] = {lok ? e0.x : 0.0f, lok ? e0.y : 0.0f, lok ? e0.z : 0.0f,
                       lok ? e0.w : 0.0f, lok ? e1.x : 0.0f, lok ? e1.y : 0.0f,
                       lok ? e1.z : 0.0f, lok ? e1.w : 0.0f};
  for (int m0 = w * kB; m0 < R; m0 += NW * kB) {
    int xm[kB];
    uint4 v[kB];
#pragma unroll
    for (int j = 0; j < kB; ++j) xm[j] = m0 + j < R ? xs[m0 + j] : -1;
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const size_t row = xm[j] >= 0 ? (size_t)xm[j] : 0;
      v[j] = *reinterpret_cast<const uint4*>(fa.W1 + row * fa.r + (size_t)pl * 8);
    }
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const bool ok = lok && xm[j] >= 0;
      const uint32_t u[4] = {ok ? v[j].x : 0u, ok ? v[j].y : 0u, ok ? v[j].z : 0u,
                             ok ? v[j].w : 0u};
      float t = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        t = fmaf(we[2 * q], __uint_as_float(u[q] << 16), t);
        t = fmaf(we[2 * q + 1], __uint_as_float(u[q] & 0xffff0000u), t);
      }
      const float tot = __uint_as_float(lane_u32(wave_iscan(__float_as_uint(t), 0u, AddF32{}), 63));
      if (lane == 0 && m0 + j < R) el[m0 + j] = xm[j] >= 0 ? tot : NAN;
    }
  }
  __syncthreads();
}

// LDS bytes of the single-tile schedule with NW wavefronts of ITEMS each.
template <int ITEMS, int NW>
constexpr size_t sched_lds_bytes() {
  return sizeof(SchedSharedT<NW>) + (size_t)64 * NW * ITEMS * 8;
}

// The single-tile schedule (N <= 64 NW ITEMS) for one workgroup of NW
// wavefronts, with sched_lds_bytes<ITEMS, NW>() bytes of LDS at smem_raw.
// FIN: see FinishArgs.
template <int ITEMS, int FIN, int NW>
__device__ void schedule_lds_body(unsigned char* smem_raw, const float* __restrict__ surv,
                                  const float* __restrict__ sps, int R, int gamma, int N, int mode,
                                  int m_cap, int32_t* __restrict__ lengths,
                                  int32_t* __restrict__ order, dspark_schedule_info* info,
                                  const FinishArgs& fa) {
  constexpr int NT = 64 * NW;
  SchedSharedT<NW>& sh = *reinterpret_cast<SchedSharedT<NW>*>(smem_raw);
  uint32_t* skey = reinterpret_cast<uint32_t*>(smem_raw + sizeof(SchedSharedT<NW>));
  int* sid = reinterpret_cast<int*>(skey + NT * ITEMS);

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  // Fused draft step: the survivals are made here first (one thread per
  // request), into the key area of LDS.  Inside the last step, the last
  // position's embedding terms go to the id area first.
  const float* sv = surv;
  if constexpr (FIN != kFinNone) {
    float* el = reinterpret_cast<float*>(sid);
    if constexpr (FIN == kFinInStep) last_embedding<NW>(fa, R, gamma, sid, el);
    float* svl = reinterpret_cast<float*>(skey);
    for (int m = threadIdx.x; m < R; m += NT) finish_request<FIN>(fa, m, gamma, svl, el);
    __syncthreads();
    sv = svl;
  }
  // striped arrangement: wave w owns [w*64*ITEMS, (w+1)*64*ITEMS), item-major inside
  uint32_t ck[ITEMS];
  int id[ITEMS];
  bool ok[ITEMS];
  int rk[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int e = w * 64 * ITEMS + i * 64 + lane;
    ok[i] = e < N;
    ck[i] = ok[i] ? key_of(sv[e]) : 0xffffffffu;
    id[i] = e;
  }
  if constexpr (FIN != kFinNone) __syncthreads();   // the keys are read before the sort reuses the area
  // The SPS entries of this thread's sorted positions, fetched now so that the
  // latency hides behind the sort.
  float spv[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int p = threadIdx.x * ITEMS + i;
    spv[i] = (p < N && mode != 2) ? sps[R + p] : 0.0f;
  }
  const float sps0 = (mode == 0 && threadIdx.x == 0) ? sps[R - 1] : 0.0f;
  // Per pass four barriers: after the ranking, after the per-digit wave
  // prefixes, after the digit scan, after the scatter.  The reload of the next
  // pass's keys needs none after it: every wave's next scatter waits behind
  // that pass's first barrier, and each wave only touches its own counter row
  // between barriers.
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 8 * pass;
    zero_my_counters(sh);
    rank_items<ITEMS>(sh, ck, ok, shift, rk);
    __syncthreads();
    wave_prefix_and_totals(sh);
    __syncthreads();
    scan_digits(sh, sh.tot);   // base[d]: items with a smaller digit
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      if (ok[i]) {
        const int d = (ck[i] >> shift) & 0xff;
        const int dst = sh.base[d] + sh.cnt[w * kDig + d] + rk[i];
        skey[dst] = ck[i];
        sid[dst] = id[i];
      }
    }
    __syncthreads();
    if (pass < 3) {
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const int e = w * 64 * ITEMS + i * 64 + lane;
        if (ok[i]) {
          ck[i] = skey[e];
          id[i] = sid[e];
        }
      }
    }
  }
  Best best;
  scan_theta<ITEMS>(
      sh, N, R, sps, sps0, mode, m_cap, order,
      [&](int p, uint32_t& k, int& i) { k = skey[p]; i = sid[p]; },
      [&](int i, int p) { sid[i] = p; }, [&](int, int i) { return spv[i]; }, best);
  write_results<NT>(R, gamma, best, sid, lengths, info);
}

}  // namespace
}  // namespace dspark
