// Hardware-aware prefix scheduler for CDNA4 (gfx950).
//
// [P1] section 二 design 2 (objective Theta = tau * SPS(B) with B = sum (1 + l_r),
// tau = sum (1 + sum_{j<=l_r} a_{r,j}); candidates sorted globally by survival)
// and section 三 challenge 2 (no early stop: every budget is evaluated).
//
// One workgroup of 1024 threads (16 wavefronts) does the whole schedule in a
// single launch, so the call costs one dispatch whatever the batch:
//   1. keys: the fp32 bit pattern of a (non-negative, so monotone in a),
//      complemented so that an ascending sort gives descending survival;
//   2. stable LSD radix sort, 4 passes of 8 bits.  Within a tile each wavefront
//      ranks its elements with ballot-based peer matching (8 ballots per item),
//      keeping per-wave digit counters in LDS; digit offsets are prefix sums
//      over (digit, wave), which keeps equal keys in id order;
//   3. exact fixed-point prefix sums q = rint(a * 2^40) (uint64) in sorted
//      order, Theta for every budget in fp64, first argmax;
//   4. inverse permutation, then l_r = #{j : rank(r, j) < m*}.
// Up to 16384 candidates the tile lives in LDS (one tile, no global traffic);
// beyond that the sort ping-pongs between two workspace buffers, tile by tile,
// with a per-pass digit histogram giving the global digit offsets.
#include "dspark_internal.h"

namespace dspark {
namespace {

constexpr int kT = 1024;          // threads
constexpr int kW = kT / 64;       // wavefronts
constexpr int kDig = 256;         // radix digits per pass
constexpr int kTileItems = 16;    // items per thread in a tile of the global path
constexpr int kTile = kT * kTileItems;
constexpr double kTauScale = 1099511627776.0;       // 2^40
constexpr double kTauInv = 1.0 / 1099511627776.0;   // 2^-40

struct SchedShared {
  int cnt[kW * kDig];        // per-wave digit counters, then offsets
  int base[kDig];            // running global digit offsets
  int tot[kDig];             // digit totals
  unsigned long long wsum[kW];
  double bval[kW];
  int bidx[kW];
  unsigned long long bsum[kW];
  unsigned long long carry;
};

__device__ __forceinline__ uint32_t key_of(float a) {
  // canonical non-negative bits (-0 -> +0), complemented: ascending = descending a
  return ~(__float_as_uint(a) & 0x7fffffffu);
}

__device__ __forceinline__ float value_of(uint32_t ck) { return __uint_as_float(~ck); }

// Exclusive scan of the 256 digit totals tot[] into base[] (wave 0 does the work).
__device__ void scan_digits(SchedShared& sh, const int* tot) {
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
    int inc = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(inc, off);
      if (lane >= off) inc += o;
    }
    const int ex = inc - s;
#pragma unroll
    for (int j = 0; j < 4; ++j) sh.base[lane * 4 + j] = ex + v[j];
  }
}

// Rank this wave's ITEMS elements by digit; rk[i] = rank among equal digits of
// this wave in (item, lane) order.  cnt row of this wave must be zero on entry.
template <int ITEMS>
__device__ __forceinline__ void rank_items(SchedShared& sh, const uint32_t (&ck)[ITEMS],
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

// Turn per-wave counters into scatter offsets: cnt[w][d] = base[d] + sum_{w'<w} cnt[w'][d];
// then advance base[d] by the tile's total of digit d.  Threads 0..255.
__device__ __forceinline__ void offsets_from_base(SchedShared& sh) {
  if (threadIdx.x < kDig) {
    const int d = threadIdx.x;
    int run = sh.base[d];
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      const int c = sh.cnt[w * kDig + d];
      sh.cnt[w * kDig + d] = run;
      run += c;
    }
    sh.base[d] = run;
  }
}

__device__ __forceinline__ void zero_my_counters(SchedShared& sh) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < kDig / 64; ++j) sh.cnt[w * kDig + lane + 64 * j] = 0;
}

// Block-wide exclusive scan of one uint64 per thread; returns the exclusive
// prefix and adds the block total to sh.carry (after the call, all threads see
// the old carry in `carry_in`).
__device__ __forceinline__ unsigned long long block_exscan_u64(SchedShared& sh,
                                                               unsigned long long v,
                                                               unsigned long long& carry_in) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  unsigned long long inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  if (lane == 63) sh.wsum[w] = inc;
  __syncthreads();
  unsigned long long before = 0;
  unsigned long long total = 0;
#pragma unroll
  for (int j = 0; j < kW; ++j) {
    const unsigned long long s = sh.wsum[j];
    if (j < w) before += s;
    total += s;
  }
  carry_in = sh.carry;
  __syncthreads();
  if (threadIdx.x == 0) sh.carry = carry_in + total;
  return before + inc - v;
}

struct Best {
  double theta;
  int m;
  unsigned long long S;   // fixed-point prefix sum at m
};

__device__ __forceinline__ void better(Best& b, const Best& o) {
  if (o.theta > b.theta || (o.theta == b.theta && o.m < b.m)) b = o;
}

// Phase 3 + 4 for a sorted array (keys ck, ids) given in blocked chunks.
// load(p, ck, id) fetches the element at sorted position p.
template <int ITEMS, typename Load, typename SetRank>
__device__ void scan_theta(SchedShared& sh, int N, int R, const float* __restrict__ sps,
                           int32_t* __restrict__ order, Load load, SetRank set_rank,
                           Best& best) {
  const int tid = threadIdx.x;
  if (tid == 0) sh.carry = 0ull;
  best.theta = -1.0;
  best.m = 0x7fffffff;
  best.S = 0ull;
  if (tid == 0) {
    best.theta = (double)R * (double)sps[R - 1];  // m = 0: tau = R
    best.m = 0;
  }
  __syncthreads();
  const unsigned long long rfx = (unsigned long long)R << 40;
  for (int c0 = 0; c0 < N; c0 += kT * ITEMS) {
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
        const double tau = __ull2double_rn(rfx + S) * kTauInv;
        const double th = tau * (double)sps[R + p];   // budget B = R + p + 1
        if (th > best.theta) {
          best.theta = th;
          best.m = p + 1;
          best.S = S;
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
  // block argmax (largest Theta, smallest m)
  const int lane = tid & 63;
  const int w = tid >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    Best o;
    o.theta = __shfl_xor(best.theta, off);
    o.m = __shfl_xor(best.m, off);
    o.S = __shfl_xor(best.S, off);
    better(best, o);
  }
  if (lane == 0) {
    sh.bval[w] = best.theta;
    sh.bidx[w] = best.m;
    sh.bsum[w] = best.S;
  }
  __syncthreads();
  best = Best{sh.bval[0], sh.bidx[0], sh.bsum[0]};
#pragma unroll
  for (int j = 1; j < kW; ++j) better(best, Best{sh.bval[j], sh.bidx[j], sh.bsum[j]});
}

__device__ void write_results(int R, int gamma, const Best& best, const int* rank,
                              int32_t* __restrict__ lengths, dspark_schedule_info* info) {
  const int m_star = best.m;
  for (int r = threadIdx.x; r < R; r += kT) {
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
template <int ITEMS>
__global__ __launch_bounds__(kT) void schedule_lds_kernel(const float* __restrict__ surv,
                                                          const float* __restrict__ sps, int R,
                                                          int gamma, int N,
                                                          int32_t* __restrict__ lengths,
                                                          int32_t* __restrict__ order,
                                                          dspark_schedule_info* info) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  SchedShared& sh = *reinterpret_cast<SchedShared*>(smem_raw);
  uint32_t* skey = reinterpret_cast<uint32_t*>(smem_raw + sizeof(SchedShared));
  int* sid = reinterpret_cast<int*>(skey + kT * ITEMS);

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  // striped arrangement: wave w owns [w*64*ITEMS, (w+1)*64*ITEMS), item-major inside
  uint32_t ck[ITEMS];
  int id[ITEMS];
  bool ok[ITEMS];
  int rk[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int e = w * 64 * ITEMS + i * 64 + lane;
    ok[i] = e < N;
    ck[i] = ok[i] ? key_of(surv[e]) : 0xffffffffu;
    id[i] = e;
  }
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 8 * pass;
    zero_my_counters(sh);
    rank_items<ITEMS>(sh, ck, ok, shift, rk);
    __syncthreads();
    // digit totals -> exclusive digit bases (single tile: the tile is the array)
    if (threadIdx.x < kDig) {
      int t = 0;
#pragma unroll
      for (int ww = 0; ww < kW; ++ww) t += sh.cnt[ww * kDig + threadIdx.x];
      sh.tot[threadIdx.x] = t;
    }
    __syncthreads();
    scan_digits(sh, sh.tot);
    __syncthreads();
    offsets_from_base(sh);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      if (ok[i]) {
        const int d = (ck[i] >> shift) & 0xff;
        const int dst = sh.cnt[w * kDig + d] + rk[i];
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
      __syncthreads();
    }
  }
  Best best;
  scan_theta<ITEMS>(
      sh, N, R, sps, order, [&](int p, uint32_t& k, int& i) { k = skey[p]; i = sid[p]; },
      [&](int i, int p) { sid[i] = p; }, best);
  write_results(R, gamma, best, sid, lengths, info);
}

// ---------------------------------------------------------------------------
// Global path: any N, tiles of kTile elements, ping-pong in workspace.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kT) void schedule_global_kernel(
    const float* __restrict__ surv, const float* __restrict__ sps, int R, int gamma, int N,
    uint32_t* __restrict__ k0, int* __restrict__ i0, uint32_t* __restrict__ k1,
    int* __restrict__ i1, int* __restrict__ rank, int32_t* __restrict__ lengths,
    int32_t* __restrict__ order, dspark_schedule_info* info) {
  __shared__ SchedShared sh;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < N; e += kT) {
    k0[e] = key_of(surv[e]);
    i0[e] = e;
  }
  __syncthreads();
  uint32_t* sk = k0;
  int* si = i0;
  uint32_t* dk = k1;
  int* di = i1;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 8 * pass;
    // digit histogram of the whole array (per-wave counters, ballot-aggregated)
    zero_my_counters(sh);
    for (int t0 = 0; t0 < N; t0 += kTile) {
      uint32_t ck[kTileItems];
      bool ok[kTileItems];
      int rk[kTileItems];
#pragma unroll
      for (int i = 0; i < kTileItems; ++i) {
        const int e = t0 + w * 64 * kTileItems + i * 64 + lane;
        ok[i] = e < N;
        ck[i] = ok[i] ? sk[e] : 0xffffffffu;
      }
      rank_items<kTileItems>(sh, ck, ok, shift, rk);
    }
    __syncthreads();
    if (threadIdx.x < kDig) {
      int t = 0;
#pragma unroll
      for (int ww = 0; ww < kW; ++ww) t += sh.cnt[ww * kDig + threadIdx.x];
      sh.tot[threadIdx.x] = t;
    }
    __syncthreads();
    scan_digits(sh, sh.tot);
    __syncthreads();
    for (int t0 = 0; t0 < N; t0 += kTile) {
      uint32_t ck[kTileItems];
      int id[kTileItems];
      bool ok[kTileItems];
      int rk[kTileItems];
      zero_my_counters(sh);
#pragma unroll
      for (int i = 0; i < kTileItems; ++i) {
        const int e = t0 + w * 64 * kTileItems + i * 64 + lane;
        ok[i] = e < N;
        ck[i] = ok[i] ? sk[e] : 0xffffffffu;
        id[i] = ok[i] ? si[e] : -1;
      }
      rank_items<kTileItems>(sh, ck, ok, shift, rk);
      __syncthreads();
      offsets_from_base(sh);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kTileItems; ++i) {
        if (ok[i]) {
          const int d = (ck[i] >> shift) & 0xff;
          const int dst = sh.cnt[w * kDig + d] + rk[i];
          dk[dst] = ck[i];
          di[dst] = id[i];
        }
      }
      __syncthreads();
    }
    uint32_t* tk = sk; sk = dk; dk = tk;
    int* ti = si; si = di; di = ti;
  }
  Best best;
  scan_theta<kTileItems>(
      sh, N, R, sps, order, [&](int p, uint32_t& k, int& i) { k = sk[p]; i = si[p]; },
      [&](int i, int p) { rank[i] = p; }, best);
  write_results(R, gamma, best, rank, lengths, info);
}

template <int ITEMS>
dspark_status launch_lds(const float* surv, const float* sps, int R, int gamma, int N,
                         int32_t* lengths, int32_t* order, dspark_schedule_info* info,
                         hipStream_t stream) {
  const size_t lds = sizeof(SchedShared) + (size_t)kT * ITEMS * 8;
  static bool attr = false;
  if (!attr) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&schedule_lds_kernel<ITEMS>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return fail(DSPARK_EDEVICE, "hipFuncSetAttribute failed for the schedule kernel");
    attr = true;
  }
  hipLaunchKernelGGL(schedule_lds_kernel<ITEMS>, dim3(1), dim3(kT), lds, stream, surv, sps, R,
                     gamma, N, lengths, order, info);
  return check_launch("schedule_lds_kernel");
}

}  // namespace

size_t schedule_workspace_bytes(int R, int gamma) {
  const size_t N = (size_t)R * (size_t)gamma;
  if (N <= (size_t)kTile) return 256;
  return 5 * N * sizeof(int32_t) + 256;
}

dspark_status launch_schedule(const float* surv, const float* sps, int R, int gamma,
                              int32_t* lengths, int32_t* order, dspark_schedule_info* info,
                              void* workspace, hipStream_t stream) {
  const int N = R * gamma;
  if (N <= kT * 1) return launch_lds<1>(surv, sps, R, gamma, N, lengths, order, info, stream);
  if (N <= kT * 2) return launch_lds<2>(surv, sps, R, gamma, N, lengths, order, info, stream);
  if (N <= kT * 4) return launch_lds<4>(surv, sps, R, gamma, N, lengths, order, info, stream);
  if (N <= kT * 8) return launch_lds<8>(surv, sps, R, gamma, N, lengths, order, info, stream);
  if (N <= kT * 16) return launch_lds<16>(surv, sps, R, gamma, N, lengths, order, info, stream);
  int* ws = reinterpret_cast<int*>(workspace);
  uint32_t* k0 = reinterpret_cast<uint32_t*>(ws);
  int* i0 = ws + N;
  uint32_t* k1 = reinterpret_cast<uint32_t*>(ws + 2 * (size_t)N);
  int* i1 = ws + 3 * (size_t)N;
  int* rank = ws + 4 * (size_t)N;
  hipLaunchKernelGGL(schedule_global_kernel, dim3(1), dim3(kT), 0, stream, surv, sps, R, gamma,
                     N, k0, i0, k1, i1, rank, lengths, order, info);
  return check_launch("schedule_global_kernel");
}

}  // namespace dspark
