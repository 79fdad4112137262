// Hardware-aware prefix scheduler for CDNA4 (gfx950).
//
// [P1] section 二 design 2 (objective Theta = tau * SPS(B) with B = sum (1 + l_r),
// tau = sum (1 + sum_{j<=l_r} a_{r,j}); candidates sorted globally by survival)
// and section 三 challenge 2 (no early stop: every budget is evaluated).
//
// Steps (both paths):
//   1. keys: the fp32 bit pattern of a (non-negative, so monotone in a),
//      complemented so that an ascending sort gives descending survival;
//   2. stable LSD radix sort, 4 passes of 8 bits.  Within a tile each wavefront
//      ranks its elements with ballot-based peer matching (8 ballots per item),
//      keeping per-wave digit counters in LDS; digit offsets are prefix sums
//      over (digit, wave), which keeps equal keys in id order;
//   3. exact fixed-point prefix sums q = rint(a * 2^40) (uint64) in sorted
//      order, Theta for every budget in fp64, first argmax;
//   4. l_r = #{j : rank(r, j) < m*}.
// Up to 8192 candidates one workgroup of 1024 threads (16 wavefronts) does it
// all in LDS in a single launch.  Beyond that the sort and the scan are spread
// over tiles of 1024 candidates on the whole device through workspace buffers
// (eleven short launches, no host sync).
#include <math.h>

#include <atomic>

#include "dspark_internal.h"
#include "packed_words.h"
#include "sched_lds.h"

namespace dspark {
namespace {

template <int ITEMS, int FIN>
__global__ __launch_bounds__(kT) void schedule_lds_kernel(const float* __restrict__ surv,
                                                          const float* __restrict__ sps, int R,
                                                          int gamma, int N, int mode,
                                                          int m_cap,
                                                          int32_t* __restrict__ lengths,
                                                          int32_t* __restrict__ order,
                                                          dspark_schedule_info* info,
                                                          FinishArgs fa) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  schedule_lds_body<ITEMS, FIN, kW>(smem_raw, surv, sps, R, gamma, N, mode, m_cap, lengths, order,
                                    info, fa);
}

// ---------------------------------------------------------------------------
// Global path (N > 8192): the same stable LSD radix sort spread over the
// device, then the scan spread over the same tiles.  Per 8-bit pass:
//   hist:    each workgroup counts the digits of its tile of kGTile candidates;
//   scatter: each workgroup derives its tile's base of every digit from all the
//            counts (or, with many tiles, reads it from one separate scan), ranks
//            its tile stably (the ballot ranking of the single-tile path) and
//            writes keys and ids to their places.
// Then: per tile, the sum of its fixed-point survivals (this launch also
// clears the lengths); per tile, the carry of the tiles before it, the prefix
// sums, Theta at each position and the tile's best; then one launch in which
// every workgroup takes m* from the tiles' results and counts its positions
// below m* into the lengths.  Eleven launches (one more beyond 512 tiles, for
// the digit scans), all on the caller's stream, no host sync.
// ---------------------------------------------------------------------------
constexpr int kGT = 256;                  // threads of a sort workgroup
constexpr int kGW = kGT / 64;
constexpr int kGItems = 4;
constexpr int kGTile = kGT * kGItems;     // candidates per tile
constexpr int kHistBatch = 32;            // tile counts a scatter thread has in flight
static_assert(kGT == kDig, "one thread per digit in the tile kernels");

__device__ __forceinline__ int tile_elem(int t, int w, int i, int lane) {
  return t * kGTile + w * 64 * kGItems + i * 64 + lane;   // (wave, item, lane) order
}

// Digit counts and bases are kept tile-major: hist[t * 256 + d].
template <bool FIRST>
__global__ __launch_bounds__(kGT) void sched_hist_kernel(const float* __restrict__ surv,
                                                         const uint32_t* __restrict__ keys,
                                                         int N, int shift,
                                                         int* __restrict__ hist) {
  __shared__ int h[kDig];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  h[threadIdx.x] = 0;
  // Every item's key is loaded before the first count (items past N read
  // element 0 and are not counted), so the loads are in flight together
  // rather than one round trip each.
  uint32_t k[kGItems];
  bool ok[kGItems];
#pragma unroll
  for (int i = 0; i < kGItems; ++i) {
    const int e = tile_elem(t, w, i, lane);
    ok[i] = e < N;
    const int ec = ok[i] ? e : 0;
    k[i] = FIRST ? key_of(surv[ec]) : keys[ec];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kGItems; ++i)
    if (ok[i]) atomicAdd(&h[(k[i] >> shift) & 0xff], 1);
  __syncthreads();
  hist[t * kDig + threadIdx.x] = h[threadIdx.x];
}

// Exclusive scan, in place, of the tile-major counts taken in (digit, tile)
// order: one workgroup, chunks of 4 * kT with carry.  Used when there are too
// many tiles for each scatter workgroup to derive its bases itself.
__global__ __launch_bounds__(kT) void sched_scan_kernel(int* __restrict__ a, int ntiles) {
  __shared__ int wtot[kW];
  __shared__ int carry;
  const int M = kDig * ntiles;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  auto at = [&](int k) -> int& { return a[(k % ntiles) * kDig + k / ntiles]; };
  if (t == 0) carry = 0;
  __syncthreads();
  for (int c0 = 0; c0 < M; c0 += 4 * kT) {
    const int b = c0 + 4 * t;
    int v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = b + j < M ? at(b + j) : 0;
    const int s = v[0] + v[1] + v[2] + v[3];
    int inc = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(inc, off);
      if (lane >= off) inc += o;
    }
    if (lane == 63) wtot[w] = inc;
    __syncthreads();
    int pre = carry, total = 0;
#pragma unroll
    for (int j = 0; j < kW; ++j) {
      pre += j < w ? wtot[j] : 0;
      total += wtot[j];
    }
    int run = pre + inc - s;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (b + j < M) at(b + j) = run;
      run += v[j];
    }
    __syncthreads();
    if (t == 0) carry += total;
    __syncthreads();
  }
}

// Tiles up to which a scatter workgroup derives its own digit bases from the
// counts (one coalesced row per tile) instead of a separate scan launch.
constexpr int kInlineTiles = 512;

// Stable scatter of tile t for the digit at `shift`.  INLINE: `hist` holds the
// counts of this pass and the bases are derived here; else it holds the bases.
template <bool FIRST, bool INLINE>
__global__ __launch_bounds__(kGT) void sched_scatter_kernel(
    const float* __restrict__ surv, const uint32_t* __restrict__ sk, const int* __restrict__ si,
    uint32_t* __restrict__ dk, int* __restrict__ di, int N, int shift, int ntiles,
    const int* __restrict__ hist) {
  __shared__ SchedShared sh;              // uses the first kGW rows of the counters
  __shared__ int wtot[kGW];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int d = threadIdx.x;              // kGT == kDig: one thread per digit below
  uint32_t ck[kGItems];
  int id[kGItems];
  bool ok[kGItems];
  int rk[kGItems];
  // Loads without branches (items past N read element 0, then take the
  // padding key), so they are in flight together.
#pragma unroll
  for (int i = 0; i < kGItems; ++i) {
    const int e = tile_elem(t, w, i, lane);
    ok[i] = e < N;
    const int ec = ok[i] ? e : 0;
    const uint32_t kv = FIRST ? key_of(surv[ec]) : sk[ec];
    const int iv = FIRST ? e : si[ec];
    ck[i] = ok[i] ? kv : 0xffffffffu;
    id[i] = ok[i] ? iv : -1;
  }
  // This tile's global base of digit d.
  int base;
  if (INLINE) {
    // The counts of every tile for digit d: kHistBatch loads in flight at a
    // time (tiles past the last read the last one and add nothing).
    int total = 0, pre = 0;
    for (int c0 = 0; c0 < ntiles; c0 += kHistBatch) {
      int hv[kHistBatch];
#pragma unroll
      for (int j = 0; j < kHistBatch; ++j)
        hv[j] = hist[min(c0 + j, ntiles - 1) * kDig + d];
#pragma unroll
      for (int j = 0; j < kHistBatch; ++j) {
        const int t2 = c0 + j;
        const int h = t2 < ntiles ? hv[j] : 0;
        total += h;
        pre += t2 < t ? h : 0;
      }
    }
    // exclusive scan of the digit totals over the 256 threads
    int inc = total;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(inc, off);
      if (lane >= off) inc += o;
    }
    if (lane == 63) wtot[w] = inc;
    __syncthreads();
    int dpre = inc - total;
#pragma unroll
    for (int j = 0; j < kGW; ++j) dpre += j < w ? wtot[j] : 0;
    base = dpre + pre;
  } else {
    base = hist[t * kDig + d];
  }
  zero_my_counters(sh);
  rank_items<kGItems>(sh, ck, ok, shift, rk);
  __syncthreads();
  {   // per digit: the tile's base, then the waves in order
    int run = base;
#pragma unroll
    for (int ww = 0; ww < kGW; ++ww) {
      const int c = sh.cnt[ww * kDig + d];
      sh.cnt[ww * kDig + d] = run;
      run += c;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kGItems; ++i) {
    if (ok[i]) {
      const int dg = (ck[i] >> shift) & 0xff;
      const int dst = sh.cnt[w * kDig + dg] + rk[i];
      dk[dst] = ck[i];
      di[dst] = id[i];
    }
  }
}

// The fixed-point scan and Theta over the sorted candidates, by tiles of kGTile
// positions (thread: four consecutive positions, 16-byte loads when aligned).
__device__ __forceinline__ void load4_sorted(const uint32_t* sk, const int* si, int N, int p0,
                                             bool vec, uint32_t (&ck)[4], int (&id)[4]) {
  if (vec && p0 + 3 < N) {
    const uint4 k4 = *reinterpret_cast<const uint4*>(sk + p0);
    const int4 i4 = *reinterpret_cast<const int4*>(si + p0);
    ck[0] = k4.x; ck[1] = k4.y; ck[2] = k4.z; ck[3] = k4.w;
    id[0] = i4.x; id[1] = i4.y; id[2] = i4.z; id[3] = i4.w;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool in = p0 + i < N;
      ck[i] = in ? sk[p0 + i] : 0xffffffffu;
      id[i] = in ? si[p0 + i] : -1;
    }
  }
}

__device__ __forceinline__ unsigned long long qfx(uint32_t ck) {
  return __double2ull_rn((double)value_of(ck) * kTauScale);
}

// Block sum of one uint64 per thread (kGT threads); every thread gets it.
__device__ __forceinline__ unsigned long long block_sum_u64(unsigned long long* red,
                                                            unsigned long long v) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  if (lane == 0) red[w] = v;
  __syncthreads();
  unsigned long long s = 0;
#pragma unroll
  for (int j = 0; j < kGW; ++j) s += red[j];
  return s;
}

// Per tile: the sum of its fixed-point survivals.
__global__ __launch_bounds__(kGT) void sched_tsum_kernel(const uint32_t* __restrict__ sk,
                                                         const int* __restrict__ si, int N,
                                                         unsigned long long* __restrict__ tsum,
                                                         int R, int32_t* __restrict__ lengths) {
  __shared__ unsigned long long red[kGW];
  // The lengths the finishing kernel counts into start at zero.
  for (int r = blockIdx.x * kGT + threadIdx.x; r < R; r += gridDim.x * kGT) lengths[r] = 0;
  const int p0 = blockIdx.x * kGTile + 4 * threadIdx.x;
  auto a16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
  uint32_t ck[4];
  int id[4];
  load4_sorted(sk, si, N, p0, a16(sk) && a16(si), ck, id);
  unsigned long long v = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) v += p0 + i < N ? qfx(ck[i]) : 0ull;
  v = block_sum_u64(red, v);
  if (threadIdx.x == 0) tsum[blockIdx.x] = v;
}

// Per tile: carry from the tiles before it, local scan, Theta at every position
// of the tile, the tile's best (largest Theta, smallest m); writes order.
struct TileBest {
  double theta;
  int m;
  int pad;
  unsigned long long S;
};

__global__ __launch_bounds__(kGT) void sched_tscan_kernel(
    const uint32_t* __restrict__ sk, const int* __restrict__ si, const float* __restrict__ sps,
    int R, int N, const unsigned long long* __restrict__ tsum, int32_t* __restrict__ order,
    TileBest* __restrict__ tbest) {
  __shared__ unsigned long long red[kGW];
  __shared__ double bth[kGW];
  __shared__ int bm[kGW];
  __shared__ unsigned long long bs[kGW];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int p0 = t * kGTile + 4 * tid;
  auto a16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
  // carry: sum of the tiles before this one (threads split the tiles)
  unsigned long long c = 0;
  for (int t2 = tid; t2 < t; t2 += kGT) c += tsum[t2];
  const unsigned long long carry = block_sum_u64(red, c);
  __syncthreads();
  uint32_t ck[4];
  int id[4];
  load4_sorted(sk, si, N, p0, a16(sk) && a16(si), ck, id);
  float sv[4];
  if (a16(sps + R) && p0 + 3 < N) {
    const float4 s4 = *reinterpret_cast<const float4*>(sps + R + p0);
    sv[0] = s4.x; sv[1] = s4.y; sv[2] = s4.z; sv[3] = s4.w;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = p0 + i < N ? sps[R + p0 + i] : 0.0f;
  }
  unsigned long long q[4];
  unsigned long long s4 = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    q[i] = p0 + i < N ? qfx(ck[i]) : 0ull;
    s4 += q[i];
  }
  // exclusive scan of s4 over the tile
  unsigned long long inc = s4;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  if (lane == 63) red[w] = inc;
  __syncthreads();
  unsigned long long S = carry + inc - s4;
#pragma unroll
  for (int j = 0; j < kGW; ++j) S += j < w ? red[j] : 0ull;
  const unsigned long long rfx = (unsigned long long)R << 40;
  Best best{-1.0, 0x7fffffff, 0ull};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = p0 + i;
    if (p < N) {
      S += q[i];
      const double th = __ull2double_rn(rfx + S) * kTauInv * (double)sv[i];
      if (th > best.theta) best = Best{th, p + 1, S};
    }
  }
  if (order) {
    if (a16(order) && p0 + 3 < N) {
      *reinterpret_cast<int4*>(order + p0) = make_int4(id[0], id[1], id[2], id[3]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (p0 + i < N) order[p0 + i] = id[i];
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    Best o;
    o.theta = __shfl_xor(best.theta, off);
    o.m = __shfl_xor(best.m, off);
    o.S = __shfl_xor(best.S, off);
    better(best, o);
  }
  if (lane == 0) {
    bth[w] = best.theta;
    bm[w] = best.m;
    bs[w] = best.S;
  }
  __syncthreads();
  if (tid == 0) {
#pragma unroll
    for (int j = 1; j < kGW; ++j) better(best, Best{bth[j], bm[j], bs[j]});
    tbest[t] = TileBest{best.theta, best.m, 0, best.S};
  }
}

// Early stop / capacity over tiles: per tile, the carry, the prefix sums and
// (early stop) the first position p whose Theta_{p+1} does not exceed
// Theta_p; writes order.  tbrk[t] = that position or INT_MAX.
__global__ __launch_bounds__(kGT) void sched_tbreak_kernel(
    const uint32_t* __restrict__ sk, const int* __restrict__ si, const float* __restrict__ sps,
    int R, int N, int mode, const unsigned long long* __restrict__ tsum,
    int32_t* __restrict__ order, int* __restrict__ tbrk) {
  __shared__ unsigned long long red[kGW];
  __shared__ int bmin[kGW];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int p0 = t * kGTile + 4 * tid;
  auto a16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
  uint32_t ck[4];
  int id[4];
  load4_sorted(sk, si, N, p0, a16(sk) && a16(si), ck, id);
  if (order) {
    if (a16(order) && p0 + 3 < N) {
      *reinterpret_cast<int4*>(order + p0) = make_int4(id[0], id[1], id[2], id[3]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (p0 + i < N) order[p0 + i] = id[i];
    }
  }
  if (mode != 1) return;   // capacity: order only (uniform per workgroup)
  unsigned long long c = 0;
  for (int t2 = tid; t2 < t; t2 += kGT) c += tsum[t2];
  const unsigned long long carry = block_sum_u64(red, c);
  __syncthreads();
  unsigned long long q[4];
  unsigned long long s4 = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    q[i] = p0 + i < N ? qfx(ck[i]) : 0ull;
    s4 += q[i];
  }
  unsigned long long inc = s4;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  if (lane == 63) red[w] = inc;
  __syncthreads();
  unsigned long long S = carry + inc - s4;
#pragma unroll
  for (int j = 0; j < kGW; ++j) S += j < w ? red[j] : 0ull;
  int brk = 0x7fffffff;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = p0 + i;
    if (p < N) {
      S += q[i];
      const double th = theta_at(R, S, sps[R + p]);
      const double th_prev = theta_at(R, S - q[i], sps[R + p - 1]);
      if (!(th > th_prev)) brk = min(brk, p);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) brk = min(brk, __shfl_xor(brk, off));
  if (lane == 0) bmin[w] = brk;
  __syncthreads();
  if (tid == 0) {
    int b = bmin[0];
#pragma unroll
    for (int j = 1; j < kGW; ++j) b = min(b, bmin[j]);
    tbrk[t] = b;
  }
}

// m* and the lengths in one launch: every workgroup takes m* from the
// per-tile results itself (one wavefront, a fixed-order reduction, so all get
// the same value), then counts its positions p < m* into l_r (cleared by the
// tile-sum kernel); workgroup 0 also writes info.
//   mode 0: the first argmax over m = 0 (tau = R) and the tiles' bests;
//   mode 1: the first break over the tiles (N if none);
//   mode 2: m_cap.
// Modes 1 and 2 take tau* from the tile sums below m*'s tile plus that tile's
// keys below m*.
__global__ __launch_bounds__(256) void sched_finish_kernel(
    const TileBest* __restrict__ tbest, const int* __restrict__ tbrk,
    const unsigned long long* __restrict__ tsum, const uint32_t* __restrict__ sk,
    const int* __restrict__ si, int ntiles, int N, int R, int gamma, int mode, int m_cap,
    const float* __restrict__ sps, dspark_schedule_info* info, int32_t* __restrict__ lengths) {
  __shared__ int s_m;
  __shared__ unsigned long long s_S;
  __shared__ double s_theta;
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int lane = tid;
    if (mode == 0) {
      Best best{-1.0, 0x7fffffff, 0ull};
      if (lane == 0) best = Best{(double)R * (double)sps[R - 1], 0, 0ull};
      for (int t = lane; t < ntiles; t += 64) better(best, Best{tbest[t].theta, tbest[t].m, tbest[t].S});
      const Best b = wave_best(best);
      if (lane == 0) {
        s_m = b.m;
        s_S = b.S;
        s_theta = b.theta;
      }
    } else {
      int m_star = m_cap;
      if (mode == 1) {
        uint32_t b = 0x7fffffffu;
        for (int t = lane; t < ntiles; t += 64) b = min(b, (uint32_t)tbrk[t]);
        m_star = (int)lane_u32(wave_iscan(b, 0x7fffffffu, MinI32{}), 63);
        if (m_star > N) m_star = N;
      }
      if (blockIdx.x == 0) {
        const int t_full = m_star / kGTile;
        unsigned long long part = 0;
        for (int t = lane; t < t_full; t += 64) part += tsum[t];
        for (int p = t_full * kGTile + lane; p < m_star; p += 64) part += qfx(sk[p]);
        const unsigned long long Sm = lane_u64(wave_iscan(part, 0ull, AddU64{}), 63);
        if (lane == 0) {
          s_S = Sm;
          s_theta = theta_at(R, Sm, mode == 1 ? sps[R + m_star - 1] : 1.0f);
        }
      }
      if (lane == 0) s_m = m_star;
    }
  }
  __syncthreads();
  const int m_star = s_m;
  if (blockIdx.x == 0 && tid == 0 && info) {
    const unsigned long long tau_fx = ((unsigned long long)R << 40) + s_S;
    info->B_star = R + m_star;
    info->m_star = m_star;
    info->tau_fx = tau_fx;
    info->tau = __ull2double_rn(tau_fx) * kTauInv;
    info->theta = s_theta;
  }
  const int p = blockIdx.x * 256 + tid;
  if (p < m_star) atomicAdd(&lengths[si[p] / gamma], 1);
}

// Fused draft step beyond the LDS path: the survivals go to memory first.
__global__ __launch_bounds__(256) void finish_kernel(FinishArgs fa, int R, int gamma) {
  const int m = blockIdx.x * 256 + threadIdx.x;
  if (m < R) finish_request<kFinAfter>(fa, m, gamma, nullptr, nullptr);
}

template <int ITEMS, int FIN>
dspark_status launch_lds(const float* surv, const float* sps, int R, int gamma, int N, int mode,
                         int m_cap, int32_t* lengths, int32_t* order, dspark_schedule_info* info,
                         const FinishArgs& fa, hipStream_t stream) {
  const size_t lds = sched_lds_bytes<ITEMS, kW>();
  // The dynamic-LDS attribute, set once per device (bit d of `done`).
  static std::atomic<unsigned long long> done{0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(DSPARK_EDEVICE, "hipGetDevice failed");
  const unsigned long long bit = dev < 64 ? 1ull << dev : 0ull;
  if (!bit || !(done.load(std::memory_order_acquire) & bit)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&schedule_lds_kernel<ITEMS, FIN>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return fail(DSPARK_EDEVICE, "hipFuncSetAttribute failed for the schedule kernel");
    done.fetch_or(bit, std::memory_order_release);
  }
  hipLaunchKernelGGL((schedule_lds_kernel<ITEMS, FIN>), dim3(1), dim3(kT), lds, stream, surv,
                     sps, R, gamma, N, mode, m_cap, lengths, order, info, fa);
  return check_launch("schedule_lds_kernel");
}

}  // namespace

// Global-path workspace: k0, i0, k1, i1, rank (Np = N rounded up to 4 each, so
// every array keeps the base's 16-byte alignment), digit counts, m*.
// Up to this many candidates the whole schedule runs in one workgroup's LDS.
constexpr int kLdsMaxN = 8192;

size_t schedule_workspace_bytes(int R, int gamma) {
  const size_t N = (size_t)R * (size_t)gamma;
  if (N <= (size_t)kLdsMaxN) return 256;
  const size_t Np = (N + 3) / 4 * 4;
  const size_t ntiles = (N + kGTile - 1) / kGTile;
  return 4 * Np * sizeof(int32_t) + (size_t)kDig * ntiles * sizeof(int32_t) +
         ntiles * (sizeof(unsigned long long) + sizeof(TileBest)) + 256;
}

// Launches of launch_schedule: one in LDS, else per pass a histogram and a
// scatter (and a digit scan beyond kInlineTiles tiles), then three.
int schedule_launch_count(int R, int gamma) {
  const long N = (long)R * gamma;
  if (N <= kLdsMaxN) return 1;
  const long ntiles = (N + kGTile - 1) / kGTile;
  return 4 * (ntiles <= kInlineTiles ? 2 : 3) + 3;
}

template <bool FIRST, bool INLINE>
void launch_scatter(int ntiles, hipStream_t stream, const float* surv, const uint32_t* sk,
                    const int* si, uint32_t* dk, int* di, int N, int shift, const int* hist) {
  hipLaunchKernelGGL((sched_scatter_kernel<FIRST, INLINE>), dim3(ntiles), dim3(kGT), 0, stream,
                     surv, sk, si, dk, di, N, shift, ntiles, hist);
}

dspark_status launch_schedule(const float* surv, const float* sps, int R, int gamma, int mode,
                              int m_cap, int32_t* lengths, int32_t* order,
                              dspark_schedule_info* info, void* workspace, hipStream_t stream) {
  const int N = R * gamma;
#define DSPARK_LDS(I) \
  launch_lds<I, kFinNone>(surv, sps, R, gamma, N, mode, m_cap, lengths, order, info, FinishArgs{}, stream)
  if (N <= kT * 1) return DSPARK_LDS(1);
  if (N <= kT * 2) return DSPARK_LDS(2);
  if (N <= kT * 4) return DSPARK_LDS(4);
  static_assert(kLdsMaxN == kT * 8, "the largest LDS variant covers kLdsMaxN");
  if (N <= kT * 8) return DSPARK_LDS(8);
#undef DSPARK_LDS
  // Workspace: keys and ids twice (Np each, so every array keeps the base's
  // 16-byte alignment), digit counts (256 x tiles), tile sums, tile bests, m*.
  const int ntiles = (N + kGTile - 1) / kGTile;
  const size_t Np = ((size_t)N + 3) / 4 * 4;
  int* ws = reinterpret_cast<int*>(workspace);
  uint32_t* k0 = reinterpret_cast<uint32_t*>(ws);
  int* i0 = ws + Np;
  uint32_t* k1 = reinterpret_cast<uint32_t*>(ws + 2 * Np);
  int* i1 = ws + 3 * Np;
  int* hist = ws + 4 * Np;
  unsigned long long* tsum =
      reinterpret_cast<unsigned long long*>(hist + (size_t)kDig * ntiles);   // 8-byte aligned
  TileBest* tbest = reinterpret_cast<TileBest*>(tsum + ntiles);
  const bool inl = ntiles <= kInlineTiles;
  // Keys and ids: surv -> (k1, i1) -> (k0, i0) -> (k1, i1) -> (k0, i0).
  uint32_t* dk[4] = {k1, k0, k1, k0};
  int* di[4] = {i1, i0, i1, i0};
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 8 * pass;
    const uint32_t* sk = pass == 0 ? nullptr : dk[pass - 1];
    const int* si = pass == 0 ? nullptr : di[pass - 1];
    if (pass == 0)
      hipLaunchKernelGGL(sched_hist_kernel<true>, dim3(ntiles), dim3(kGT), 0, stream, surv, sk, N,
                         shift, hist);
    else
      hipLaunchKernelGGL(sched_hist_kernel<false>, dim3(ntiles), dim3(kGT), 0, stream, surv, sk,
                         N, shift, hist);
    if (!inl) hipLaunchKernelGGL(sched_scan_kernel, dim3(1), dim3(kT), 0, stream, hist, ntiles);
    if (pass == 0) {
      if (inl) launch_scatter<true, true>(ntiles, stream, surv, sk, si, dk[0], di[0], N, shift, hist);
      else launch_scatter<true, false>(ntiles, stream, surv, sk, si, dk[0], di[0], N, shift, hist);
    } else {
      if (inl) launch_scatter<false, true>(ntiles, stream, surv, sk, si, dk[pass], di[pass], N, shift, hist);
      else launch_scatter<false, false>(ntiles, stream, surv, sk, si, dk[pass], di[pass], N, shift, hist);
    }
    dspark_status st = check_launch("schedule sort pass");
    if (st != DSPARK_OK) return st;
  }
  hipLaunchKernelGGL(sched_tsum_kernel, dim3(ntiles), dim3(kGT), 0, stream, k0, i0, N, tsum, R,
                     lengths);
  int* tbrk = reinterpret_cast<int*>(tbest);   // one int per tile in the tile-best area
  if (mode == 0)
    hipLaunchKernelGGL(sched_tscan_kernel, dim3(ntiles), dim3(kGT), 0, stream, k0, i0, sps, R, N,
                       tsum, order, tbest);
  else
    hipLaunchKernelGGL(sched_tbreak_kernel, dim3(ntiles), dim3(kGT), 0, stream, k0, i0, sps, R,
                       N, mode, tsum, order, tbrk);
  hipLaunchKernelGGL(sched_finish_kernel, dim3((N + 255) / 256), dim3(256), 0, stream, tbest, tbrk,
                     tsum, k0, i0, ntiles, N, R, gamma, mode, m_cap, sps, info, lengths);
  return check_launch("schedule scan");
}

dspark_status launch_draft_finish(const unsigned long long* words_last, int S, int V,
                                  const float* sh, const float* se, const float* sts_temp, int R,
                                  int gamma, int32_t* tokens, float* conf, float* surv,
                                  const float* sps, int32_t* lengths, int32_t* order,
                                  dspark_schedule_info* info, void* sched_ws, hipStream_t stream) {
  const FinishArgs fa{words_last, S, V, sh, se, sts_temp, tokens, conf, surv};
  const int N = R * gamma;
  if (N <= kT * 1) return launch_lds<1, kFinAfter>(nullptr, sps, R, gamma, N, 0, 0, lengths, order, info, fa, stream);
  if (N <= kT * 2) return launch_lds<2, kFinAfter>(nullptr, sps, R, gamma, N, 0, 0, lengths, order, info, fa, stream);
  if (N <= kT * 4) return launch_lds<4, kFinAfter>(nullptr, sps, R, gamma, N, 0, 0, lengths, order, info, fa, stream);
  if (N <= kT * 8) return launch_lds<8, kFinAfter>(nullptr, sps, R, gamma, N, 0, 0, lengths, order, info, fa, stream);
  hipLaunchKernelGGL(finish_kernel, dim3((R + 255) / 256), dim3(256), 0, stream, fa, R, gamma);
  const dspark_status st = check_launch("finish_kernel");
  if (st != DSPARK_OK) return st;
  return launch_schedule(surv, sps, R, gamma, 0, 0, lengths, order, info, sched_ws, stream);
}

}  // namespace dspark
