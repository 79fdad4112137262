// Verification side for CDNA4 (gfx950).
//
// [P1] section 三 challenge 3: every verified token is one flattened element,
// the within-sequence dependencies travel in a marker tensor; [P3] Figure 1:
// the target verifies anchor + kept prefix in parallel, accepts the prefix its
// own predictions match and emits a corrected token; [P1] section 二 design 2:
// the acceptance label 1 - TV(p_draft, p_target).
//
//   verify_pack:   cu_seqlens = exclusive scan of (1 + l_r) (one workgroup,
//                  chunks of 1024 with a carry), then one thread per (r, j)
//                  writes token (anchor or draft j), position pos0[r] + j and
//                  the request id r; up to 1024 requests both in one launch;
//   verify_greedy: one workgroup per flattened row takes the target's argmax
//                  (16-byte loads, per-thread running max in increasing v,
//                  smallest id on ties), then one thread per request walks
//                  its drafts against those argmaxes;
//   accept_prob:   one workgroup per row pair, two passes over V in base 2:
//                  online (max, sum of 2^x) of both rows, four values per
//                  rescale, then sum_v min(p, q).  With aligned rows (V a
//                  multiple of 4) 512 threads keep the first part of the pair
//                  in registers and LDS between the passes (about half of it
//                  at the DeepSeek-V4 vocabulary), so the second pass reads
//                  only the rest from memory; else 1024 threads read both rows
//                  twice.  Reductions use a fixed tree, so results are
//                  deterministic.
#include <atomic>
#include <math.h>

#include "dspark_internal.h"

namespace dspark {
namespace {

constexpr int kPackT = 1024;
constexpr int kRowT = 256;
constexpr int kRowW = kRowT / 64;
constexpr int kRowU = 4;   // loads in flight per thread in the row argmax
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int clamp_len(int l, int gamma) { return min(max(l, 0), gamma); }

__global__ __launch_bounds__(kPackT) void verify_scan_kernel(const int32_t* __restrict__ lengths,
                                                             int R, int gamma,
                                                             int32_t* __restrict__ cu) {
  __shared__ int wtot[kPackT / 64];
  __shared__ int carry;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  if (t == 0) carry = 0;
  __syncthreads();
  for (int c0 = 0; c0 < R; c0 += kPackT) {
    const int r = c0 + t;
    const int v = r < R ? 1 + clamp_len(lengths[r], gamma) : 0;
    int inc = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(inc, off);
      if (lane >= off) inc += o;
    }
    if (lane == 63) wtot[w] = inc;
    __syncthreads();
    int pre = carry, total = 0;
#pragma unroll
    for (int j = 0; j < kPackT / 64; ++j) {
      pre += j < w ? wtot[j] : 0;
      total += wtot[j];
    }
    if (r < R) cu[r] = pre + inc - v;
    __syncthreads();
    if (t == 0) carry += total;
    __syncthreads();
  }
  if (t == 0) cu[R] = carry;
}

__global__ __launch_bounds__(256) void verify_scatter_kernel(
    const int32_t* __restrict__ anchors, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ lengths, const int32_t* __restrict__ pos0,
    const int32_t* __restrict__ cu, int R, int gamma, int32_t* __restrict__ flat_tokens,
    int32_t* __restrict__ flat_pos, int32_t* __restrict__ flat_req) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  const int per = 1 + gamma;
  if (e >= (long long)R * per) return;
  const int r = (int)(e / per);
  const int j = (int)(e % per);
  if (j > clamp_len(lengths[r], gamma)) return;
  const int dst = cu[r] + j;
  flat_tokens[dst] = j == 0 ? anchors[r] : tokens[(size_t)r * gamma + j - 1];
  if (flat_pos) flat_pos[dst] = (pos0 ? pos0[r] : 0) + j;
  if (flat_req) flat_req[dst] = r;
}

// The whole flattening in one workgroup when R <= kPackT: the scan of the
// sequence lengths, then every (r, j) element scattered by the same threads
// (one launch instead of two: at these sizes the work is a few microseconds
// and the second launch cost as much again).
__global__ __launch_bounds__(kPackT) void verify_pack_small_kernel(
    const int32_t* __restrict__ anchors, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ lengths, const int32_t* __restrict__ pos0, int R, int gamma,
    int32_t* __restrict__ cu, int32_t* __restrict__ flat_tokens, int32_t* __restrict__ flat_pos,
    int32_t* __restrict__ flat_req) {
  __shared__ int wtot[kPackT / 64];
  __shared__ int scu[kPackT];
  __shared__ int slen[kPackT];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int len = t < R ? clamp_len(lengths[t], gamma) : 0;
  const int v = t < R ? 1 + len : 0;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  if (lane == 63) wtot[w] = inc;
  __syncthreads();
  int pre = 0, total = 0;
#pragma unroll
  for (int j = 0; j < kPackT / 64; ++j) {
    pre += j < w ? wtot[j] : 0;
    total += wtot[j];
  }
  if (t < R) {
    cu[t] = pre + inc - v;
    scu[t] = pre + inc - v;
    slen[t] = len;
  }
  if (t == 0) cu[R] = total;
  __syncthreads();
  const int per = 1 + gamma;
  for (int e = t; e < R * per; e += kPackT) {
    const int r = e / per;
    const int j = e - r * per;
    if (j > slen[r]) continue;
    const int dst = scu[r] + j;
    flat_tokens[dst] = j == 0 ? anchors[r] : tokens[(size_t)r * gamma + j - 1];
    if (flat_pos) flat_pos[dst] = (pos0 ? pos0[r] : 0) + j;
    if (flat_req) flat_req[dst] = r;
  }
}

// Running (max, smallest index) of one thread, merged in a fixed tree.
__device__ __forceinline__ void take(float& bv, int& bi, float v, int i) {
  const bool t = (v > bv) | ((v == bv) & (i < bi));   // selects, no branch
  bv = t ? v : bv;
  bi = t ? i : bi;
}

__global__ __launch_bounds__(kRowT) void verify_argmax_kernel(const float* __restrict__ logits,
                                                              const int32_t* __restrict__ cu,
                                                              int R, int V, int vec,
                                                              int32_t* __restrict__ amax) {
  __shared__ float sv[kRowW];
  __shared__ int si[kRowW];
  const int row = blockIdx.x;
  if (row >= cu[R]) return;   // rows past the batch are not read
  const int t = threadIdx.x;
  const float* z = logits + (size_t)row * V;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  if (vec) {
    // Each row is read once: non-temporal loads, kRowU of them in flight per
    // thread before any is used (one per thread leaves the memory system
    // underfed).  take() is a lexicographic max, so the order of the elements
    // does not matter.
    // The next batch's loads are issued before this batch is compared, so a
    // thread's loads never drain between batches.
    const v4f* z4 = reinterpret_cast<const v4f*>(z);
    const int n4 = V >> 2;
    int p = t;
    constexpr int kStep = kRowU * kRowT;
    if (p + (kRowU - 1) * kRowT < n4) {
      v4f q[kRowU];
#pragma unroll
      for (int u = 0; u < kRowU; ++u) q[u] = __builtin_nontemporal_load(z4 + p + u * kRowT);
      for (;;) {
        const int pn = p + kStep;
        const bool more = pn + (kRowU - 1) * kRowT < n4;
        v4f qn[kRowU];
        // past the last whole batch the next loads re-read this batch (in
        // bounds) and are not used
        const int pl = more ? pn : p;
#pragma unroll
        for (int u = 0; u < kRowU; ++u) qn[u] = __builtin_nontemporal_load(z4 + pl + u * kRowT);
        __builtin_amdgcn_sched_barrier(0);   // next loads issued before the compares
#pragma unroll
        for (int u = 0; u < kRowU; ++u) {
          const int e = 4 * (p + u * kRowT);
          take(bv, bi, q[u].x, e);
          take(bv, bi, q[u].y, e + 1);
          take(bv, bi, q[u].z, e + 2);
          take(bv, bi, q[u].w, e + 3);
        }
        p = pn;
        if (!more) break;
#pragma unroll
        for (int u = 0; u < kRowU; ++u) q[u] = qn[u];
      }
    }
    for (; p < n4; p += kRowT) {
      const v4f q = __builtin_nontemporal_load(z4 + p);
      take(bv, bi, q.x, 4 * p);
      take(bv, bi, q.y, 4 * p + 1);
      take(bv, bi, q.z, 4 * p + 2);
      take(bv, bi, q.w, 4 * p + 3);
    }
  } else {
    for (int v = t; v < V; v += kRowT) take(bv, bi, z[v], v);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    take(bv, bi, ov, oi);
  }
  if ((t & 63) == 0) {
    sv[t >> 6] = bv;
    si[t >> 6] = bi;
  }
  __syncthreads();
  if (t == 0) {
    for (int j = 1; j < kRowW; ++j) take(bv, bi, sv[j], si[j]);
    amax[row] = bi < V ? bi : 0;
  }
}

__global__ __launch_bounds__(256) void verify_accept_kernel(const int32_t* __restrict__ amax,
                                                            const int32_t* __restrict__ cu,
                                                            const int32_t* __restrict__ tokens,
                                                            int R, int gamma,
                                                            int32_t* __restrict__ accepted,
                                                            int32_t* __restrict__ next_token) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= R) return;
  const int s = cu[r];
  const int l = clamp_len(cu[r + 1] - s - 1, gamma);
  int a = 0;
  while (a < l && tokens[(size_t)r * gamma + a] == amax[s + a]) ++a;
  accepted[r] = a;
  next_token[r] = amax[s + a];
}

// Acceptance probability in base 2: with k = log2(e) / T and x' = k x, p_v =
// 2^(x'_v - L) where L = m + log2(sum 2^(x' - m)), so the kernel keeps (max,
// sum of 2^(x' - max)) pairs and uses the hardware 2^x.
constexpr int kAccT = 1024;
constexpr int kAccW = kAccT / 64;
constexpr int kAccU = 2;   // loop iterations whose loads are in flight together

struct MaxSum {
  float m;
  float s;
};

__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ MaxSum merge_ms(MaxSum a, MaxSum b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return {m, 0.0f};
  return {m, a.s * exp2_(a.m - m) + b.s * exp2_(b.m - m)};
}

// Fold four scaled values into a running pair (one rescale per four).
__device__ __forceinline__ void add4(MaxSum& a, float x0, float x1, float x2, float x3) {
  const float nm = fmaxf(fmaxf(a.m, fmaxf(x0, x1)), fmaxf(x2, x3));
  if (nm == -INFINITY) return;   // nothing finite yet
  a.s = a.s * exp2_(a.m - nm) + ((exp2_(x0 - nm) + exp2_(x1 - nm)) + (exp2_(x2 - nm) + exp2_(x3 - nm)));
  a.m = nm;
}

__device__ __forceinline__ MaxSum block_ms(MaxSum v, MaxSum* sh) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    MaxSum o{__shfl_xor(v.m, off), __shfl_xor(v.s, off)};
    v = merge_ms(v, o);
  }
  const int t = threadIdx.x;
  if ((t & 63) == 0) sh[t >> 6] = v;
  __syncthreads();
  MaxSum r = sh[0];
#pragma unroll
  for (int j = 1; j < kAccW; ++j) r = merge_ms(r, sh[j]);
  __syncthreads();
  return r;
}

// Holding variant for 16-byte aligned rows: 512 threads (one workgroup per
// CU), and each thread keeps its first kAccReg iterations of both rows in
// registers and the next kAccLds in LDS between the two passes, so the second
// pass re-reads only the rest of the row pair.
constexpr int kAccRT = 512;
constexpr int kAccRW = kAccRT / 64;
constexpr int kAccReg = 24;   // iterations per thread held in registers
constexpr int kAccLds = 8;    // iterations per thread held in LDS
constexpr int kAccRU = 4;     // streamed iterations whose loads are in flight together
static_assert(kAccLds % kAccRU == 0, "the LDS-held iterations go in whole batches");
constexpr size_t kAccLdsBytes = (size_t)kAccLds * 2 * kAccRT * sizeof(v4f);

template <int NW>
__device__ __forceinline__ MaxSum block_ms_w(MaxSum v, MaxSum* sh) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    MaxSum o{__shfl_xor(v.m, off), __shfl_xor(v.s, off)};
    v = merge_ms(v, o);
  }
  const int t = threadIdx.x;
  if ((t & 63) == 0) sh[t >> 6] = v;
  __syncthreads();
  MaxSum r = sh[0];
#pragma unroll
  for (int j = 1; j < NW; ++j) r = merge_ms(r, sh[j]);
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kAccRT) void accept_prob_hold_kernel(const float* __restrict__ zd,
                                                                 const float* __restrict__ zt,
                                                                 int V, float k2,
                                                                 float* __restrict__ out) {
  __shared__ MaxSum shd[kAccRW];
  __shared__ MaxSum sht[kAccRW];
  __shared__ float ssum[kAccRW];
  extern __shared__ v4f held[];   // [kAccLds][2][kAccRT]: a thread's own slots only
  const int t = threadIdx.x;
  const int row = blockIdx.x;
  const v4f* a4 = reinterpret_cast<const v4f*>(zd + (size_t)row * V);
  const v4f* b4 = reinterpret_cast<const v4f*>(zt + (size_t)row * V);
  const int V4 = V >> 2;
  const v4f ninf = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  // The held part: entry t + u * kAccRT of each row for u < kAccReg (past the
  // row: entry 0 read and replaced by -inf, which adds nothing to either pass).
  v4f xr[kAccReg], yr[kAccReg];
#pragma unroll
  for (int u = 0; u < kAccReg; ++u) {
    const int p = t + u * kAccRT;
    const int pc = p < V4 ? p : 0;
    xr[u] = a4[pc];
    yr[u] = b4[pc];
  }
#pragma unroll
  for (int u = 0; u < kAccReg; ++u) {
    const bool in = t + u * kAccRT < V4;
    xr[u] = in ? xr[u] : ninf;
    yr[u] = in ? yr[u] : ninf;
  }
  MaxSum md{-INFINITY, 0.0f}, mt{-INFINITY, 0.0f};
#pragma unroll
  for (int u = 0; u < kAccReg; ++u) {
    add4(md, xr[u].x * k2, xr[u].y * k2, xr[u].z * k2, xr[u].w * k2);
    add4(mt, yr[u].x * k2, yr[u].y * k2, yr[u].z * k2, yr[u].w * k2);
  }
  // The LDS-held part: batches of kAccRU iterations, kept after their use.
#pragma unroll
  for (int u0 = kAccReg; u0 < kAccReg + kAccLds; u0 += kAccRU) {
    v4f x[kAccRU], y[kAccRU];
#pragma unroll
    for (int u = 0; u < kAccRU; ++u) {
      const int p = t + (u0 + u) * kAccRT;
      const int pc = p < V4 ? p : 0;
      x[u] = a4[pc];
      y[u] = b4[pc];
    }
#pragma unroll
    for (int u = 0; u < kAccRU; ++u) {
      const bool in = t + (u0 + u) * kAccRT < V4;
      x[u] = in ? x[u] : ninf;
      y[u] = in ? y[u] : ninf;
      add4(md, x[u].x * k2, x[u].y * k2, x[u].z * k2, x[u].w * k2);
      add4(mt, y[u].x * k2, y[u].y * k2, y[u].z * k2, y[u].w * k2);
      held[((u0 - kAccReg + u) * 2) * kAccRT + t] = x[u];
      held[((u0 - kAccReg + u) * 2 + 1) * kAccRT + t] = y[u];
    }
  }
  // The streamed rest, read twice (kept in the caches after the first read).
  const int p0 = t + (kAccReg + kAccLds) * kAccRT;
  {
    int p = p0;
    for (; p + (kAccRU - 1) * kAccRT < V4; p += kAccRU * kAccRT) {
      v4f x[kAccRU], y[kAccRU];
#pragma unroll
      for (int u = 0; u < kAccRU; ++u) {
        x[u] = a4[p + u * kAccRT];
        y[u] = b4[p + u * kAccRT];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kAccRU; ++u) {
        add4(md, x[u].x * k2, x[u].y * k2, x[u].z * k2, x[u].w * k2);
        add4(mt, y[u].x * k2, y[u].y * k2, y[u].z * k2, y[u].w * k2);
      }
    }
    for (; p < V4; p += kAccRT) {
      const v4f x = a4[p];
      const v4f y = b4[p];
      add4(md, x.x * k2, x.y * k2, x.z * k2, x.w * k2);
      add4(mt, y.x * k2, y.y * k2, y.z * k2, y.w * k2);
    }
  }
  md = block_ms_w<kAccRW>(md, shd);
  mt = block_ms_w<kAccRW>(mt, sht);
  const float Ld = md.m + __log2f(md.s);
  const float Lt = mt.m + __log2f(mt.s);
  auto term = [&](float x, float y) {
    return fminf(exp2_(fmaf(x, k2, -Ld)), exp2_(fmaf(y, k2, -Lt)));
  };
  float acc = 0.0f;
#pragma unroll
  for (int u = 0; u < kAccReg; ++u)
    acc += (term(xr[u].x, yr[u].x) + term(xr[u].y, yr[u].y)) +
           (term(xr[u].z, yr[u].z) + term(xr[u].w, yr[u].w));
#pragma unroll
  for (int u = 0; u < kAccLds; ++u) {
    const v4f x = held[(u * 2) * kAccRT + t];
    const v4f y = held[(u * 2 + 1) * kAccRT + t];
    acc += (term(x.x, y.x) + term(x.y, y.y)) + (term(x.z, y.z) + term(x.w, y.w));
  }
  {
    int p = p0;
    for (; p + (kAccRU - 1) * kAccRT < V4; p += kAccRU * kAccRT) {
      v4f x[kAccRU], y[kAccRU];
#pragma unroll
      for (int u = 0; u < kAccRU; ++u) {
        x[u] = __builtin_nontemporal_load(a4 + p + u * kAccRT);
        y[u] = __builtin_nontemporal_load(b4 + p + u * kAccRT);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kAccRU; ++u)
        acc += (term(x[u].x, y[u].x) + term(x[u].y, y[u].y)) +
               (term(x[u].z, y[u].z) + term(x[u].w, y[u].w));
    }
    for (; p < V4; p += kAccRT) {
      const v4f x = __builtin_nontemporal_load(a4 + p);
      const v4f y = __builtin_nontemporal_load(b4 + p);
      acc += (term(x.x, y.x) + term(x.y, y.y)) + (term(x.z, y.z) + term(x.w, y.w));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if ((t & 63) == 0) ssum[t >> 6] = acc;
  __syncthreads();
  if (t == 0) {
    float s = 0.0f;
    for (int j = 0; j < kAccRW; ++j) s += ssum[j];
    out[row] = s;
  }
}

__global__ __launch_bounds__(kAccT) void accept_prob_kernel(const float* __restrict__ zd,
                                                            const float* __restrict__ zt, int V,
                                                            float k2, int vec,
                                                            float* __restrict__ out) {
  __shared__ MaxSum shd[kAccW];
  __shared__ MaxSum sht[kAccW];
  __shared__ float ssum[kAccW];
  const int t = threadIdx.x;
  {
    const int row = blockIdx.x;
    const float* a = zd + (size_t)row * V;
    const float* b = zt + (size_t)row * V;
    MaxSum md{-INFINITY, 0.0f}, mt{-INFINITY, 0.0f};
    if (vec) {
      // kAccU iterations' loads of both rows in flight before the first use
      // (same element order as one at a time).  The rows are read again by the
      // second pass, so these loads keep their lines.
      const v4f* a4 = reinterpret_cast<const v4f*>(a);
      const v4f* b4 = reinterpret_cast<const v4f*>(b);
      const int V4 = V >> 2;
      int p = t;
      for (; p + (kAccU - 1) * kAccT < V4; p += kAccU * kAccT) {
        v4f x[kAccU], y[kAccU];
#pragma unroll
        for (int u = 0; u < kAccU; ++u) {
          x[u] = a4[p + u * kAccT];
          y[u] = b4[p + u * kAccT];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kAccU; ++u) {
          add4(md, x[u].x * k2, x[u].y * k2, x[u].z * k2, x[u].w * k2);
          add4(mt, y[u].x * k2, y[u].y * k2, y[u].z * k2, y[u].w * k2);
        }
      }
      for (; p < V4; p += kAccT) {
        const v4f x = a4[p];
        const v4f y = b4[p];
        add4(md, x.x * k2, x.y * k2, x.z * k2, x.w * k2);
        add4(mt, y.x * k2, y.y * k2, y.z * k2, y.w * k2);
      }
    } else {
      for (int v = t; v < V; v += kAccT) {
        add4(md, a[v] * k2, -INFINITY, -INFINITY, -INFINITY);
        add4(mt, b[v] * k2, -INFINITY, -INFINITY, -INFINITY);
      }
    }
    md = block_ms(md, shd);
    mt = block_ms(mt, sht);
    const float Ld = md.m + __log2f(md.s);
    const float Lt = mt.m + __log2f(mt.s);
    float acc = 0.0f;
    auto term = [&](float x, float y) {
      return fminf(exp2_(fmaf(x, k2, -Ld)), exp2_(fmaf(y, k2, -Lt)));
    };
    if (vec) {
      // The second and last read of the rows: non-temporal, kAccU in flight.
      const v4f* a4 = reinterpret_cast<const v4f*>(a);
      const v4f* b4 = reinterpret_cast<const v4f*>(b);
      const int V4 = V >> 2;
      int p = t;
      for (; p + (kAccU - 1) * kAccT < V4; p += kAccU * kAccT) {
        v4f x[kAccU], y[kAccU];
#pragma unroll
        for (int u = 0; u < kAccU; ++u) {
          x[u] = __builtin_nontemporal_load(a4 + p + u * kAccT);
          y[u] = __builtin_nontemporal_load(b4 + p + u * kAccT);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kAccU; ++u)
          acc += (term(x[u].x, y[u].x) + term(x[u].y, y[u].y)) +
                 (term(x[u].z, y[u].z) + term(x[u].w, y[u].w));
      }
      for (; p < V4; p += kAccT) {
        const v4f x = __builtin_nontemporal_load(a4 + p);
        const v4f y = __builtin_nontemporal_load(b4 + p);
        acc += (term(x.x, y.x) + term(x.y, y.y)) + (term(x.z, y.z) + term(x.w, y.w));
      }
    } else {
      for (int v = t; v < V; v += kAccT) acc += term(a[v], b[v]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if ((t & 63) == 0) ssum[t >> 6] = acc;
    __syncthreads();
    if (t == 0) {
      float s = 0.0f;
      for (int j = 0; j < kAccW; ++j) s += ssum[j];
      out[row] = s;
    }
  }
}

}  // namespace

dspark_status launch_verify_pack(const int32_t* anchors, const int32_t* tokens,
                                 const int32_t* lengths, const int32_t* pos0, int R, int gamma,
                                 int32_t* flat_tokens, int32_t* flat_pos, int32_t* flat_req,
                                 int32_t* cu_seqlens, hipStream_t stream) {
  if (R <= kPackT && (long long)R * (1 + gamma) <= (1LL << 20)) {
    hipLaunchKernelGGL(verify_pack_small_kernel, dim3(1), dim3(kPackT), 0, stream, anchors, tokens,
                       lengths, pos0, R, gamma, cu_seqlens, flat_tokens, flat_pos, flat_req);
    return check_launch("verify_pack");
  }
  hipLaunchKernelGGL(verify_scan_kernel, dim3(1), dim3(kPackT), 0, stream, lengths, R, gamma,
                     cu_seqlens);
  const long long n = (long long)R * (1 + gamma);
  hipLaunchKernelGGL(verify_scatter_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     stream, anchors, tokens, lengths, pos0, cu_seqlens, R, gamma, flat_tokens,
                     flat_pos, flat_req);
  return check_launch("verify_pack");
}

dspark_status launch_verify_greedy(const float* target_logits, const int32_t* cu_seqlens,
                                   const int32_t* tokens, int R, int gamma, int V,
                                   int32_t* target_argmax, int32_t* accepted,
                                   int32_t* next_token, hipStream_t stream) {
  const int rows = R * (1 + gamma);
  const int vec = (V % 4 == 0) && ((reinterpret_cast<uintptr_t>(target_logits) & 15u) == 0);
  hipLaunchKernelGGL(verify_argmax_kernel, dim3(rows), dim3(kRowT), 0, stream, target_logits,
                     cu_seqlens, R, V, vec, target_argmax);
  hipLaunchKernelGGL(verify_accept_kernel, dim3((R + 255) / 256), dim3(256), 0, stream,
                     target_argmax, cu_seqlens, tokens, R, gamma, accepted, next_token);
  return check_launch("verify_greedy");
}

dspark_status launch_accept_prob(const float* draft_logits, const float* target_logits, int n,
                                 int V, float temperature, float* out, hipStream_t stream) {
  auto a16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
  const int vec = (V % 4 == 0) && a16(draft_logits) && a16(target_logits);
  // One workgroup per row pair: aligned rows of a multiple of four entries
  // take the holding variant (about half of each row pair stays on chip
  // between the passes); others the 1024-thread kernel, which reads both rows
  // twice.  (Measured on the latter: capping the grid so that workgroups loop
  // over rows, or limiting workgroups per CU, was slower or no faster.)
  const float k2 = 1.44269504088896341f / temperature;   // log2(e) / T
  if (vec) {
    // The dynamic-LDS attribute, set once per device (bit d of `done`).
    static std::atomic<unsigned long long> done{0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(DSPARK_EDEVICE, "hipGetDevice failed");
    const unsigned long long bit = dev < 64 ? 1ull << dev : 0ull;
    if (!bit || !(done.load(std::memory_order_acquire) & bit)) {
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(&accept_prob_hold_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kAccLdsBytes) != hipSuccess)
        return fail(DSPARK_EDEVICE, "hipFuncSetAttribute failed for accept_prob_hold_kernel");
      done.fetch_or(bit, std::memory_order_release);
    }
    hipLaunchKernelGGL(accept_prob_hold_kernel, dim3(n), dim3(kAccRT), kAccLdsBytes, stream,
                       draft_logits, target_logits, V, k2, out);
    return check_launch("accept_prob_hold_kernel");
  }
  hipLaunchKernelGGL(accept_prob_kernel, dim3(n), dim3(kAccT), 0, stream, draft_logits,
                     target_logits, V, k2, vec, out);
  return check_launch("accept_prob_kernel");
}

}  // namespace dspark
