// Confidence head, STS calibration and prefix survival for CDNA4 (gfx950).
//
// [P1] section 二 design 2 (confidence head, sequential temperature scaling,
// survival products); [P4] (fp32 confidences):
//   s_{m,k} = w_h . h_{m,k} + w_e . W1[x_{k-1}]     (x_0 = anchor)
//   c_{m,k} = 1 / (1 + exp(-s_{m,k} / T_k))
//   a_{m,j} = c_{m,1} * ... * c_{m,j}               (fp32, left to right)
//
// Token ids are checked on the device: a position whose x_{k-1} lies outside
// [0, V) gets c = NaN (and so does its survival and every later one).
//
// The work is a dot product of length d + r per (request, position), bound by
// the HBM read of h.  One workgroup handles all gamma positions of one
// request, so the survival products are a short sequential tail in the same
// workgroup.  In the main kernels (16-byte aligned h and w_conf, d a multiple
// of 8, d <= 16384) thread t takes the 16-byte pieces t (and t + 1024) of a
// row, loads the matching fp32 w_h piece once, and applies it to that piece of
// up to eight positions' rows, whose loads are all in flight together: w_h,
// twice the bytes of an h row, is read once per request instead of once per
// position.  The loads are buffer loads, so the tails (pieces past d,
// positions past gamma) read zeros without a branch: a load on a branch would
// make the compiler drain every load in flight where the branch joins.  The
// token is read first and the W1-row loads issue behind the h loads, so that
// chain overlaps the h stream.  Lanes reduce with a fixed shuffle tree and the
// wavefront parts are added in a fixed order, so results are deterministic.
// Other shapes take a general kernel that splits each position's row over
// wavefronts.
#include <math.h>

#include "dspark_internal.h"
#include "raw_buffer.h"

namespace dspark {
namespace {

constexpr int kMaxGamma = 64;

__device__ __forceinline__ float bf16_lo(unsigned int w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned int w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Sum of w[i] * x[i] (x bf16) over this lane's share of elements [i0, i1):
// 16-byte pieces strided by the wavefront (vec: i0, i1 multiples of 8 and both
// arrays 16-byte aligned), eight pieces per lane in flight per round.
__device__ __forceinline__ float dot_part(const float* __restrict__ w,
                                          const uint16_t* __restrict__ x, int i0, int i1,
                                          bool vec, int lane) {
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (vec) {
    const int p1 = i1 >> 3;
    for (int p = (i0 >> 3) + lane; p < p1; p += 512) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int pp = p + 64 * u;
        if (pp < p1) {
          const u32x4 hv = *reinterpret_cast<const u32x4*>(x + 8 * pp);
          const float4 w0 = *reinterpret_cast<const float4*>(w + 8 * pp);
          const float4 w1 = *reinterpret_cast<const float4*>(w + 8 * pp + 4);
          float a = acc[u & 3];
          a = fmaf(w0.x, bf16_lo(hv.x), a);
          a = fmaf(w0.y, bf16_hi(hv.x), a);
          a = fmaf(w0.z, bf16_lo(hv.y), a);
          a = fmaf(w0.w, bf16_hi(hv.y), a);
          a = fmaf(w1.x, bf16_lo(hv.z), a);
          a = fmaf(w1.y, bf16_hi(hv.z), a);
          a = fmaf(w1.z, bf16_lo(hv.w), a);
          a = fmaf(w1.w, bf16_hi(hv.w), a);
          acc[u & 3] = a;
        }
      }
    }
  } else {
    for (int i = i0 + lane; i < i1; i += 64)
      acc[0] = fmaf(w[i], __uint_as_float((unsigned)x[i] << 16), acc[0]);
  }
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// Element range [lo, hi) of part j of P over n elements, in whole pieces of 8
// when vec.
__device__ __forceinline__ void part_range(int n, int P, int j, bool vec, int& lo, int& hi) {
  if (vec) {
    const int n8 = n >> 3;
    lo = 8 * (int)(((long long)n8 * j) / P);
    hi = 8 * (int)(((long long)n8 * (j + 1)) / P);
  } else {
    lo = (int)(((long long)n * j) / P);
    hi = (int)(((long long)n * (j + 1)) / P);
  }
}

// One workgroup per request.  With P wavefronts per position and G positions
// per round (G * P wavefronts), wavefront w takes part w % P of position
// w / P; part P - 1 also adds the W1-row term.
__global__ __launch_bounds__(1024) void confidence_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ W1,
    const int32_t* __restrict__ anchors, const int32_t* __restrict__ tokens,
    const float* __restrict__ w_conf, const float* __restrict__ sts_temp, int gamma, int d,
    int V, int r, int P, int vec_h, int vec_e, float* __restrict__ conf,
    float* __restrict__ surv) {
  __shared__ float parts[1024 / 64];
  __shared__ float cval[kMaxGamma];
  const int m = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int G = (blockDim.x >> 6) / P;   // positions per round
  const float* w_h = w_conf;
  const float* w_e = w_conf + d;
  float a = 1.0f;   // running survival product (thread 0)
  for (int k0 = 0; k0 < gamma; k0 += G) {
    const int kk = wave / P;
    const int j = wave % P;
    const int k = k0 + kk;
    if (kk < G && k < gamma) {
      int x = 0;
      if (j == P - 1) x = k == 0 ? anchors[m] : tokens[(size_t)m * gamma + k - 1];
      int lo, hi;
      part_range(d, P, j, vec_h, lo, hi);
      float part = dot_part(w_h, h + ((size_t)m * gamma + k) * d, lo, hi, vec_h, lane);
      if (j == P - 1) {
        if (x >= 0 && x < V) part += dot_part(w_e, W1 + (size_t)x * r, 0, r, vec_e, lane);
        else part = NAN;
      }
      const float s = wave_sum(part);
      if (lane == 0) parts[wave] = s;
    }
    __syncthreads();
    if ((int)threadIdx.x < G && k0 + (int)threadIdx.x < gamma) {
      const int kt = k0 + threadIdx.x;
      float s = 0.0f;
      for (int jj = 0; jj < P; ++jj) s += parts[threadIdx.x * P + jj];
      const float t = sts_temp ? sts_temp[kt] : 1.0f;
      const float c = 1.0f / (1.0f + expf(-(s / t)));
      conf[(size_t)m * gamma + kt] = c;
      cval[threadIdx.x] = c;
    }
    __syncthreads();
    if (surv && threadIdx.x == 0) {
      const int kn = min(G, gamma - k0);
      for (int q = 0; q < kn; ++q) {
        const int kt = k0 + q;
        a = kt == 0 ? cval[q] : a * cval[q];
        surv[(size_t)m * gamma + kt] = a;
      }
    }
    __syncthreads();
  }
}

// ---- one workgroup per request, w_h read once for all positions ----
constexpr int kRowThreads = 1024;
constexpr int kRowWaves = kRowThreads / 64;

__device__ __forceinline__ float dot8(const u32x4 w0, const u32x4 w1, const u32x4 hv, float a) {
  a = fmaf(__uint_as_float(w0.x), bf16_lo(hv.x), a);
  a = fmaf(__uint_as_float(w0.y), bf16_hi(hv.x), a);
  a = fmaf(__uint_as_float(w0.z), bf16_lo(hv.y), a);
  a = fmaf(__uint_as_float(w0.w), bf16_hi(hv.y), a);
  a = fmaf(__uint_as_float(w1.x), bf16_lo(hv.z), a);
  a = fmaf(__uint_as_float(w1.y), bf16_hi(hv.z), a);
  a = fmaf(__uint_as_float(w1.z), bf16_lo(hv.w), a);
  a = fmaf(__uint_as_float(w1.w), bf16_hi(hv.w), a);
  return a;
}

// Loads of this thread's share of w_h . h[m, k0 + q, :], q < G: PJ pieces per
// row (piece tid + 1024 j), each with its w_h piece.  rh covers the request's
// gamma rows of h, rw the d floats of w_h.
template <int G, int PJ>
struct HDot {
  u32x4 w[PJ][2];
  u32x4 hv[PJ][G];
  __device__ __forceinline__ void load(Rsrc rh, Rsrc rw, int k0, int gamma, int d, int tid) {
    const int n8 = d >> 3;
#pragma unroll
    for (int j = 0; j < PJ; ++j) {
      const int p = tid + j * kRowThreads;
      const uint32_t wo = p < n8 ? (uint32_t)p * 32u : kOff;
      w[j][0] = ld16(rw, wo);
      w[j][1] = ld16(rw, wo + 16u);
#pragma unroll
      for (int q = 0; q < G; ++q) {
        const uint32_t ho = (p < n8 && k0 + q < gamma)
                                ? ((uint32_t)(k0 + q) * (uint32_t)d + 8u * (uint32_t)p) * 2u
                                : kOff;
        hv[j][q] = ld16(rh, ho);
      }
    }
  }
  __device__ __forceinline__ void sum(float (&acc)[G]) const {
#pragma unroll
    for (int q = 0; q < G; ++q) {
      float a = 0.0f;
#pragma unroll
      for (int j = 0; j < PJ; ++j) a = dot8(w[j][0], w[j][1], hv[j][q], a);
      acc[q] = a;
    }
  }
};

// Sum over the wavefront by a DPP scan (lanes of a row of 16, then rows
// through broadcasts of lanes 15 and 31; a fixed order), read from lane 63.
// Unlike a shuffle tree it needs no LDS round trip per step, which matters
// when every lane reduces several values.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xf,
                                                        false));
}
__device__ __forceinline__ float wave_total(float v) {
  v = dpp_add<0x111, 0xf>(v);   // row_shr:1
  v = dpp_add<0x112, 0xf>(v);   // row_shr:2
  v = dpp_add<0x114, 0xf>(v);   // row_shr:4
  v = dpp_add<0x118, 0xf>(v);   // row_shr:8
  v = dpp_add<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// acc[q] summed over the workgroup: a fixed DPP scan per wavefront, then the
// wavefront parts in wavefront order by thread q (result in out[q]).
template <int G>
__device__ __forceinline__ void block_sums(const float (&acc)[G], float (*part)[G], int lane,
                                           int wave, int tid, float& out) {
#pragma unroll
  for (int q = 0; q < G; ++q) {
    const float s = wave_total(acc[q]);
    if (lane == 0) part[wave][q] = s;
  }
  __syncthreads();
  out = 0.0f;
  if (tid < G) {
#pragma unroll
    for (int w = 0; w < kRowWaves; ++w) out += part[w][tid];
  }
}

template <int PJ>
constexpr int row_positions() { return PJ == 1 ? 8 : 4; }

// Whole confidence head for one request per workgroup: positions in rounds of
// G; wavefront q < G also takes the embedding term of position k0 + q.
template <int PJ>
__global__ __launch_bounds__(kRowThreads) void confidence_rows_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ W1,
    const int32_t* __restrict__ anchors, const int32_t* __restrict__ tokens,
    const float* __restrict__ w_conf, const float* __restrict__ sts_temp, int gamma, int d,
    int V, int r, float* __restrict__ conf, float* __restrict__ surv) {
  constexpr int G = row_positions<PJ>();
  __shared__ float part[kRowWaves][G];
  __shared__ float epart[G];
  __shared__ float cval[G];
  const int m = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Rsrc rh = rsrc_of(h + (size_t)m * gamma * d, (size_t)gamma * d * 2);
  const Rsrc rw = rsrc_of(w_conf, (size_t)d * 4);
  const Rsrc rwe = rsrc_of(w_conf + d, (size_t)r * 4);
  // this lane's 16-byte piece of a W1 row and its two of w_e (zeros past r)
  const uint32_t eo = lane * 8 < r ? (uint32_t)lane * 16u : kOff;
  const uint32_t weo = lane * 8 < r ? (uint32_t)lane * 32u : kOff;
  float a = 1.0f;   // running survival product (thread 0)
  for (int k0 = 0; k0 < gamma; k0 += G) {
    const int ke = k0 + wave;
    const bool emb = wave < G && ke < gamma;
    // x_{ke-1} (x_0 = anchor), both candidates read without a branch
    const int kc = min(ke, gamma - 1);
    const int xa = anchors[m];
    const int xt = tokens[(size_t)m * gamma + (kc > 0 ? kc - 1 : 0)];
    const int x = kc == 0 ? xa : xt;
    HDot<G, PJ> hd;
    hd.load(rh, rw, k0, gamma, d, tid);
    // W1 row of token x: zeros for an invalid token.
    const bool ok = emb && x >= 0 && x < V;
    const Rsrc re = rsrc_of(W1 + (ok ? (size_t)x * r : 0), ok ? (size_t)r * 2 : 0);
    const u32x4 ev = ld16(re, eo);
    const u32x4 we0 = ld16(rwe, weo);
    const u32x4 we1 = ld16(rwe, weo + 16u);
    float acc[G];
    hd.sum(acc);
    const float es = wave_total(dot8(we0, we1, ev, 0.0f));
    if (emb && lane == 0) epart[wave] = ok ? es : NAN;
    float s;
    block_sums<G>(acc, part, lane, wave, tid, s);
    if (tid < G && k0 + tid < gamma) {
      const int kt = k0 + tid;
      s += epart[tid];
      const float t = sts_temp ? sts_temp[kt] : 1.0f;
      const float c = 1.0f / (1.0f + expf(-(s / t)));
      conf[(size_t)m * gamma + kt] = c;
      cval[tid] = c;
    }
    __syncthreads();
    if (surv && tid == 0) {
      const int kn = min(G, gamma - k0);
      for (int q = 0; q < kn; ++q) {
        const int kt = k0 + q;
        a = kt == 0 ? cval[q] : a * cval[q];
        surv[(size_t)m * gamma + kt] = a;
      }
    }
    __syncthreads();
  }
}

// Prologue of the fused draft step in the same shape: w_h . h[m, k, :] for
// every position of request m into sh, and a grid-stride clear of the packed
// words the step kernels combine into.
template <int PJ>
__global__ __launch_bounds__(kRowThreads) void conf_prologue_rows_kernel(
    const uint16_t* __restrict__ h, const float* __restrict__ w_h, int gamma, int d,
    float* __restrict__ sh, uint4* __restrict__ words, size_t nclear) {
  constexpr int G = row_positions<PJ>();
  __shared__ float part[kRowWaves][G];
  const int m = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Rsrc rh = rsrc_of(h + (size_t)m * gamma * d, (size_t)gamma * d * 2);
  const Rsrc rw = rsrc_of(w_h, (size_t)d * 4);
  HDot<G, PJ> hd;
  hd.load(rh, rw, 0, gamma, d, tid);
  for (size_t i = (size_t)blockIdx.x * kRowThreads + tid; i < nclear;
       i += (size_t)gridDim.x * kRowThreads)
    words[i] = make_uint4(0u, 0u, 0u, 0u);
  for (int k0 = 0; k0 < gamma; k0 += G) {
    if (k0 > 0) hd.load(rh, rw, k0, gamma, d, tid);
    float acc[G];
    hd.sum(acc);
    float s;
    block_sums<G>(acc, part, tid & 63, wave, tid, s);
    if (tid < G && k0 + tid < gamma) sh[(size_t)m * gamma + k0 + tid] = s;
    __syncthreads();
  }
}

// The row kernels' conditions: 16-byte pieces of h and w_h (and of w_e and the
// W1 rows for the full head), at most two pieces per thread, and each
// request's h rows addressable with 32-bit offsets.
int row_pieces(const uint16_t* h, const float* w_conf, int gamma, int d) {
  auto a16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
  if (d % 8 != 0 || !a16(h) || !a16(w_conf)) return 0;
  if ((size_t)gamma * d * 2 >= kMaxRsrcBytes) return 0;
  const int n8 = d / 8;
  return n8 <= kRowThreads ? 1 : n8 <= 2 * kRowThreads ? 2 : 0;
}

// Prologue of the fused draft step: the token-independent part of every
// confidence logit, w_h . h[m, k, :], one workgroup of four wavefronts per
// (request, position) (each wavefront a quarter of the row, so every lane has
// only a few 16-byte pieces in flight; the quarters are added in a fixed
// order), and a grid-stride clear of the packed words the step kernels
// combine into.
constexpr int kProWaves = 4;

__global__ __launch_bounds__(64 * kProWaves) void conf_prologue_kernel(
    const uint16_t* __restrict__ h, const float* __restrict__ w_h, int n_dots, int d, int vec,
    float* __restrict__ sh, uint4* __restrict__ words, size_t nclear) {
  __shared__ float part[kProWaves];
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nclear;
       i += (size_t)gridDim.x * blockDim.x)
    words[i] = make_uint4(0u, 0u, 0u, 0u);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int t = blockIdx.x; t < n_dots; t += gridDim.x) {
    int lo, hi;
    part_range(d, kProWaves, wave, vec, lo, hi);
    const float s = wave_sum(dot_part(w_h, h + (size_t)t * d, lo, hi, vec, lane));
    if (lane == 0) part[wave] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
      float a = 0.0f;
#pragma unroll
      for (int j = 0; j < kProWaves; ++j) a += part[j];
      sh[t] = a;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void survival_kernel(const float* __restrict__ conf, int R,
                                                       int gamma, float* __restrict__ surv) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= R) return;
  float a = 1.0f;
  for (int k = 0; k < gamma; ++k) {
    const float c = conf[(size_t)m * gamma + k];
    a = k == 0 ? c : a * c;
    surv[(size_t)m * gamma + k] = a;
  }
}

}  // namespace

dspark_status launch_confidence(const uint16_t* h, const uint16_t* W1, const int32_t* anchors,
                                const int32_t* tokens, const float* w_conf, const float* sts_temp,
                                int R, int gamma, int d, int V, int r, float* conf, float* surv,
                                hipStream_t stream) {
  auto a16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
  const int vec_h = (d % 8 == 0) && a16(h) && a16(w_conf);
  const int vec_e = (r % 8 == 0) && (d % 4 == 0) && a16(W1) && a16(w_conf);
  const int pj = row_pieces(h, w_conf, gamma, d);
  if (pj > 0 && vec_e && r <= 512) {
    if (pj == 1)
      hipLaunchKernelGGL(confidence_rows_kernel<1>, dim3(R), dim3(kRowThreads), 0, stream, h, W1,
                         anchors, tokens, w_conf, sts_temp, gamma, d, V, r, conf, surv);
    else
      hipLaunchKernelGGL(confidence_rows_kernel<2>, dim3(R), dim3(kRowThreads), 0, stream, h, W1,
                         anchors, tokens, w_conf, sts_temp, gamma, d, V, r, conf, surv);
    return check_launch("confidence_rows_kernel");
  }
  // P wavefronts per position, G positions per round, at most 16 wavefronts.
  const int P = gamma < 16 ? 16 / gamma : 1;
  const int G = gamma < 16 ? gamma : 16;
  hipLaunchKernelGGL(confidence_kernel, dim3(R), dim3(64 * P * G), 0, stream, h, W1, anchors,
                     tokens, w_conf, sts_temp, gamma, d, V, r, P, vec_h, vec_e, conf, surv);
  return check_launch("confidence_kernel");
}

dspark_status launch_conf_prologue(const uint16_t* h, const float* w_h, int R, int gamma, int d,
                                   float* sh, unsigned long long* words, size_t n_words,
                                   hipStream_t stream) {
  auto a16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
  const int vec = (d % 8 == 0) && a16(h) && a16(w_h);
  const int n_dots = R * gamma;
  const size_t nclear = (n_words + 1) / 2;   // 16-byte stores (the area is rounded up)
  const int pj = row_pieces(h, w_h, gamma, d);
  if (pj > 0) {
    if (pj == 1)
      hipLaunchKernelGGL(conf_prologue_rows_kernel<1>, dim3(R), dim3(kRowThreads), 0, stream, h,
                         w_h, gamma, d, sh, reinterpret_cast<uint4*>(words), nclear);
    else
      hipLaunchKernelGGL(conf_prologue_rows_kernel<2>, dim3(R), dim3(kRowThreads), 0, stream, h,
                         w_h, gamma, d, sh, reinterpret_cast<uint4*>(words), nclear);
    return check_launch("conf_prologue_rows_kernel");
  }
  size_t blocks = (size_t)n_dots;
  const size_t cblocks = (nclear + 64 * kProWaves - 1) / (64 * kProWaves);
  if (cblocks > blocks) blocks = cblocks;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(conf_prologue_kernel, dim3((unsigned)blocks), dim3(64 * kProWaves), 0,
                     stream, h, w_h, n_dots, d, vec, sh, reinterpret_cast<uint4*>(words), nclear);
  return check_launch("conf_prologue_kernel");
}

dspark_status launch_survival(const float* conf, int R, int gamma, float* surv,
                              hipStream_t stream) {
  hipLaunchKernelGGL(survival_kernel, dim3((R + 255) / 256), dim3(256), 0, stream, conf, R,
                     gamma, surv);
  return check_launch("survival_kernel");
}

}  // namespace dspark
