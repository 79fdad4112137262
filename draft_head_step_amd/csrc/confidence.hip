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
// workgroup.  Each position's h row is split over P = 16 / gamma wavefronts
// (P >= 1), so that every lane has only a few 16-byte pieces of h (8 bf16, with
// the matching two float4 pieces of w_h) and issues them all at once; the
// token is read first so that the W1-row chain overlaps the h stream.  Lanes
// reduce with a fixed shuffle tree and the P parts are added in a fixed order,
// so results are deterministic.
#include <math.h>

#include "dspark_internal.h"

namespace dspark {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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
