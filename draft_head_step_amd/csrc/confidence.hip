// Confidence head, STS calibration and prefix survival for CDNA4 (gfx950).
//
// [P1] section 二 design 2 (confidence head, sequential temperature scaling,
// survival products); [P4] (fp32 confidences):
//   s_{m,k} = w_h . h_{m,k} + w_e . W1[x_{k-1}]     (x_0 = anchor)
//   c_{m,k} = 1 / (1 + exp(-s_{m,k} / T_k))
//   a_{m,j} = c_{m,1} * ... * c_{m,j}               (fp32, left to right)
//
// The work is a dot product of length d + r per (request, position), bound by
// the HBM read of h.  One workgroup handles all gamma positions of one
// request (one wavefront per position), so the survival products are a short
// sequential tail in the same workgroup.  Each lane streams 16-byte pieces of h
// (8 bf16) with the matching two float4 pieces of w_h, four pieces in flight;
// the wavefront reduces with a fixed shuffle tree, so results are deterministic.
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

// Sum of w[i] * x[i] (x bf16) over this lane's share of [0, n): 16-byte pieces
// strided by the wavefront, four independent partial sums so that several
// loads are in flight per lane.
__device__ __forceinline__ float dot_part(const float* __restrict__ w,
                                          const uint16_t* __restrict__ x, int n, bool vec,
                                          int lane) {
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  int tail_from = 0;
  if (vec) {
    const int n8 = n >> 3;
    int p = lane;
    for (; p + 192 < n8; p += 256) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int pp = p + 64 * u;
        const u32x4 hv = *reinterpret_cast<const u32x4*>(x + 8 * pp);
        const float4 w0 = *reinterpret_cast<const float4*>(w + 8 * pp);
        const float4 w1 = *reinterpret_cast<const float4*>(w + 8 * pp + 4);
        float a = acc[u];
        a = fmaf(w0.x, bf16_lo(hv.x), a);
        a = fmaf(w0.y, bf16_hi(hv.x), a);
        a = fmaf(w0.z, bf16_lo(hv.y), a);
        a = fmaf(w0.w, bf16_hi(hv.y), a);
        a = fmaf(w1.x, bf16_lo(hv.z), a);
        a = fmaf(w1.y, bf16_hi(hv.z), a);
        a = fmaf(w1.z, bf16_lo(hv.w), a);
        a = fmaf(w1.w, bf16_hi(hv.w), a);
        acc[u] = a;
      }
    }
    for (; p < n8; p += 64) {
      const u32x4 hv = *reinterpret_cast<const u32x4*>(x + 8 * p);
      const float4 w0 = *reinterpret_cast<const float4*>(w + 8 * p);
      const float4 w1 = *reinterpret_cast<const float4*>(w + 8 * p + 4);
      float a = acc[0];
      a = fmaf(w0.x, bf16_lo(hv.x), a);
      a = fmaf(w0.y, bf16_hi(hv.x), a);
      a = fmaf(w0.z, bf16_lo(hv.y), a);
      a = fmaf(w0.w, bf16_hi(hv.y), a);
      a = fmaf(w1.x, bf16_lo(hv.z), a);
      a = fmaf(w1.y, bf16_hi(hv.z), a);
      a = fmaf(w1.z, bf16_lo(hv.w), a);
      a = fmaf(w1.w, bf16_hi(hv.w), a);
      acc[0] = a;
    }
    tail_from = 8 * n8;
  }
  for (int i = tail_from + lane; i < n; i += 64)
    acc[1] = fmaf(w[i], __uint_as_float((unsigned)x[i] << 16), acc[1]);
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// One workgroup per request, one wavefront per draft position (looping when
// gamma exceeds the wavefront count).
__global__ __launch_bounds__(1024) void confidence_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ W1,
    const int32_t* __restrict__ anchors, const int32_t* __restrict__ tokens,
    const float* __restrict__ w_conf, const float* __restrict__ sts_temp, int gamma, int d,
    int V, int r, int vec_h, int vec_e, float* __restrict__ conf, float* __restrict__ surv) {
  __shared__ float cval[kMaxGamma];
  const int m = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const float* w_h = w_conf;
  const float* w_e = w_conf + d;
  float a = 1.0f;   // running survival product (thread 0)
  for (int k0 = 0; k0 < gamma; k0 += kMaxGamma) {
    const int kn = min(kMaxGamma, gamma - k0);
    for (int kk = wave; kk < kn; kk += nwaves) {
      const int k = k0 + kk;
      int x = k == 0 ? anchors[m] : tokens[(size_t)m * gamma + k - 1];
      x = min(max(x, 0), V - 1);
      float part = dot_part(w_h, h + ((size_t)m * gamma + k) * d, d, vec_h, lane);
      part += dot_part(w_e, W1 + (size_t)x * r, r, vec_e, lane);
      const float s = wave_sum(part);
      if (lane == 0) {
        const float t = sts_temp ? sts_temp[k] : 1.0f;
        const float c = 1.0f / (1.0f + expf(-(s / t)));
        conf[(size_t)m * gamma + k] = c;
        cval[kk] = c;
      }
    }
    __syncthreads();
    if (surv && threadIdx.x == 0) {
      for (int kk = 0; kk < kn; ++kk) {
        const int k = k0 + kk;
        a = k == 0 ? cval[kk] : a * cval[kk];
        surv[(size_t)m * gamma + k] = a;
      }
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
  const int waves = gamma < 16 ? gamma : 16;
  hipLaunchKernelGGL(confidence_kernel, dim3(R), dim3(64 * waves), 0, stream, h, W1, anchors,
                     tokens, w_conf, sts_temp, gamma, d, V, r, vec_h, vec_e, conf, surv);
  return check_launch("confidence_kernel");
}

dspark_status launch_survival(const float* conf, int R, int gamma, float* surv,
                              hipStream_t stream) {
  hipLaunchKernelGGL(survival_kernel, dim3((R + 255) / 256), dim3(256), 0, stream, conf, R,
                     gamma, surv);
  return check_launch("survival_kernel");
}

}  // namespace dspark
