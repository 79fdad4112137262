// RNN head for CDNA4 (gfx950): the Markov head's alternative sequential stage
// ([P3] part 01: a recurrent in-block state updated by a gate over the
// concatenated history state, previous-token embedding and backbone hidden
// state; [P1] section 二 design 1: the RNN head remembers the whole prefix).
// The pages give no equations; the reading implemented (the same as the CPU
// oracle's):
//   u_k = [s_{k-1}; e_k; h_k],  e_k = W1[x_{k-1}] (x_0 = anchor),  s_0 = 0
//   g_k = sigmoid(G u_k + b_g),  c_k = e_k + tanh(C u_k + b_c)
//   s_k = g_k * c_k + (1 - g_k) * s_{k-1},  z_k = base_k + bf16(s_k) W2
// with U = [G; C] stored [2r, 2r + d] bf16 (columns: the s, e and h blocks).
//
// A call is 2 gamma + 2 launches:
//   rnn_pre_kernel     P[m, k, :] = U[:, h block] h[m, k] + b for every
//                      position at once (the token-independent part, one GEMM
//                      of Rgamma x d by d x 2r on MFMA), and the clears;
//   per step k:
//     rnn_state_kernel the rest of the pre-activations, U[:, s and e blocks]
//                      [bf16(s_{k-1}); e_k] (a GEMM of R x 2r by 2r x 2r), then
//                      the gate, candidate and blend; the new state goes to
//                      the other half of a ping-pong pair (other workgroups
//                      still read the old one), in fp32 and in bf16;
//     the Markov step kernel with the bf16 state rows as its GEMM rows in
//                      place of the gathered W1 rows (bias, select, argmax);
//   last_tokens_kernel (in markov_step.hip).
//
// GEMM tiles: 32 x 32 outputs per workgroup of four wavefronts, each taking a
// quarter of K with operands loaded straight from memory in the MFMA's register
// layout (16 bytes per lane per K step); the quarters are added in a fixed
// order through LDS, so results are deterministic.
#include <math.h>

#include "markov_types.h"
#include "packed_words.h"

namespace dspark {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGW = 4;   // wavefronts per GEMM workgroup (K split four ways)

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// fp32 -> bf16 bits, to nearest even.
__device__ __forceinline__ uint16_t to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Sums the four wavefronts' partial tiles (NA accumulators each) in a fixed
// order; wavefront 0 returns with the totals.  `red` holds kGW * NA * 16 * 64 floats.
template <int NA>
__device__ __forceinline__ void reduce_waves(f32x16 (&acc)[NA], float* red, int wave, int lane) {
  if (wave > 0) {
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int q = 0; q < 16; ++q) red[(((wave - 1) * NA + a) * 16 + q) * 64 + lane] = acc[a][q];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 1; w < kGW; ++w)
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[a][q] += red[(((w - 1) * NA + a) * 16 + q) * 64 + lane];
  }
}

// K range [lo, hi) of wavefront w: quarters of K in whole 16-wide MFMA steps.
__device__ __forceinline__ void k_quarter(int K, int w, int& lo, int& hi) {
  const int steps = (K + 15) / 16;
  lo = 16 * (steps * w / kGW);
  hi = 16 * (steps * (w + 1) / kGW);
}

// 16 bytes of row `row` of a [rows, ld] bf16 matrix at column k (k % 8 == 0):
// zeros past the row's K columns or past the last row.
__device__ __forceinline__ u32x4 load8(const uint16_t* __restrict__ p, int ld, int row, int rows,
                                       int k, int K) {
  if (row >= rows || k >= K) return u32x4{0u, 0u, 0u, 0u};
  return *reinterpret_cast<const u32x4*>(p + (size_t)row * ld + k);
}

// P[t, n] = b[n] + sum_k h[t, k] U[n, 2r + k]  for t < Rgamma, n < 2r; the first
// workgroups also clear the packed words and the initial state.
__global__ __launch_bounds__(64 * kGW) void rnn_pre_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ U, const float* __restrict__ b,
    int M, int r, int d, float* __restrict__ P, uint4* __restrict__ clear, size_t nclear) {
  __shared__ float red[(kGW - 1) * 16 * 64];
  const int tid = threadIdx.x;
  const size_t nb = (size_t)gridDim.x * gridDim.y;
  const size_t bid = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
  for (size_t i = bid * blockDim.x + tid; i < nclear; i += nb * blockDim.x)
    clear[i] = make_uint4(0u, 0u, 0u, 0u);
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int t0 = blockIdx.x * 32, n0 = blockIdx.y * 32;
  const int ldu = 2 * r + d;
  const uint16_t* Uh = U + 2 * r;   // the h block: U[n, 2r + k]
  int lo, hi;
  k_quarter(d, wave, lo, hi);
  f32x16 acc[1] = {f32x16{}};
  // D[t][n]: A = h rows (t), B = U rows (n); lane (col, half) supplies row col,
  // K elements 8 half .. 8 half + 7 of each 16-wide step.
#pragma unroll 4
  for (int k = lo; k < hi; k += 16) {
    const u32x4 a = load8(h, d, t0 + col, M, k + 8 * half, d);
    const u32x4 bb = load8(Uh, ldu, n0 + col, 2 * r, k + 8 * half, d);
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(bb), acc[0], 0, 0, 0);
  }
  reduce_waves<1>(acc, red, wave, lane);
  if (wave == 0) {
    const int n = n0 + col;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int t = t0 + 8 * (q >> 2) + 4 * half + (q & 3);
      if (t < M) P[(size_t)t * 2 * r + n] = acc[0][q] + b[n];
    }
  }
}

// One gated update at step k for requests m0 .. m0+31 and units n0 .. n0+31:
// gate and candidate pre-activations over the s and e blocks (K = 2r), plus P,
// then s_new = g (e + tanh(pre_c)) + (1 - g) s_old.  At step 0 the old state is
// s_0 = 0 (s_old and sb_old NULL).
__global__ __launch_bounds__(64 * kGW) void rnn_state_kernel(
    const uint16_t* __restrict__ W1, const uint16_t* __restrict__ U, const float* __restrict__ P,
    const int32_t* __restrict__ anchors, const unsigned long long* __restrict__ prev, int sub,
    int R, int gamma, int V, int r, int d, int k, const float* __restrict__ s_old,
    const uint16_t* __restrict__ sb_old, float* __restrict__ s_new, uint16_t* __restrict__ sb_new) {
  __shared__ float red[(kGW - 1) * 2 * 16 * 64];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int m0 = blockIdx.x * 32, n0 = blockIdx.y * 32;
  const int ldu = 2 * r + d;
  // Token x_{k-1} of this lane's A row (request m0 + col); -1 if invalid.
  const int ma = m0 + col;
  int xa = -1;
  if (ma < R) {
    if (!prev) {
      const int a = anchors[ma];
      xa = (a >= 0 && a < V) ? a : -1;
    } else {
      xa = read_token(prev, ma, sub, V);
    }
  }
  int lo, hi;
  k_quarter(2 * r, wave, lo, hi);
  f32x16 acc[2] = {f32x16{}, f32x16{}};   // gate, candidate
#pragma unroll 4
  for (int kk = lo; kk < hi; kk += 16) {
    const int ke = kk + 8 * half;
    u32x4 a;
    if (ke < r) a = sb_old ? load8(sb_old, r, ma, R, ke, r) : u32x4{0u, 0u, 0u, 0u};
    else a = xa >= 0 ? load8(W1, r, xa, V, ke - r, r) : u32x4{0u, 0u, 0u, 0u};
    const u32x4 bg = load8(U, ldu, n0 + col, 2 * r, ke, 2 * r);
    const u32x4 bc = load8(U, ldu, r + n0 + col, 2 * r, ke, 2 * r);
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(bg), acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(bc), acc[1], 0, 0, 0);
  }
  reduce_waves<2>(acc, red, wave, lane);
  if (wave != 0) return;
  // The last unit tile may run past r (r % 32 == 16): those lanes still take
  // part in the shuffles below and store nothing.
  const int n = n0 + col;
  const bool n_ok = n < r;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int ml = 8 * (q >> 2) + 4 * half + (q & 3);
    const int m = m0 + ml;
    const int xm = __shfl(xa, ml);
    if (m >= R || !n_ok) continue;
    const size_t pt = ((size_t)m * gamma + k) * 2 * r;
    const float pg = acc[0][q] + P[pt + n];
    const float pc = acc[1][q] + P[pt + r + n];
    const float e = xm >= 0 ? __uint_as_float((uint32_t)W1[(size_t)xm * r + n] << 16) : 0.0f;
    const float g = 1.0f / (1.0f + expf(-pg));
    const float c = e + tanhf(pc);
    const float so = s_old ? s_old[(size_t)m * r + n] : 0.0f;
    const float sn = g * c + (1.0f - g) * so;
    s_new[(size_t)m * r + n] = sn;
    sb_new[(size_t)m * r + n] = to_bf16(sn);
  }
}

}  // namespace

size_t rnn_workspace_bytes(int R, int gamma, int V, int r) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t words = plan_markov(R, gamma, V, r, DSPARK_GREEDY, false).ws_bytes;
  const size_t P = (size_t)R * gamma * 2 * r * sizeof(float);
  const size_t s32 = (size_t)2 * R * r * sizeof(float);
  const size_t s16 = (size_t)2 * R * r * sizeof(uint16_t);
  return up(words) + up(P) + up(s32) + up(s16);
}

RnnBuffers rnn_buffers(void* workspace, int R, int gamma, int V, int r) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  unsigned char* ws = reinterpret_cast<unsigned char*>(workspace);
  const size_t words = plan_markov(R, gamma, V, r, DSPARK_GREEDY, false).ws_bytes;
  const size_t pb = (size_t)R * gamma * 2 * r * sizeof(float);
  const size_t s32 = (size_t)2 * R * r * sizeof(float);
  RnnBuffers B;
  B.words = reinterpret_cast<unsigned long long*>(ws);
  B.words_bytes = words;
  B.P = reinterpret_cast<float*>(ws + up(words));
  float* s = reinterpret_cast<float*>(ws + up(words) + up(pb));
  uint16_t* sb = reinterpret_cast<uint16_t*>(ws + up(words) + up(pb) + up(s32));
  B.s[0] = s;
  B.s[1] = s + (size_t)R * r;
  B.sb[0] = sb;
  B.sb[1] = sb + (size_t)R * r;
  return B;
}

dspark_status launch_rnn_pre(const uint16_t* h, const uint16_t* U, const float* b, int R,
                             int gamma, int r, int d, const RnnBuffers& B, size_t n_words,
                             hipStream_t stream) {
  const int M = R * gamma;
  const dim3 grid((M + 31) / 32, (2 * r) / 32);
  hipLaunchKernelGGL(rnn_pre_kernel, grid, dim3(64 * kGW), 0, stream, h, U, b, M, r, d, B.P,
                     reinterpret_cast<uint4*>(B.words), (n_words + 1) / 2);
  return check_launch("rnn_pre_kernel");
}

dspark_status launch_rnn_state(const uint16_t* W1, const uint16_t* U, const int32_t* anchors,
                               const unsigned long long* prev, int sub, int R, int gamma, int V,
                               int r, int d, int k, const RnnBuffers& B, float* s_out,
                               hipStream_t stream) {
  const dim3 grid((R + 31) / 32, (r + 31) / 32);
  const int o = k & 1, nw = (k + 1) & 1;   // state before step k in half o, after it in nw
  hipLaunchKernelGGL(rnn_state_kernel, grid, dim3(64 * kGW), 0, stream, W1, U, B.P, anchors, prev,
                     sub, R, gamma, V, r, d, k, k == 0 ? nullptr : B.s[o],
                     k == 0 ? nullptr : B.sb[o], s_out ? s_out : B.s[nw], B.sb[nw]);
  return check_launch("rnn_state_kernel");
}

}  // namespace dspark
