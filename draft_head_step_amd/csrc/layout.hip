// W2 storage conversion for CDNA4 (gfx950).
//
// The step kernels take the r x V projection W2 of [P1] section 二 design 1
// (Markov-head equation) stored column by column: element (i, v) at
// W2[v * r + i], so that each vocabulary entry's r values are contiguous (the
// MFMA operand layout).  A caller holding W2 row by row (element (i, v) at
// w2_rv[i * V + v]) converts it once, when the weights are loaded.
//
// A tiled transpose through LDS: a workgroup of 256 threads moves a 64 x 64
// tile, reading 64 consecutive v of each i (128 bytes per row) and writing 64
// consecutive i of each v; the LDS rows are padded by one element so the
// transposed reads spread over the banks.  Tails in either dimension are
// bounds-checked.  Off the drafting path, bound by HBM.
#include "dspark_internal.h"

namespace dspark {
namespace {

constexpr int kTT = 64;        // tile edge
constexpr int kTThreads = 256;

__global__ __launch_bounds__(kTThreads) void w2_store_from_rv_kernel(const uint16_t* __restrict__ src,
                                                                    uint16_t* __restrict__ dst,
                                                                    int r, int V) {
  __shared__ uint16_t tile[kTT][kTT + 1];
  const int v0 = blockIdx.x * kTT;
  const int i0 = blockIdx.y * kTT;
  const int tx = threadIdx.x & (kTT - 1);
  const int ty = threadIdx.x / kTT;    // 0..3
#pragma unroll
  for (int j = 0; j < kTT; j += kTThreads / kTT) {
    const int i = i0 + ty + j;
    const int v = v0 + tx;
    if (i < r && v < V) tile[ty + j][tx] = src[(size_t)i * V + v];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kTT; j += kTThreads / kTT) {
    const int v = v0 + ty + j;
    const int i = i0 + tx;
    if (i < r && v < V) dst[(size_t)v * r + i] = tile[tx][ty + j];
  }
}

}  // namespace

dspark_status launch_w2_store_from_rv(const uint16_t* w2_rv, uint16_t* w2_store, int r, int V,
                                      hipStream_t stream) {
  const dim3 grid((unsigned)((V + kTT - 1) / kTT), (unsigned)((r + kTT - 1) / kTT));
  hipLaunchKernelGGL(w2_store_from_rv_kernel, grid, dim3(kTThreads), 0, stream, w2_rv, w2_store,
                     r, V);
  return check_launch("w2_store_from_rv_kernel");
}

}  // namespace dspark
