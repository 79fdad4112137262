// Markov-head refinement step for CDNA4 (gfx950).
//
// One draft position k of every request at once ([P1] section 二 design 1,
// Markov-head equation; [P3] part 01; [P4] logits bias):
//   e_m  = W1[x_{k-1,m}, :]                      gather, x_0 = anchor
//   z_mv = base[m, k, v] + sum_i e_mi * W2(i, v)  bf16 MFMA, fp32 accumulation
//   x_k  = argmax_v z_mv  |  argmax_v z_mv / T - ln(-ln u_mv)
//
// Design (HBM-bound: W2, base and the uniforms are each read once per step):
//   * The bias GEMM is computed transposed, bias^T[v, m] = W2^T[v, :] . e_m, so
//     that both MFMA operands are K-contiguous rows of the [V, r] stores of W1
//     and W2, and so that every lane's accumulators cover four consecutive
//     vocabulary entries of one request: the base / uniform reads of the
//     epilogue are 16-byte vector loads in exactly the accumulator layout.
//   * Each wave owns 32 requests and keeps their gathered W1 rows (the MFMA B
//     operand) in registers for the whole kernel.  A workgroup of NW waves
//     shares 32-column chunks of W2 staged through LDS (double-buffered, rows
//     padded by 16 bytes so the MFMA A-operand reads hit distinct banks).
//   * Each workgroup walks a contiguous group of chunks and keeps a running
//     (max, argmax) per request; a second tiny kernel reduces the per-group
//     partials to the token.  No float atomics: the result is deterministic.
//   * Workgroup ids are decoded so that the R-blocks sharing a V group land on
//     the same XCD (ids congruent mod 8) and are dispatched together, so the
//     second and later reads of a W2 chunk hit that XCD's L2.
#include <math.h>

#include "dspark_internal.h"

namespace dspark {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 32;         // vocabulary rows of W2 per MFMA tile
constexpr int kMaxGroups = 1024;   // upper bound on V groups (sizes the workspace)

__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// Running argmax with smallest-index tie-break.
__device__ __forceinline__ void merge_best(float& bv, int& bi, float ov, int oi) {
  if (ov > bv || (ov == bv && oi < bi)) {
    bv = ov;
    bi = oi;
  }
}

__device__ __forceinline__ float gumbel_noise(float u) {
  // -ln(-ln u); logf is accurate to a few ulp relative to its result, so w stays
  // accurate for u close to 1 where the noise is largest.
  const float w = -logf(u);
  return -logf(w);
}

template <int RK, int NW, int MODE>
__global__ __launch_bounds__(NW * 64) void markov_step_kernel(
    const uint16_t* __restrict__ W1, const uint16_t* __restrict__ W2,
    const float* __restrict__ base, const float* __restrict__ unif,
    const int32_t* __restrict__ prev, int prev_stride, int R, int gamma, int V, int r, int k,
    float inv_t, int n_rblocks, int n_vgroups, int cpg, int n_chunks, int vec4,
    float2* __restrict__ partials, float* __restrict__ bias_out) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int KS = RK / 16;                          // MFMA K steps at the compiled bucket
  constexpr int NT = NW * 64;                          // threads per workgroup
  constexpr int PMAX = (4 * RK + NT - 1) / NT;         // 16-byte W2 pieces per thread per chunk

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int col = lane & 31;

  // XCD-aware decode of the workgroup id.
  const int id = blockIdx.x;
  const int q = id >> 3;
  const int rb = q % n_rblocks;
  const int vg = (q / n_rblocks) * 8 + (id & 7);
  if (vg >= n_vgroups) return;
  const int c_begin = vg * cpg;
  const int c_end = min(c_begin + cpg, n_chunks);

  const int ksteps = r >> 4;
  const int pitch = r + 8;                              // bf16 per LDS row (16-byte pad)
  const int buf_elems = kChunk * pitch;
  uint16_t* lds = reinterpret_cast<uint16_t*>(smem);

  // ---- gather: this lane's request row of W1 becomes the MFMA B operand ----
  const int m = rb * (NW * 32) + wave * 32 + col;
  const bool m_ok = m < R;
  bf16x8 e[KS];
  {
    int x = m_ok ? prev[(size_t)m * prev_stride] : 0;
    x = min(max(x, 0), V - 1);                          // out-of-range ids never fault
    const uint16_t* er = W1 + (size_t)x * r + half * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (s < ksteps && m_ok) {
        e[s] = ld_bf16x8(er + s * 16);
      } else {
        e[s] = bf16x8{};
      }
    }
  }

  // ---- W2 chunk staging: piece p of a chunk is 8 consecutive bf16 of one row ----
  const int pieces = 4 * r;                            // 16-byte pieces per chunk (32 rows)
  const int ppr = r >> 3;                              // pieces per row
  int loff[PMAX];
  int prow[PMAX];
#pragma unroll
  for (int j = 0; j < PMAX; ++j) {
    const int p = tid + j * NT;
    const int row = p / ppr;
    prow[j] = p < pieces ? row : kChunk;                // kChunk marks "no piece"
    loff[j] = row * pitch + (p - row * ppr) * 8;
  }
  u32x4 stage[PMAX];
  auto load_chunk = [&](int c) {
    const int v0 = c * kChunk;
    const uint16_t* src = W2 + (size_t)v0 * r;
#pragma unroll
    for (int j = 0; j < PMAX; ++j) {
      const int p = tid + j * NT;
      if (prow[j] < kChunk && v0 + prow[j] < V) {
        stage[j] = *reinterpret_cast<const u32x4*>(src + (size_t)p * 8);
      } else {
        stage[j] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_chunk = [&](int b) {
    uint16_t* dst = lds + b * buf_elems;
#pragma unroll
    for (int j = 0; j < PMAX; ++j) {
      if (prow[j] < kChunk) *reinterpret_cast<u32x4*>(dst + loff[j]) = stage[j];
    }
  };

  const size_t row_off = ((size_t)(m_ok ? m : 0) * gamma + k) * (size_t)V;
  const float* brow = base + row_off;
  const float* urow = (MODE == DSPARK_SAMPLE) ? unif + row_off : nullptr;
  float* bout = bias_out ? bias_out + row_off : nullptr;

  float best = -INFINITY;
  int best_i = 0x7fffffff;

  if (c_begin < c_end) load_chunk(c_begin);
  for (int c = c_begin; c < c_end; ++c) {
    const int b = (c - c_begin) & 1;
    store_chunk(b);
    __syncthreads();
    if (c + 1 < c_end) load_chunk(c + 1);

    // Epilogue inputs first, so their HBM latency overlaps the MFMAs.
    const int v0 = c * kChunk;
    float bv[16];
    float uv[16];
    if (m_ok) {
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const int v = v0 + 8 * jq + 4 * half;
        if (vec4 && v + 3 < V) {
          const float4 t = *reinterpret_cast<const float4*>(brow + v);
          bv[4 * jq + 0] = t.x; bv[4 * jq + 1] = t.y; bv[4 * jq + 2] = t.z; bv[4 * jq + 3] = t.w;
          if (MODE == DSPARK_SAMPLE) {
            const float4 w = *reinterpret_cast<const float4*>(urow + v);
            uv[4 * jq + 0] = w.x; uv[4 * jq + 1] = w.y; uv[4 * jq + 2] = w.z; uv[4 * jq + 3] = w.w;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool ok = v + i < V;
            bv[4 * jq + i] = ok ? brow[v + i] : 0.f;
            if (MODE == DSPARK_SAMPLE) uv[4 * jq + i] = ok ? urow[v + i] : 0.5f;
          }
        }
      }
    }

    // Bias tile: 32 vocabulary rows x 32 requests, K = r.
    const uint16_t* abase = lds + b * buf_elems + col * pitch + half * 8;
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (s < ksteps) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(abase + s * 16);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, e[s], acc, 0, 0, 0);
      }
    }

    // Fused bias-add + select.  Lane holds rows v0 + 8*jq + 4*half + i of column m.
    if (m_ok) {
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const int v = v0 + 8 * jq + 4 * half;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int vi = v + i;
          if (vi < V) {
            const float z = bv[4 * jq + i] + acc[4 * jq + i];
            float s;
            if (MODE == DSPARK_SAMPLE) {
              s = z * inv_t + gumbel_noise(uv[4 * jq + i]);
            } else {
              s = z;
            }
            if (s > best) {
              best = s;
              best_i = vi;
            }
          }
        }
        if (bout) {
          if (vec4 && v + 3 < V) {
            *reinterpret_cast<float4*>(bout + v) =
                make_float4(acc[4 * jq], acc[4 * jq + 1], acc[4 * jq + 2], acc[4 * jq + 3]);
          } else {
            for (int i = 0; i < 4; ++i)
              if (v + i < V) bout[v + i] = acc[4 * jq + i];
          }
        }
      }
    }
  }

  // Lanes l and l^32 hold the same request: merge, then one lane writes the partial.
  const float ov = __shfl_xor(best, 32);
  const int oi = __shfl_xor(best_i, 32);
  merge_best(best, best_i, ov, oi);
  if (m_ok && half == 0) {
    partials[(size_t)m * n_vgroups + vg] = make_float2(best, __int_as_float(best_i));
  }
}

// One wave per request: reduce the per-group partials to x_k.
__global__ __launch_bounds__(256) void argmax_reduce_kernel(const float2* __restrict__ partials,
                                                            int R, int n_vgroups, int V,
                                                            int gamma, int k,
                                                            int32_t* __restrict__ tokens) {
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (m >= R) return;
  float best = -INFINITY;
  int best_i = 0x7fffffff;
  for (int g = lane; g < n_vgroups; g += 64) {
    const float2 p = partials[(size_t)m * n_vgroups + g];
    merge_best(best, best_i, p.x, __float_as_int(p.y));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(best, off);
    const int oi = __shfl_xor(best_i, off);
    merge_best(best, best_i, ov, oi);
  }
  if (lane == 0) tokens[(size_t)m * gamma + k] = best_i < V ? best_i : 0;
}

template <int RK, int NW, int MODE>
dspark_status launch_step_t(const MarkovPlan& p, dim3 grid, size_t lds, hipStream_t stream,
                            const uint16_t* W1, const uint16_t* W2, const float* base,
                            const float* unif, const int32_t* prev, int prev_stride, int R,
                            int gamma, int V, int r, int k, float inv_t, int vec4,
                            float2* partials, float* bias_out) {
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&markov_step_kernel<RK, NW, MODE>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)(2 * kChunk * (RK + 8) * 2)) != hipSuccess) {
      return fail(DSPARK_EDEVICE, "hipFuncSetAttribute failed for the Markov step kernel");
    }
    attr_set = true;
  }
  hipLaunchKernelGGL((markov_step_kernel<RK, NW, MODE>), grid, dim3(NW * 64), lds, stream, W1,
                     W2, base, unif, prev, prev_stride, R, gamma, V, r, k, inv_t, p.n_rblocks,
                     p.n_vgroups, p.cpg, p.n_chunks, vec4, partials, bias_out);
  return check_launch("markov_step_kernel");
}

template <int RK, int NW>
dspark_status dispatch_mode(int mode, const MarkovPlan& p, dim3 grid, size_t lds,
                            hipStream_t stream, const uint16_t* W1, const uint16_t* W2,
                            const float* base, const float* unif, const int32_t* prev,
                            int prev_stride, int R, int gamma, int V, int r, int k, float inv_t,
                            int vec4, float2* partials, float* bias_out) {
  if (mode == DSPARK_SAMPLE)
    return launch_step_t<RK, NW, DSPARK_SAMPLE>(p, grid, lds, stream, W1, W2, base, unif, prev,
                                                prev_stride, R, gamma, V, r, k, inv_t, vec4,
                                                partials, bias_out);
  return launch_step_t<RK, NW, DSPARK_GREEDY>(p, grid, lds, stream, W1, W2, base, unif, prev,
                                              prev_stride, R, gamma, V, r, k, inv_t, vec4,
                                              partials, bias_out);
}

template <int RK>
dspark_status dispatch_nw(int mode, const MarkovPlan& p, dim3 grid, size_t lds,
                          hipStream_t stream, const uint16_t* W1, const uint16_t* W2,
                          const float* base, const float* unif, const int32_t* prev,
                          int prev_stride, int R, int gamma, int V, int r, int k, float inv_t,
                          int vec4, float2* partials, float* bias_out) {
  switch (p.nw) {
    case 1:
      return dispatch_mode<RK, 1>(mode, p, grid, lds, stream, W1, W2, base, unif, prev,
                                  prev_stride, R, gamma, V, r, k, inv_t, vec4, partials, bias_out);
    case 2:
      return dispatch_mode<RK, 2>(mode, p, grid, lds, stream, W1, W2, base, unif, prev,
                                  prev_stride, R, gamma, V, r, k, inv_t, vec4, partials, bias_out);
    case 4:
      return dispatch_mode<RK, 4>(mode, p, grid, lds, stream, W1, W2, base, unif, prev,
                                  prev_stride, R, gamma, V, r, k, inv_t, vec4, partials, bias_out);
    default:
      return dispatch_mode<RK, 8>(mode, p, grid, lds, stream, W1, W2, base, unif, prev,
                                  prev_stride, R, gamma, V, r, k, inv_t, vec4, partials, bias_out);
  }
}

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  return (s && *s) ? atoi(s) : dflt;
}

}  // namespace

MarkovPlan plan_markov(int R, int gamma, int V, int r) {
  (void)gamma;
  MarkovPlan p{};
  p.rk = r <= 64 ? 64 : r <= 128 ? 128 : r <= 256 ? 256 : 512;
  const int waves_needed = (R + 31) / 32;
  int nw = waves_needed >= 8 ? 8 : waves_needed >= 4 ? 4 : waves_needed >= 2 ? 2 : 1;
  const int nw_env = env_int("DSPARK_MARKOV_NW", 0);
  if (nw_env == 1 || nw_env == 2 || nw_env == 4 || nw_env == 8) nw = nw_env;
  p.nw = nw;
  p.n_rblocks = (R + 32 * nw - 1) / (32 * nw);
  p.n_chunks = (V + kChunk - 1) / kChunk;
  const int max_groups = p.n_chunks < kMaxGroups ? p.n_chunks : kMaxGroups;
  // Default: about 256 workgroups in flight (one per CU), split between the R blocks.
  int target = env_int("DSPARK_MARKOV_WG", 256);
  if (target < 8) target = 8;
  int groups = (target + p.n_rblocks - 1) / p.n_rblocks;
  groups = (groups + 7) / 8 * 8;
  if (groups > max_groups) groups = max_groups;
  if (groups < 1) groups = 1;
  p.cpg = (p.n_chunks + groups - 1) / groups;
  p.n_vgroups = (p.n_chunks + p.cpg - 1) / p.cpg;
  p.ws_bytes = (size_t)R * (size_t)max_groups * sizeof(float2);
  return p;
}

dspark_status launch_markov_draft(const uint16_t* W1, const uint16_t* W2, const float* base,
                                  const int32_t* anchors, int R, int gamma, int V, int r,
                                  int mode, float temperature, const float* uniforms,
                                  int32_t* tokens, float* bias_out, void* workspace,
                                  const dspark_step_events* events, hipStream_t stream) {
  const MarkovPlan p = plan_markov(R, gamma, V, r);
  float2* partials = reinterpret_cast<float2*>(workspace);
  const int padded_groups = (p.n_vgroups + 7) / 8 * 8;
  const dim3 grid(padded_groups * p.n_rblocks);
  const size_t lds = 2 * kChunk * (size_t)(r + 8) * 2;
  const float inv_t = mode == DSPARK_SAMPLE ? 1.0f / temperature : 1.0f;
  auto a16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
  const int vec4 = (V % 4 == 0) && a16(base) && (!uniforms || a16(uniforms)) &&
                   (!bias_out || a16(bias_out));
  for (int k = 0; k < gamma; ++k) {
    const int32_t* prev = k == 0 ? anchors : tokens + (k - 1);
    const int prev_stride = k == 0 ? 1 : gamma;
    if (events && k < events->count && events->begin && events->begin[k]) {
      if (hipEventRecord(reinterpret_cast<hipEvent_t>(events->begin[k]), stream) != hipSuccess)
        return fail(DSPARK_EDEVICE, "hipEventRecord failed");
    }
    dspark_status st;
    switch (p.rk) {
      case 64:
        st = dispatch_nw<64>(mode, p, grid, lds, stream, W1, W2, base, uniforms, prev,
                             prev_stride, R, gamma, V, r, k, inv_t, vec4, partials, bias_out);
        break;
      case 128:
        st = dispatch_nw<128>(mode, p, grid, lds, stream, W1, W2, base, uniforms, prev,
                              prev_stride, R, gamma, V, r, k, inv_t, vec4, partials, bias_out);
        break;
      case 256:
        st = dispatch_nw<256>(mode, p, grid, lds, stream, W1, W2, base, uniforms, prev,
                              prev_stride, R, gamma, V, r, k, inv_t, vec4, partials, bias_out);
        break;
      default:
        st = dispatch_nw<512>(mode, p, grid, lds, stream, W1, W2, base, uniforms, prev,
                              prev_stride, R, gamma, V, r, k, inv_t, vec4, partials, bias_out);
        break;
    }
    if (st != DSPARK_OK) return st;
    if (events && k < events->count && events->end && events->end[k]) {
      if (hipEventRecord(reinterpret_cast<hipEvent_t>(events->end[k]), stream) != hipSuccess)
        return fail(DSPARK_EDEVICE, "hipEventRecord failed");
    }
    hipLaunchKernelGGL(argmax_reduce_kernel, dim3((R + 3) / 4), dim3(256), 0, stream, partials,
                       R, p.n_vgroups, V, gamma, k, tokens);
    st = check_launch("argmax_reduce_kernel");
    if (st != DSPARK_OK) return st;
  }
  return DSPARK_OK;
}

}  // namespace dspark
