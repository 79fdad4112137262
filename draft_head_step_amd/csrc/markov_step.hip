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

// Workgroup barrier that orders LDS only.  __syncthreads() also fences global
// memory, which makes the compiler wait for every outstanding global load
// (vmcnt(0)) at each barrier and would drain the prefetch pipeline; the waves
// here share nothing through global memory inside a launch.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Running argmax with smallest-index tie-break.
__device__ __forceinline__ void merge_best(float& bv, int& bi, float ov, int oi) {
  if (ov > bv || (ov == bv && oi < bi)) {
    bv = ov;
    bi = oi;
  }
}

// Prefetch depths, in 32-column chunks, of W2 (register staging ring) and of
// the base / uniform epilogue inputs.  With rank 512 the gathered W1 rows alone
// take 128 VGPRs per lane; the 4-wave variant runs one wave per SIMD and spends
// the registers that frees on deeper prefetch instead.
template <int RK, int NW>
constexpr bool deep_variant() { return RK == 512 && NW == 4; }
template <int RK, int NW>
constexpr int w2_depth() { return deep_variant<RK, NW>() ? 2 : 1; }
template <int RK, int NW>
constexpr int epi_depth() { return deep_variant<RK, NW>() ? 3 : 1; }
constexpr int lcm_small(int a, int b) { return (a % b == 0) ? a : (b % a == 0) ? b : a * b; }

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
  constexpr int PPR = RK / 8;                          // 16-byte pieces per LDS row
  constexpr int PIECES = kChunk * PPR;                 // pieces per chunk
  constexpr int PMAX = (PIECES + NT - 1) / NT;         // pieces per thread per chunk
  constexpr int PITCH = RK + 8;                        // bf16 per LDS row (16-byte pad)
  constexpr int BUF = kChunk * PITCH;                  // bf16 per LDS buffer
  constexpr int WD = w2_depth<RK, NW>();                // W2 staging slots (chunks in flight)
  constexpr int PD = epi_depth<RK, NW>();
  constexpr int NS = PD + 1;                           // epilogue register slots
  constexpr int UNR = lcm_small(WD, NS);               // unroll keeping slot indices static

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
  const int rpieces = r >> 3;                          // pieces at or beyond are stored as zeros
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

  // ---- W2 chunk staging: piece p = (row, 8-element column block) of a chunk ----
  u32x4 stage[WD][PMAX];
  auto load_chunk = [&](int c, u32x4 (&st)[PMAX]) {
    const int v0 = c * kChunk;
#pragma unroll
    for (int j = 0; j < PMAX; ++j) {
      const int p = tid + j * NT;
      const int row = p / PPR;
      const int cp = p % PPR;
      if (p < PIECES && cp < rpieces && v0 + row < V) {
        st[j] = *reinterpret_cast<const u32x4*>(W2 + (size_t)(v0 + row) * r + cp * 8);
      } else {
        st[j] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_chunk = [&](int b, const u32x4 (&st)[PMAX]) {
    uint16_t* dst = lds + b * BUF;
#pragma unroll
    for (int j = 0; j < PMAX; ++j) {
      const int p = tid + j * NT;
      if (p < PIECES) *reinterpret_cast<u32x4*>(dst + (p / PPR) * PITCH + (p % PPR) * 8) = st[j];
    }
  };

  const size_t row_off = ((size_t)(m_ok ? m : 0) * gamma + k) * (size_t)V;
  const float* brow = base + row_off;
  const float* urow = (MODE == DSPARK_SAMPLE) ? unif + row_off : nullptr;
  float* bout = bias_out ? bias_out + row_off : nullptr;

  // Epilogue inputs of chunk c in the accumulator layout: element 4*jq + i is
  // vocabulary entry c*32 + 8*jq + 4*half + i of this lane's request.
  float eb[NS][16];
  float eu[NS][16];
  auto load_epi = [&](int c, float (&bv)[16], float (&uv)[16]) {
    if (!m_ok) return;
    const int v0 = c * kChunk;
    if (vec4 && v0 + kChunk <= V) {
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const int v = v0 + 8 * jq + 4 * half;
        const float4 t = *reinterpret_cast<const float4*>(brow + v);
        bv[4 * jq + 0] = t.x; bv[4 * jq + 1] = t.y; bv[4 * jq + 2] = t.z; bv[4 * jq + 3] = t.w;
        if (MODE == DSPARK_SAMPLE) {
          const float4 w = *reinterpret_cast<const float4*>(urow + v);
          uv[4 * jq + 0] = w.x; uv[4 * jq + 1] = w.y; uv[4 * jq + 2] = w.z; uv[4 * jq + 3] = w.w;
        }
      }
    } else {
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int v = v0 + 8 * jq + 4 * half + i;
          const bool ok = v < V;
          bv[4 * jq + i] = ok ? brow[v] : 0.f;
          if (MODE == DSPARK_SAMPLE) uv[4 * jq + i] = ok ? urow[v] : 0.5f;
        }
      }
    }
  };

  float best = -INFINITY;
  int best_i = 0x7fffffff;
  // Selection score of one element.  Sampling: z/T - ln(-ln u) with the hardware
  // base-2 logarithm (relative error ~1e-7 over the whole open unit interval).
  auto score = [&](float b, float a, float u) {
    const float z = b + a;
    if (MODE == DSPARK_SAMPLE) {
      constexpr float kLn2 = 0.693147180559945309f;
      const float w = -kLn2 * __builtin_amdgcn_logf(u);      // -ln u  (> 0)
      return fmaf(-kLn2, __builtin_amdgcn_logf(w), z * inv_t);
    }
    return z;
  };

  // One chunk: stage W2 into LDS, prefetch, bias tile on MFMA, fused select.
  auto body = [&](int c, u32x4 (&st)[PMAX], float (&cb)[16], float (&cu)[16], float (&pb)[16],
                  float (&pu)[16]) {
    const int b = (c - c_begin) & 1;
    store_chunk(b, st);
    lds_barrier();
    if (c + WD < c_end) load_chunk(c + WD, st);        // the slot just stored is free again
    if (c + PD < c_end) load_epi(c + PD, pb, pu);

    // Bias tile: 32 vocabulary rows x 32 requests over the compiled K = RK.  The
    // steps beyond r multiply zero-filled LDS columns by zero E registers, so the
    // loop has no branches and the LDS reads pipeline ahead of the MFMAs.
    const uint16_t* abase = lds + b * BUF + col * PITCH + half * 8;
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(abase + s * 16);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, e[s], acc, 0, 0, 0);
    }

    // Fused bias-add + select.  Lane holds rows v0 + 8*jq + 4*half + i of column m.
    const int v0 = c * kChunk;
    if (m_ok) {
      const int vl = v0 + 4 * half;
      if (v0 + kChunk <= V) {
#pragma unroll
        for (int qq = 0; qq < 16; ++qq) {
          const float sc = score(cb[qq], acc[qq], cu[qq]);
          if (sc > best) {
            best = sc;
            best_i = vl + 8 * (qq >> 2) + (qq & 3);
          }
        }
      } else {
#pragma unroll
        for (int qq = 0; qq < 16; ++qq) {
          const int vi = vl + 8 * (qq >> 2) + (qq & 3);
          const float sc = score(cb[qq], acc[qq], cu[qq]);
          if (vi < V && sc > best) {
            best = sc;
            best_i = vi;
          }
        }
      }
      if (bout) {
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          const int v = v0 + 8 * jq + 4 * half;
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
  };

#pragma unroll
  for (int t = 0; t < WD; ++t)
    if (c_begin + t < c_end) load_chunk(c_begin + t, stage[t]);
#pragma unroll
  for (int t = 0; t < PD; ++t)
    if (c_begin + t < c_end) load_epi(c_begin + t, eb[t], eu[t]);
  // Unrolled so that every register-slot index is static.
  for (int c0 = c_begin; c0 < c_end; c0 += UNR) {
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      if (c0 + j < c_end)
        body(c0 + j, stage[j % WD], eb[j % NS], eu[j % NS], eb[(j + PD) % NS], eu[(j + PD) % NS]);
    }
  }

  // Lanes l and l^32 hold the same request: merge, then one lane writes the partial.
  const float ov = __shfl_xor(best, 32);
  const int oi = __shfl_xor(best_i, 32);
  merge_best(best, best_i, ov, oi);
  if (m_ok && half == 0) {
    partials[(size_t)vg * R + m] = make_float2(best, __int_as_float(best_i));
  }
}

// Reduce the per-group partials [group][request] to x_k: one wave per request,
// lanes stride over the groups (independent loads), then a fixed shuffle tree.
__global__ __launch_bounds__(256) void argmax_reduce_kernel(const float2* __restrict__ partials,
                                                            int R, int n_vgroups, int V,
                                                            int gamma, int k,
                                                            int32_t* __restrict__ tokens) {
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (m >= R) return;
  float best = -INFINITY;
  int best_i = 0x7fffffff;
#pragma unroll 4
  for (int g = lane; g < n_vgroups; g += 64) {
    const float2 p = partials[(size_t)g * R + m];
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
                            (int)lds) != hipSuccess) {
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

// Workgroups of the step kernel that fit on one CU (cached per instantiation).
template <int RK, int NW, int MODE>
int blocks_per_cu_t() {
  static int cached = 0;
  if (!cached) {
    int nb = 0;
    const size_t lds = 2 * kChunk * (size_t)(RK + 8) * 2;
    hipFuncSetAttribute(reinterpret_cast<const void*>(&markov_step_kernel<RK, NW, MODE>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &nb, reinterpret_cast<const void*>(&markov_step_kernel<RK, NW, MODE>), NW * 64,
            lds) != hipSuccess || nb < 1)
      nb = 1;
    cached = nb;
  }
  return cached;
}

template <int RK>
int blocks_per_cu_nw(int nw, int mode) {
  const bool s = mode == DSPARK_SAMPLE;
  switch (nw) {
    case 1: return s ? blocks_per_cu_t<RK, 1, DSPARK_SAMPLE>() : blocks_per_cu_t<RK, 1, DSPARK_GREEDY>();
    case 2: return s ? blocks_per_cu_t<RK, 2, DSPARK_SAMPLE>() : blocks_per_cu_t<RK, 2, DSPARK_GREEDY>();
    case 4: return s ? blocks_per_cu_t<RK, 4, DSPARK_SAMPLE>() : blocks_per_cu_t<RK, 4, DSPARK_GREEDY>();
    default: return s ? blocks_per_cu_t<RK, 8, DSPARK_SAMPLE>() : blocks_per_cu_t<RK, 8, DSPARK_GREEDY>();
  }
}

int blocks_per_cu(int rk, int nw, int mode) {
  switch (rk) {
    case 64: return blocks_per_cu_nw<64>(nw, mode);
    case 128: return blocks_per_cu_nw<128>(nw, mode);
    case 256: return blocks_per_cu_nw<256>(nw, mode);
    default: return blocks_per_cu_nw<512>(nw, mode);
  }
}

int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    return 256;
  return n;
}

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  return (s && *s) ? atoi(s) : dflt;
}

}  // namespace

MarkovPlan plan_markov(int R, int gamma, int V, int r, int mode, bool for_launch) {
  (void)gamma;
  MarkovPlan p{};
  p.rk = r <= 64 ? 64 : r <= 128 ? 128 : r <= 256 ? 256 : 512;
  const int waves_needed = (R + 31) / 32;
  int nw = waves_needed >= 8 ? 8 : waves_needed >= 4 ? 4 : waves_needed >= 2 ? 2 : 1;
  // Rank-512 sampling: the 8-wave kernel would spill; the 4-wave, one-wave-per-SIMD
  // variant with deeper prefetch is used instead.
  if (p.rk == 512 && mode == DSPARK_SAMPLE && nw == 8) nw = 4;
  const int nw_env = env_int("DSPARK_MARKOV_NW", 0);
  if (nw_env == 1 || nw_env == 2 || nw_env == 4 || nw_env == 8) nw = nw_env;
  p.nw = nw;
  p.n_rblocks = (R + 32 * nw - 1) / (32 * nw);
  p.n_chunks = (V + kChunk - 1) / kChunk;
  const int max_groups = p.n_chunks < kMaxGroups ? p.n_chunks : kMaxGroups;
  p.ws_bytes = (size_t)R * (size_t)max_groups * sizeof(float2);
  if (!for_launch) return p;
  // One wave of workgroups: as many as fit on the device at once, split between
  // the R blocks (each V group is walked by n_rblocks workgroups).
  int target = env_int("DSPARK_MARKOV_WG", 0);
  if (target <= 0) target = device_cus() * blocks_per_cu(p.rk, nw, mode);
  if (target < 8) target = 8;
  int groups = (target + p.n_rblocks - 1) / p.n_rblocks;
  groups = (groups + 7) / 8 * 8;
  if (groups > max_groups) groups = max_groups;
  if (groups < 1) groups = 1;
  p.cpg = (p.n_chunks + groups - 1) / groups;
  p.n_vgroups = (p.n_chunks + p.cpg - 1) / p.cpg;
  return p;
}

dspark_status launch_markov_draft(const uint16_t* W1, const uint16_t* W2, const float* base,
                                  const int32_t* anchors, int R, int gamma, int V, int r,
                                  int mode, float temperature, const float* uniforms,
                                  int32_t* tokens, float* bias_out, void* workspace,
                                  const dspark_step_events* events, hipStream_t stream) {
  const MarkovPlan p = plan_markov(R, gamma, V, r, mode, true);
  float2* partials = reinterpret_cast<float2*>(workspace);
  const int padded_groups = (p.n_vgroups + 7) / 8 * 8;
  const dim3 grid(padded_groups * p.n_rblocks);
  const size_t lds = 2 * kChunk * (size_t)(p.rk + 8) * 2;   // two W2 chunk buffers
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
