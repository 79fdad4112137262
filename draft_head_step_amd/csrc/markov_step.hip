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
//   * A wave owns 32 requests and keeps their gathered W1 rows (MFMA B operand)
//     in registers for the whole launch.  The workgroup's waves share 32-column
//     chunks of W2 staged through LDS (double-buffered, rows padded by 16 bytes
//     so the A-operand reads hit distinct banks).
//   * Each workgroup walks a group of chunks keeping a running (max, argmax)
//     per request, then folds it into one packed 64-bit word per request with
//     an integer atomic max (order-independent, so results are deterministic).
//     The next step reads its input tokens from those words (and its first V
//     group stores them to the output); a small launch unpacks the last
//     step.  A call is gamma + 2 launches: clear, the steps,
//     unpack.  (A last-arriving workgroup could do the unpack, but the
//     device-scope release fence it needs costs more than the launch.)
//   * Workgroup ids are decoded so that the R-blocks sharing a V group land on
//     the same XCD (ids congruent mod 8) and are dispatched together, so the
//     second and later reads of a W2 chunk hit that XCD's L2.
//   * Loads run ahead of use through register rings (W2 staging, epilogue
//     inputs).  The steady-state loop body is branch-free: every load is a raw
//     buffer load issued unconditionally (the hardware range check turns the
//     tail, padding and rank-padding reads into zeros) and validity is applied
//     with selects, because a load on a conditional path makes the compiler's
//     wait-count analysis assume the worst and drain the whole ring (vmcnt(0))
//     at the next use.  Groups are padded to the unroll factor, prefetches stay
//     inside the group, and scheduling barriers keep each chunk's arithmetic
//     in its own iteration so the waits count the ring from the back.
//   * Rank 512: the gathered rows take 128 VGPRs per lane.  Either one wave per
//     SIMD with deeper rings ("plain", 4 waves), or K-split wave pairs (each
//     wave holds one K half, 64 VGPRs, two waves per SIMD; partial tiles are
//     exchanged through LDS and the epilogue of chunk c-1 runs beside the MFMAs
//     of chunk c).
#include <math.h>

#include <mutex>
#include <type_traits>

#include <hip/hip_ext.h>

#include "dspark_internal.h"

namespace dspark {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 32;         // vocabulary rows of W2 per MFMA tile
constexpr int kMaxGroups = 1024;   // upper bound on V groups (sizes the workspace)
// Internal mode: greedy on the Markov bias alone (no base logits are read).
constexpr int kBiasOnly = 2;

__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// Workgroup barrier that orders LDS only.  __syncthreads() also fences global
// memory, which makes the compiler wait for every outstanding global load at
// each barrier; the waves here share nothing through global memory in a launch.
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

// Per-step results are kept as one 64-bit word per request, combined across
// workgroups with an unsigned atomic max: the score in the high half (mapped
// to an unsigned key that orders like the float, -0 taken as +0) and the
// complement of the token id in the low half, so equal scores keep the
// smallest id -- the same order as merge_best, independent of arrival order.
// A cleared word (0) is below every packed value and decodes to token 0.
// Each request has S words (1 or kMaxSubWords, chosen per call) and V group g
// combines into word g % S.  The atomics of a launch all land at its end, R x
// (V groups) of them on R x S words.  With many groups per request (small R,
// e.g. 64 requests x 512 groups) one word per request serialises them on a few
// lines (measured: 25.0 us per launch at S = 1 or 4, 21.7 us at S = 16); with
// fewer groups, reading S words at the start of the next step costs more than
// the contention saves (DeepSeek-V4 shape, 128 groups: 74.5 us at S = 1, 76.2 at 16).
constexpr int kMaxSubWords = 16;
constexpr int kSubWordsAboveGroups = 256;
__device__ __forceinline__ unsigned long long pack_best(float v, int i) {
  const uint32_t b = __float_as_uint(v + 0.0f);
  const uint32_t key = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)key << 32) | (unsigned long long)(0xffffffffu - (uint32_t)i);
}

__device__ __forceinline__ int unpack_token(unsigned long long w, int V) {
  const uint32_t i = 0xffffffffu - (uint32_t)w;
  return i < (uint32_t)V ? (int)i : 0;
}

// Token of request m from its S packed words (S a power of two).  The two
// sizes the launch picks load all their words before combining them (one
// memory round trip); other sizes (tuning overrides) take the plain loop.
__device__ __forceinline__ int read_token(const unsigned long long* w, int m, int S, int V) {
  unsigned long long b = 0;
  if (S == 1) {
    b = w[m];
  } else if (S == kMaxSubWords) {   // 16-byte loads, all issued first
    const ulonglong2* p = reinterpret_cast<const ulonglong2*>(w + (size_t)m * S);
    ulonglong2 v[kMaxSubWords / 2];
#pragma unroll
    for (int j = 0; j < kMaxSubWords / 2; ++j) v[j] = p[j];
#pragma unroll
    for (int j = 0; j < kMaxSubWords / 2; ++j) {
      b = v[j].x > b ? v[j].x : b;
      b = v[j].y > b ? v[j].y : b;
    }
  } else {   // S even: 16-byte loads
    const ulonglong2* p = reinterpret_cast<const ulonglong2*>(w + (size_t)m * S);
    for (int j = 0; j < S / 2; ++j) {
      const ulonglong2 v = p[j];
      b = v.x > b ? v.x : b;
      b = v.y > b ? v.y : b;
    }
  }
  return unpack_token(b, V);
}

// Where a step kernel takes its input tokens and leaves its results.
struct StepIO {
  const int32_t* anchors;              // step 0: x_0
  const unsigned long long* prev;      // steps > 0: packed results of step k-1 [R][sub]
  unsigned long long* best;            // packed results of step k, cleared before step 0
  int32_t* tokens;                     // [R][gamma]
  int gamma;
  int k;
  int sub;                             // words per request (power of two)
};

// Token x_{k-1} of request m (step 0: the anchor).  The first V group of each
// R block also stores it to tokens, which completes step k-1 there.
__device__ __forceinline__ int step_input(const StepIO& io, int m, bool m_ok, bool writer,
                                          int V) {
  if (!m_ok) return 0;
  if (!io.prev) return io.anchors[m];
  const int x = read_token(io.prev, m, io.sub, V);
  if (writer) io.tokens[(size_t)m * io.gamma + io.k - 1] = x;
  return x;
}


// Selection score of z = b + a.  Sampling compares the Gumbel-max score in
// base 2: (z/T - ln(-ln u)) / ln 2 = z * log2(e)/T - log2(-log2 u) + const, the
// same argmax, with two hardware base-2 logarithms (relative error ~1e-7 over
// the open unit interval) and one fma.  `kscale` is log2(e)/T.
template <int MODE>
__device__ __forceinline__ float select_score(float b, float a, float u, float kscale) {
  if (MODE == DSPARK_SAMPLE) {
    const float g = __builtin_amdgcn_logf(-__builtin_amdgcn_logf(u));
    return fmaf(b + a, kscale, -g);
  }
  return b + a;
}

// Running argmax of one lane.  Element q of a chunk is vocabulary entry
// (chunk)*32 + lane offset + 8*(q/4) + (q%4).  Per element only the score and
// q are kept (q is an inline constant); the iteration whose chunk raised the
// maximum is recorded once per chunk and the id is rebuilt at the end.  Chunks
// arrive in increasing v and q runs in increasing v within a chunk, so a
// strict comparison keeps the smallest id among equal maxima.
struct Argmax {
  float best = -INFINITY;
  int q = 0;
  int iter = -1;
};

template <int MODE, int N, bool MASKED>
__device__ __forceinline__ void select_chunk(Argmax& am, const float* cb, const float* z,
                                             const float* cu, float kscale, int iter, int lim) {
  const float before = am.best;
#pragma unroll
  for (int q = 0; q < N; ++q) {
    const float sc = select_score<MODE>(cb[q], z[q], cu[q], kscale);
    // MASKED: only elements with in-chunk offset below lim are valid (the chunk
    // that crosses V, padding iterations with lim <= 0).
    const bool take = MASKED ? (sc > am.best && 8 * (q >> 2) + (q & 3) < lim) : sc > am.best;
    if (take) {
      am.best = sc;
      am.q = q;
    }
  }
  if (am.best != before) am.iter = iter;
}

// Vocabulary id of an Argmax (0x7fffffff if nothing was taken).
__device__ __forceinline__ int argmax_id(const Argmax& am, int c0, int cstep, int lane_off) {
  return am.iter < 0 ? 0x7fffffff
                     : (c0 + am.iter * cstep) * kChunk + lane_off + 8 * (am.q >> 2) + (am.q & 3);
}

// ---- raw buffer access ----
// Buffer loads take one scalar resource (base, size) and a 32-bit per-lane
// byte offset.  Offsets at or past the size read as zero instead of faulting,
// which replaces every clamp and select of the tail, padding and rank-padding
// cases; the per-lane offsets stay fixed over the loop (chunk steps are a
// uniform add), so the ring needs no 64-bit address registers.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;     // untyped dword access (gfx9 family)
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ Rsrc make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ u32x4 buf_load16(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float buf_load4(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
// Four-byte load of a stream read once (non-temporal: the line is not kept in
// the caches).  The uniform part of the offset rides in soffset, which the
// range check does not cover: an out-of-range lane must carry it in `off`.
__device__ __forceinline__ float buf_load4_nt(Rsrc r, uint32_t off, int soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 2));
}

// Element (m, k, v) of base / uniforms / bias_out is at float offset
// k_off + m * row_stride + (v / 32) * cstride + (v % 32) * vstride in either
// layout; block_rsrc covers [block start, total).  Byte offsets inside one R
// block of one step fit in 32 bits (checked on the host).
struct Addr {
  size_t k_off, row_stride, cstride, vstride, total;
};

// Buffer resource over the rows of R block `rb` (first row rb * rows) at step k.
__device__ __forceinline__ Rsrc block_rsrc(const float* arr, const Addr& ad, int rb, int rows) {
  const size_t off = ad.k_off + (size_t)rb * rows * ad.row_stride;
  const size_t rem = ad.total > off ? (ad.total - off) * 4 : 0;
  return make_rsrc(arr + off, rem > 0xfffffff0u ? 0xfffffff0u : (uint32_t)rem);
}

// W2 chunk staging.  Piece p = tid + j * NT of the 32 x RK chunk is row p / PPR,
// 8-element block p % PPR; since NT is a multiple of PPR the block is the same
// for all j and the row advances by NT / PPR.  Blocks past r carry an offset
// past the buffer, rows past V land past it, so both read as zeros.
template <int RK, int NT>
__device__ __forceinline__ uint32_t w2_lane_offset(int tid, int r) {
  constexpr int PPR = RK / 8;
  const int cp = tid % PPR;
  return cp < (r >> 3) ? (uint32_t)((tid / PPR) * r + cp * 8) * 2u : kOutOfRange;
}

template <int RK, int NT, int PMAX>
__device__ __forceinline__ void w2_load(u32x4 (&st)[PMAX], Rsrc rw2, uint32_t lane_off, int cc,
                                        int r) {
  constexpr int PPR = RK / 8;
  const uint32_t off = lane_off + (uint32_t)cc * (uint32_t)(kChunk * r * 2);
#pragma unroll
  for (int j = 0; j < PMAX; ++j) st[j] = buf_load16(rw2, off + (uint32_t)(j * (NT / PPR) * r * 2));
}

template <int RK, int NT, int PMAX>
__device__ __forceinline__ void w2_store(uint16_t* dst, const u32x4 (&st)[PMAX], int tid) {
  constexpr int PPR = RK / 8;
  constexpr int PIECES = kChunk * PPR;
  constexpr int PITCH = RK + 8;
#pragma unroll
  for (int j = 0; j < PMAX; ++j) {
    const int p = tid + j * NT;
    if (PIECES % NT == 0 || p < PIECES)
      *reinterpret_cast<u32x4*>(dst + (p / PPR) * PITCH + (p % PPR) * 8) = st[j];
  }
}

// Rank 512: a W2 row is 1 KB, one wave-wide 16-byte load, so the chunk is staged
// by direct loads into LDS (buffer_load ... lds): lane l's 16 bytes land at
// M0 + 16 l, the row pitch keeps its 16-byte pad, and out-of-range lanes (blocks
// past r, rows past V) write zeros.  No registers hold the data and no LDS
// stores are issued; wave w stages rows w, w + NW, ...
//
// The load is issued from inline assembly on purpose.  The compiler does not
// know it writes LDS, so it adds no drain before the LDS reads that follow.
// The kernels instead wait for it explicitly (vmcnt, then a barrier) before
// reading a stage buffer.  The compiler's own vmcnt waits for ordinary loads
// stay correct: loads retire in issue order, so VMEM ops it does not see only
// make a wait stricter.
constexpr int kPitch512 = 512 + 8;

__device__ __forceinline__ uint32_t w2_dma_lane_offset(int lane, int r) {
  return lane * 8 < r ? (uint32_t)lane * 16u : kOutOfRange;
}

// Raw buffer descriptor words (base, stride 0, size in bytes, untyped dwords).
__device__ __forceinline__ u32x4 raw_desc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, (uint32_t)kRsrcWord3};
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

template <int NW>
__device__ __forceinline__ void w2_dma(uint16_t* buf, u32x4 dw2, uint32_t lane_off, int cc, int r,
                                       int wave) {
#pragma unroll
  for (int j = 0; j < kChunk / NW; ++j) {
    const int row = wave + j * NW;
    const uint32_t voff = lane_off + (uint32_t)((cc * kChunk + row) * r) * 2u;
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(dw2), "{m0}"(lds_addr(buf + row * kPitch512))
                 : "memory");
  }
}

// s_waitcnt vmcnt(min(N, 63)), other counters untouched (gfx9 encoding).  A
// smaller count only waits longer, so clamping keeps it correct.
template <int N0>
__device__ __forceinline__ void wait_vmcnt() {
  constexpr int N = N0 < 63 ? N0 : 63;
  static_assert(N >= 0, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}

// How the epilogue reads the logits and uniforms of a chunk.
//   kEpiScalar  row-major, four-byte loads (any alignment);
//   kEpiVec4    row-major, 16-byte loads (each row's 128-byte slice of a chunk
//               takes four instructions per half-wave);
//   kEpiCol     column-tiled: for one vocabulary entry the 32 requests of a
//               tile are 128 contiguous bytes, so every four-byte load
//               instruction reads whole lines, which go non-temporal.
constexpr int kEpiScalar = 0;
constexpr int kEpiVec4 = 1;
constexpr int kEpiCol = 2;

// VMEM instructions one epi_load issues (they count in vmcnt with the DMA).
// Exact for the 16-byte and column paths (the column loads differ in soffset
// only, which no merge combines); the scalar path's consecutive four-byte
// loads may be merged by the compiler, so waits never rely on that count.
template <int MODE, int EPI, int NJ>
constexpr int epi_load_count() {
  return MODE == kBiasOnly ? 0 : (EPI == kEpiVec4 ? NJ : 4 * NJ) * (MODE == DSPARK_SAMPLE ? 2 : 1);
}

// Epilogue inputs of NJ accumulator groups (jq = j0 .. j0+NJ-1) of one chunk for
// one lane: element 4*j + i is vocabulary entry v0 + 8*(j0+j) + 4*half + i; `off`
// is the lane's byte offset of entry v0 + 8*j0 + 4*half and `vs` the byte
// distance between consecutive entries of the column layout.
template <int MODE, int EPI, int NJ>
__device__ __forceinline__ void epi_load(float (&bv)[4 * NJ], float (&uv)[4 * NJ], Rsrc rbase,
                                         Rsrc runif, uint32_t off, int vs) {
  if (MODE == kBiasOnly) {
#pragma unroll
    for (int j = 0; j < 4 * NJ; ++j) bv[j] = 0.0f;
    return;
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    if (EPI == kEpiCol) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int so = (8 * j + i) * vs;
        bv[4 * j + i] = buf_load4_nt(rbase, off, so);
        if (MODE == DSPARK_SAMPLE) uv[4 * j + i] = buf_load4_nt(runif, off, so);
      }
    } else if (EPI == kEpiVec4) {
      const float4 t = __builtin_bit_cast(float4, buf_load16(rbase, off + 32u * j));
      bv[4 * j + 0] = t.x; bv[4 * j + 1] = t.y; bv[4 * j + 2] = t.z; bv[4 * j + 3] = t.w;
      if (MODE == DSPARK_SAMPLE) {
        const float4 w = __builtin_bit_cast(float4, buf_load16(runif, off + 32u * j));
        uv[4 * j + 0] = w.x; uv[4 * j + 1] = w.y; uv[4 * j + 2] = w.z; uv[4 * j + 3] = w.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bv[4 * j + i] = buf_load4(rbase, off + 32u * j + 4u * i);
        if (MODE == DSPARK_SAMPLE) uv[4 * j + i] = buf_load4(runif, off + 32u * j + 4u * i);
      }
    }
  }
}

constexpr int lcm_small(int a, int b) { return (a % b == 0) ? a : (b % a == 0) ? b : a * b; }

// Scheduling template for one chunk's MFMA chain (masks: 0x100 LDS read,
// 0x008 MFMA, 0x002 VALU): kLdsAhead A-operand reads first, then per K-step
// one MFMA, the next read and two VALU instructions, then the last MFMAs.
constexpr int kLdsAhead = 4;

template <int KS>
__device__ __forceinline__ void mfma_pipeline() {
  __builtin_amdgcn_sched_group_barrier(0x100, kLdsAhead, 0);
#pragma unroll
  for (int s = 0; s < KS - kLdsAhead; ++s) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
  }
#pragma unroll
  for (int s = 0; s < kLdsAhead; ++s) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
  }
}

// Number of leading iterations of a group whose chunks lie wholly inside V: all
// n_valid, unless the group's last chunk is the one that crosses V.
__device__ __forceinline__ int n_whole(int c0, int cstep, int n_valid, int V) {
  const int last = c0 + (n_valid - 1) * cstep;
  return (last + 1) * kChunk <= V ? n_valid : n_valid - 1;
}

// ---------------------------------------------------------------------------
// Plain kernel: a wave owns 32 requests over the full K.
// ---------------------------------------------------------------------------
template <int RK, int NW>
constexpr bool plain_deep() { return RK == 512 && NW == 4; }
// W1 rows of all the workgroup's tiles are staged through LDS, in one round if
// they fit in the CU's LDS, else in two (the first half of the waves, then the
// second half, through the same area).
template <int RK, int NW, int TW>
constexpr int plain_gather_rounds() {
  return (size_t)NW * TW * 32 * RK * 2 <= 160 * 1024 ? 1 : 2;
}
template <int RK, int NW, int TW>
constexpr size_t plain_lds_bytes() {
  const size_t stage = (size_t)(RK == 512 ? (plain_deep<RK, NW>() ? 3 : 2) : 2) * 32 * (RK + 8) * 2;
  const size_t gather = (size_t)NW / plain_gather_rounds<RK, NW, TW>() * TW * 32 * RK * 2;
  return stage > gather ? stage : gather;
}
template <int RK, int NW>
constexpr int plain_wd() { return plain_deep<RK, NW>() ? 2 : 1; }   // W2 chunks staged ahead
template <int RK, int NW>
constexpr int plain_pd() { return plain_deep<RK, NW>() ? 3 : 1; }   // epilogue chunks ahead
template <int RK, int NW>
constexpr int plain_unroll() { return lcm_small(plain_wd<RK, NW>(), plain_pd<RK, NW>() + 1); }

// Rank 512 keeps 128 VGPRs of W1 rows per lane and its LDS stages hold one
// workgroup per CU, so two waves per SIMD is the occupancy that can ever run.
// Saying so lets the compiler spend registers on a deeper LDS-read pipeline
// instead of packing for an occupancy the launch never reaches.
template <int RK>
constexpr int plain_max_waves() { return RK == 512 ? 2 : 8; }

template <int RK, int NW, int MODE, int EPI, bool BIAS, int TW>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(1, plain_max_waves<RK>()))) void markov_step_kernel(
    const uint16_t* __restrict__ W1, const uint16_t* __restrict__ W2,
    const float* __restrict__ base, const float* __restrict__ unif,
    StepIO io, int R, int V, int r, float inv_t, int n_rblocks, int n_vgroups, int cpg,
    int cstep, int n_chunks, Addr ad, float* __restrict__ bias_out) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int KS = RK / 16;
  constexpr int NT = NW * 64;
  constexpr int ROWS = NW * 32 * TW;
  constexpr int PMAX = (kChunk * (RK / 8) + NT - 1) / NT;
  constexpr int PITCH = RK + 8;
  constexpr int BUF = kChunk * PITCH;
  constexpr int WD = plain_wd<RK, NW>();
  constexpr int PD = plain_pd<RK, NW>();
  constexpr int NS = PD + 1;
  constexpr int UNR = plain_unroll<RK, NW>();
  constexpr bool DMA = RK == 512;                  // W2 staged by direct loads into LDS
  constexpr int NBUF = DMA ? WD + 1 : 2;           // LDS stage buffers
  static_assert(TW == 1 || !DMA, "two tiles per wave only with register staging");
  // W1 rows staged through LDS (see plain_gather_rounds).
  constexpr int GROUNDS = plain_gather_rounds<RK, NW, TW>();
  constexpr int GWPR = NW / GROUNDS;                 // waves staging per round
  static_assert(NW % GROUNDS == 0 && (size_t)GWPR * TW * 32 * RK * 2 <= 160 * 1024,
                "W1 staging must fit the CU's LDS");
  // vmcnt at the top of an iteration that leaves only the loads issued after
  // the DMA of its own chunk outstanding (0 with bias stores in flight).
  constexpr int EL = epi_load_count<MODE, EPI, 4>();
  // The scalar epilogue's four-byte loads may be merged by the compiler into
  // fewer instructions, so only the 16-byte and column paths have a count to
  // rely on.
  constexpr int DMA_WAIT = (BIAS || EPI == kEpiScalar) ? 0 : EL + (WD - 1) * (kChunk / NW + EL);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int col = lane & 31;
  const float kscale = inv_t * 1.44269504088896341f;   // log2(e) / T

  const int id = blockIdx.x;
  const int q = id >> 3;
  const int rb = q % n_rblocks;
  const int vg = (q / n_rblocks) * 8 + (id & 7);
  if (vg >= n_vgroups) return;
  // Iteration i (0 <= i < cpg, a multiple of UNR) handles chunk c0 + i * cstep:
  // contiguous groups (cstep 1) or groups strided across V (cstep = number of
  // groups).  Iterations past the group's n_valid chunks are masked, and
  // prefetches are clamped to the group's last chunk.
  const int c0 = cstep == 1 ? vg * cpg : vg;
  const int n_valid = cstep == 1 ? min(cpg, n_chunks - c0) : (n_chunks - 1 - vg) / cstep + 1;
  auto chunk = [&](int i) { return c0 + min(i, n_valid - 1) * cstep; };
  uint16_t* lds = reinterpret_cast<uint16_t*>(smem);

  // Tile t of this wave holds requests (wave * TW + t) * 32 + col of the R block.
  int m[TW];
  bool m_ok[TW];
  int xt[TW];
  uint32_t e_off[TW];
  bf16x8 e[TW][KS];
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    const int m_loc = (wave * TW + t) * 32 + col;
    m[t] = rb * ROWS + m_loc;
    m_ok[t] = m[t] < R;
    // Row-major rows past R lie past the block's range; column-layout rows
    // past R would alias the next entries, so they are sent out of range.
    e_off[t] = (EPI == kEpiCol && !m_ok[t])
                   ? kOutOfRange
                   : (uint32_t)(m_loc * ad.row_stride + 4 * half * ad.vstride) * 4u;
    int x = step_input(io, m[t], m_ok[t], vg == 0 && half == 0, V);
    xt[t] = min(max(x, 0), V - 1);                      // out-of-range ids never fault
  }

  const Rsrc rw2 = make_rsrc(W2, (uint32_t)V * (uint32_t)r * 2u);
  const u32x4 dw2 = raw_desc(W2, (uint32_t)V * (uint32_t)r * 2u);
  const uint32_t w2_off = DMA ? w2_dma_lane_offset(lane, r) : w2_lane_offset<RK, NT>(tid, r);
  const Rsrc rbase = MODE == kBiasOnly ? make_rsrc(W2, 0u) : block_rsrc(base, ad, rb, ROWS);
  const Rsrc runif = MODE == DSPARK_SAMPLE ? block_rsrc(unif, ad, rb, ROWS) : rbase;
  const uint32_t e_cb = (uint32_t)ad.cstride * 4u;
  const size_t vstride = EPI == kEpiCol ? ad.vstride : 1;
  const int e_vs = (int)vstride * 4;

  u32x4 stage[DMA ? 1 : WD][DMA ? 1 : PMAX];
  float eb[NS][TW][16];
  float eu[NS][TW][16];
  f32x16 accs[2][TW];
  Argmax am[TW];
  static_assert(UNR % 2 == 0 && UNR % NS == 0, "the unroll must cycle the rings");

  // Fused bias-add + select of iteration i.  Rows past R are never written, so
  // they need no mask.
  auto finish = [&](auto masked, int i, const f32x16 (&acc)[TW], const float (&cb)[TW][16],
                    const float (&cu)[TW][16]) {
    constexpr bool MASKED = decltype(masked)::value;
    const int cv = (c0 + i * cstep) * kChunk;
    const int vlim = i < n_valid ? V : 0;
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      float av[16];
#pragma unroll
      for (int qq = 0; qq < 16; ++qq) av[qq] = acc[t][qq];
      select_chunk<MODE, 16, MASKED>(am[t], cb[t], av, cu[t], kscale, i, vlim - cv - 4 * half);
      if (BIAS && m_ok[t]) {
        float* oc =
            bias_out + ad.k_off + (size_t)m[t] * ad.row_stride + (size_t)chunk(i) * ad.cstride;
#pragma unroll
        for (int qq = 0; qq < 16; ++qq) {
          const int o = 8 * (qq >> 2) + 4 * half + (qq & 3);
          if (cv + o < vlim) oc[o * vstride] = acc[t][qq];
        }
      }
    }
  };

  // Iteration i: stage chunk i, run its MFMAs into one accumulator, finish
  // iteration i-1 from the other beside them (the select does not wait for this
  // chunk's MFMAs), then refill the epilogue slot it freed with iteration i + PD.
  // Iteration i's epilogue inputs live in slot i % NS.
  auto body = [&](auto masked, auto first, int i, auto& st, f32x16 (&acc)[TW],
                  const f32x16 (&pacc)[TW], float (&pb)[TW][16], float (&pu)[TW][16]) {
    const int b = NBUF == 2 ? (i & 1) : i % NBUF;
    if constexpr (DMA) {
      // This wave's rows of chunk i have landed; the barrier publishes all rows.
      if constexpr (decltype(first)::value) wait_vmcnt<0>();
      else wait_vmcnt<DMA_WAIT>();
      lds_barrier();
      w2_dma<NW>(lds + ((i + WD) % NBUF) * BUF, dw2, w2_off, chunk(i + WD), r, wave);
    } else {
      w2_store<RK, NT, PMAX>(lds + b * BUF, st, tid);
      lds_barrier();
      w2_load<RK, NT, PMAX>(st, rw2, w2_off, chunk(i + WD), r);
    }
    __builtin_amdgcn_sched_barrier(0);   // issue the prefetch before the MFMAs

    // Bias tile: 32 vocabulary rows x 32 requests over the compiled K = RK
    // (steps past r multiply zero-filled LDS columns by zero registers).
    // With two tiles per wave each A read feeds two MFMAs.
    const uint16_t* abase = lds + b * BUF + col * PITCH + half * 8;
#pragma unroll
    for (int t = 0; t < TW; ++t) acc[t] = f32x16{};
#pragma unroll
    for (int s0 = 0; s0 < KS; s0 += 4) {
      bf16x8 a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const bf16x8*>(abase + (s0 + i) * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < TW; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], e[t][s0 + i], acc[t], 0, 0, 0);
    }
    if (!decltype(first)::value || i >= 1) finish(masked, i - 1, pacc, pb, pu);
    // Rank 512: LDS reads run kLdsAhead K-steps ahead of the MFMAs, and the
    // previous chunk's select fills the issue slots between them (measured
    // slower at rank 256, where the compiler's own order wins).
    if constexpr (RK == 512) mfma_pipeline<KS>();
#pragma unroll
    for (int t = 0; t < TW; ++t)
      epi_load<MODE, EPI, 4>(pb[t], pu[t], rbase, runif, e_off[t] + (uint32_t)chunk(i + PD) * e_cb,
                             e_vs);
    // Keep each chunk's arithmetic in its own iteration: hoisting the noise of
    // a prefetched chunk next to its load would wait for that load.
    __builtin_amdgcn_sched_barrier(0);
  };

  // W1 rows through LDS: each wave copies its tiles' rows (32 x RK bf16 each)
  // with direct loads that move whole rows (1 KB per instruction: 512 / RK
  // rows); piece c of row q sits in slot c ^ (q mod pieces per row), so the
  // one-row-per-lane reads spread over the banks.  Wave w stages in round
  // w / GWPR into slot w % GWPR of the area.
  constexpr int PPR = RK / 8;       // 16-byte pieces per row
  constexpr int RPI = 64 / PPR;     // rows per direct load
  const int gslot = wave % GWPR;
  auto gather_issue = [&]() {
    const u32x4 dw1 = raw_desc(W1, (uint32_t)V * (uint32_t)r * 2u);
    const int c = lane % PPR;
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      uint16_t* greg = lds + (gslot * TW + t) * 32 * RK;
#pragma unroll
      for (int i = 0; i < 32 / RPI; ++i) {
        const int q = i * RPI + lane / PPR;
        const int xq = __shfl(xt[t], q);
        const bool okq = rb * ROWS + (wave * TW + t) * 32 + q < R;
        const int piece = c ^ (q & (PPR - 1));
        const uint32_t voff = (okq && piece * 8 < r)
                                  ? (uint32_t)xq * (uint32_t)r * 2u + (uint32_t)(piece * 16)
                                  : kOutOfRange;
        asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                     :
                     : "v"(voff), "s"(dw1), "{m0}"(lds_addr(greg + i * RPI * RK))
                     : "memory");
      }
    }
  };
  // Waits for everything this wave issued (the compiler may merge the scalar
  // epilogue loads, so a count of them is not reliable), then reads the rows.
  auto gather_read = [&]() {
    wait_vmcnt<0>();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      const uint16_t* greg = lds + (gslot * TW + t) * 32 * RK + col * RK;
#pragma unroll
      for (int s = 0; s < KS; ++s)
        e[t][s] = *reinterpret_cast<const bf16x8*>(greg + (((2 * s + half) ^ (col & (PPR - 1))) * 8));
    }
  };
  // Prologue loads in the order they are consumed (oldest first), so that the
  // waits at the top of the loop can count them from the back.
  auto prologue = [&]() {
#pragma unroll
    for (int t = 0; t < (WD > PD ? WD : PD); ++t) {
      if (t < WD) {
        if constexpr (DMA) w2_dma<NW>(lds + t * BUF, dw2, w2_off, chunk(t), r, wave);
        else w2_load<RK, NT, PMAX>(stage[t % (DMA ? 1 : WD)], rw2, w2_off, chunk(t), r);
      }
      if (t < PD) {
#pragma unroll
        for (int u = 0; u < TW; ++u)
          epi_load<MODE, EPI, 4>(eb[t][u], eu[t][u], rbase, runif,
                                 e_off[u] + (uint32_t)chunk(t) * e_cb, e_vs);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Register-staged W2: the prologue goes first and lands while the rows are
  // staged.  Direct-to-LDS W2 writes the area the rows pass through, so it
  // starts after the last round.  The barrier after each round frees the area
  // for the next round or for the stage buffers.
  if constexpr (!DMA) prologue();
#pragma unroll
  for (int rd = 0; rd < GROUNDS; ++rd) {
    if (wave / GWPR == rd) {
      gather_issue();
      gather_read();
    }
    lds_barrier();
  }
  if constexpr (DMA) prologue();
  // The first UNR iterations (the first has nothing to finish) and those from
  // n_main on use the masked select; in between every finished chunk lies
  // wholly inside V.
  const int n_main = n_whole(c0, cstep, n_valid, V) / UNR * UNR;
#pragma unroll
  for (int j = 0; j < UNR; ++j)
    body(std::true_type{}, std::true_type{}, j, stage[DMA ? 0 : j % WD], accs[j & 1],
         accs[(j + 1) & 1], eb[(j + NS - 1) % NS], eu[(j + NS - 1) % NS]);
  int i0 = UNR;
  for (; i0 < n_main; i0 += UNR) {
#pragma unroll
    for (int j = 0; j < UNR; ++j)
      body(std::false_type{}, std::false_type{}, i0 + j, stage[DMA ? 0 : j % WD], accs[j & 1],
           accs[(j + 1) & 1], eb[(j + NS - 1) % NS], eu[(j + NS - 1) % NS]);
  }
  for (; i0 < cpg; i0 += UNR) {
#pragma unroll
    for (int j = 0; j < UNR; ++j)
      body(std::true_type{}, std::false_type{}, i0 + j, stage[DMA ? 0 : j % WD], accs[j & 1],
           accs[(j + 1) & 1], eb[(j + NS - 1) % NS], eu[(j + NS - 1) % NS]);
  }
  // cpg is a multiple of UNR: the last iteration used accs[1] and slot NS - 1.
  finish(std::true_type{}, cpg - 1, accs[1], eb[NS - 1], eu[NS - 1]);
  if constexpr (DMA) wait_vmcnt<0>();   // no direct load lands in LDS after exit

  // Lanes l and l^32 hold the same request: merge, then one lane publishes.
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    float best = am[t].best;
    int best_i = argmax_id(am[t], c0, cstep, 4 * half);
    const float ov = __shfl_xor(best, 32);
    const int oi = __shfl_xor(best_i, 32);
    merge_best(best, best_i, ov, oi);
    if (m_ok[t] && half == 0)
      atomicMax(io.best + (size_t)m[t] * io.sub + (vg & (io.sub - 1)), pack_best(best, best_i));
  }
}

// ---------------------------------------------------------------------------
// K-split kernel (rank 512): wave pairs share 32 requests, one K half each.
// After its MFMAs each wave hands the half-tile it does not finish (groups
// jq outside {2kh, 2kh+1}) to its partner through a double-buffered LDS slot;
// the epilogue of chunk c-1 runs in iteration c beside the MFMAs of chunk c,
// so one barrier per chunk orders everything.  At the end the pair merges its
// halves through LDS and writes one partial per request and V group.
// ---------------------------------------------------------------------------
constexpr int kSplitWD = 1;
constexpr int kSplitPD = 1;
constexpr int kSplitUnroll = lcm_small(kSplitWD, kSplitPD + 1);

constexpr int kSplitBufs = kSplitWD + 1;   // LDS stage buffers (direct loads run WD ahead)

// W1 staging per wave: 32 rows x 256 bf16 (its K half of rank 512).
constexpr int kGatherWave = 32 * 256;

template <int NP>
constexpr size_t ksplit_lds_bytes() {
  const size_t loop = (size_t)kSplitBufs * kChunk * kPitch512 * 2 + (size_t)2 * (2 * NP) * 64 * 8 * 4;
  const size_t gather = (size_t)(2 * NP) * kGatherWave * 2;
  return loop > gather ? loop : gather;
}

// One K-split workgroup (its LDS stages and exchange buffer) fills a CU's LDS:
// at most two waves per SIMD.
template <int NP, int MODE, int EPI, bool BIAS>
__global__ __launch_bounds__(NP * 128)
__attribute__((amdgpu_waves_per_eu(1, 2))) void markov_step_ksplit_kernel(
    const uint16_t* __restrict__ W1, const uint16_t* __restrict__ W2,
    const float* __restrict__ base, const float* __restrict__ unif,
    StepIO io, int R, int V, int r, float inv_t, int n_rblocks, int n_vgroups, int cpg,
    int cstep, int n_chunks, Addr ad, float* __restrict__ bias_out) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int RK = 512;
  constexpr int NW = 2 * NP;
  constexpr int NT = NW * 64;
  constexpr int ROWS = NP * 32;
  constexpr int KH = RK / 32;                          // MFMA K steps per half
  constexpr int PMAX = (kChunk * (RK / 8) + NT - 1) / NT;
  constexpr int PITCH = RK + 8;
  constexpr int BUF = kChunk * PITCH;
  constexpr int WD = kSplitWD;
  constexpr int PD = kSplitPD;
  constexpr int NS = PD + 1;
  constexpr int UNR = kSplitUnroll;
  constexpr int NBUF = kSplitBufs;
  constexpr int EL = epi_load_count<MODE, EPI, 2>();
  // vmcnt at the top of an iteration that leaves only the loads issued after
  // the DMA of its own chunk outstanding (0 with bias stores in flight, and 0
  // with the scalar epilogue, whose four-byte loads the compiler may merge
  // into fewer instructions).  With WD = 1 those are the previous iteration's
  // epilogue loads, which also retires the epilogue inputs this iteration uses.
  constexpr int DMA_WAIT = (BIAS || EPI == kEpiScalar) ? 0 : EL + (WD - 1) * (kChunk / NW + EL);
  static_assert(PITCH == kPitch512, "rank-512 pitch");

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int col = lane & 31;
  const float kscale = inv_t * 1.44269504088896341f;   // log2(e) / T
  const int pair = wave >> 1;
  const int kh = wave & 1;

  const int id = blockIdx.x;
  const int q = id >> 3;
  const int rb = q % n_rblocks;
  const int vg = (q / n_rblocks) * 8 + (id & 7);
  if (vg >= n_vgroups) return;
  const int c0 = cstep == 1 ? vg * cpg : vg;
  const int n_valid = cstep == 1 ? min(cpg, n_chunks - c0) : (n_chunks - 1 - vg) / cstep + 1;
  auto chunk = [&](int i) { return c0 + min(i, n_valid - 1) * cstep; };
  uint16_t* lds = reinterpret_cast<uint16_t*>(smem);
  float* xbuf = reinterpret_cast<float*>(smem + (size_t)NBUF * BUF * 2);   // [2][NW][64][8]

  const int m_loc = pair * 32 + col;
  const int m = rb * ROWS + m_loc;
  const bool m_ok = m < R;
  // W1 rows, staged through LDS before anything else uses it: each wave copies
  // its 32 rows' K half (32 x 512 B) with direct loads that each move two
  // contiguous row halves (a row-major gather straight into registers touches
  // 32 lines per instruction).  Piece c of row q is stored in slot c ^ q, so
  // the reads below, one row per lane, spread over the banks.  The W2
  // prologue waits behind this (the staging area covers the stage buffers).
  bf16x8 e[KH];
  {
    int x = step_input(io, m, m_ok, vg == 0 && kh == 0 && half == 0, V);
    x = min(max(x, 0), V - 1);
    const u32x4 dw1 = raw_desc(W1, (uint32_t)V * (uint32_t)r * 2u);
    uint16_t* greg = lds + wave * kGatherWave;
    const int c = lane & 31;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int q = 2 * i + (lane >> 5);
      const int xq = __shfl(x, q);
      const bool okq = rb * ROWS + pair * 32 + q < R;
      const int piece = c ^ q;
      const uint32_t voff = (okq && kh * 256 + piece * 8 < r)
                                ? (uint32_t)xq * (uint32_t)r * 2u + (uint32_t)(kh * 512 + piece * 16)
                                : kOutOfRange;
      asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                   :
                   : "v"(voff), "s"(dw1), "{m0}"(lds_addr(greg + 2 * i * 256))
                   : "memory");
    }
    wait_vmcnt<0>();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < KH; ++s)
      e[s] = *reinterpret_cast<const bf16x8*>(greg + col * 256 + (((2 * s + half) ^ col) & 31) * 8);
    lds_barrier();   // every wave has its rows before the stage buffers are reused
  }

  const u32x4 dw2 = raw_desc(W2, (uint32_t)V * (uint32_t)r * 2u);
  const uint32_t w2_off = w2_dma_lane_offset(lane, r);
  const Rsrc rbase = MODE == kBiasOnly ? make_rsrc(W2, 0u) : block_rsrc(base, ad, rb, ROWS);
  const Rsrc runif = MODE == DSPARK_SAMPLE ? block_rsrc(unif, ad, rb, ROWS) : rbase;
  const uint32_t e_off =
      (EPI == kEpiCol && !m_ok)
          ? kOutOfRange
          : (uint32_t)(m_loc * ad.row_stride + (16 * kh + 4 * half) * ad.vstride) * 4u;
  const uint32_t e_cb = (uint32_t)ad.cstride * 4u;
  const size_t vstride = EPI == kEpiCol ? ad.vstride : 1;
  const int e_vs = (int)vstride * 4;

  float eb[NS][8];
  float eu[NS][8];
  float own[8];
  Argmax am;

  // Epilogue of iteration i: own half-tile + partner's from xbuf slot xs.
  auto epilogue = [&](auto masked, int i, int xs, const float (&cb)[8], const float (&cu)[8]) {
    constexpr bool MASKED = decltype(masked)::value;
    const float* px = xbuf + (((size_t)xs * NW + (wave ^ 1)) * 64 + lane) * 8;
    const float4 p0 = *reinterpret_cast<const float4*>(px);
    const float4 p1 = *reinterpret_cast<const float4*>(px + 4);
    const float part[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    const int cv = (c0 + i * cstep) * kChunk;
    const int vlim = i < n_valid ? V : 0;
    float z[8];
#pragma unroll
    for (int qq = 0; qq < 8; ++qq) z[qq] = part[qq] + own[qq];
    select_chunk<MODE, 8, MASKED>(am, cb, z, cu, kscale, i, vlim - cv - 16 * kh - 4 * half);
    if (BIAS && m_ok) {
      float* oc = bias_out + ad.k_off + (size_t)m * ad.row_stride + (size_t)chunk(i) * ad.cstride;
#pragma unroll
      for (int qq = 0; qq < 8; ++qq) {
        const int o = 16 * kh + 8 * (qq >> 2) + 4 * half + (qq & 3);
        if (cv + o < vlim) oc[o * vstride] = z[qq];
      }
    }
  };

  auto body = [&](auto masked, auto first, int t, float (&pb)[8], float (&pu)[8], float (&nb)[8],
                  float (&nu)[8]) {
    // This wave's rows of chunk t have landed; the barrier publishes all rows.
    if constexpr (decltype(first)::value) wait_vmcnt<0>();
    else wait_vmcnt<DMA_WAIT>();
    lds_barrier();
    w2_dma<NW>(lds + ((t + WD) % NBUF) * BUF, dw2, w2_off, chunk(t + WD), r, wave);
    __builtin_amdgcn_sched_barrier(0);

    // Wave kh reads the chunk's rows as col ^ 16*kh, so its own 16 rows always
    // land in acc[0..7] and the partner's in acc[8..15] (constant indices).
    const uint16_t* abase =
        lds + (t % NBUF) * BUF + (col ^ (16 * kh)) * PITCH + half * 8 + kh * KH * 16;
    f32x16 acc = {};
#pragma unroll
    for (int s0 = 0; s0 < KH; s0 += 4) {
      bf16x8 a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const bf16x8*>(abase + (s0 + i) * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], e[s0 + i], acc, 0, 0, 0);
    }
    // Epilogue of the previous chunk (its partner half was written before this
    // iteration's barrier).  At t = 0 there is none (a uniform branch with no
    // memory loads).
    if (!decltype(first)::value || t >= 1) epilogue(masked, t - 1, (t - 1) & 1, pb, pu);
    mfma_pipeline<KH>();
    // Hand the other half-tile to the partner; keep ours for the next iteration.
    float* px = xbuf + (((size_t)(t & 1) * NW + wave) * 64 + lane) * 8;
    *reinterpret_cast<float4*>(px) = make_float4(acc[8], acc[9], acc[10], acc[11]);
    *reinterpret_cast<float4*>(px + 4) = make_float4(acc[12], acc[13], acc[14], acc[15]);
#pragma unroll
    for (int qq = 0; qq < 8; ++qq) own[qq] = acc[qq];
    // The slot of iteration t-1 is free now: refill it with iteration t + PD.
    epi_load<MODE, EPI, 2>(nb, nu, rbase, runif, e_off + (uint32_t)chunk(t + PD) * e_cb, e_vs);
    __builtin_amdgcn_sched_barrier(0);
  };

#pragma unroll
  for (int t = 0; t < (WD > PD ? WD : PD); ++t) {
    if (t < WD) w2_dma<NW>(lds + t * BUF, dw2, w2_off, chunk(t), r, wave);
    if (t < PD)
      epi_load<MODE, EPI, 2>(eb[t], eu[t], rbase, runif, e_off + (uint32_t)chunk(t) * e_cb, e_vs);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Iteration t's epilogue inputs live in slot t % NS; iteration t finishes
  // iteration t-1 and refills that slot with iteration t + PD.
  // The first UNR iterations (the first has no previous chunk) and those from
  // n_main on run the masked select; in between every epilogue's chunk lies
  // wholly inside V.
  const int n_main = n_whole(c0, cstep, n_valid, V) / UNR * UNR;
#pragma unroll
  for (int j = 0; j < UNR; ++j)
    body(std::true_type{}, std::true_type{}, j, eb[(j + NS - 1) % NS],
         eu[(j + NS - 1) % NS], eb[(j + PD) % NS], eu[(j + PD) % NS]);
  int i0 = UNR;
  for (; i0 < n_main; i0 += UNR) {
#pragma unroll
    for (int j = 0; j < UNR; ++j)
      body(std::false_type{}, std::false_type{}, i0 + j, eb[(j + NS - 1) % NS],
           eu[(j + NS - 1) % NS], eb[(j + PD) % NS], eu[(j + PD) % NS]);
  }
  for (; i0 < cpg; i0 += UNR) {
#pragma unroll
    for (int j = 0; j < UNR; ++j)
      body(std::true_type{}, std::false_type{}, i0 + j, eb[(j + NS - 1) % NS],
           eu[(j + NS - 1) % NS], eb[(j + PD) % NS], eu[(j + PD) % NS]);
  }
  // No direct load may land in LDS after this point (the merge below reuses
  // stage memory, and the workgroup's LDS is released at exit).
  wait_vmcnt<0>();
  lds_barrier();   // the partner's last half-tile
  // cpg is a multiple of UNR (hence of NS): the last iteration's slot is NS - 1.
  epilogue(std::true_type{}, cpg - 1, (cpg - 1) & 1, eb[NS - 1], eu[NS - 1]);

  float best = am.best;
  int best_i = argmax_id(am, c0, cstep, 16 * kh + 4 * half);
  const float ov = __shfl_xor(best, 32);
  const int oi = __shfl_xor(best_i, 32);
  merge_best(best, best_i, ov, oi);
  // Merge the pair's two halves through LDS (the W2 staging area is free: every
  // wave finished its MFMAs before the barrier above), one partial per group.
  float2* xch = reinterpret_cast<float2*>(smem);
  if (kh == 1 && half == 0) xch[pair * 32 + col] = make_float2(best, __int_as_float(best_i));
  lds_barrier();
  if (kh == 0 && half == 0 && m_ok) {
    const float2 o = xch[pair * 32 + col];
    merge_best(best, best_i, o.x, __float_as_int(o.y));
    atomicMax(io.best + (size_t)m * io.sub + (vg & (io.sub - 1)), pack_best(best, best_i));
  }
}

__global__ __launch_bounds__(256) void clear_words_kernel(uint4* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// tokens[m][k] from the packed results of the last step.
__global__ __launch_bounds__(256) void last_tokens_kernel(const unsigned long long* __restrict__ w,
                                                          int S, int R, int V, int gamma, int k,
                                                          int32_t* __restrict__ tokens) {
  const int m = blockIdx.x * 256 + threadIdx.x;
  if (m < R) tokens[(size_t)m * gamma + k] = read_token(w, m, S, V);
}

// ---- host side: kernel variants ----

using StepKernel = void (*)(const uint16_t*, const uint16_t*, const float*, const float*,
                            StepIO, int, int, int, float, int, int, int, int, int, Addr, float*);

struct StepVariant {
  StepKernel fn;
  int threads;
  size_t lds;
  int rows;     // requests per workgroup
  int unroll;   // chunks per group must be a multiple of this
};

template <int RK, int NW, int MODE, int EPI, bool BIAS, int TW = 1>
StepVariant plain_variant() {
  return {&markov_step_kernel<RK, NW, MODE, EPI, BIAS, TW>, NW * 64, plain_lds_bytes<RK, NW, TW>(),
          NW * 32 * TW, plain_unroll<RK, NW>()};
}
template <int NP, int MODE, int EPI, bool BIAS>
StepVariant ksplit_variant() {
  return {&markov_step_ksplit_kernel<NP, MODE, EPI, BIAS>, NP * 128, ksplit_lds_bytes<NP>(),
          NP * 32, kSplitUnroll};
}

template <int RK, int MODE, int EPI, bool BIAS>
StepVariant plain_by_nw(int nw, int tw) {
  // Two tiles per wave: bias-only GEMM at ranks 128 and 256, 4 or 8 waves, no
  // bias output (the only combinations built; with the logits streams as well
  // the registers spill).
  if constexpr ((RK == 128 || RK == 256) && !BIAS && MODE == kBiasOnly) {
    if (tw == 2) return nw == 8 ? plain_variant<RK, 8, MODE, EPI, BIAS, 2>()
                                : plain_variant<RK, 4, MODE, EPI, BIAS, 2>();
  }
  switch (nw) {
    case 1: return plain_variant<RK, 1, MODE, EPI, BIAS>();
    case 2: return plain_variant<RK, 2, MODE, EPI, BIAS>();
    case 4: return plain_variant<RK, 4, MODE, EPI, BIAS>();
    default: return plain_variant<RK, 8, MODE, EPI, BIAS>();
  }
}
template <int MODE, int EPI, bool BIAS>
StepVariant pick3(const MarkovPlan& p) {
  if (p.ksplit) {
    switch (p.nw / 2) {
      case 1: return ksplit_variant<1, MODE, EPI, BIAS>();
      case 2: return ksplit_variant<2, MODE, EPI, BIAS>();
      default: return ksplit_variant<4, MODE, EPI, BIAS>();
    }
  }
  switch (p.rk) {
    case 64: return plain_by_nw<64, MODE, EPI, BIAS>(p.nw, p.tw);
    case 128: return plain_by_nw<128, MODE, EPI, BIAS>(p.nw, p.tw);
    case 256: return plain_by_nw<256, MODE, EPI, BIAS>(p.nw, p.tw);
    default: return plain_by_nw<512, MODE, EPI, BIAS>(p.nw, p.tw);
  }
}
template <int MODE>
StepVariant pick2(const MarkovPlan& p, int epi, bool bias) {
  switch (epi) {
    case kEpiCol: return bias ? pick3<MODE, kEpiCol, true>(p) : pick3<MODE, kEpiCol, false>(p);
    case kEpiVec4: return bias ? pick3<MODE, kEpiVec4, true>(p) : pick3<MODE, kEpiVec4, false>(p);
    default: return bias ? pick3<MODE, kEpiScalar, true>(p) : pick3<MODE, kEpiScalar, false>(p);
  }
}
StepVariant pick_variant(const MarkovPlan& p, int mode, int epi, bool bias) {
  // No logits stream: the epilogue mode only decides where the bias goes.
  if (mode == kBiasOnly) {
    if (!bias) return pick3<kBiasOnly, kEpiVec4, false>(p);
    return epi == kEpiCol ? pick3<kBiasOnly, kEpiCol, true>(p) : pick3<kBiasOnly, kEpiVec4, true>(p);
  }
  return mode == DSPARK_SAMPLE ? pick2<DSPARK_SAMPLE>(p, epi, bias)
                               : pick2<DSPARK_GREEDY>(p, epi, bias);
}

// Per-kernel launch attributes and occupancy, resolved once per variant and
// device (host threads may call concurrently).
struct VariantState {
  StepKernel fn;
  int device;
  int blocks_per_cu;
};
VariantState g_states[512];
int g_nstates = 0;
std::mutex g_states_mu;

int prepare_variant(const StepVariant& v) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  std::lock_guard<std::mutex> lock(g_states_mu);
  for (int i = 0; i < g_nstates; ++i)
    if (g_states[i].fn == v.fn && g_states[i].device == dev) return g_states[i].blocks_per_cu;
  const void* f = reinterpret_cast<const void*>(v.fn);
  if (hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)v.lds) != hipSuccess)
    return -1;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, f, v.threads, v.lds) != hipSuccess || nb < 1)
    nb = 1;
  if (g_nstates < 512) g_states[g_nstates++] = {v.fn, dev, nb};
  return nb;
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
  (void)for_launch;
  MarkovPlan p{};
  p.rk = r <= 64 ? 64 : r <= 128 ? 128 : r <= 256 ? 256 : 512;
  const int waves_needed = (R + 31) / 32;
  int nw = waves_needed >= 8 ? 8 : waves_needed >= 4 ? 4 : waves_needed >= 2 ? 2 : 1;
  // Choices measured on MI355X.  Rank 512 sampling: K-split wave pairs (a
  // plain wave would need the whole SIMD); rank 512 greedy: eight plain waves;
  // up to 64 requests: two-wave workgroups, at most two per CU (fewer,
  // longer groups).  DSPARK_MARKOV_KSPLIT / _NW / _WG / _STRIDED override the
  // choice for tuning (and DSPARK_MARKOV_SUBWORDS the words per request).
  if (p.rk == 512 && mode == DSPARK_SAMPLE && nw == 8) nw = 4;
  const int ks_env = env_int("DSPARK_MARKOV_KSPLIT", -1);
  p.ksplit = p.rk == 512 && (ks_env < 0 ? mode == DSPARK_SAMPLE : ks_env != 0);
  if (p.ksplit) nw = 2 * (waves_needed >= 4 ? 4 : waves_needed >= 2 ? 2 : 1);
  const int nw_env = env_int("DSPARK_MARKOV_NW", 0);
  if (!p.ksplit && (nw_env == 1 || nw_env == 2 || nw_env == 4 || nw_env == 8)) nw = nw_env;
  p.nw = nw;
  // Two tiles per wave halve the LDS reads per MFMA: the bias-only GEMM at
  // ranks 128-256 (DSPARK_MARKOV_TW=1 turns it off).  With bias output the
  // table has no such variant; the launch then falls back to one tile and
  // recomputes the R blocks from the variant's rows.
  const int tw_env = env_int("DSPARK_MARKOV_TW", 0);
  p.tw = (tw_env == 1 || tw_env == 2) ? tw_env : (mode == kBiasOnly ? 2 : 1);
  if (p.ksplit || (p.rk != 128 && p.rk != 256) || (nw != 4 && nw != 8) || mode != kBiasOnly)
    p.tw = 1;
  const int rows = p.ksplit ? nw / 2 * 32 : nw * 32 * p.tw;
  p.n_rblocks = (R + rows - 1) / rows;
  p.n_chunks = (V + kChunk - 1) / kChunk;
  // packed per-step results [gamma][R][S], sized for the largest S
  p.ws_bytes = (size_t)gamma * (size_t)R * kMaxSubWords * 8;
  return p;
}

dspark_status launch_markov_draft(const uint16_t* W1, const uint16_t* W2, const float* base,
                                  const int32_t* anchors, int R, int gamma, int V, int r,
                                  int layout, int mode, float temperature,
                                  const float* uniforms, int32_t* tokens, float* bias_out,
                                  void* workspace, const dspark_step_events* events,
                                  hipStream_t stream) {
  // No base logits: greedy on the Markov bias alone.
  const int kmode = base ? mode : kBiasOnly;
  MarkovPlan p = plan_markov(R, gamma, V, r, kmode, true);
  auto a16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
  const bool tiled = layout == DSPARK_LAYOUT_TILED;
  const bool vec4 = V % 4 == 0 && a16(base) && (!uniforms || a16(uniforms)) &&
                    (!bias_out || a16(bias_out));
  const int epi = tiled ? kEpiCol : vec4 ? kEpiVec4 : kEpiScalar;
  const StepVariant var = pick_variant(p, kmode, epi, bias_out != nullptr);
  p.n_rblocks = (R + var.rows - 1) / var.rows;   // the variant's requests per workgroup
  const int bpc = prepare_variant(var);
  if (bpc < 0) return fail(DSPARK_EDEVICE, "hipFuncSetAttribute failed for the Markov step kernel");

  // One wave of workgroups: as many as fit on the device at once, split between
  // the R blocks (each V group is walked by n_rblocks workgroups).  Groups hold
  // a multiple of the kernel's unroll factor of chunks.
  const int max_groups = p.n_chunks < kMaxGroups ? p.n_chunks : kMaxGroups;
  int target = env_int("DSPARK_MARKOV_WG", 0);
  if (target <= 0) target = device_cus() * (p.n_rblocks == 1 && R <= 64 && bpc > 2 ? 2 : bpc);
  if (target < 8) target = 8;
  int groups = (target + p.n_rblocks - 1) / p.n_rblocks;
  groups = (groups + 7) / 8 * 8;
  if (groups > max_groups) groups = max_groups;
  if (groups < 1) groups = 1;
  p.cpg = (p.n_chunks + groups - 1) / groups;
  p.cpg = (p.cpg + var.unroll - 1) / var.unroll * var.unroll;
  // Contiguous groups: group g owns chunks [g*cpg, (g+1)*cpg).  Strided groups:
  // group g owns chunks g, g + G, g + 2G, ... (all G groups in flight read one
  // contiguous window of W2 and of the logits at a time).
  // Strided groups measured faster for the tiled layout at R >= 128 (sampling
  // and long blocks); row-major rows are far apart whichever way V is split.
  const int st_env = env_int("DSPARK_MARKOV_STRIDED", -1);
  const bool strided = st_env < 0 ? (tiled && R >= 128) : st_env != 0;
  p.n_vgroups = strided ? groups : (p.n_chunks + p.cpg - 1) / p.cpg;
  const int cstep = strided ? groups : 1;

  unsigned long long* packed = reinterpret_cast<unsigned long long*>(workspace);
  int sub = p.n_vgroups > kSubWordsAboveGroups ? kMaxSubWords : 1;
  const int sub_env = env_int("DSPARK_MARKOV_SUBWORDS", 0);
  if (sub_env == 1 || sub_env == 2 || sub_env == 4 || sub_env == 8 || sub_env == 16) sub = sub_env;
  const size_t words = (size_t)R * sub;
  const size_t nclear = ((size_t)gamma * words + 1) / 2;   // 16-byte stores
  const size_t cblocks = (nclear + 255) / 256;
  hipLaunchKernelGGL(clear_words_kernel, dim3(cblocks < 1024 ? (unsigned)cblocks : 1024u),
                     dim3(256), 0, stream, reinterpret_cast<uint4*>(workspace), nclear);
  const int padded_groups = (p.n_vgroups + 7) / 8 * 8;
  const dim3 grid(padded_groups * p.n_rblocks);
  const float inv_t = mode == DSPARK_SAMPLE ? 1.0f / temperature : 1.0f;
  // Column-tiled [gamma][C][32][R]: one step is C * 32 * R floats, and each
  // launch's range ends with its own step (rows past R are sent past it).
  const size_t step_floats = (size_t)p.n_chunks * kChunk * R;
  Addr ad;
  ad.row_stride = tiled ? 1 : (size_t)gamma * V;
  ad.cstride = tiled ? (size_t)kChunk * R : (size_t)kChunk;
  ad.vstride = tiled ? (size_t)R : 1;
  ad.total = (size_t)R * gamma * V;
  for (int k = 0; k < gamma; ++k) {
    const StepIO io{anchors, k == 0 ? nullptr : packed + (size_t)(k - 1) * words,
                    packed + (size_t)k * words, tokens, gamma, k, sub};
    ad.k_off = tiled ? (size_t)k * step_floats : (size_t)k * V;
    if (tiled) ad.total = ad.k_off + step_floats;
    // Timing hooks ride on the dispatch itself (start / stop timestamps of the
    // kernel's packet), so they add no marker packets between kernels.
    hipEvent_t ev_begin = nullptr, ev_end = nullptr;
    if (events && k < events->count) {
      if (events->begin) ev_begin = reinterpret_cast<hipEvent_t>(events->begin[k]);
      if (events->end) ev_end = reinterpret_cast<hipEvent_t>(events->end[k]);
    }
    hipExtLaunchKernelGGL(var.fn, grid, dim3(var.threads), (uint32_t)var.lds, stream, ev_begin,
                          ev_end, 0u, W1, W2, base, uniforms, io, R, V, r, inv_t, p.n_rblocks,
                          p.n_vgroups, p.cpg, cstep, p.n_chunks, ad, bias_out);
    dspark_status st = check_launch("markov_step_kernel");
    if (st != DSPARK_OK) return st;
  }
  hipLaunchKernelGGL(last_tokens_kernel, dim3((R + 255) / 256), dim3(256), 0, stream,
                     packed + (size_t)(gamma - 1) * words, sub, R, V, gamma, gamma - 1,
                     tokens);
  return check_launch("last_tokens_kernel");
}

}  // namespace dspark
