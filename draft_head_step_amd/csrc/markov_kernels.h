// Markov-head refinement step kernels for CDNA4 (gfx950).  Included by the
// markov_pick_*.hip units, each of which instantiates one slice of the variant
// table (they compile in parallel).
//
// One draft position k of every request at once ([P1] section 二 design 1,
// Markov-head equation; [P3] part 01; [P4] logits bias):
//   e_m  = W1[x_{k-1,m}, :]                      gather, x_0 = anchor
//   z_mv = base[m, k, v] + sum_i e_mi * W2(i, v)  bf16 MFMA, fp32 accumulation
//   x_k  = argmax_v z_mv  |  argmax_v z_mv / T - ln(-ln u_mv)
//
// Design (HBM-bound: W2, base and the uniforms are each read once per step):
//   * Both MFMA operands are K-contiguous rows of the [V, r] stores of W1 and
//     W2.  With the column-tiled logits (and with none) the tile is computed
//     transposed, bias^T[v, m] = W2^T[v, :] . e_m: each lane's accumulators are
//     one request and 16 vocabulary entries, and one four-byte load of an
//     entry for the tile's 32 requests reads a whole 128-byte line.  With
//     row-major logits the operands swap, bias[m, v] = e_m . W2(:, v): each
//     lane's accumulators are one vocabulary entry and 16 requests, and one
//     four-byte load of one request's 32 entries across a half-wave reads a
//     whole line.  The register layouts of the two operands are the same, so
//     the swap costs nothing; only the selection keeps one running maximum per
//     request row instead of one per lane, and merges them across lanes once.
//   * A wave owns 32 requests and keeps their gathered W1 rows (one MFMA
//     operand) in registers for the whole launch.  The workgroup's waves share
//     32-column chunks of W2 staged through LDS (double-buffered, rows padded
//     by 16 bytes so the operand reads hit distinct banks).
//   * Each workgroup walks a group of chunks keeping a running (max, argmax)
//     per request, then folds it into one packed 64-bit word per request with
//     an integer atomic max (order-independent, so results are deterministic).
//     The next step reads its input tokens from those words (and its first V
//     group stores them to the output).
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
//   * Rank 512: the gathered rows take 128 VGPRs per lane.  Either a plain
//     wave holds them all (two waves per SIMD at most), or K-split wave pairs
//     (each wave holds one K half, 64 VGPRs; partial tiles are exchanged
//     through LDS and the epilogue of chunk c-1 runs beside the MFMAs of
//     chunk c).
//   * Ids are checked: a request whose input token is outside [0, V) gathers a
//     zero row and publishes the poison word, so its tokens read -1.
#pragma once

#include <math.h>

#include <type_traits>

#include "markov_types.h"
#include "packed_words.h"
#include "sched_lds.h"

namespace dspark {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

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
// The same merge without a branch (so that shuffles feeding several merges
// can all be in flight at once).
__device__ __forceinline__ void merge_best_sel(float& bv, int& bi, float ov, int oi) {
  const bool take = (ov > bv) | ((ov == bv) & (oi < bi));
  bv = take ? ov : bv;
  bi = take ? oi : bi;
}

// Token x_{k-1} of request m (step 0: the anchor), or -1 if it is not a valid
// id.  The first V group of each R block also stores it to tokens, which
// completes step k-1 there.
__device__ __forceinline__ int step_input(const StepIO& io, int m, bool m_ok, bool writer,
                                          int V) {
  if (!m_ok) return -1;
  if (!io.prev) {
    const int a = io.anchors[m];
    return (a >= 0 && a < V) ? a : -1;
  }
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

// Running argmax of one lane over one request (requests on the lanes).
// Element q of a chunk is vocabulary entry (chunk)*32 + lane offset + 8*(q/4)
// + (q%4).  Per element only the score and q are kept (q is an inline
// constant); the iteration whose chunk raised the maximum is recorded once per
// chunk and the id is rebuilt at the end.  Chunks arrive in increasing v and q
// runs in increasing v within a chunk, so a strict comparison keeps the
// smallest id among equal maxima.
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

// Running argmaxes of one lane over N requests (vocabulary entries on the
// lanes): one entry per chunk for each row, so a row keeps its best score and
// the iteration it came from.
template <int N>
struct RowArgmax {
  float best[N];
  int iter[N];
  __device__ RowArgmax() {
#pragma unroll
    for (int q = 0; q < N; ++q) {
      best[q] = -INFINITY;
      iter[q] = -1;
    }
  }
};

template <int MODE, int N, bool MASKED>
__device__ __forceinline__ void select_rows(RowArgmax<N>& am, const float* cb, const float* z,
                                            const float* cu, float kscale, int iter,
                                            bool entry_ok) {
#pragma unroll
  for (int q = 0; q < N; ++q) {
    const float sc = select_score<MODE>(cb[q], z[q], cu[q], kscale);
    const bool take = MASKED ? (sc > am.best[q] && entry_ok) : sc > am.best[q];
    am.best[q] = take ? sc : am.best[q];
    am.iter[q] = take ? iter : am.iter[q];
  }
}

// Merges the N rows' (score, id) across the 32 lanes of each half-wave (lane
// col = vocabulary entry).  Halving steps over lane bits 4, 3, ...: a lane
// keeps half of its rows (the upper half if its bit is set) and merges in its
// partner's best of the same rows, until it holds one row; full merges over
// the remaining low lane bits follow.  On return v[0] / id[0] hold the result
// for row merged_row(lane), the lane's bits 4 down to 5 - log2(N) read as a
// binary number; the lanes whose lower bits are zero (merged_publisher) hold
// each row once.
template <int N>
__device__ __forceinline__ void merge_rows(float (&v)[N], int (&id)[N], int lane) {
  // A lane sends its partner the half it drops (the half the partner keeps),
  // and every shuffle of a level is issued before any merge: the merges are
  // branch-free selects, so the shuffles do not wait for each other.  The
  // halves are picked by bit masks, not by selects between array elements
  // (which the compiler turns into a dynamically indexed scratch load).
#pragma unroll
  for (int lvl = 0; (N >> lvl) > 1; ++lvl) {
    constexpr int NH = N / 2;
    const int mask = 16 >> lvl;
    const int H = (N >> lvl) / 2;
    const int hi = (lane & mask) ? -1 : 0;   // all ones: this lane keeps the upper half
    float ov[NH];
    int oi[NH];
#pragma unroll
    for (int p = 0; p < H; ++p) {
      const int lv = __float_as_int(v[p]), hv = __float_as_int(v[H + p]);
      ov[p] = __shfl_xor(__int_as_float((lv & hi) | (hv & ~hi)), mask);
      oi[p] = __shfl_xor((id[p] & hi) | (id[H + p] & ~hi), mask);
    }
#pragma unroll
    for (int p = 0; p < H; ++p) {
      const int lv = __float_as_int(v[p]), hv = __float_as_int(v[H + p]);
      float mv = __int_as_float((hv & hi) | (lv & ~hi));
      int mi = (id[H + p] & hi) | (id[p] & ~hi);
      merge_best_sel(mv, mi, ov[p], oi[p]);
      v[p] = mv;
      id[p] = mi;
    }
  }
  constexpr int LOG = N == 16 ? 4 : N == 8 ? 3 : N == 4 ? 2 : N == 2 ? 1 : 0;
#pragma unroll
  for (int mask = 16 >> LOG; mask >= 1; mask >>= 1) {
    const float ov = __shfl_xor(v[0], mask);
    const int oi = __shfl_xor(id[0], mask);
    merge_best_sel(v[0], id[0], ov, oi);
  }
}

// Row index (0..N-1) a lane holds after merge_rows, and whether it publishes it.
template <int N>
__device__ __forceinline__ int merged_row(int lane) {
  constexpr int LOG = N == 16 ? 4 : N == 8 ? 3 : N == 4 ? 2 : N == 2 ? 1 : 0;
  return ((lane & 31) >> (5 - LOG)) & (N - 1);
}
template <int N>
__device__ __forceinline__ bool merged_publisher(int lane) {
  constexpr int LOG = N == 16 ? 4 : N == 8 ? 3 : N == 4 ? 2 : N == 2 ? 1 : 0;
  return (lane & ((1 << (5 - LOG)) - 1)) == 0;
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
// Four-byte load of a stream read once (non-temporal: the line is not kept in
// the caches).  The uniform part of the offset rides in soffset, which the
// range check does not cover: an out-of-range lane must carry it in `off`.
__device__ __forceinline__ float buf_load4_nt(Rsrc r, uint32_t off, int soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 2));
}

// Keeps a value in a VGPR as computed, so the compiler cannot move a uniform
// part of a buffer offset into the (unchecked) scalar offset.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm("" : "+v"(x));
  return x;
}

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

// VMEM instructions one epi_load issues for NJ accumulator groups (they count
// in vmcnt with the direct loads).  Every load is a separate four-byte load:
// the column layout's loads differ only in soffset and the row layout's in an
// opaque per-lane offset, so the compiler merges none of them.
template <int MODE, int EPI, int NJ>
constexpr int epi_load_count() {
  return MODE == kBiasOnly || EPI == kEpiNone ? 0 : 4 * NJ * (MODE == DSPARK_SAMPLE ? 2 : 1);
}

// Epilogue inputs of NJ accumulator groups of one chunk for one lane.
//   kEpiCol (requests on the lanes): element 4*j + i is vocabulary entry
//     v0 + 8*j + 4*half + i of the lane's request; `off` is the lane's byte
//     offset of entry v0 + 4*half and `vs` the byte distance between
//     consecutive entries, which rides in soffset (always in range: the
//     layout pads the last chunk).
//   kEpiRow (entries on the lanes): element 4*j + i is request row
//     8*j + 4*half + i of the lane's entry; `off` is the lane's byte offset of
//     its entry in row 4*half and `vs` the byte distance between rows.  Every
//     offset stays in the per-lane register, so rows past R and entries past
//     the end of the array fail the range check and read zero.
template <int MODE, int EPI, int NJ>
__device__ __forceinline__ void epi_load(float (&bv)[4 * NJ], float (&uv)[4 * NJ], Rsrc rbase,
                                         Rsrc runif, uint32_t off, uint32_t vs) {
  if (MODE == kBiasOnly || EPI == kEpiNone) {
#pragma unroll
    for (int j = 0; j < 4 * NJ; ++j) bv[j] = 0.0f;
    return;
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (EPI == kEpiCol) {
        const int so = (8 * j + i) * (int)vs;
        bv[4 * j + i] = buf_load4_nt(rbase, off, so);
        if (MODE == DSPARK_SAMPLE) uv[4 * j + i] = buf_load4_nt(runif, off, so);
      } else {
        const uint32_t o = opaque(off + (uint32_t)(8 * j + i) * vs);
        bv[4 * j + i] = buf_load4_nt(rbase, o, 0);
        if (MODE == DSPARK_SAMPLE) uv[4 * j + i] = buf_load4_nt(runif, o, 0);
      }
    }
  }
}

constexpr int lcm_small(int a, int b) { return (a % b == 0) ? a : (b % a == 0) ? b : a * b; }

// Scheduling template for one chunk's MFMA chain (masks: 0x100 LDS read,
// 0x008 MFMA, 0x002 VALU): kLdsAhead operand reads first, then per K-step
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

// Embedding part of the confidence logit ([P1] section 二 design 2, confidence
// head: the w_e . W1[x_{k-1}] term) for the 32 rows one wave has staged in LDS:
// COLS bf16 per row from K offset k0, source piece p of row q stored in slot
// p ^ (q & (COLS/8 - 1)).  Each lane takes one 16-byte piece (its eight w_e
// values stay in registers) of RPP rows per pass; the lanes of a row add their
// products in a fixed shuffle order.  Row q is request mbase + q, its token is
// lane q's x (NaN is written for an invalid token).  The 32 / RPP passes are
// shared out over the first V groups of the R block (this workgroup takes the
// passes congruent to `share` mod `nshare`): done by one workgroup alone they
// would make it finish well after the others.
template <int COLS>
constexpr int conf_embed_passes() { return 32 / (64 / (COLS / 8)); }

template <int COLS>
__device__ __forceinline__ void conf_embed_part(const uint16_t* greg, const float* __restrict__ w_e,
                                                int k0, int r, int mbase, int R, int x,
                                                float* __restrict__ se, int gamma, int k, int slot,
                                                int lane, int share, int nshare) {
  constexpr int PPR = COLS / 8;
  constexpr int RPP = 64 / PPR;
  const int c = lane % PPR;
  const int kk = k0 + c * 8;
  float w[8];
  if (kk < r) {   // r is a multiple of 16: a piece is wholly inside or outside
    const float4 a = *reinterpret_cast<const float4*>(w_e + kk);
    const float4 b = *reinterpret_cast<const float4*>(w_e + kk + 4);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) w[t] = 0.0f;
  }
#pragma unroll 1
  for (int ps = share; ps < 32 / RPP; ps += nshare) {
    const int q = ps * RPP + lane / PPR;
    const u32x4 v = *reinterpret_cast<const u32x4*>(greg + q * COLS + ((c ^ (q & (PPR - 1))) * 8));
    float p = w[0] * bf_lo(v.x);
    p = fmaf(w[1], bf_hi(v.x), p);
    p = fmaf(w[2], bf_lo(v.y), p);
    p = fmaf(w[3], bf_hi(v.y), p);
    p = fmaf(w[4], bf_lo(v.z), p);
    p = fmaf(w[5], bf_hi(v.z), p);
    p = fmaf(w[6], bf_lo(v.w), p);
    p = fmaf(w[7], bf_hi(v.w), p);
#pragma unroll
    for (int o = 1; o < PPR; o <<= 1) p += __shfl_xor(p, o);
    const int xq = __shfl(x, q);
    const int m = mbase + q;
    if (c == 0 && m < R) se[((size_t)m * gamma + k) * 2 + slot] = xq >= 0 ? p : NAN;
  }
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
  constexpr bool ROWF = EPI == kEpiRow;            // vocabulary entries on the lanes
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
  static_assert(TW == 1 || !ROWF, "two tiles per wave only with requests on the lanes");
  // W1 rows staged through LDS (see plain_gather_rounds).
  constexpr int GROUNDS = plain_gather_rounds<RK, NW, TW>();
  constexpr int GWPR = NW / GROUNDS;                 // waves staging per round
  static_assert(NW % GROUNDS == 0 && (size_t)GWPR * TW * 32 * RK * 2 <= 160 * 1024,
                "W1 staging must fit the CU's LDS");
  // vmcnt at the top of an iteration that leaves only the loads issued after
  // the DMA of its own chunk outstanding (0 with bias stores in flight).
  constexpr int EL = epi_load_count<MODE, EPI, 4>();
  constexpr int DMA_WAIT = BIAS ? 0 : EL + (WD - 1) * (kChunk / NW + EL);

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
  // Iteration i (0 <= i < n_valid rounded up to a multiple of UNR) handles
  // chunk c0 + i * cstep: contiguous groups (cstep 1) or groups strided across
  // V (cstep = number of groups).  Iterations past the group's n_valid chunks
  // are masked, and prefetches are clamped to the group's last chunk.
  const int c0 = cstep == 1 ? vg * cpg : vg;
  const int n_valid = cstep == 1 ? min(cpg, n_chunks - c0) : (n_chunks - 1 - vg) / cstep + 1;
  auto chunk = [&](int i) { return c0 + min(i, n_valid - 1) * cstep; };
  uint16_t* lds = reinterpret_cast<uint16_t*>(smem);

  // Tile t of this wave holds requests (wave * TW + t) * 32 + (0..31) of the R
  // block; lane col gathers the row of request tbase + col.
  int tbase[TW];
  bool m_ok[TW];
  int xt[TW];
  uint32_t e_off[TW];
  bf16x8 e[TW][KS];
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    const int t_loc = (wave * TW + t) * 32;
    tbase[t] = rb * ROWS + t_loc;
    m_ok[t] = tbase[t] + col < R;
    if (ROWF) {
      // entries on the lanes: the lane's entry col in row 4*half of the tile
      e_off[t] = (uint32_t)((t_loc + 4 * half) * ad.row_stride + col) * 4u;
    } else {
      // Column-layout rows past R would alias the next entries, so they are
      // sent out of range.
      e_off[t] = (EPI == kEpiCol && !m_ok[t])
                     ? kOutOfRange
                     : (uint32_t)((t_loc + col) * ad.row_stride + 4 * half * ad.vstride) * 4u;
    }
    xt[t] = step_input(io, tbase[t] + col, m_ok[t], vg == 0 && half == 0, V);
  }

  const Rsrc rw2 = make_rsrc(W2, (uint32_t)V * (uint32_t)r * 2u);
  const u32x4 dw2 = raw_desc(W2, (uint32_t)V * (uint32_t)r * 2u);
  const uint32_t w2_off = DMA ? w2_dma_lane_offset(lane, r) : w2_lane_offset<RK, NT>(tid, r);
  const Rsrc rbase = (MODE == kBiasOnly || EPI == kEpiNone) ? make_rsrc(W2, 0u)
                                                             : block_rsrc(base, ad, rb, ROWS);
  const Rsrc runif = MODE == DSPARK_SAMPLE ? block_rsrc(unif, ad, rb, ROWS) : rbase;
  const uint32_t e_cb = (uint32_t)ad.cstride * 4u;
  const size_t vstride = EPI == kEpiCol ? ad.vstride : 1;
  const uint32_t e_vs = ROWF ? (uint32_t)ad.row_stride * 4u : (uint32_t)vstride * 4u;

  u32x4 stage[DMA ? 1 : WD][DMA ? 1 : PMAX];
  float eb[NS][TW][16];
  float eu[NS][TW][16];
  f32x16 accs[2][TW];
  Argmax am[TW];
  RowArgmax<ROWF ? 16 : 1> ram[TW];
  static_assert(UNR % 2 == 0 && UNR % NS == 0, "the unroll must cycle the rings");

  // Fused bias-add + select of iteration i.  Rows past R are never published,
  // so they need no mask.
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
      if constexpr (ROWF) {
        select_rows<MODE, 16, MASKED>(ram[t], cb[t], av, cu[t], kscale, i, cv + col < vlim);
        if (BIAS) {
#pragma unroll
          for (int qq = 0; qq < 16; ++qq) {
            const int mq = tbase[t] + 8 * (qq >> 2) + 4 * half + (qq & 3);
            if (mq < R && cv + col < vlim)
              bias_out[ad.k_off + (size_t)mq * ad.row_stride + (size_t)chunk(i) * ad.cstride +
                       col] = acc[t][qq];
          }
        }
      } else {
        select_chunk<MODE, 16, MASKED>(am[t], cb[t], av, cu[t], kscale, i, vlim - cv - 4 * half);
        if (BIAS && m_ok[t]) {
          float* oc = bias_out + ad.k_off + (size_t)(tbase[t] + col) * ad.row_stride +
                      (size_t)chunk(i) * ad.cstride;
#pragma unroll
          for (int qq = 0; qq < 16; ++qq) {
            const int o = 8 * (qq >> 2) + 4 * half + (qq & 3);
            if (cv + o < vlim) oc[o * ad.vstride] = acc[t][qq];
          }
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
    // Requests on the lanes: W2 is the first operand (bias^T); entries on the
    // lanes: the gathered rows are.  With two tiles per wave each W2 read
    // feeds two MFMAs.
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
          acc[t] = ROWF ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(e[t][s0 + i], a[i], acc[t], 0, 0, 0)
                        : __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], e[t][s0 + i], acc[t], 0, 0, 0);
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
  // w / GWPR into slot w % GWPR of the area.  Rows of requests past R, or with
  // an invalid token, read as zeros.
  constexpr int PPR = RK / 8;       // 16-byte pieces per row
  constexpr int RPI = 64 / PPR;     // rows per direct load
  const int gslot = wave % GWPR;
  const uint32_t w1_bytes = io.dense ? (uint32_t)R * (uint32_t)r * 2u : (uint32_t)V * (uint32_t)r * 2u;
  // Source byte offset of the 16-byte piece that direct load i of tile t moves
  // for this lane (out of range for a row that reads as zeros).
  auto gather_voff = [&](int t, int i) -> uint32_t {
    const int c = lane % PPR;
    const int qq = i * RPI + lane / PPR;
    const int xq = __shfl(xt[t], qq);
    const int mq = tbase[t] + qq;
    const bool okq = mq < R && (io.dense != nullptr || xq >= 0);
    const int src = io.dense ? mq : xq;
    const int piece = c ^ (qq & (PPR - 1));
    return (okq && piece * 8 < r) ? (uint32_t)src * (uint32_t)r * 2u + (uint32_t)(piece * 16)
                                  : kOutOfRange;
  };
  auto gather_issue = [&]() {
    const u32x4 dw1 = raw_desc(io.dense ? io.dense : W1, w1_bytes);
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      uint16_t* greg = lds + (gslot * TW + t) * 32 * RK;
#pragma unroll
      for (int i = 0; i < 32 / RPI; ++i) {
        const uint32_t voff = gather_voff(t, i);
        asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                     :
                     : "v"(voff), "s"(dw1), "{m0}"(lds_addr(greg + i * RPI * RK))
                     : "memory");
      }
    }
  };
  // Second round: the same pieces are loaded at the start, beside the first
  // round's direct loads, into the registers that will hold the rows (a lane
  // has KS pieces of 16 bytes per tile, as many as its MFMA operand), and are
  // written where the direct loads would put them once the first round has
  // read the area.  So only one round waits for the memory system.
  static_assert(32 / RPI == KS, "a lane's gathered pieces fill its operand registers");
  auto gather_prefetch = [&]() {
    const Rsrc rw1 = make_rsrc(io.dense ? io.dense : W1, w1_bytes);
#pragma unroll
    for (int t = 0; t < TW; ++t)
#pragma unroll
      for (int i = 0; i < KS; ++i)
        e[t][i] = __builtin_bit_cast(bf16x8, buf_load16(rw1, opaque(gather_voff(t, i))));
  };
  auto gather_put = [&]() {
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      uint16_t* greg = lds + (gslot * TW + t) * 32 * RK;
#pragma unroll
      for (int i = 0; i < KS; ++i)
        *reinterpret_cast<bf16x8*>(greg + i * RPI * RK + lane * 8) = e[t][i];
    }
  };
  // Waits for everything this wave issued, then reads the rows (and, in the
  // fused draft step, the first V groups share out the confidence head's
  // embedding term over them).
  auto gather_read = [&]() {
    wait_vmcnt<0>();
    __builtin_amdgcn_sched_barrier(0);
    const int nshare = min(n_vgroups, conf_embed_passes<RK>());
    if (io.se && vg < nshare) {
#pragma unroll
      for (int t = 0; t < TW; ++t)
        conf_embed_part<RK>(lds + (gslot * TW + t) * 32 * RK, io.w_e, 0, r, tbase[t], R, xt[t],
                            io.se, io.gamma, io.k, 0, lane, vg, nshare);
      // the plain kernel holds whole rows: the second K half is empty
      if (vg == 0) {
#pragma unroll
        for (int t = 0; t < TW; ++t)
          if (half == 0 && m_ok[t]) io.se[((size_t)(tbase[t] + col) * io.gamma + io.k) * 2 + 1] = 0.0f;
      }
    }
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
  if constexpr (GROUNDS == 2) {
    if (wave >= GWPR) gather_prefetch();
  }
  if constexpr (!DMA) prologue();
#pragma unroll
  for (int rd = 0; rd < GROUNDS; ++rd) {
    if (wave / GWPR == rd) {
      if (rd == 0) gather_issue();
      else gather_put();
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
  // Iterations past n_valid (rounded up to the unroll) would only repeat the
  // group's last chunk under a mask: a short last group stops early instead of
  // finishing last.
  const int n_iter = (n_valid + UNR - 1) / UNR * UNR;
  for (; i0 < n_iter; i0 += UNR) {
#pragma unroll
    for (int j = 0; j < UNR; ++j)
      body(std::true_type{}, std::false_type{}, i0 + j, stage[DMA ? 0 : j % WD], accs[j & 1],
           accs[(j + 1) & 1], eb[(j + NS - 1) % NS], eu[(j + NS - 1) % NS]);
  }
  // n_iter is a multiple of UNR: the last iteration used accs[1] and slot NS - 1.
  finish(std::true_type{}, n_iter - 1, accs[1], eb[NS - 1], eu[NS - 1]);
  if constexpr (DMA) wait_vmcnt<0>();   // no direct load lands in LDS after exit

#pragma unroll
  for (int t = 0; t < TW; ++t) {
    if constexpr (ROWF) {
      // Entries on the lanes: merge each row across the half-wave's 32 entries;
      // the publishing lanes then hold distinct rows.
      float bv[16];
      int bi[16];
#pragma unroll
      for (int qq = 0; qq < 16; ++qq) {
        bv[qq] = ram[t].best[qq];
        bi[qq] = ram[t].iter[qq] < 0 ? 0x7fffffff
                                     : (c0 + ram[t].iter[qq] * cstep) * kChunk + col;
      }
      merge_rows<16>(bv, bi, lane);
      const int qf = merged_row<16>(lane);
      const int ml = 8 * (qf >> 2) + 4 * half + (qf & 3);   // request tbase + ml
      const int xm = __shfl(xt[t], ml);
      const int mq = tbase[t] + ml;
      if (merged_publisher<16>(lane) && mq < R)
        atomicMax(io.best + (size_t)mq * io.sub + (vg & (io.sub - 1)),
                  xm >= 0 ? pack_best(bv[0], bi[0]) : kPoison);
    } else {
      // Lanes l and l^32 hold the same request: merge, then one lane publishes.
      float best = am[t].best;
      int best_i = argmax_id(am[t], c0, cstep, 4 * half);
      const float ov = __shfl_xor(best, 32);
      const int oi = __shfl_xor(best_i, 32);
      merge_best(best, best_i, ov, oi);
      if (m_ok[t] && half == 0)
        atomicMax(io.best + (size_t)(tbase[t] + col) * io.sub + (vg & (io.sub - 1)),
                  xt[t] >= 0 ? pack_best(best, best_i) : kPoison);
    }
  }
}

// ---------------------------------------------------------------------------
// K-split kernel (rank 512): wave pairs share 32 requests, one K half each.
// After its MFMAs each wave hands the half-tile it does not finish to its
// partner through a double-buffered LDS slot; the epilogue of chunk c-1 runs
// in iteration c beside the MFMAs of chunk c, so one barrier per chunk orders
// everything.  Requests on the lanes: each wave finishes 16 vocabulary rows of
// the tile and the pair merges its two (max, argmax) at the end.  Entries on
// the lanes: each wave finishes 16 requests of the tile and publishes them.
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

// The fused draft step's finishing work inside its last step (see StepIO),
// on a workgroup with no step work: x_{gamma-2} (the anchors when gamma = 1)
// from the previous step's words, the last position's embedding term from
// W1 and w_e, then the confidences, survivals and the schedule.
template <int NW>
__device__ void finish_in_step(const StepIO& io, const FinParams& fp, const uint16_t* W1, int R,
                               int V, int r, unsigned char* smem) {
  const FinishArgs fa{io.prev, io.sub, V, fp.sh, io.se, fp.sts, nullptr, fp.conf, fp.surv,
                      io.anchors, W1, io.w_e, r};
  schedule_lds_body<kFinStepItems, kFinInStep, NW>(smem, nullptr, fp.sps, R, io.gamma,
                                                   R * io.gamma, 0, 0, fp.lengths, fp.order,
                                                   fp.info, fa);
}

// The K-split step for one workgroup.  FIN: the fused draft step's last step
// (see FinParams), instantiated in a kernel of its own so that the other steps
// run without it.
template <int NP, int MODE, int EPI, bool BIAS, bool FIN>
__device__ __forceinline__ void ksplit_step(
    const uint16_t* __restrict__ W1, const uint16_t* __restrict__ W2,
    const float* __restrict__ base, const float* __restrict__ unif,
    const StepIO& io, int R, int V, int r, float inv_t, int n_rblocks, int n_vgroups, int cpg,
    int cstep, int n_chunks, const Addr& ad, float* __restrict__ bias_out, const FinParams& fp,
    unsigned char* smem) {
  constexpr bool ROWF = EPI == kEpiRow;
  constexpr int RK = 512;
  constexpr int NW = 2 * NP;
  constexpr int ROWS = NP * 32;
  constexpr int KH = RK / 32;                          // MFMA K steps per half
  constexpr int PITCH = RK + 8;
  constexpr int BUF = kChunk * PITCH;
  constexpr int WD = kSplitWD;
  constexpr int PD = kSplitPD;
  constexpr int NS = PD + 1;
  constexpr int UNR = kSplitUnroll;
  constexpr int NBUF = kSplitBufs;
  constexpr int EL = epi_load_count<MODE, EPI, 2>();
  // vmcnt at the top of an iteration that leaves only the loads issued after
  // the DMA of its own chunk outstanding (0 with bias stores in flight).  With
  // WD = 1 those are the previous iteration's epilogue loads, which also
  // retires the epilogue inputs this iteration uses.
  constexpr int DMA_WAIT = BIAS ? 0 : EL + (WD - 1) * (kChunk / NW + EL);
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
  if (vg >= n_vgroups) {
    if constexpr (FIN) {
      static_assert(!BIAS, "the fused step has no bias output");
      static_assert(sched_lds_bytes<kFinStepItems, NW>() <= ksplit_lds_bytes<NP>(),
                    "the finishing schedule fits in the step workgroup's LDS");
      if (rb == 0 && vg == n_vgroups) finish_in_step<NW>(io, fp, W1, R, V, r, smem);
    }
    return;
  }
  const int c0 = cstep == 1 ? vg * cpg : vg;
  const int n_valid = cstep == 1 ? min(cpg, n_chunks - c0) : (n_chunks - 1 - vg) / cstep + 1;
  auto chunk = [&](int i) { return c0 + min(i, n_valid - 1) * cstep; };
  uint16_t* lds = reinterpret_cast<uint16_t*>(smem);
  float* xbuf = reinterpret_cast<float*>(smem + (size_t)NBUF * BUF * 2);   // [2][NW][64][8]

  const int pbase = rb * ROWS + pair * 32;          // the pair's first request
  const bool m_ok = pbase + col < R;                // lane col's gathered request
  // W1 rows, staged through LDS before anything else uses it: each wave copies
  // its 32 rows' K half (32 x 512 B) with direct loads that each move two
  // contiguous row halves (a row-major gather straight into registers touches
  // 32 lines per instruction).  Piece c of row q is stored in slot c ^ q, so
  // the reads below, one row per lane, spread over the banks.  The W2
  // prologue waits behind this (the staging area covers the stage buffers).
  // Requests on the lanes: lane col takes row col.  Entries on the lanes: wave
  // kh's lane col takes row col ^ 16 kh, so that the rows it finishes (tile
  // rows 0-15 of its product) are requests 16 kh .. 16 kh + 15.
  bf16x8 e[KH];
  const int x = step_input(io, pbase + col, m_ok, vg == 0 && kh == 0 && half == 0, V);
  {
    const u32x4 dw1 = io.dense ? raw_desc(io.dense, (uint32_t)R * (uint32_t)r * 2u)
                               : raw_desc(W1, (uint32_t)V * (uint32_t)r * 2u);
    uint16_t* greg = lds + wave * kGatherWave;
    const int c = lane & 31;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int qq = 2 * i + (lane >> 5);
      const int xq = __shfl(x, qq);
      const int mq = pbase + qq;
      const bool okq = mq < R && (io.dense != nullptr || xq >= 0);
      const int src = io.dense ? mq : xq;
      const int piece = c ^ qq;
      const uint32_t voff = (okq && kh * 256 + piece * 8 < r)
                                ? (uint32_t)src * (uint32_t)r * 2u + (uint32_t)(kh * 512 + piece * 16)
                                : kOutOfRange;
      asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                   :
                   : "v"(voff), "s"(dw1), "{m0}"(lds_addr(greg + 2 * i * 256))
                   : "memory");
    }
    wait_vmcnt<0>();
    __builtin_amdgcn_sched_barrier(0);
    const int nshare = min(n_vgroups, conf_embed_passes<256>());
    if (io.se && vg < nshare)
      conf_embed_part<256>(greg, io.w_e, kh * 256, r, pbase, R, x, io.se, io.gamma, io.k, kh, lane,
                           vg, nshare);
    __builtin_amdgcn_sched_barrier(0);
    const int er = ROWF ? (col ^ (16 * kh)) : col;
#pragma unroll
    for (int s = 0; s < KH; ++s)
      e[s] = *reinterpret_cast<const bf16x8*>(greg + er * 256 + (((2 * s + half) ^ er) & 31) * 8);
    lds_barrier();   // every wave has its rows before the stage buffers are reused
  }

  const u32x4 dw2 = raw_desc(W2, (uint32_t)V * (uint32_t)r * 2u);
  const uint32_t w2_off = w2_dma_lane_offset(lane, r);
  const Rsrc rbase = (MODE == kBiasOnly || EPI == kEpiNone) ? make_rsrc(W2, 0u)
                                                             : block_rsrc(base, ad, rb, ROWS);
  const Rsrc runif = MODE == DSPARK_SAMPLE ? block_rsrc(unif, ad, rb, ROWS) : rbase;
  // The lane's own epilogue elements: requests on the lanes, request col and
  // entries 16 kh + 8 j + 4 half + i; entries on the lanes, entry col and
  // requests 16 kh + 8 j + 4 half + i of the pair.
  const uint32_t e_off =
      ROWF ? (uint32_t)((pair * 32 + 16 * kh + 4 * half) * ad.row_stride + col) * 4u
           : ((EPI == kEpiCol && !m_ok)
                  ? kOutOfRange
                  : (uint32_t)((pair * 32 + col) * ad.row_stride + (16 * kh + 4 * half) * ad.vstride) * 4u);
  const uint32_t e_cb = (uint32_t)ad.cstride * 4u;
  const uint32_t e_vs = ROWF ? (uint32_t)ad.row_stride * 4u
                             : (uint32_t)(EPI == kEpiCol ? ad.vstride : 1) * 4u;

  float eb[NS][8];
  float eu[NS][8];
  float own[8];
  Argmax am;
  RowArgmax<ROWF ? 8 : 1> ram;

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
    if constexpr (ROWF) {
      select_rows<MODE, 8, MASKED>(ram, cb, z, cu, kscale, i, cv + col < vlim);
      if (BIAS) {
#pragma unroll
        for (int qq = 0; qq < 8; ++qq) {
          const int mq = pbase + 16 * kh + 8 * (qq >> 2) + 4 * half + (qq & 3);
          if (mq < R && cv + col < vlim)
            bias_out[ad.k_off + (size_t)mq * ad.row_stride + (size_t)chunk(i) * ad.cstride + col] =
                z[qq];
        }
      }
    } else {
      select_chunk<MODE, 8, MASKED>(am, cb, z, cu, kscale, i, vlim - cv - 16 * kh - 4 * half);
      if (BIAS && m_ok) {
        float* oc = bias_out + ad.k_off + (size_t)(pbase + col) * ad.row_stride +
                    (size_t)chunk(i) * ad.cstride;
#pragma unroll
        for (int qq = 0; qq < 8; ++qq) {
          const int o = 16 * kh + 8 * (qq >> 2) + 4 * half + (qq & 3);
          if (cv + o < vlim) oc[o * ad.vstride] = z[qq];
        }
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

    // Requests on the lanes: wave kh reads the chunk's rows as col ^ 16*kh, so
    // its own 16 entries always land in acc[0..7] and the partner's in
    // acc[8..15] (constant indices).  Entries on the lanes: the gathered rows
    // carry that permutation instead.
    const uint16_t* abase =
        lds + (t % NBUF) * BUF + (ROWF ? col : (col ^ (16 * kh))) * PITCH + half * 8 + kh * KH * 16;
    f32x16 acc = {};
#pragma unroll
    for (int s0 = 0; s0 < KH; s0 += 4) {
      bf16x8 a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const bf16x8*>(abase + (s0 + i) * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc = ROWF ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(e[s0 + i], a[i], acc, 0, 0, 0)
                   : __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], e[s0 + i], acc, 0, 0, 0);
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
  // As in the plain kernel, a short last group stops after its own chunks.
  const int n_iter = (n_valid + UNR - 1) / UNR * UNR;
  for (; i0 < n_iter; i0 += UNR) {
#pragma unroll
    for (int j = 0; j < UNR; ++j)
      body(std::true_type{}, std::false_type{}, i0 + j, eb[(j + NS - 1) % NS],
           eu[(j + NS - 1) % NS], eb[(j + PD) % NS], eu[(j + PD) % NS]);
  }
  // No direct load may land in LDS after this point (the merge below reuses
  // stage memory, and the workgroup's LDS is released at exit).
  wait_vmcnt<0>();
  lds_barrier();   // the partner's last half-tile
  // n_iter is a multiple of UNR (hence of NS): the last iteration's slot is NS - 1.
  epilogue(std::true_type{}, n_iter - 1, (n_iter - 1) & 1, eb[NS - 1], eu[NS - 1]);

  if constexpr (ROWF) {
    // Each wave holds its 16 requests over all the chunk entries: merge each
    // row across the half-wave's 32 entries and publish.
    float bv[8];
    int bi[8];
#pragma unroll
    for (int qq = 0; qq < 8; ++qq) {
      bv[qq] = ram.best[qq];
      bi[qq] = ram.iter[qq] < 0 ? 0x7fffffff : (c0 + ram.iter[qq] * cstep) * kChunk + col;
    }
    merge_rows<8>(bv, bi, lane);
    const int qf = merged_row<8>(lane);
    const int ml = 16 * kh + 8 * (qf >> 2) + 4 * half + (qf & 3);   // request pbase + ml
    const int xm = __shfl(x, ml);
    const int mq = pbase + ml;
    if (merged_publisher<8>(lane) && mq < R)
      atomicMax(io.best + (size_t)mq * io.sub + (vg & (io.sub - 1)),
                xm >= 0 ? pack_best(bv[0], bi[0]) : kPoison);
  } else {
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
      atomicMax(io.best + (size_t)(pbase + col) * io.sub + (vg & (io.sub - 1)),
                x >= 0 ? pack_best(best, best_i) : kPoison);
    }
  }
  if constexpr (FIN) {
    // The workgroup that publishes last unpacks x_{gamma-1} of every request.
    // The results are agent-scope atomics, complete once each wave's memory
    // counter drains; then one count per workgroup, and the last reads the
    // words with agent-scope loads (all S of a request in flight together:
    // past S the last word again, which leaves the maximum unchanged).  No
    // cache-wide write-back or invalidate, which would cost the workgroups
    // still streaming their L2 contents.
    wait_vmcnt<0>();
    __syncthreads();
    int* last = reinterpret_cast<int*>(smem);
    if (tid == 0)
      last[0] = __hip_atomic_fetch_add(fp.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                (unsigned int)(n_rblocks * n_vgroups - 1);
    __syncthreads();
    if (last[0]) {
      for (int m = tid; m < R; m += NW * 64) {
        const unsigned long long* wm = io.best + (size_t)m * io.sub;
        unsigned long long w[kMaxSubWords];
#pragma unroll
        for (int j = 0; j < kMaxSubWords; ++j)
          w[j] = __hip_atomic_load(wm + min(j, io.sub - 1), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        unsigned long long b = 0;
#pragma unroll
        for (int j = 0; j < kMaxSubWords; ++j) b = w[j] > b ? w[j] : b;
        io.tokens[(size_t)m * io.gamma + io.k] = unpack_token(b, V);
      }
    }
  }
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
  ksplit_step<NP, MODE, EPI, BIAS, false>(W1, W2, base, unif, io, R, V, r, inv_t, n_rblocks,
                                          n_vgroups, cpg, cstep, n_chunks, ad, bias_out,
                                          FinParams{}, smem);
}

// The fused draft step's last step: the same, plus the finishing work.
template <int NP, int MODE, int EPI>
__global__ __launch_bounds__(NP * 128)
__attribute__((amdgpu_waves_per_eu(1, 2))) void markov_step_ksplit_fin_kernel(
    const uint16_t* __restrict__ W1, const uint16_t* __restrict__ W2,
    const float* __restrict__ base, const float* __restrict__ unif,
    StepIO io, int R, int V, int r, float inv_t, int n_rblocks, int n_vgroups, int cpg,
    int cstep, int n_chunks, Addr ad, float* __restrict__ bias_out, FinParams fp) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  ksplit_step<NP, MODE, EPI, false, true>(W1, W2, base, unif, io, R, V, r, inv_t, n_rblocks,
                                          n_vgroups, cpg, cstep, n_chunks, ad, bias_out, fp,
                                          smem);
}

// ---- variant tables ----

template <int RK, int NW, int MODE, int EPI, bool BIAS, int TW = 1>
StepVariant plain_variant() {
  return {&markov_step_kernel<RK, NW, MODE, EPI, BIAS, TW>, NW * 64, plain_lds_bytes<RK, NW, TW>(),
          NW * 32 * TW, plain_unroll<RK, NW>()};
}
template <int NP, int MODE, int EPI, bool BIAS>
StepVariant ksplit_variant() {
  StepFinKernel fin = nullptr;
  if constexpr (!BIAS) fin = &markov_step_ksplit_fin_kernel<NP, MODE, EPI>;
  return {&markov_step_ksplit_kernel<NP, MODE, EPI, BIAS>, NP * 128, ksplit_lds_bytes<NP>(),
          NP * 32, kSplitUnroll, fin};
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
  // Sampling at ranks 256-512 keeps two epilogue streams and its rows in
  // registers: eight waves (two per SIMD) would spill, so it runs four.
  constexpr bool NO8 = MODE == DSPARK_SAMPLE && RK >= 256;
  switch (nw) {
    case 1: return plain_variant<RK, 1, MODE, EPI, BIAS>();
    case 2: return plain_variant<RK, 2, MODE, EPI, BIAS>();
    case 4: return plain_variant<RK, 4, MODE, EPI, BIAS>();
    default: return plain_variant<RK, NO8 ? 4 : 8, MODE, EPI, BIAS>();
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

}  // namespace
}  // namespace dspark
