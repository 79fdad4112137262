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
//                      of Rgamma x d by d x 2r on MFMA, LDS-tiled, K split in
//                      up to four partial sums), and the clears;
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
// Every sum is taken in a fixed order (K quarters, K splits), so results are
// deterministic.
#include <math.h>

#include <algorithm>
#include <atomic>

#include "markov_types.h"
#include "packed_words.h"
#include "raw_buffer.h"

namespace dspark {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// fp32 -> bf16 bits, to nearest even.
__device__ __forceinline__ uint16_t to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---- the token-independent pre-activations (one GEMM over every position) ----
// P_s[t, n] = [s == 0] b[n] + sum_{k in split s} h[t, k] U[n, 2r + k], for
// t < M = R gamma, n < 2r.  Tiles of 128 positions x 128 units per workgroup of
// four wavefronts (2 x 2, each 64 x 64 as 2 x 2 MFMA tiles), K in stages of 64.
// Stages go straight from memory into a ring of four LDS buffers (direct loads,
// no registers held), three stages in flight while one is multiplied: the GEMM
// is bound by the latency of its operand reads, so what counts is how many
// bytes each CU keeps in flight.  K is split over `splits` workgroups (about
// one workgroup per CU in all); the state update adds the partial sums in split
// order.  Work items are (split, position tile, unit tile) in that order, dealt
// to the eight XCDs in contiguous ranges, so the workgroups sharing a tile of h
// (and the unit tiles of one split) run under one L2.
constexpr int kPBM = 128, kPBN = 128, kPBK = 64;
constexpr int kPRows = kPBM + kPBN;
constexpr int kPStage = kPRows * kPBK;            // bf16 per LDS stage (32 KB)
constexpr int kPNB = 4;                           // LDS stages in the ring
constexpr int kPD = kPNB - 1;                     // stages in flight
constexpr int kPDma = kPRows / 8 / 4;             // direct loads per wave per stage
constexpr int kXcds = 8;
constexpr int kMaxSplits = 4;
static_assert(kPDma == 8, "each wave moves 64 rows per stage, 8 per load");

__device__ __forceinline__ u32x4 raw_desc(const void* p, size_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t n = (uint32_t)(bytes < kMaxRsrcBytes ? bytes : kMaxRsrcBytes);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, n, (uint32_t)kRsrcWord3};
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// Workgroup barrier ordering LDS only (__syncthreads also fences global memory,
// which would make every barrier wait for all loads in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}

// Direct loads of one stage: wave w fills LDS rows 64 w .. 64 w + 63 (rows
// 0..127 the h tile, 128..255 the U tile), eight rows of 128 bytes per load,
// lane l taking 16 bytes of row 8 i + l / 8.  LDS slot q of a row holds piece
// q ^ (row & 7) of the row's 64 columns, so the fragment reads below (32 rows
// at one piece) spread over the banks.  off[i] is the lane's byte offset in
// its resource (kOff past the matrix); columns past d read as zero.
__device__ __forceinline__ void pre_dma(uint16_t* stage, u32x4 desc, const uint32_t (&off)[kPDma],
                                        int kcol, int d, bool live, int wave) {
  const bool ok = live && kcol < d;
  const uint32_t kb = 2u * (uint32_t)(kcol & ~63);
#pragma unroll
  for (int i = 0; i < kPDma; ++i) {
    const uint32_t voff = ok ? off[i] + kb : kOff;
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(desc), "{m0}"(lds_addr(stage + (wave * 64 + 8 * i) * kPBK))
                 : "memory");
  }
}

// One stage: wavefront (wm, wn) multiplies its 64 x 64 block over the stage's 64 K.
__device__ __forceinline__ void pre_mma(const uint16_t* __restrict__ buf, int wm, int wn, int col,
                                        int half, f32x16 (&acc)[2][2]) {
  const uint16_t* A = buf + (wm * 64 + col) * kPBK;
  const uint16_t* B = buf + (kPBM + wn * 64 + col) * kPBK;
  const int sw = col & 7;   // rows 32 i + col: row & 7 == col & 7
#pragma unroll
  for (int ks = 0; ks < kPBK / 16; ++ks) {
    const int slot = ((2 * ks + half) ^ sw) * 8;
    u32x4 a[2], bb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      a[i] = *reinterpret_cast<const u32x4*>(A + i * 32 * kPBK + slot);
      bb[i] = *reinterpret_cast<const u32x4*>(B + i * 32 * kPBK + slot);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[i]), as_bf16x8(bb[j]),
                                                             acc[i][j], 0, 0, 0);
  }
}

__global__ __launch_bounds__(256) void rnn_pre_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ U, const float* __restrict__ b,
    int M, int r, int d, int splits, int items, float* __restrict__ P, uint4* __restrict__ clear,
    size_t nclear) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* lds = reinterpret_cast<uint16_t*>(smem);
  const int tid = threadIdx.x;
  for (size_t i = (size_t)blockIdx.x * 256 + tid; i < nclear; i += (size_t)gridDim.x * 256)
    clear[i] = make_uint4(0u, 0u, 0u, 0u);
  const int per = (items + kXcds - 1) / kXcds;
  const int item = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (item >= items) return;
  const int N = 2 * r, ldu = 2 * r + d;
  const int ntm = (M + kPBM - 1) / kPBM, ntn = (N + kPBN - 1) / kPBN;
  const int sp = item / (ntm * ntn);
  const int t0 = (item / ntn) % ntm * kPBM, n0 = item % ntn * kPBN;
  const int nst = (d + kPBK - 1) / kPBK;
  const int st0 = nst * sp / splits, st1 = nst * (sp + 1) / splits;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;
  // This wave's direct-load rows and their offsets (waves 0, 1: h; 2, 3: U).
  const int tn = min(kPBM, M - t0), nn = min(kPBN, N - n0);
  const uint16_t* Uh = U + 2 * r;   // the h block: U[n, 2r + k]
  const u32x4 desc = wave < 2 ? raw_desc(h + (size_t)t0 * d, (size_t)tn * d * 2)
                              : raw_desc(Uh + (size_t)n0 * ldu, ((size_t)(nn - 1) * ldu + d) * 2);
  const int piece = (lane & 7) ^ ((lane >> 3) & 7);   // LDS slot lane & 7 of row 8 i + lane / 8
  const int kp = 8 * piece;                           // the piece's first column in a stage
  uint32_t off[kPDma];
#pragma unroll
  for (int i = 0; i < kPDma; ++i) {
    const int lr = (wave & 1) * 64 + 8 * i + (lane >> 3);   // row within the operand tile
    off[i] = wave < 2 ? (lr < tn ? (uint32_t)lr * (uint32_t)d * 2u + 2u * kp : kOff)
                      : (lr < nn ? (uint32_t)lr * (uint32_t)ldu * 2u + 2u * kp : kOff);
  }
  f32x16 acc[2][2] = {{f32x16{}, f32x16{}}, {f32x16{}, f32x16{}}};
  if (st0 < st1) {
    // Every iteration issues exactly kPDma loads per wave (stages past the
    // split read zeros), so stage st has landed once at most (kPD - 1) kPDma
    // loads of this wave are outstanding.
#pragma unroll
    for (int j = 0; j < kPD; ++j)
      pre_dma(lds + j * kPStage, desc, off, (st0 + j) * kPBK + kp, d, st0 + j < st1, wave);
    for (int st = st0; st < st1; ++st) {
      const int i = st - st0;
      wait_vmcnt<(kPD - 1) * kPDma>();
      lds_barrier();   // the stage is complete, and every wave is done with the buffer refilled next
      pre_dma(lds + ((i + kPD) % kPNB) * kPStage, desc, off, (st + kPD) * kPBK + kp, d,
              st + kPD < st1, wave);
      __builtin_amdgcn_sched_barrier(0);
      pre_mma(lds + (i % kPNB) * kPStage, wm, wn, col, half, acc);
    }
    wait_vmcnt<0>();   // no direct load may land after this point
  }
  // The bias is loaded before any store and without a branch: a load on a
  // conditional path would make every later store wait for all stores before it.
  float* Ps = P + (size_t)sp * M * N;
  float bn[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float bv = b[min(n0 + wn * 64 + 32 * j + col, N - 1)];
    bn[j] = sp == 0 ? bv : 0.0f;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + 32 * j + col;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int t = t0 + wm * 64 + 32 * i + 8 * (q >> 2) + 4 * half + (q & 3);
        if (t < M && n < N) Ps[(size_t)t * N + n] = acc[i][j][q] + bn[j];
      }
  }
}

// ---- one gated update ----
// Step k for requests m0 .. m0+15 and units n0 .. n0+15: gate and candidate
// pre-activations over the s and e blocks (K = 2r, an eighth per wavefront, on
// 16 x 16 x 32 MFMA tiles), plus the P partials; then
// s_new = g (e + tanh(pre_c)) + (1 - g) s_old.  At step 0 the old state is
// s_0 = 0 (s_old and sb_old NULL).  The update is latency-bound (one small GEMM
// per step), so every load is issued as early as it can be, all before the
// first MFMA: the U operands before the previous tokens are read, then those of
// the element-wise part (P partials, embedding entries, old state) and the
// state / embedding operands.  Small tiles give R/16 x r/16
// workgroups (512 at R = 256, r = 512), so the loads spread over the whole chip.
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kSW = 8;      // wavefronts per update workgroup
constexpr int kSB = 4;      // 32-wide K steps per wavefront: its whole eighth of K = 2r
static_assert(kSW * kSB * 32 >= 2 * DSPARK_MAX_RANK, "one batch of loads covers K");
constexpr int kSPad = 17;   // LDS pitch of the partial tiles (floats)

__global__ __launch_bounds__(64 * kSW) void rnn_state_kernel(
    const uint16_t* __restrict__ W1, const uint16_t* __restrict__ U, const float* __restrict__ P,
    int splits, const int32_t* __restrict__ anchors, const unsigned long long* __restrict__ prev,
    int sub, int R, int gamma, int V, int r, int d, int k, const float* __restrict__ s_old,
    const uint16_t* __restrict__ sb_old, float* __restrict__ s_new, uint16_t* __restrict__ sb_new) {
  __shared__ float red[kSW * 2 * 16 * kSPad];
  __shared__ int xs[16];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, c16 = lane & 15, quad = lane >> 4;
  // Tiles (request tile mt, unit tile nt), unit-tile major, dealt to the eight
  // XCDs in contiguous ranges: the request tiles sharing a U tile run under one
  // L2, which then fetches that tile once.
  const int nmt = (R + 15) / 16, items = nmt * (r / 16);
  const int per = (items + kXcds - 1) / kXcds;
  const int item = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (item >= items) return;
  const int m0 = item % nmt * 16, n0 = item / nmt * 16;
  const int nm = min(16, R - m0);
  const int ldu = 2 * r + d;
  const int steps = (2 * r + 31) / 32;
  const int lo = 32 * (steps * wave / kSW), hi = 32 * (steps * (wave + 1) / kSW);
  // Every load below is a buffer load whose out-of-range offset reads as zero,
  // so no loaded value passes through a select (which would make the compiler
  // wait for it where the select is placed).  Everything that does not depend
  // on the previous tokens is issued before they are read: the U operands (gate
  // rows n0 + c16, candidate rows r + n0 + c16, over the s and e blocks), the
  // s-block operands from the old bf16 state, the P partials and the old state.
  const Rsrc rug = rsrc_of(U + (size_t)n0 * ldu, ((size_t)15 * ldu + 2 * r) * 2);
  const Rsrc ruc = rsrc_of(U + (size_t)(r + n0) * ldu, ((size_t)15 * ldu + 2 * r) * 2);
  const Rsrc rsb = rsrc_of(sb_old ? sb_old + (size_t)m0 * r : W1, sb_old ? (size_t)nm * r * 2 : 0);
  u32x4 bg[kSB], bc[kSB], a_s[kSB];
#pragma unroll
  for (int u = 0; u < kSB; ++u) {
    const int kk = lo + 32 * u, ke = kk + 8 * quad;
    const bool in = kk < hi;
    const uint32_t o = in ? ((uint32_t)c16 * (uint32_t)ldu + (uint32_t)ke) * 2u : kOff;
    bg[u] = ld16(rug, o);
    bc[u] = ld16(ruc, o);
    a_s[u] = ld16(rsb, (in && c16 < nm && ke < r) ? ((uint32_t)c16 * (uint32_t)r + (uint32_t)ke) * 2u
                                                  : kOff);
  }
  // Element-wise operands of this thread's output (threads 0..255: request
  // m0 + tid / 16, unit n0 + tid % 16).
  const int en = tid & 15, el = (tid >> 4) & 15;
  const int n = n0 + en, me = m0 + el;
  const bool eok = tid < 256 && el < nm;
  const size_t pstride = (size_t)R * gamma * 2 * r;
  float pg[kMaxSplits], pc[kMaxSplits];
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp) {
    const bool use = sp < splits;
    const Rsrc rp = rsrc_of(P + (use ? sp * pstride : 0) + ((size_t)m0 * gamma + k) * 2 * r,
                            ((size_t)(nm - 1) * gamma * 2 * r + 2 * r) * 4);
    const uint32_t o = (eok && use) ? ((uint32_t)el * (uint32_t)(gamma * 2 * r) + (uint32_t)n) * 4u
                                    : kOff;
    pg[sp] = ld4f(rp, o);
    pc[sp] = ld4f(rp, o + (o == kOff ? 0u : 4u * (uint32_t)r));
  }
  const Rsrc rso = rsrc_of(s_old ? s_old + (size_t)m0 * r : P, s_old ? (size_t)nm * r * 4 : 0);
  const float so = ld4f(rso, eok ? ((uint32_t)el * (uint32_t)r + (uint32_t)n) * 4u : kOff);
  // Token x_{k-1} of each of the 16 requests; -1 if invalid.
  if (tid < 16) {
    const int m = m0 + tid;
    int x = -1;
    if (m < R) {
      if (!prev) {
        const int a = anchors[m];
        x = (a >= 0 && a < V) ? a : -1;
      } else {
        x = read_token(prev, m, sub, V);
      }
    }
    xs[tid] = x;
  }
  __syncthreads();
  // The token-dependent loads: the e-block operands from the embedding row of
  // x_{k-1} (complementary to the s-block lanes: one of the two reads zero),
  // and this thread's embedding entry.
  const Rsrc rw1 = rsrc_of(W1, (size_t)V * r * 2);
  const int xa = xs[c16];
  u32x4 a[kSB];
#pragma unroll
  for (int u = 0; u < kSB; ++u) {
    const int kk = lo + 32 * u, ke = kk + 8 * quad;
    const uint32_t oe = (kk < hi && c16 < nm && ke >= r && xa >= 0)
                            ? ((uint32_t)xa * (uint32_t)r + (uint32_t)(ke - r)) * 2u : kOff;
    a[u] = ld16(rw1, oe);
  }
  const int xe = xs[el];
  const uint32_t w1e = ld2(rw1, (eok && xe >= 0) ? ((uint32_t)xe * (uint32_t)r + (uint32_t)n) * 2u
                                                 : kOff);
  __builtin_amdgcn_sched_barrier(0);   // every load issued before the first MFMA
#pragma unroll
  for (int u = 0; u < kSB; ++u) a[u] |= a_s[u];
  const float e = __uint_as_float(w1e << 16);
  f32x4 acc[2] = {f32x4{}, f32x4{}};   // gate, candidate
#pragma unroll
  for (int u = 0; u < kSB; ++u) {
    acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[u]), as_bf16x8(bg[u]), acc[0], 0,
                                                      0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[u]), as_bf16x8(bc[u]), acc[1], 0,
                                                      0, 0);
  }
  // Partial tiles to LDS as [wave][gate / candidate][request][unit]; lane l
  // holds unit l % 16 of requests 4 (l / 16) .. +3.
#pragma unroll
  for (int gc = 0; gc < 2; ++gc)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      red[((wave * 2 + gc) * 16 + 4 * quad + i) * kSPad + c16] = acc[gc][i];
  __syncthreads();
  if (!eok) return;
  float ag = red[(0 * 16 + el) * kSPad + en], ac = red[(1 * 16 + el) * kSPad + en];
#pragma unroll
  for (int w = 1; w < kSW; ++w) {
    ag += red[((w * 2 + 0) * 16 + el) * kSPad + en];
    ac += red[((w * 2 + 1) * 16 + el) * kSPad + en];
  }
  float g_pre = pg[0], c_pre = pc[0];
#pragma unroll
  for (int sp = 1; sp < kMaxSplits; ++sp) {
    g_pre += pg[sp];
    c_pre += pc[sp];
  }
  const float g = 1.0f / (1.0f + expf(-(ag + g_pre)));
  const float c = e + tanhf(ac + c_pre);
  const float sn = g * c + (1.0f - g) * so;
  s_new[(size_t)me * r + n] = sn;
  sb_new[(size_t)me * r + n] = to_bf16(sn);
}

}  // namespace

int rnn_pre_splits(int R, int gamma, int r, int d) {
  const long tiles = (long)((R * gamma + kPBM - 1) / kPBM) * ((2 * r + kPBN - 1) / kPBN);
  const long nst = (d + kPBK - 1) / kPBK;
  long sp = (256 + tiles / 2) / tiles;   // about one workgroup per CU
  sp = std::min<long>(sp, kMaxSplits);
  sp = std::min<long>(sp, std::max<long>(1, nst / 4));   // four K stages per split at least
  return (int)std::max<long>(1, sp);
}

size_t rnn_workspace_bytes(int R, int gamma, int V, int r, int d) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t words = plan_markov(R, gamma, V, r, DSPARK_GREEDY, false).ws_bytes;
  const size_t P = (size_t)rnn_pre_splits(R, gamma, r, d) * R * gamma * 2 * r * sizeof(float);
  const size_t s32 = (size_t)2 * R * r * sizeof(float);
  const size_t s16 = (size_t)2 * R * r * sizeof(uint16_t);
  return up(words) + up(P) + up(s32) + up(s16);
}

RnnBuffers rnn_buffers(void* workspace, int R, int gamma, int V, int r, int d) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  unsigned char* ws = reinterpret_cast<unsigned char*>(workspace);
  const size_t words = plan_markov(R, gamma, V, r, DSPARK_GREEDY, false).ws_bytes;
  RnnBuffers B;
  B.splits = rnn_pre_splits(R, gamma, r, d);
  const size_t pb = (size_t)B.splits * R * gamma * 2 * r * sizeof(float);
  const size_t s32 = (size_t)2 * R * r * sizeof(float);
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
  const int items = B.splits * ((M + kPBM - 1) / kPBM) * ((2 * r + kPBN - 1) / kPBN);
  const int per = (items + kXcds - 1) / kXcds;
  const size_t lds = (size_t)kPNB * kPStage * sizeof(uint16_t);
  // The dynamic-LDS attribute, set once per device (bit d of `done`).
  static std::atomic<unsigned long long> done{0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(DSPARK_EDEVICE, "hipGetDevice failed");
  const unsigned long long bit = dev < 64 ? 1ull << dev : 0ull;
  if (!bit || !(done.load(std::memory_order_acquire) & bit)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&rnn_pre_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return fail(DSPARK_EDEVICE, "hipFuncSetAttribute failed for the pre-activation kernel");
    done.fetch_or(bit, std::memory_order_release);
  }
  hipLaunchKernelGGL(rnn_pre_kernel, dim3(per * kXcds), dim3(256), lds, stream, h, U, b, M, r, d,
                     B.splits, items, B.P, reinterpret_cast<uint4*>(B.words), (n_words + 1) / 2);
  return check_launch("rnn_pre_kernel");
}

dspark_status launch_rnn_state(const uint16_t* W1, const uint16_t* U, const int32_t* anchors,
                               const unsigned long long* prev, int sub, int R, int gamma, int V,
                               int r, int d, int k, const RnnBuffers& B, float* s_out,
                               hipStream_t stream) {
  const int items = (R + 15) / 16 * (r / 16);
  const dim3 grid((items + kXcds - 1) / kXcds * kXcds);
  const int o = k & 1, nw = (k + 1) & 1;   // state before step k in half o, after it in nw
  hipLaunchKernelGGL(rnn_state_kernel, grid, dim3(64 * kSW), 0, stream, W1, U, B.P, B.splits,
                     anchors, prev, sub, R, gamma, V, r, d, k, k == 0 ? nullptr : B.s[o],
                     k == 0 ? nullptr : B.sb[o], s_out ? s_out : B.s[nw], B.sb[nw]);
  return check_launch("rnn_state_kernel");
}

}  // namespace dspark
