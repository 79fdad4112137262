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

#include "markov_types.h"
#include "packed_words.h"

namespace dspark {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// fp32 -> bf16 bits, to nearest even.
__device__ __forceinline__ uint16_t to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---- branch-free loads ----
// A guarded load (if in range, load, else zero) puts every load in a basic
// block of its own, and the compiler then waits for all outstanding loads at
// the joins.  Here tails read as zero without branches: buffer loads whose
// per-lane offset lies past the resource's size return zeros, and a clamped
// in-range address whose value is then replaced by zero (a select).
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;        // untyped dword access (gfx9 family)
constexpr uint32_t kOff = 0x80000000u;        // an offset past every resource below
constexpr size_t kMaxRsrcBytes = 0x7ffffff0u;

__device__ __forceinline__ Rsrc rsrc_of(const void* p, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0,
                                           (int)(bytes < kMaxRsrcBytes ? bytes : kMaxRsrcBytes),
                                           kRsrcWord3);
}
// Keeps a per-lane offset in a VGPR, so that no uniform part of it moves into
// the scalar offset (which the range check does not cover).
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm("" : "+v"(x));
  return x;
}
__device__ __forceinline__ u32x4 ld16(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, opaque(off), 0, 0));
}
__device__ __forceinline__ u32x4 zero_unless(bool ok, u32x4 v) {
  return ok ? v : u32x4{0u, 0u, 0u, 0u};
}

// ---- the token-independent pre-activations (one GEMM over every position) ----
// P_s[t, n] = [s == 0] b[n] + sum_{k in split s} h[t, k] U[n, 2r + k], for
// t < M = R gamma, n < 2r.  Tiles of 128 positions x 128 units per workgroup of
// four wavefronts (2 x 2, each 64 x 64 as 2 x 2 MFMA tiles), K in stages of 64
// through double-buffered LDS (global -> registers -> LDS, the loads of the
// next two stages in flight while the current one is multiplied).  K is split over
// `splits` workgroups; the state update adds the partial sums in split order.
// Work items are (split, position tile, unit tile) in that order, dealt to the
// eight XCDs in contiguous ranges, so the workgroups sharing a tile of h (and
// the unit tiles of one split) run under one L2.
constexpr int kPBM = 128, kPBN = 128, kPBK = 64;
constexpr int kPLd = kPBK + 8;           // LDS row pitch in bf16: 144 bytes, rows 4 banks apart
constexpr int kPRows = kPBM + kPBN;
constexpr int kPLoads = kPRows * kPBK / 8 / 256;   // 16-byte loads per thread per stage
constexpr int kXcds = 8;
constexpr int kMaxSplits = 4;
static_assert(kPLoads == 8, "four h rows and four U rows per thread and stage");

// Stage loads of one thread: rows lrow + 32 j of the h tile and of the U tile,
// 16 bytes at column k.  oh / ou are the rows' byte offsets in their resources
// (kOff for rows past the matrix); columns past d read as zero.
__device__ __forceinline__ void pre_load(Rsrc rh, Rsrc ru, const uint32_t (&oh)[4],
                                         const uint32_t (&ou)[4], int k, int d,
                                         u32x4 (&v)[kPLoads]) {
  const bool kok = k < d;
  const uint32_t kb = 2u * (uint32_t)k;
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = ld16(rh, kok ? oh[j] + kb : kOff);
#pragma unroll
  for (int j = 0; j < 4; ++j) v[4 + j] = ld16(ru, kok ? ou[j] + kb : kOff);
}

__device__ __forceinline__ void pre_store(uint16_t* __restrict__ buf, int row, int kc,
                                          const u32x4 (&v)[kPLoads]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    *reinterpret_cast<u32x4*>(buf + (row + 32 * j) * kPLd + kc) = v[j];
    *reinterpret_cast<u32x4*>(buf + (kPBM + row + 32 * j) * kPLd + kc) = v[4 + j];
  }
}

// One stage: wavefront (wm, wn) multiplies its 64 x 64 block over the stage's 64 K.
__device__ __forceinline__ void pre_mma(const uint16_t* __restrict__ buf, int wm, int wn, int col,
                                        int half, f32x16 (&acc)[2][2]) {
  const uint16_t* A = buf + (wm * 64 + col) * kPLd + 8 * half;
  const uint16_t* B = buf + (kPBM + wn * 64 + col) * kPLd + 8 * half;
#pragma unroll
  for (int ks = 0; ks < kPBK / 16; ++ks) {
    u32x4 a[2], bb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      a[i] = *reinterpret_cast<const u32x4*>(A + i * 32 * kPLd + 16 * ks);
      bb[i] = *reinterpret_cast<const u32x4*>(B + i * 32 * kPLd + 16 * ks);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[i]), as_bf16x8(bb[j]),
                                                             acc[i][j], 0, 0, 0);
  }
}

__global__ __launch_bounds__(256, 2) void rnn_pre_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ U, const float* __restrict__ b,
    int M, int r, int d, int splits, int items, float* __restrict__ P, uint4* __restrict__ clear,
    size_t nclear) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][kPRows * kPLd];
  const int tid = threadIdx.x;
  for (size_t i = (size_t)blockIdx.x * 256 + tid; i < nclear; i += (size_t)gridDim.x * 256)
    clear[i] = make_uint4(0u, 0u, 0u, 0u);
  const int per = (items + kXcds - 1) / kXcds;
  const int item = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (blockIdx.x / kXcds >= per || item >= items) return;
  const int N = 2 * r, ldu = 2 * r + d;
  const int ntm = (M + kPBM - 1) / kPBM, ntn = (N + kPBN - 1) / kPBN;
  const int sp = item / (ntm * ntn);
  const int t0 = (item / ntn) % ntm * kPBM, n0 = item % ntn * kPBN;
  const int nst = (d + kPBK - 1) / kPBK;
  const int st0 = nst * sp / splits, st1 = nst * (sp + 1) / splits;
  const uint16_t* Uh = U + 2 * r;   // the h block: U[n, 2r + k]
  // loads: thread tid takes rows tid / 8 + 32 j of each operand tile, 16 bytes at kc
  const int lrow = tid >> 3, kc = 8 * (tid & 7);
  const int tn = min(kPBM, M - t0), nn = min(kPBN, N - n0);
  const Rsrc rh = rsrc_of(h + (size_t)t0 * d, (size_t)tn * d * 2);
  const Rsrc ru = rsrc_of(Uh + (size_t)n0 * ldu, ((size_t)(nn - 1) * ldu + d) * 2);
  uint32_t oh[4], ou[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = lrow + 32 * j;
    oh[j] = row < tn ? (uint32_t)row * (uint32_t)d * 2u : kOff;
    ou[j] = row < nn ? (uint32_t)row * (uint32_t)ldu * 2u : kOff;
  }
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;
  f32x16 acc[2][2] = {{f32x16{}, f32x16{}}, {f32x16{}, f32x16{}}};
  // Two stages of loads in flight: while stage st is multiplied from one LDS
  // buffer, stage st + 1 waits in registers for the other buffer and stage
  // st + 2 is being fetched.  The loads are issued unconditionally (a stage
  // past the split's end reads zeros without touching memory): a load issued
  // on one path only would make the compiler wait for every load in flight.
  if (st0 < st1) {
    auto kat = [&](int st) { return st < st1 ? st * kPBK + kc : d; };
    u32x4 v0[kPLoads], v1[kPLoads];
    pre_load(rh, ru, oh, ou, kat(st0), d, v0);
    pre_load(rh, ru, oh, ou, kat(st0 + 1), d, v1);
    pre_store(lds[0], lrow, kc, v0);
    __syncthreads();
    for (int st = st0; st < st1; st += 2) {
      pre_load(rh, ru, oh, ou, kat(st + 2), d, v0);
      pre_mma(lds[0], wm, wn, col, half, acc);
      if (st + 1 >= st1) break;
      pre_store(lds[1], lrow, kc, v1);
      __syncthreads();
      pre_load(rh, ru, oh, ou, kat(st + 3), d, v1);
      pre_mma(lds[1], wm, wn, col, half, acc);
      if (st + 2 >= st1) break;
      pre_store(lds[0], lrow, kc, v0);
      __syncthreads();
    }
  }
  float* Ps = P + (size_t)sp * M * N;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + 32 * j + col;
    if (n >= N) continue;
    const float bn = sp == 0 ? b[n] : 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int t = t0 + wm * 64 + 32 * i + 8 * (q >> 2) + 4 * half + (q & 3);
        if (t < M) Ps[(size_t)t * N + n] = acc[i][j][q] + bn;
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

// U operands of one wavefront's K share: gate rows n0 + c16 and candidate rows
// r + n0 + c16 over the s and e blocks.  Steps past the share (a uniform test)
// load column 0 and are replaced by zeros.
__device__ __forceinline__ void state_load_u(const uint16_t* __restrict__ U, int ldu, int r,
                                             int n0, int c16, int quad, int lo, int hi,
                                             u32x4 (&bg)[kSB], u32x4 (&bc)[kSB]) {
  const uint16_t* ug = U + (size_t)(n0 + c16) * ldu + 8 * quad;
  const uint16_t* uc = ug + (size_t)r * ldu;
#pragma unroll
  for (int u = 0; u < kSB; ++u) {
    const int kk = lo + 32 * u;
    const bool in = kk < hi;
    const int kc = in ? kk : 0;
    bg[u] = zero_unless(in, *reinterpret_cast<const u32x4*>(ug + kc));
    bc[u] = zero_unless(in, *reinterpret_cast<const u32x4*>(uc + kc));
  }
}

__global__ __launch_bounds__(64 * kSW) void rnn_state_kernel(
    const uint16_t* __restrict__ W1, const uint16_t* __restrict__ U, const float* __restrict__ P,
    int splits, const int32_t* __restrict__ anchors, const unsigned long long* __restrict__ prev,
    int sub, int R, int gamma, int V, int r, int d, int k, const float* __restrict__ s_old,
    const uint16_t* __restrict__ sb_old, float* __restrict__ s_new, uint16_t* __restrict__ sb_new) {
  __shared__ float red[kSW * 2 * 16 * kSPad];
  __shared__ int xs[16];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, c16 = lane & 15, quad = lane >> 4;
  const int m0 = blockIdx.x * 16, n0 = blockIdx.y * 16;
  const int ldu = 2 * r + d;
  const int steps = (2 * r + 31) / 32;
  const int lo = 32 * (steps * wave / kSW), hi = 32 * (steps * (wave + 1) / kSW);
  u32x4 bg[kSB], bc[kSB];
  state_load_u(U, ldu, r, n0, c16, quad, lo, hi, bg, bc);
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
  // Element-wise operands of this thread's output (threads 0..255: request
  // m0 + tid / 16, unit n0 + tid % 16), loaded now and combined after the GEMM.
  const int en = tid & 15, el = (tid >> 4) & 15;
  const int n = n0 + en, me = m0 + el;
  const bool eok = tid < 256 && me < R && n < r;
  const size_t pstride = (size_t)R * gamma * 2 * r;
  float pg[kMaxSplits], pc[kMaxSplits];
  const size_t pt = eok ? ((size_t)me * gamma + k) * 2 * r + n : 0;
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp) {
    const bool use = eok && sp < splits;
    const size_t o = (sp < splits ? (size_t)sp * pstride : 0) + pt;
    const float vg = P[o], vc = P[o + r];
    pg[sp] = use ? vg : 0.0f;
    pc[sp] = use ? vc : 0.0f;
  }
  const int xe = xs[el];
  const bool e_ok = eok && xe >= 0;
  const uint16_t w1e = W1[e_ok ? (size_t)xe * r + n : 0];
  const float e = e_ok ? __uint_as_float((uint32_t)w1e << 16) : 0.0f;
  const bool so_ok = eok && s_old != nullptr;
  const float sov = (so_ok ? s_old : P)[so_ok ? (size_t)me * r + n : 0];
  const float so = so_ok ? sov : 0.0f;
  const int ma = m0 + c16;
  const int xa = xs[c16];
  // State / embedding operands: the s block from the old bf16 state, the e
  // block from the embedding row of x_{k-1}; invalid ones load W1[0] and are
  // replaced by zeros.
  const bool s_ok = sb_old != nullptr && ma < R;
  u32x4 a[kSB];
#pragma unroll
  for (int u = 0; u < kSB; ++u) {
    const int kk = lo + 32 * u;
    const bool in = kk < hi;
    const int ke = (in ? kk : 0) + 8 * quad;
    const bool from_s = ke < r;
    const bool ok = in && (from_s ? s_ok : xa >= 0);
    const uint16_t* src = !ok ? W1 : from_s ? sb_old + (size_t)ma * r + ke
                                            : W1 + (size_t)xa * r + (ke - r);
    a[u] = zero_unless(ok, *reinterpret_cast<const u32x4*>(src));
  }
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
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      red[((wave * 2 + a) * 16 + 4 * quad + i) * kSPad + c16] = acc[a][i];
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
  long sp = (2L * 256 + tiles - 1) / tiles;   // about two workgroups per CU
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
  hipLaunchKernelGGL(rnn_pre_kernel, dim3(per * kXcds), dim3(256), 0, stream, h, U, b, M, r, d,
                     B.splits, items, B.P, reinterpret_cast<uint4*>(B.words), (n_words + 1) / 2);
  return check_launch("rnn_pre_kernel");
}

dspark_status launch_rnn_state(const uint16_t* W1, const uint16_t* U, const int32_t* anchors,
                               const unsigned long long* prev, int sub, int R, int gamma, int V,
                               int r, int d, int k, const RnnBuffers& B, float* s_out,
                               hipStream_t stream) {
  const dim3 grid((R + 15) / 16, (r + 15) / 16);
  const int o = k & 1, nw = (k + 1) & 1;   // state before step k in half o, after it in nw
  hipLaunchKernelGGL(rnn_state_kernel, grid, dim3(64 * kSW), 0, stream, W1, U, B.P, B.splits,
                     anchors, prev, sub, R, gamma, V, r, d, k, k == 0 ? nullptr : B.s[o],
                     k == 0 ? nullptr : B.sb[o], s_out ? s_out : B.s[nw], B.sb[nw]);
  return check_launch("rnn_state_kernel");
}

}  // namespace dspark
