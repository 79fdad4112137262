// Packed per-step results of the Markov-head draft, shared by the step
// kernels and the kernels that read their last results.
//
// A step's result for request m is one 64-bit word combined across workgroups
// with an unsigned atomic max: the selection score in the high half (mapped to
// an unsigned key that orders like the float, -0 taken as +0) and the
// complement of the token id in the low half, so equal scores keep the
// smallest id whatever order the workgroups arrive in.  Each request has S
// words (1 or kMaxSubWords, chosen per call) and V group g combines into word
// g % S; a reader takes the maximum of the S words.
//
// Ids are checked on the device: a request whose input token lies outside
// [0, V) (a bad anchor, or a bad token of the step before) publishes kPoison,
// which is above every packed score (the largest key a score can map to is
// that of +inf) and decodes to -1, so every later step of that request, and
// its output tokens, carry -1.  A cleared word (0), or any word whose id is
// not below V, also decodes to -1.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace dspark {

constexpr int kMaxSubWords = 16;
constexpr int kSubWordsAboveGroups = 256;
constexpr unsigned long long kPoison = 0xffffffff00000000ull;

__device__ __forceinline__ unsigned long long pack_best(float v, int i) {
  const uint32_t b = __float_as_uint(v + 0.0f);
  const uint32_t key = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)key << 32) | (unsigned long long)(0xffffffffu - (uint32_t)i);
}

__device__ __forceinline__ int unpack_token(unsigned long long w, int V) {
  const uint32_t i = 0xffffffffu - (uint32_t)w;
  return i < (uint32_t)V ? (int)i : -1;
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

}  // namespace dspark
