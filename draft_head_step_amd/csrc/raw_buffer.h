// Branch-free loads for CDNA4 (gfx950), shared by the RNN-head and the
// scheduler kernels.
//
// A guarded load (if in range, load, else zero) puts every load in a basic
// block of its own, and the compiler then waits for all outstanding loads at
// the joins; a select on a loaded value makes it wait where the select is
// placed.  Here tails read as zero without branches or selects: buffer loads
// whose per-lane offset lies past the resource's size return zeros.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace dspark {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;        // untyped dword access (gfx9 family)
constexpr uint32_t kOff = 0x80000000u;        // an offset past every resource below
constexpr size_t kMaxRsrcBytes = 0x80000000u;  // every resource here is at most 2^31 bytes

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
__device__ __forceinline__ float ld4f(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, opaque(off), 0, 0));
}
__device__ __forceinline__ uint32_t ld2(Rsrc r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, opaque(off), 0, 0);
}

}  // namespace
}  // namespace dspark
