// Shared device helpers for libmcsparse (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mcs {

typedef uint16_t bf16_t;  // raw bf16 storage

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;  // masked score: exp2 of it is exactly 0

// Word 3 of a raw buffer resource on gfx9-family parts (32-bit data format);
// loads past num_records return zeros.
constexpr int kBufferFlags = 0x00020000;

// s_waitcnt immediate for vmcnt(0) with expcnt / lgkmcnt left at their
// maximum (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8]). Used after LDS-DMA loads, whose completion the compiler
// does not track through registers.
constexpr int kWaitVmcnt0 = 0x0F70;

// A raw buffer resource whose base and size are wave-uniform (SGPRs). The
// explicit readfirstlane keeps the compiler from treating the descriptor as
// divergent, which would wrap every buffer load in a waterfall loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void *base, uint32_t bytes) {
  const uint64_t v = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), 0, n, kBufferFlags);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
  __bf16 h = (__bf16)x;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroups are dealt to the 8 XCDs round-robin by id. Remap so that XCD x
// runs a contiguous range of logical work items: neighbouring items (query
// tiles of one head, or sibling query groups) then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int per = nblocks >> 3, rem = nblocks & 7;
  const int xcd = bid & 7, local = bid >> 3;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

}  // namespace mcs
