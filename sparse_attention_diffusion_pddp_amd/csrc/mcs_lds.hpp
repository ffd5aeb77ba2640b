// LDS tile helpers shared by the attention and selection kernels (gfx950):
// the XOR swizzle of 16-byte chunks, LDS-DMA buffer loads, the transposing
// LDS read and the cross-half lane exchange.
#pragma once

#include "mcs_common.hpp"

namespace mcs {

// K (and V) tiles sit in LDS row-major (one row = one key), each 16-byte chunk
// c of row k stored at chunk c ^ swz(k). With it, the 32 keys x one chunk of
// a K fragment read and the 4 keys x 32 bytes of a transposing V read both
// spread over all banks.
template <int CH>
__device__ __forceinline__ int swz(int k) {
  return (((k & 3) << 1) | ((k >> 2) & 1) | (((k >> 3) & 1) << 3)) & (CH - 1);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposing LDS read (gfx950 ds_read_b64_tr_b16). Inside each group of 16
// lanes, with M[j] the four 16-bit values at lane j's address, lane i
// receives M[4e + i/4][i % 4] as element e (e = 0..3).
// (The host compilation pass of this file never sees gfx950 builtins: a
// kernel template mentioning them would silently lose its host launch stub.)
__device__ __forceinline__ s16x4 lds_read_tr16(const bf16_t *p) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
#else
  return s16x4{};
#endif
}

// Every lane gets {x of its lane in the low half (lanes 0-31), x of its lane
// in the high half}: one v_permlane32_swap on two copies of x instead of an
// LDS round trip. Written as inline asm because this toolchain's builtin for
// the instruction returns the first register's result for both outputs.
// The s_nops cover the VALU-write-then-permlane wait states.
__device__ __forceinline__ void cross_half(float x, float &lo, float &hi) {
#if defined(__HIP_DEVICE_COMPILE__)
  lo = x;
  hi = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(lo), "+v"(hi));
#else
  lo = hi = x;
#endif
}

// 16-byte buffer load of each lane straight into LDS at lds + 16 * lane.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, void *lds, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, 0, 0, 0);
#endif
}

}  // namespace mcs
