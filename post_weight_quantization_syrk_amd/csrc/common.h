// Shared device-side definitions for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace gptq {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// bf16 bit pattern -> float (exact widening).
__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// LDS transpose read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i supplies the address of 4 consecutive 16-bit elements; lane j
// receives element j%4 of the chunks addressed by lanes 4e + j/4, e = 0..3.
// Used with lane i addressing row (i/4), columns 4*(i%4)..+3 of a row-major
// 4 x 16 block, lane j receives column j, rows 0..3.
__device__ __forceinline__ s16x4 lds_read_tr16(const void* lds_generic_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_generic_ptr));
}

__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Broadcast lane `SRC` (0..15) of each 16-lane row to the whole row (DPP
// row_newbcast): a VGPR-to-VGPR move, no scalar register involved.
template <int SRC>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(
      __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + SRC, 0xF, 0xF, false));
}

}  // namespace gptq
