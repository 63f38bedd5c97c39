// Device-side helpers shared by the HIP kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lazyattn {

// ---- 64-bit block word (layout documented in include/lazy_attn.h) --------
struct BlockWord {
  uint32_t block_id;
  int32_t pos0;
  int32_t n_valid;
  bool causal;
};

__device__ __forceinline__ BlockWord unpack_word(uint64_t w) {
  BlockWord b;
  b.block_id = static_cast<uint32_t>(w);
  b.pos0 = static_cast<int32_t>((w >> 32) & 0xFFFFFFull);
  b.n_valid = static_cast<int32_t>((w >> 56) & 0x7Full) + 1;
  b.causal = (w >> 63) != 0;
  return b;
}

// ---- bf16 <-> fp32 --------------------------------------------------------
// Widening is exact: a bf16 value is the top half of its fp32 bit pattern.
__device__ __forceinline__ float bf16_lo(uint32_t packed) {
  return __uint_as_float(packed << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t packed) {
  return __uint_as_float(packed & 0xFFFF0000u);
}

// Round two fp32 values to bf16 (round-to-nearest-even) and pack lo | hi<<16.
// gfx950 has a native instruction (v_cvt_pk_bf16_f32) for this conversion.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return static_cast<uint16_t>(pack_bf16x2(x, 0.0f) & 0xFFFFu);
}

// ---- wave-level reductions (wave64) ---------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace lazyattn
