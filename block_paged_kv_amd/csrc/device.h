// Device-side helpers shared by the gfx950 kernels of libpagedkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedkv.h"

namespace pagedkv {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

// bf16 is carried as raw 16-bit patterns; a 32-bit word holds two of them,
// the lower-addressed element in the low half.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats -> packed bf16 pair (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float float2v __attribute__((ext_vector_type(2)));
  const float2v f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// Two bf16 products summed into a float accumulator (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Lane permutation inside a 16-lane DPP row.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}

// Sum over aligned groups of R lanes (R in {1,2,4,8,16}); every lane of a
// group receives the group total. quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror and row_mirror pair each lane with a partner in the
// other half of its current group.
template <int R>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (R >= 2) x += dpp_mov<0xB1>(x);
  if constexpr (R >= 4) x += dpp_mov<0x4E>(x);
  if constexpr (R >= 8) x += dpp_mov<0x141>(x);
  if constexpr (R >= 16) x += dpp_mov<0x140>(x);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

typedef short shortx4_t __attribute__((ext_vector_type(4)));

// Transposing LDS read (ds_read_b64_tr_b16). Within each 16-lane group, lane
// j receives, for k = 0..3, element j % 4 of the 8-byte row addressed by lane
// 4k + j / 4: when lane j addresses row r0 + j / 4, columns c0 + 4 (j % 4) ..
// +3 of a row-major 16-bit matrix, it receives rows r0 .. r0+3 of column
// c0 + j.
__device__ __forceinline__ uint2 ds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) shortx4_t lds_shortx4_t;
  const shortx4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t*)(p));
  return __builtin_bit_cast(uint2, r);
}

// Maximum over the four lanes l % 16 + 16k (k = 0..3) that hold one matrix
// column of an MFMA 16x16 accumulator: v_permlane32_swap pairs lane l with
// l ^ 32 and v_permlane16_swap pairs l with l ^ 16; each returns both halves
// of the pair.
__device__ __forceinline__ float max_across_groups(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
  const unsigned w = __float_as_uint(x);
  const auto r16 = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
}

// Eight E4M3 codes (bytes of v, low first) to eight bf16 values, exactly:
// every E4M3 value is a bf16 value. v_cvt_scalef32_pk_bf16_fp8 converts one
// 16-bit half of a word (two codes) and multiplies by 2^exponent(scale); a
// scale of 1 leaves the values as they are.
template <bool HI>
__device__ __forceinline__ uint32_t widen_e4m3x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
__device__ __forceinline__ uint4 widen_e4m3x8(const uint2& v) {
  return make_uint4(widen_e4m3x2<false>(v.x), widen_e4m3x2<true>(v.x),
                    widen_e4m3x2<false>(v.y), widen_e4m3x2<true>(v.y));
}

// 16 zero bytes in the code object: the load source of key rows a tile or
// stage does not attend, so those LDS rows hold finite zeros.
__device__ __attribute__((aligned(16))) const uint4 kZeroChunk = {0u, 0u, 0u, 0u};

// global_load_lds_dwordx4: each lane copies 16 bytes from global memory to
// LDS byte offset m0 + 16 * lane (m0 wave-uniform). Issued as assembly so that
// the compiler leaves the vector-memory counter to the kernel's own pipeline
// (it would otherwise drain every outstanding load before each LDS read).
// Two address forms: a 64-bit address per lane, or a wave-uniform 64-bit base
// (held in scalar registers) plus a 32-bit byte offset per lane.
__device__ __forceinline__ void lds_dma16(const void* gaddr, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(m0), "v"(gaddr) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(m0), "v"(voff), "s"(base) : "memory", "m0");
}

// Streaming forms (the nt cache policy: lines marked for early eviction), for
// data a kernel reads exactly once, such as the decode kernels' K/V stages. A
// plain read stream of a 2 GiB buffer, contiguous or in random 8 KiB chunks,
// measured about 6.9 TB/s with the policy and 6.1-6.3 TB/s without.
__device__ __forceinline__ void lds_dma16_stream(const void* gaddr, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
               :: "s"(m0), "v"(gaddr) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma16_stream(const void* base, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
               :: "s"(m0), "v"(voff), "s"(base) : "memory", "m0");
}

// LDS byte offset of a __shared__ location: the low half of its generic
// address (the high half is the LDS aperture).
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

}  // namespace pagedkv
