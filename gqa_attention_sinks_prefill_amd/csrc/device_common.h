// Device-side building blocks shared by the sink-attention kernels (gfx950).
//
// Register layouts of the two bf16 MFMA shapes used here (wave64):
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//     A: lane l holds row l%32, k = 8*(l/32) .. +7   (8 bf16 = 16 bytes)
//     B: lane l holds col l%32, k = 8*(l/32) .. +7
//     D: lane l holds col l%32, rows 8*(i/4) + 4*(l/32) + i%4, i = 0..15
//   v_mfma_f32_16x16x32_bf16  D[16x16] += A[16x32] * B[32x16]
//     A: lane l holds row l%16, k = 8*(l/16) .. +7
//     B: lane l holds col l%16, k = 8*(l/16) .. +7
//     D: lane l holds col l%16, rows 4*(l/16) + i, i = 0..3
// The contraction index k may be permuted freely as long as A and B use the
// same permutation; the kernels use that freedom to feed the softmax output
// (in D layout) straight back as the B operand of the P.V product.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sinkattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16_t mfma_32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma_16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Two floats -> two bf16 (round to nearest even), low half = lo.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over the lane pair (l, l ^ 32).  permlane32_swap exchanges the
// upper half of one register with the lower half of the other; with both
// operands equal, every lane ends up holding its own value and its partner's.
__device__ __forceinline__ float pair32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Same over (l, l ^ 16): permlane16_swap exchanges odd 16-lane rows of one
// register with even rows of the other.
__device__ __forceinline__ float pair16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ u32x4_t load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// Raw buffer resource over `num_bytes` bytes from `base` (dword 3 = the CDNA
// default data format).  A load whose offset lies past num_bytes returns zero
// and does not touch memory, which is how tiles are padded at sequence ends.
constexpr int kBufferWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, num_bytes, kBufferWord3);
}
// Cache policy of a load: 0 = default, kNonTemporal = streaming data that is
// read once (the "nt" bit).
constexpr int kNonTemporal = 2;
template <int kPolicy = 0>
__device__ __forceinline__ u32x4_t buffer_load16(__amdgpu_buffer_rsrc_t r, int byte_offset) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, kPolicy);
}

// Direct global -> LDS copy through a buffer resource: every lane moves 16
// bytes from byte_offset + wave_offset into LDS at lds_base + 16 * lane (lanes
// past the resource's end write zeros).  lds_base and wave_offset must be
// wave-uniform.  Completion is tracked by vmcnt.
template <int kPolicy = 0>
__device__ __forceinline__ void buffer_load16_lds(__amdgpu_buffer_rsrc_t r, void* lds_base,
                                                  int byte_offset, int wave_offset = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds_base, 16, byte_offset, wave_offset, 0,
      kPolicy);
}

// Wait until this wave's outstanding vector-memory operations (including the
// LDS copies above) have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element (i & 3) of the 8-byte pieces addressed by lanes
// 4k + (i >> 2), k = 0..3, as its elements k = 0..3.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2_t lds_read_tr16(const void* p) {
  s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, r);
}

// Transposing 8-bit LDS read (ds_read_b64_tr_b8).  Within each group of 16
// lanes, lane i receives byte (i & 7) of the 8-byte pieces addressed by lanes
// 2k + (i >> 3), k = 0..7, as its bytes k = 0..7 (established by an in-bounds
// probe of the instruction).
typedef int i32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2_t lds_read_tr8(const void* p) {
  i32x2_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2_t*)(p));
  return __builtin_bit_cast(u32x2_t, r);
}

// Two OCP E4M3 codes (bytes 0-1 of `w`, or 2-3 when HI) -> two bf16, exactly
// (every E4M3 value is a bf16 value).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
// Eight codes (two words) -> the eight bf16 of one MFMA operand.
__device__ __forceinline__ u32x4_t fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  return u32x4_t{fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0), fp8x2_to_bf16x2<false>(w1),
                 fp8x2_to_bf16x2<true>(w1)};
}

// max of three floats in one instruction (v_max3_f32)
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Store of a result no kernel of this launch reads back (the "nt" bit):
// streamed out rather than kept in the cache.  Under a saturating read
// stream, plain stores of the split-decode states were acknowledged so late
// that the waves' waits for their next copies stalled on them.
__device__ __forceinline__ void store_nt(float* p, float v) { __builtin_nontemporal_store(v, p); }


}  // namespace sinkattn
