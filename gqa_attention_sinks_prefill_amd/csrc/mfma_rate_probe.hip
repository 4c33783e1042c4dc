// Matrix-pipe reference for the benchmark (not part of the attention
// library): the bf16 MFMA rate one plain kernel sustains on this GPU when
// every SIMD does nothing but independent v_mfma_f32_32x32x16_bf16, with the
// operands either taken from a bf16 tensor (changing from one instruction to
// the next, as the prefill's do) or all equal to 1.0.  The two rates differ by
// how much power the operand bits draw, which sets the clock the chip holds.
//
// int mfma_rate_probe(const void* operands, int64_t bytes, int32_t blocks,
//                     int32_t iters, uint32_t* out, void* stream)
//   operands: device bf16 data, 16-byte aligned, bytes >= 16384 (each wave
//   reads its 16 A and B fragments from one 16 KB window of it), or null for
//   operands of 1.0.  blocks: workgroups of 256 threads (2 per CU fill every
//   SIMD with 2 waves).  iters: loop trips of 16 MFMAs per wave.  out: device,
//   `blocks` uint32 (written only if the folded result equals a constant the
//   sums never reach, so the MFMAs cannot be dropped).  Returns 0, -1 for bad
//   arguments, -3 if the launch fails.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
constexpr int kThreads = 256;

__device__ __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__global__ __launch_bounds__(kThreads, 2) void mfma_kernel(const u32x4_t* __restrict__ ops,
                                                           int64_t windows, int iters,
                                                           uint32_t* out) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  u32x4_t a[8], b[8];
  if (ops != nullptr) {
    const u32x4_t* w = ops + (wave % windows) * 1024;   // 16 KB: 16 fragments x 64 lanes
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = w[i * 64 + lane];
      b[i] = w[(8 + i) * 64 + lane];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = b[i] = u32x4_t{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  }
  f32x16_t acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j & 3] = mfma(a[j & 7], b[(3 * j) & 7], acc[j & 3]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[j][i];
  if (s == 1.5e38f) out[blockIdx.x] = 1u;
}

}  // namespace

extern "C" int mfma_rate_probe(const void* operands, int64_t bytes, int32_t blocks, int32_t iters,
                               uint32_t* out, void* stream) {
  if (!out || blocks <= 0 || iters <= 0) return -1;
  if (operands != nullptr &&
      (bytes < 16384 || reinterpret_cast<uintptr_t>(operands) % 16 != 0))
    return -1;
  hipLaunchKernelGGL(mfma_kernel, dim3(blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4_t*>(operands),
                     operands != nullptr ? bytes / 16384 : int64_t(1), iters, out);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
