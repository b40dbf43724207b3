// Measurement helper (not part of the library): the int8 (and bf16) MFMA
// rate and the shader clock the device holds when waves do nothing but
// v_mfma_i32_32x32x32_i8 (or v_mfma_f32_32x32x16_bf16), with no memory
// traffic.  Set beside the GEMM's
// counters it separates the cost of the matrix instructions themselves from
// the cost of feeding them.
//
// Each wave keeps 8 independent 32x32 accumulators and cycles through four
// A and two B fragments of pseudo-random bytes (fixed per lane), so
// consecutive MFMAs see different operands, as in a GEMM.  One launch does
// blocks x 4 waves x iters x 8 MFMAs of 65536 operations each.  Every wave
// writes one int32 per lane (the sum of its accumulators), so the work is
// observable: with iters doubled every sum doubles exactly.
#include <hip/hip_runtime.h>

#include <cstdint>

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

namespace {

__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// 4 fragments of 16 bytes with values in [-64, 63] (no int32 overflow for
// any iters below 2^20: 8 x 32 x 64 x 64 x 2^20 < 2^31 per accumulator).
__device__ __forceinline__ v4i frag(uint32_t seed) {
  v4i f;
  for (int i = 0; i < 4; ++i) f[i] = int(mix(seed * 4u + uint32_t(i)) & 0xbfbfbfbfu);
  return f;
}

__global__ __launch_bounds__(256, 2) void mfma_i8_loop(int iters, int* __restrict__ out) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  const v4i a0 = frag(t * 8u + 0), a1 = frag(t * 8u + 1), a2 = frag(t * 8u + 2), a3 = frag(t * 8u + 3);
  const v4i b0 = frag(t * 8u + 4), b1 = frag(t * 8u + 5);
  v16i acc[8];
  for (int j = 0; j < 8; ++j)
    for (int e = 0; e < 16; ++e) acc[j][e] = 0;
  for (int i = 0; i < iters; ++i) {
    acc[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, b0, acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, b1, acc[1], 0, 0, 0);
    acc[2] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a2, b0, acc[2], 0, 0, 0);
    acc[3] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a3, b1, acc[3], 0, 0, 0);
    acc[4] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, b1, acc[4], 0, 0, 0);
    acc[5] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, b0, acc[5], 0, 0, 0);
    acc[6] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a2, b1, acc[6], 0, 0, 0);
    acc[7] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a3, b0, acc[7], 0, 0, 0);
  }
  int s = 0;
  for (int j = 0; j < 8; ++j)
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  out[t] = s;
}

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// The same loop on v_mfma_f32_32x32x16_bf16 (32768 flops each), for the
// bf16 matmul of the weight-only path.  Fragments hold bf16 values in
// [1, 2) (pseudo-random mantissas), so sums stay finite for any iters; each
// lane writes the int32 bits of its float sum.
__device__ __forceinline__ v4i frag_bf16(uint32_t seed) {
  v4i f;
  for (int i = 0; i < 4; ++i) f[i] = int((mix(seed * 4u + uint32_t(i)) & 0x007f007fu) | 0x3f803f80u);
  return f;
}

__global__ __launch_bounds__(256, 2) void mfma_bf16_loop(int iters, int* __restrict__ out) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  const v8bf a0 = __builtin_bit_cast(v8bf, frag_bf16(t * 8u + 0)), a1 = __builtin_bit_cast(v8bf, frag_bf16(t * 8u + 1));
  const v8bf a2 = __builtin_bit_cast(v8bf, frag_bf16(t * 8u + 2)), a3 = __builtin_bit_cast(v8bf, frag_bf16(t * 8u + 3));
  const v8bf b0 = __builtin_bit_cast(v8bf, frag_bf16(t * 8u + 4)), b1 = __builtin_bit_cast(v8bf, frag_bf16(t * 8u + 5));
  v16f acc[8];
  for (int j = 0; j < 8; ++j)
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  for (int i = 0; i < iters; ++i) {
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[1], 0, 0, 0);
    acc[2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, b0, acc[2], 0, 0, 0);
    acc[3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a3, b1, acc[3], 0, 0, 0);
    acc[4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[4], 0, 0, 0);
    acc[5] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc[5], 0, 0, 0);
    acc[6] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, b1, acc[6], 0, 0, 0);
    acc[7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a3, b0, acc[7], 0, 0, 0);
  }
  float s = 0.f;
  for (int j = 0; j < 8; ++j)
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  out[t] = __float_as_int(s);
}

}  // namespace

// blocks workgroups of 256 threads; out holds blocks * 256 int32.
extern "C" int mfma_rate_launch(int blocks, int iters, int* out, hipStream_t stream) {
  if (blocks <= 0 || iters < 0 || iters >= (1 << 20) || out == nullptr) return 1;
  hipLaunchKernelGGL(mfma_i8_loop, dim3(unsigned(blocks)), dim3(256), 0, stream, iters, out);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

// The bf16 loop; out holds blocks * 256 int32 (float bits).
extern "C" int mfma_rate_launch_bf16(int blocks, int iters, int* out, hipStream_t stream) {
  if (blocks <= 0 || iters < 0 || iters >= (1 << 20) || out == nullptr) return 1;
  hipLaunchKernelGGL(mfma_bf16_loop, dim3(unsigned(blocks)), dim3(256), 0, stream, iters, out);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}
