// Internal launchers shared between the C-ABI layer and the kernel files.
// Every launcher assumes its arguments were validated by the ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convrot {

// Two fp32 -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// The int8 code of a value v of a row whose scale is s (the scale's rule is
// s = absmax / 127): code = round_half_away(v / s), taken as one fused
// multiply-add and a byte pick.  rb = RN(1 / s) raised by two units in the
// last place, so that |v * rb| exceeds |v / s| strictly, by at most 2^-21 of
// it; fma(v, rb, 1.5 * 2^23) rounds v * rb to an integer once (the unit in
// the last place there is 1, ties to even) and its low byte is that integer
// in two's complement.  An exact tie n + 1/2 therefore rounds away from
// zero, as the definition does, and a code differs from the definition only
// where |v / s| lies within 2^-21 of a boundary below it (one further from
// zero).  Valid for s in [2^-100, 2^122) or s = 0 (all codes 0); smaller
// scales are lifted by 2^64 with their values.  The identities are checked
// on the host (tests/host/quotient_identities.c).
constexpr float kCodeMagic = 12582912.0f;  // 1.5 * 2^23
constexpr float kTinyScale = 0x1p-100f;    // below it, lift values and scale by 2^64

__device__ __forceinline__ float code_rcp(float s) {
  return s > 0.f ? __uint_as_float(__float_as_uint(1.0f / s) + 2u) : 0.f;
}

// The word whose low byte is the code of v (rb from code_rcp, possibly
// carrying a sign flip shared with v).
__device__ __forceinline__ uint32_t code_bits(float v, float rb) {
  return __float_as_uint(__builtin_fmaf(v, rb, kCodeMagic));
}

// The low bytes of four words, in order, as one word.
__device__ __forceinline__ uint32_t pack4_lo(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);  // a0 b0 0 0
  const uint32_t hi = __builtin_amdgcn_perm(d, c, 0x0c0c0400u);  // c0 d0 0 0
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);             // a0 b0 c0 d0
}

// x bf16 [rows, K] (in_dtype 1) or fp32 (in_dtype 0) -> codes int8 [rows, K]
// with |code| <= qmax and fp32 scale [rows].  log2g = log2(group size).
hipError_t launch_rotate_quant(const void* x, int in_dtype, int64_t rows, int64_t K, int log2g,
                               int8_t* codes, float* scale, hipStream_t stream);

// Fast path for bf16 activations with group 256 (K a multiple of 256 up to
// 16384); returns hipErrorNotSupported without launching for other shapes.
hipError_t launch_rotate_quant_g256(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, float* x_scale,
                                    hipStream_t stream);

// Fast path for bf16 activations with group 16 or 1 (log2g 4 or 0) and
// K <= 8192; returns hipErrorNotSupported without launching otherwise.
hipError_t launch_rotate_quant_small(const uint16_t* x, int64_t M, int64_t K, int log2g, int8_t* xq, float* x_scale,
                                     hipStream_t stream);

// RMSNorm with (1 + w) weights, then the activation rotate-and-quantize of
// its bf16 output (bf16 input only).  y_norm, if not null, receives the
// normalised bf16 row.
hipError_t launch_rmsnorm_rotate_quant(const uint16_t* x, const float* norm_w, float eps, int64_t rows, int64_t K,
                                       int log2g, int8_t* codes, float* scale, uint16_t* y_norm,
                                       hipStream_t stream);

// Fast path of the above for group 256 (same shapes as launch_rotate_quant_g256).
hipError_t launch_rmsnorm_rotate_quant_g256(const uint16_t* x, const float* norm_w, float eps, int64_t M,
                                            int64_t K, int8_t* xq, float* x_scale, uint16_t* y_norm,
                                            hipStream_t stream);

// int4 weight preparation with the per-row clip search; clip_index may be null.
hipError_t launch_quantize_weight_i4(const void* w, int in_dtype, int64_t rows, int64_t K, int log2g,
                                     uint8_t* wq4, float* scale, int32_t* clip_index, hipStream_t stream);

// Weight-only path: codes (int8 [rows, K] or packed int4 [rows, K/2]) and
// row scales -> the un-rotated weight as bf16 [rows, K].
hipError_t launch_dequantize_weight(const void* wq, int wbits, const float* w_scale, int64_t rows, int64_t K,
                                    int log2g, uint16_t* out, hipStream_t stream);

// Fast path of the above for group 256 (K a multiple of 256); returns
// hipErrorNotSupported without launching otherwise.
hipError_t launch_dequantize_g256(const void* wq, int wbits, const float* w_scale, int64_t rows, int64_t K,
                                  uint16_t* out, hipStream_t stream);

// y = bf16(x . w^T) for bf16 x [M, K] and w [N, K], fp32 accumulation
// (the matmul of the weight-only path).
hipError_t launch_gemm_bf16(const uint16_t* x, const uint16_t* w, int64_t M, int64_t N, int64_t K, uint16_t* y,
                            hipStream_t stream);

// One weight matrix of a GEMM launch and its outputs (row stride ldy
// elements); acc and y may each be null, the same way for every output.
struct GemmOutDesc {
  const void* wq;
  const float* w_scale;
  int N, ldy;
  int32_t* acc;
  uint16_t* y;
};

// acc_o = xq . wq_o^T (int32), optional bf16 epilogue, for 1..8 weight
// matrices sharing the quantized input, in one launch.  wbits 8 or 4.
hipError_t launch_gemm_multi(const int8_t* xq, const float* x_scale, int wbits, int64_t M, int64_t K,
                             const GemmOutDesc* outs, int n_outs, hipStream_t stream);

// acc = xq . wq^T (int32), optional bf16 epilogue.  wbits 8 or 4.
hipError_t launch_gemm(const int8_t* xq, const float* x_scale, const void* wq, int wbits,
                       const float* w_scale, int64_t M, int64_t N, int64_t K, int32_t* acc_out,
                       uint16_t* y, hipStream_t stream);

}  // namespace convrot
