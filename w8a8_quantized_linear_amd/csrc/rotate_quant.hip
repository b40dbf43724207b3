// Fused group-wise Hadamard rotation + per-row quantization on gfx950.
//
// One row (an activation token, or an output row of a weight) is held in the
// registers of TPT threads; every thread owns C chunks of 16 consecutive
// elements (chunk c = t + TPT * j).  A group of g <= 256 elements is g/16
// consecutive chunks, so it sits in g/16 consecutive lanes of one 16-lane row
// of the wavefront.  The fast Walsh-Hadamard transform then runs as:
//   - stages over element-index bits 0..3: butterflies inside a thread's 16
//     registers;
//   - stages over bits 4..7: butterflies between lanes t and t ^ (1 << b-4)
//     (cross-lane exchange within the 16-lane row).
// The transform is left unnormalised (sums of +-x); for even log2(g) the 1/sqrt(g)
// is a power of two and is folded exactly into the scale, for odd log2(g) it
// is applied per element.
//
// The row's absmax is reduced across the TPT threads (wave shuffles, then LDS
// across waves), after which every code is decided in fp32:
//   scale = absmax / 127,  code = round_half_away(value / scale)
// as stated for ConvRot int8 checkpoints ("MOSS-Image Qwen3.5-9B text encoder,
// INT8 (W8A8, ConvRot)", file table rows "Quantized" and "Matmul"); the
// quotient and rounding are one fma and a byte pick (code_rcp, code_bits),
// the rule every int8 code of the library follows.
//
// MODE_I4 runs the int4 weight preparation of "MossInt4" ("Format"): the same
// rotation, then a per-row clip search over c = 1.00 .. 0.50 with fp64 error
// sums, codes in [-7, 7] packed two per byte (low nibble = even column).
#include "convrot_internal.h"

#include <math.h>

namespace convrot {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

enum { IN_F32 = 0, IN_BF16 = 1 };
enum { MODE_I8 = 0, MODE_I4 = 1 };

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

template <int IN>
__device__ __forceinline__ void load_chunk(const void* base, int64_t elem_off, float (&v)[16]) {
  if constexpr (IN == IN_BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem_off);
    uint4 a = p[0], b = p[1];
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = bf16_lo(w[i]);
      v[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem_off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 f = p[i];
      v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
  }
}

// Butterflies over element bits 0..min(log2g, 4)-1 inside one chunk.
__device__ __forceinline__ void fwht_in_register(float (&v)[16], int log2g) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if (b < log2g) {
      const int h = 1 << b;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (!(i & h)) {
          float a = v[i], c = v[i + h];
          v[i] = a + c;
          v[i + h] = a - c;
        }
      }
    }
  }
}

// Butterflies over element bits 4..log2g-1: partner lane differs in bit b-4.
__device__ __forceinline__ void fwht_cross_lane(float (&v)[16], int log2g, int lane) {
#pragma unroll
  for (int b = 4; b < 8; ++b) {
    if (b < log2g) {
      const int m = 1 << (b - 4);
      const bool high = (lane & m) != 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = __shfl_xor(v[i], m);
        v[i] = high ? (p - v[i]) : (v[i] + p);
      }
    }
  }
}

template <int TPT>
__device__ __forceinline__ float row_max(float v, float* red) {
  constexpr int kIn = TPT < 64 ? TPT : 64;
#pragma unroll
  for (int off = kIn / 2; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  if constexpr (TPT > 64) {
    const int wave = threadIdx.x / 64;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    const int first = (threadIdx.x / TPT) * (TPT / 64);
    float r = red[first];
#pragma unroll
    for (int w = 1; w < TPT / 64; ++w) r = fmaxf(r, red[first + w]);
    __syncthreads();
    v = r;
  }
  return v;
}

template <int TPT>
__device__ __forceinline__ double row_sum(double v, double* red) {
  constexpr int kIn = TPT < 64 ? TPT : 64;
#pragma unroll
  for (int off = kIn / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  if constexpr (TPT > 64) {
    const int wave = threadIdx.x / 64;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    const int first = (threadIdx.x / TPT) * (TPT / 64);
    double r = red[first];
#pragma unroll
    for (int w = 1; w < TPT / 64; ++w) r += red[first + w];
    __syncthreads();
    v = r;
  }
  return v;
}

template <int TPT, int C, int IN, int MODE, bool NORM>
__global__ __launch_bounds__(kThreads) void rotate_quant_kernel(const void* __restrict__ x, int64_t rows,
                                                                int64_t K, int log2g, float inv_sqrt_g,
                                                                float pow2_norm, void* __restrict__ codes,
                                                                float* __restrict__ scale,
                                                                int32_t* __restrict__ clip_index,
                                                                const float* __restrict__ norm_w, float eps,
                                                                uint16_t* __restrict__ y_norm) {
  static_assert(!NORM || (IN == IN_BF16 && MODE == MODE_I8), "the norm front end takes bf16 activations");
  constexpr int P = kThreads / TPT;  // rows per workgroup
  __shared__ float red_f[kWaves];
  __shared__ double red_d[kWaves];

  const int t = threadIdx.x % TPT;
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * P + threadIdx.x / TPT;
  const bool row_ok = row < rows;
  const int64_t nchunks = K / 16;
  const bool odd = (log2g & 1) != 0;

  float v[C][16];
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int64_t c = t + int64_t(TPT) * j;
    if (row_ok && c < nchunks) {
      load_chunk<IN>(x, row * K + c * 16, v[j]);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[j][i] = 0.f;
    }
  }

  if constexpr (NORM) {
    // RMSNorm with (1 + w) weights; the rotation below sees its bf16 output.
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < C; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) ss = __builtin_fma(double(v[j][i]), double(v[j][i]), ss);
    ss = row_sum<TPT>(ss, red_d);
    const float ms = float(ss / double(K));
    const float r = 1.0f / sqrtf(ms + eps);
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const int64_t c = t + int64_t(TPT) * j;
      if (c < nchunks) {
        uint32_t yw[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float w0 = norm_w[c * 16 + 2 * i], w1 = norm_w[c * 16 + 2 * i + 1];
          yw[i] = pack_bf16x2((v[j][2 * i] * r) * (1.0f + w0), (v[j][2 * i + 1] * r) * (1.0f + w1));
          v[j][2 * i] = __uint_as_float(yw[i] << 16);
          v[j][2 * i + 1] = __uint_as_float(yw[i] & 0xffff0000u);
        }
        if (y_norm != nullptr && row_ok) {
          uint4* dst = reinterpret_cast<uint4*>(y_norm + row * K + c * 16);
          dst[0] = make_uint4(yw[0], yw[1], yw[2], yw[3]);
          dst[1] = make_uint4(yw[4], yw[5], yw[6], yw[7]);
        }
      }
    }
  }

  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < C; ++j) {
    fwht_in_register(v[j], log2g);
    fwht_cross_lane(v[j], log2g, lane);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (odd) v[j][i] *= inv_sqrt_g;
      amax = fmaxf(amax, fabsf(v[j][i]));
    }
  }
  amax = row_max<TPT>(amax, red_f);

  if constexpr (MODE == MODE_I8) {
    // v holds rotated values times 1/pow2_norm (exact power of two), so
    // value/scale is the same quotient as v / (amax_v / 127).
    float s_v = amax / 127.0f;
    float out_mul = pow2_norm;
    if (s_v < kTinyScale && s_v > 0.f) {
      // Tiny row (uniform: amax is the row's): lift values and scale by 2^64
      // so the reciprocal stays finite; for a normal s_v the quotients are
      // exactly the unlifted ones.
#pragma unroll
      for (int j = 0; j < C; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) v[j][i] *= 0x1p64f;
      s_v = (amax * 0x1p64f) / 127.0f;
      out_mul = pow2_norm * 0x1p-64f;
    }
    if (row_ok && t == 0) scale[row] = s_v * out_mul;
    const float rb = code_rcp(s_v);
    int8_t* out = static_cast<int8_t*>(codes);
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const int64_t c = t + int64_t(TPT) * j;
      uint32_t q[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) q[i] = code_bits(v[j][i], rb);
      if (row_ok && c < nchunks) {
        uint4 o;
        o.x = pack4_lo(q[0], q[1], q[2], q[3]);
        o.y = pack4_lo(q[4], q[5], q[6], q[7]);
        o.z = pack4_lo(q[8], q[9], q[10], q[11]);
        o.w = pack4_lo(q[12], q[13], q[14], q[15]);
        *reinterpret_cast<uint4*>(out + row * K + c * 16) = o;
      }
    }
  } else {
    // int4 clip search on the normalised rotated values.
#pragma unroll
    for (int j = 0; j < C; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) v[j][i] *= pow2_norm;
    const float amax_n = amax * pow2_norm;
    int best_i = 0;
    double best_e = 0.0;
    float best_s = 0.f;
    for (int ci = 0; ci <= 50; ++ci) {
      const float s = float(double(amax_n) * double(100 - ci) / 700.0);
      double e = 0.0;
#pragma unroll
      for (int j = 0; j < C; ++j) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float r = (s == 0.f) ? 0.f : roundf(v[j][i] / s);
          r = fminf(fmaxf(r, -7.f), 7.f);
          double d = double(r) * double(s) - double(v[j][i]);
          e += d * d;
        }
      }
      e = row_sum<TPT>(e, red_d);
      if (ci == 0 || e < best_e) {
        best_e = e;
        best_i = ci;
        best_s = s;
      }
    }
    if (row_ok && t == 0) {
      scale[row] = best_s;
      if (clip_index) clip_index[row] = best_i;
    }
    uint8_t* out = static_cast<uint8_t*>(codes);
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const int64_t c = t + int64_t(TPT) * j;
      uint32_t packed[2] = {0u, 0u};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float r = (best_s == 0.f) ? 0.f : roundf(v[j][i] / best_s);
        r = fminf(fmaxf(r, -7.f), 7.f);
        packed[i / 8] |= (uint32_t(int(r)) & 0xfu) << (4 * (i % 8));
      }
      if (row_ok && c < nchunks) {
        *reinterpret_cast<uint2*>(out + row * (K / 2) + c * 8) = make_uint2(packed[0], packed[1]);
      }
    }
  }
}

template <int IN, int MODE, bool NORM = false>
hipError_t dispatch(const void* x, int64_t rows, int64_t K, int log2g, void* codes, float* scale,
                    int32_t* clip_index, hipStream_t stream, const float* norm_w = nullptr, float eps = 0.f,
                    uint16_t* y_norm = nullptr) {
  const int64_t nchunks = K / 16;
  const float inv_sqrt_g = float(1.0 / sqrt(double(1 << log2g)));
  const float pow2_norm = (log2g & 1) ? 1.0f : ldexpf(1.0f, -(log2g / 2));
  int tpt = 256, c = 1;
  if (nchunks <= 256) {
    tpt = 16;
    while (tpt < nchunks) tpt *= 2;
  } else {
    c = int((nchunks + 255) / 256);
  }
  const int per_block = kThreads / tpt;
  const dim3 grid(unsigned((rows + per_block - 1) / per_block));
#define CONVROT_RQ(TPT_, C_)                                                                          \
  hipLaunchKernelGGL((rotate_quant_kernel<TPT_, C_, IN, MODE, NORM>), grid, dim3(kThreads), 0, stream, x, rows, \
                     K, log2g, inv_sqrt_g, pow2_norm, codes, scale, clip_index, norm_w, eps, y_norm)
  switch (tpt * 16 + c) {
    case 16 * 16 + 1: CONVROT_RQ(16, 1); break;
    case 32 * 16 + 1: CONVROT_RQ(32, 1); break;
    case 64 * 16 + 1: CONVROT_RQ(64, 1); break;
    case 128 * 16 + 1: CONVROT_RQ(128, 1); break;
    case 256 * 16 + 1: CONVROT_RQ(256, 1); break;
    case 256 * 16 + 2: CONVROT_RQ(256, 2); break;
    case 256 * 16 + 3: CONVROT_RQ(256, 3); break;
    case 256 * 16 + 4: CONVROT_RQ(256, 4); break;
    case 256 * 16 + 5: CONVROT_RQ(256, 5); break;
    case 256 * 16 + 6: CONVROT_RQ(256, 6); break;
    case 256 * 16 + 7: CONVROT_RQ(256, 7); break;
    case 256 * 16 + 8: CONVROT_RQ(256, 8); break;
    default: return hipErrorInvalidValue;
  }
#undef CONVROT_RQ
  return hipGetLastError();
}

// Weight-only path: undo the rotation of a stored row.  Codes (int8, or
// packed int4 with the low nibble first) are exact in fp32, and so is their
// unnormalised transform t (|t| <= 256 * 128); the value is then
// s_w * (t * 2^-(log2g/2)) with one rounding for even log2(g) (the power of
// two is exact), or (t / sqrt(g)) * s_w for odd log2(g), and is rounded to
// bf16.  ("MOSS-Image Qwen3.5-9B text encoder, INT8 (W8A8, ConvRot)", file
// table row "Matmul": its weight-only mode expands the codes into a bf16 weight.)
template <int TPT, int C, bool W4>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const void* __restrict__ wq,
                                                           const float* __restrict__ w_scale, int64_t rows,
                                                           int64_t K, int log2g, float inv_sqrt_g, float pow2_norm,
                                                           uint16_t* __restrict__ out) {
  constexpr int P = kThreads / TPT;
  const int t = threadIdx.x % TPT;
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * P + threadIdx.x / TPT;
  const bool row_ok = row < rows;
  const int64_t nchunks = K / 16;
  const bool odd = (log2g & 1) != 0;

  float v[C][16];
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int64_t c = t + int64_t(TPT) * j;
#pragma unroll
    for (int i = 0; i < 16; ++i) v[j][i] = 0.f;
    if (row_ok && c < nchunks) {
      if constexpr (W4) {
        const uint2 b = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(wq) + row * (K / 2) + c * 8);
        const uint32_t w[2] = {b.x, b.y};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int nib = int((w[i / 8] >> (4 * (i % 8))) & 0xfu);
          v[j][i] = float(nib >= 8 ? nib - 16 : nib);
        }
      } else {
        const uint4 b = *reinterpret_cast<const uint4*>(static_cast<const int8_t*>(wq) + row * K + c * 16);
        const uint32_t w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 16; ++i) v[j][i] = float(int8_t(w[i / 4] >> (8 * (i % 4))));
      }
    }
  }
  const float s = row_ok ? w_scale[row] : 0.f;
#pragma unroll
  for (int j = 0; j < C; ++j) {
    fwht_in_register(v[j], log2g);
    fwht_cross_lane(v[j], log2g, lane);
    const int64_t c = t + int64_t(TPT) * j;
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // fma with +0 rounds like the product and turns a -0 (zero scale,
      // negative transform) into the +0 that the dense product gives.
      const float a = odd ? __builtin_fmaf(v[j][2 * i] * inv_sqrt_g, s, 0.0f)
                          : __builtin_fmaf(s, v[j][2 * i] * pow2_norm, 0.0f);
      const float b = odd ? __builtin_fmaf(v[j][2 * i + 1] * inv_sqrt_g, s, 0.0f)
                          : __builtin_fmaf(s, v[j][2 * i + 1] * pow2_norm, 0.0f);
      o[i] = pack_bf16x2(a, b);
    }
    if (row_ok && c < nchunks) {
      uint4* dst = reinterpret_cast<uint4*>(out + row * K + c * 16);
      dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
      dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
  }
}

template <bool W4>
hipError_t dispatch_dequant(const void* wq, const float* w_scale, int64_t rows, int64_t K, int log2g,
                            uint16_t* out, hipStream_t stream) {
  const int64_t nchunks = K / 16;
  const float inv_sqrt_g = float(1.0 / sqrt(double(1 << log2g)));
  const float pow2_norm = (log2g & 1) ? 1.0f : ldexpf(1.0f, -(log2g / 2));
  int tpt = 256, c = 1;
  if (nchunks <= 256) {
    tpt = 16;
    while (tpt < nchunks) tpt *= 2;
  } else {
    c = int((nchunks + 255) / 256);
  }
  const int per_block = kThreads / tpt;
  const dim3 grid(unsigned((rows + per_block - 1) / per_block));
#define CONVROT_DQ(TPT_, C_)                                                                            \
  hipLaunchKernelGGL((dequant_kernel<TPT_, C_, W4>), grid, dim3(kThreads), 0, stream, wq, w_scale, rows, K, \
                     log2g, inv_sqrt_g, pow2_norm, out)
  switch (tpt * 16 + c) {
    case 16 * 16 + 1: CONVROT_DQ(16, 1); break;
    case 32 * 16 + 1: CONVROT_DQ(32, 1); break;
    case 64 * 16 + 1: CONVROT_DQ(64, 1); break;
    case 128 * 16 + 1: CONVROT_DQ(128, 1); break;
    case 256 * 16 + 1: CONVROT_DQ(256, 1); break;
    case 256 * 16 + 2: CONVROT_DQ(256, 2); break;
    case 256 * 16 + 3: CONVROT_DQ(256, 3); break;
    case 256 * 16 + 4: CONVROT_DQ(256, 4); break;
    case 256 * 16 + 5: CONVROT_DQ(256, 5); break;
    case 256 * 16 + 6: CONVROT_DQ(256, 6); break;
    case 256 * 16 + 7: CONVROT_DQ(256, 7); break;
    case 256 * 16 + 8: CONVROT_DQ(256, 8); break;
    default: return hipErrorInvalidValue;
  }
#undef CONVROT_DQ
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequantize_weight(const void* wq, int wbits, const float* w_scale, int64_t rows, int64_t K,
                                    int log2g, uint16_t* out, hipStream_t stream) {
  if (log2g == 8) {
    const hipError_t e = launch_dequantize_g256(wq, wbits, w_scale, rows, K, out, stream);
    if (e != hipErrorNotSupported) return e;
  }
  if (wbits == 4) return dispatch_dequant<true>(wq, w_scale, rows, K, log2g, out, stream);
  return dispatch_dequant<false>(wq, w_scale, rows, K, log2g, out, stream);
}

hipError_t launch_rotate_quant(const void* x, int in_dtype, int64_t rows, int64_t K, int log2g, int8_t* codes,
                               float* scale, hipStream_t stream) {
  if (in_dtype == IN_BF16 && log2g == 8) {
    const hipError_t e =
        launch_rotate_quant_g256(static_cast<const uint16_t*>(x), rows, K, codes, scale, stream);
    if (e != hipErrorNotSupported) return e;
  }
  if (in_dtype == IN_BF16 && (log2g == 4 || log2g == 0)) {
    const hipError_t e =
        launch_rotate_quant_small(static_cast<const uint16_t*>(x), rows, K, log2g, codes, scale, stream);
    if (e != hipErrorNotSupported) return e;
  }
  if (in_dtype == IN_BF16) return dispatch<IN_BF16, MODE_I8>(x, rows, K, log2g, codes, scale, nullptr, stream);
  return dispatch<IN_F32, MODE_I8>(x, rows, K, log2g, codes, scale, nullptr, stream);
}

hipError_t launch_rmsnorm_rotate_quant(const uint16_t* x, const float* norm_w, float eps, int64_t rows, int64_t K,
                                       int log2g, int8_t* codes, float* scale, uint16_t* y_norm,
                                       hipStream_t stream) {
  if (log2g == 8) {
    const hipError_t e = launch_rmsnorm_rotate_quant_g256(x, norm_w, eps, rows, K, codes, scale, y_norm, stream);
    if (e != hipErrorNotSupported) return e;
  }
  return dispatch<IN_BF16, MODE_I8, true>(x, rows, K, log2g, codes, scale, nullptr, stream, norm_w, eps, y_norm);
}

hipError_t launch_quantize_weight_i4(const void* w, int in_dtype, int64_t rows, int64_t K, int log2g,
                                     uint8_t* wq4, float* scale, int32_t* clip_index, hipStream_t stream) {
  if (in_dtype == IN_BF16) return dispatch<IN_BF16, MODE_I4>(w, rows, K, log2g, wq4, scale, clip_index, stream);
  return dispatch<IN_F32, MODE_I4>(w, rows, K, log2g, wq4, scale, clip_index, stream);
}

}  // namespace convrot
