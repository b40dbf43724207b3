// Fast path of the activation rotate-and-quantize pass for group 256 (the
// group size of ConvRot int8 checkpoints: "MOSS-Image Qwen3.5-9B text encoder,
// INT8 (W8A8, ConvRot)", file table rows "Quantized" and "Matmul").
//
// One token row is held in the registers of TW wavefronts (TW = 1 for
// short rows, more for longer rows or few tokens); each lane owns C chunks
// of 16 consecutive bf16 values and a
// group of 256 values lives in 16 consecutive lanes (one DPP row).  No LDS
// and no barrier is needed when TW = 1.  A workgroup takes one group of
// tokens; a launch covers at most 2^30 groups (larger M takes several).
//
// Walsh-Hadamard transform of a group (unnormalised; the 1/16 is a power of
// two and is folded exactly into the scale):
//   - element-index bits 0..3: butterflies inside the lane's 16 registers;
//   - bits 4..7: butterflies between lanes, one v_fmac_f32_dpp per value and
//     stage.  The four lane pairings are XOR 1, 2, 7 and 8 (DPP quad_perm,
//     row_half_mirror, row_ror:8), a basis of GF(2)^4; lane i therefore loads
//     and stores chunk u(i) = i ^ (bit 2 of i ? 3 : 0) of its group, which
//     makes these pairings the standard Sylvester butterflies in u.  Every
//     lane computes v + c * partner with c = +-1 by lane, so the values carry
//     a known per-lane sign (-1)^popcount(u); it is applied for free in the
//     quantization (the sign is folded into the reciprocal and the scale).
//
// Quantization per element: scale = absmax / 127 (fp32, correctly rounded)
// and code = round_half_away(value / scale), taken as one fused multiply-add
// and a byte pick (code_rcp, code_bits in convrot_internal.h): the code is
// the low byte of fma(v, rb, 1.5 * 2^23) with rb = RN(1 / scale) raised by
// two units in the last place.  Exact ties round away from zero; a code
// differs from the definition only where the exact quotient lies within
// 2^-21 of a rounding boundary below it.  This takes 1.75 VALU instructions
// per value (the fma and 3/4 of a byte permute), against 6.75 for a
// correctly rounded quotient and rounding.  Scales below 2^-100 are lifted
// by 2^64 with their values first.
#include "convrot_internal.h"

#include <cstdint>
#include <cstdlib>
#include <mutex>

namespace convrot {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// v += c * v[partner lane] for 16 registers, one DPP stage.  The s_nop
// covers the DPP read-after-VALU-write hazard for values written just
// before the block; inside the block each register is read once.
#define CONVROT_DPP_STAGE(CTRL)                                                                        \
  asm volatile("s_nop 1\n\t"                                                                           \
               "v_fmac_f32_dpp %0, %0, %16 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"      \
               "v_fmac_f32_dpp %1, %1, %16 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"      \
               "v_fmac_f32_dpp %2, %2, %16 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"      \
               "v_fmac_f32_dpp %3, %3, %16 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"      \
               "v_fmac_f32_dpp %4, %4, %16 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"      \
               "v_fmac_f32_dpp %5, %5, %16 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"      \
               "v_fmac_f32_dpp %6, %6, %16 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"      \
               "v_fmac_f32_dpp %7, %7, %16 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"      \
               "v_fmac_f32_dpp %8, %8, %16 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"      \
               "v_fmac_f32_dpp %9, %9, %16 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"      \
               "v_fmac_f32_dpp %10, %10, %16 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"    \
               "v_fmac_f32_dpp %11, %11, %16 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"    \
               "v_fmac_f32_dpp %12, %12, %16 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"    \
               "v_fmac_f32_dpp %13, %13, %16 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"    \
               "v_fmac_f32_dpp %14, %14, %16 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"    \
               "v_fmac_f32_dpp %15, %15, %16 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1"        \
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]),   \
                 "+v"(v[7]), "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]),             \
                 "+v"(v[13]), "+v"(v[14]), "+v"(v[15])                                                  \
               : "v"(c))

__device__ __forceinline__ void stage_xor1(float (&v)[16], float c) { CONVROT_DPP_STAGE("quad_perm:[1,0,3,2]"); }
__device__ __forceinline__ void stage_xor2(float (&v)[16], float c) { CONVROT_DPP_STAGE("quad_perm:[2,3,0,1]"); }
__device__ __forceinline__ void stage_xor7(float (&v)[16], float c) { CONVROT_DPP_STAGE("row_half_mirror"); }
__device__ __forceinline__ void stage_xor8(float (&v)[16], float c) { CONVROT_DPP_STAGE("row_ror:8"); }
#undef CONVROT_DPP_STAGE

// Butterflies over element-index bits 1..3 inside one lane (bit 0 is done
// while unpacking the bf16 pairs).
__device__ __forceinline__ void fwht16_rest(float (&v)[16]) {
#pragma unroll
  for (int h = 2; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (!(i & h)) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
}

// m = max(m, |a|, |b|) in one instruction (the operands come out of the DPP
// asm blocks, so the compiler would otherwise add NaN-quieting moves).
__device__ __forceinline__ void max3_abs(float& m, float a, float b) {
  asm("v_max3_f32 %0, |%1|, |%2|, %0" : "+v"(m) : "v"(a), "v"(b));
}

// bf16 rounding (to nearest even) of v, as an fp32 value: one convert that
// puts v's bf16 in the high half of the word and +0 in the low half.
__device__ __forceinline__ float round_bf16(float v) { return __uint_as_float(pack_bf16x2(0.0f, v)); }

// One token per TW waves.  WALK (TW = 1 only): a workgroup of the resident
// grid walks the tokens, its wave w taking w + 4 * (blockIdx.x + i *
// gridDim.x) for i = 0, 1, ..., so set-up (the RMSNorm factors in LDS) is
// paid once per workgroup rather than once per four tokens.  The waves of a
// workgroup then run their loops independently: nothing after the set-up
// waits on a barrier.
template <int C, int TW, bool NORM, bool WALK = false>
__global__ __launch_bounds__(kThreads) void rotate_quant_g256_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                                     int K, int8_t* __restrict__ xq,
                                                                     float* __restrict__ x_scale,
                                                                     const float* __restrict__ norm_w, float eps,
                                                                     uint16_t* __restrict__ y_norm) {
  static_assert(TW == 1 || TW == 2 || TW == 4, "waves per token");
  static_assert(!WALK || TW == 1, "a walking wave holds whole tokens");
  constexpr int P = kWaves / TW;  // tokens per workgroup iteration
  __shared__ float red[kWaves];
  __shared__ double red_d[kWaves];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wt = wave % TW;  // this wave's index within its token
  const int g = lane & 15;
  // chunk of the group this lane loads and stores (see header)
  const int u = g ^ ((g & 4) ? 3 : 0);
  const int chunk_lane = (lane & ~15) + u;
  // per-stage partner coefficients (-1)^u_k and the final sign (-1)^popcount(u)
  const float c0 = (u & 1) ? -1.f : 1.f;
  const float c1 = (u & 2) ? -1.f : 1.f;
  const float c2 = (u & 4) ? -1.f : 1.f;
  const float c3 = (u & 8) ? -1.f : 1.f;
  const float sgn = c0 * c1 * c2 * c3;

  // element offset of chunk j of this lane inside a token row
  auto chunk_off = [&](int j) { return (j * (64 * TW) + wt * 64 + chunk_lane) * 16; };
  // A row of K = 256 * G values fills G of the 4 * C * TW group slots
  // (group of chunk j: (j * TW + wt) * 4 + lane / 16); the rest stay zero
  // and are neither loaded nor stored.  Uniform over a 16-lane group.
  const int nvalid = K >> 8;
  auto slot_ok = [&](int j) { return ((j * TW + wt) * 4 + (lane >> 4)) < nvalid; };
  // Every slot in use (the common widths: 16, 32, 48 and 64 groups): plain
  // loads, with no zero fill to keep for the masked case.
  const bool full = nvalid == 4 * C * TW;  // uniform

  auto load = [&](u32x4 (&raw)[C][2], int64_t tok) {
    if (tok < M) {
      const uint16_t* row = x + tok * K;
      if (full) {
#pragma unroll
        for (int j = 0; j < C; ++j) {
          const u32x4* p = reinterpret_cast<const u32x4*>(row + chunk_off(j));
          raw[j][0] = __builtin_nontemporal_load(p);
          raw[j][1] = __builtin_nontemporal_load(p + 1);
        }
        return;
      }
#pragma unroll
      for (int j = 0; j < C; ++j) {
        if (slot_ok(j)) {
          const u32x4* p = reinterpret_cast<const u32x4*>(row + chunk_off(j));
          raw[j][0] = __builtin_nontemporal_load(p);
          raw[j][1] = __builtin_nontemporal_load(p + 1);
        } else {
          raw[j][0] = u32x4{0u, 0u, 0u, 0u};
          raw[j][1] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };

  // RMSNorm: the factors 1 + w of the columns a lane owns are fixed across
  // tokens.  Up to 48 KB they are kept in LDS, where they cost no
  // occupancy: entry ((j * TW + t) * 4 + q) * 64 + l holds columns
  // [4q, 4q + 4) of chunk j of lane l of the token's wave t, so a wave's
  // 16-byte reads are consecutive.  The workgroup fills it together.
  // Larger rows (K = 16384) keep them in registers, as LDS would then
  // limit occupancy more than registers do.
  constexpr bool kW1Lds = NORM && C * TW * 4096 <= 49152;
  __shared__ float4 w1s[kW1Lds ? C * TW * 4 * 64 : 1];
  float w1r[NORM && !kW1Lds ? C : 1][16];
  if constexpr (kW1Lds) {
#pragma unroll
    for (int k = 0; k < C * TW; ++k) {
      const int e = k * kThreads + threadIdx.x;  // < C * TW * 256
      const int l = e & 63, q = (e >> 6) & 3, jt = e >> 8;
      const int lg = l & 15, lu = lg ^ ((lg & 4) ? 3 : 0);
      const int col = ((jt / TW) * (64 * TW) + (jt % TW) * 64 + (l & ~15) + lu) * 16 + 4 * q;
      const float4 f = col < K ? *reinterpret_cast<const float4*>(norm_w + col) : make_float4(0.f, 0.f, 0.f, 0.f);
      w1s[e] = make_float4(1.0f + f.x, 1.0f + f.y, 1.0f + f.z, 1.0f + f.w);
    }
    __syncthreads();
  } else if constexpr (NORM) {
#pragma unroll
    for (int j = 0; j < C; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 f = slot_ok(j) ? *reinterpret_cast<const float4*>(norm_w + chunk_off(j) + 4 * q)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
        w1r[j][4 * q + 0] = 1.0f + f.x;
        w1r[j][4 * q + 1] = 1.0f + f.y;
        w1r[j][4 * q + 2] = 1.0f + f.z;
        w1r[j][4 * q + 3] = 1.0f + f.w;
      }
  }

  // Normalise (NORM), rotate and quantize the token held in raw.
  auto process = [&](const u32x4 (&raw)[C][2], int64_t tok) {
    float v[C][16];
    if constexpr (NORM) {
      float f[C][16];  // the row as loaded
#pragma unroll
      for (int j = 0; j < C; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t w = raw[j][i >> 2][i & 3];
          f[j][2 * i] = __uint_as_float(w << 16);
          f[j][2 * i + 1] = __uint_as_float(w & 0xffff0000u);
        }
      // mean square in fp64 (each square of a bf16 value is exact there),
      // then y = bf16_rne((x * r) * (1 + w)) with r = 1 / sqrt(ms + eps)
      double ss = 0.0;
#pragma unroll
      for (int j = 0; j < C; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const double d = f[j][i];
          ss = __builtin_fma(d, d, ss);
        }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
      if constexpr (TW > 1) {
        if (lane == 0) red_d[wave] = ss;
        __syncthreads();
        const int first = (wave / TW) * TW;
        ss = red_d[first];
#pragma unroll
        for (int w2 = 1; w2 < TW; ++w2) ss += red_d[first + w2];
        __syncthreads();
      }
      const float ms = float(ss / double(K));
      const float r = 1.0f / sqrtf(ms + eps);
      // An index the compiler cannot see through, so the walking kernel
      // reads the factors from LDS for each token instead of holding all
      // of them in registers across its loop (16 per chunk).
      int wl = lane;
      if constexpr (WALK) asm volatile("" : "+v"(wl));
      const bool want_y = y_norm != nullptr && tok < M;
#pragma unroll
      for (int j = 0; j < C; ++j) {
        float y[16];  // the normalised values, rounded to bf16
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float w1[4];
          if constexpr (kW1Lds) {
            const float4 wf = w1s[((j * TW + wt) * 4 + q) * 64 + wl];
            w1[0] = wf.x, w1[1] = wf.y, w1[2] = wf.z, w1[3] = wf.w;
          } else {
#pragma unroll
            for (int h = 0; h < 4; ++h) w1[h] = w1r[j][4 * q + h];
          }
#pragma unroll
          for (int h = 0; h < 4; ++h) y[4 * q + h] = round_bf16((f[j][4 * q + h] * r) * w1[h]);
        }
        if (want_y && slot_ok(j)) {
          uint32_t p[8];  // the high halves of consecutive pairs
#pragma unroll
          for (int i = 0; i < 8; ++i)
            p[i] = __builtin_amdgcn_perm(__float_as_uint(y[2 * i + 1]), __float_as_uint(y[2 * i]), 0x07060302u);
          u32x4* dst = reinterpret_cast<u32x4*>(y_norm + tok * K + chunk_off(j));
          dst[0] = u32x4{p[0], p[1], p[2], p[3]};
          dst[1] = u32x4{p[4], p[5], p[6], p[7]};
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {  // the bit-0 butterfly
          v[j][2 * i] = y[2 * i] + y[2 * i + 1];
          v[j][2 * i + 1] = y[2 * i] - y[2 * i + 1];
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < C; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) {  // unpack a bf16 pair and do the bit-0 butterfly
          const uint32_t w = raw[j][i >> 2][i & 3];
          const float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xffff0000u);
          v[j][2 * i] = lo + hi;
          v[j][2 * i + 1] = lo - hi;
        }
    }

    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      fwht16_rest(v[j]);
      stage_xor1(v[j], c0);
      stage_xor2(v[j], c1);
      stage_xor7(v[j], c2);
      stage_xor8(v[j], c3);
#pragma unroll
      for (int i = 0; i < 16; i += 2) max3_abs(amax, v[j][i], v[j][i + 1]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if constexpr (TW > 1) {
      if (lane == 0) red[wave] = amax;
      __syncthreads();
      const int first = (wave / TW) * TW;
#pragma unroll
      for (int w2 = 0; w2 < TW; ++w2) amax = fmaxf(amax, red[first + w2]);
      __syncthreads();
    }
    float s = amax / 127.0f;  // scale of the unnormalised values
    float out_mul = 0.0625f;  // 1/sqrt(256), exact
    if (s < kTinyScale && s > 0.f) {
      // Tiny row (the branch is uniform: amax is the token's).  Lift values
      // and scale by 2^64 so 1/s stays finite and the quotient identity
      // holds; for a normal s the quotients are exactly the unlifted ones.
#pragma unroll
      for (int j = 0; j < C; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) v[j][i] *= 0x1p64f;
      s = (amax * 0x1p64f) / 127.0f;
      out_mul = 0x1p-68f;
    }
    const float dr = sgn * code_rcp(s);  // the lane's sign folded into the reciprocal
    if (tok < M) {
      if (wt == 0 && lane == 0) x_scale[tok] = s * out_mul;
      int8_t* out = xq + tok * K;
#pragma unroll
      for (int j = 0; j < C; ++j) {
        if (!slot_ok(j)) continue;  // past the row's end
        uint32_t q[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) q[i] = code_bits(v[j][i], dr);
        const u32x4 o = {pack4_lo(q[0], q[1], q[2], q[3]), pack4_lo(q[4], q[5], q[6], q[7]),
                         pack4_lo(q[8], q[9], q[10], q[11]), pack4_lo(q[12], q[13], q[14], q[15])};
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(out + chunk_off(j)));
      }
    }
  };

  u32x4 raw[C][2];
  if constexpr (WALK) {
    const int64_t stride = int64_t(gridDim.x) * kWaves;
    for (int64_t tok = int64_t(blockIdx.x) * kWaves + wave; tok < M; tok += stride) {  // uniform per wave
      load(raw, tok);
      process(raw, tok);
    }
  } else {
    const int64_t tok = int64_t(blockIdx.x) * P + wave / TW;
    load(raw, tok);
    process(raw, tok);
  }
}

template <int C, int TW, bool NORM>
hipError_t launch(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, float* xs, const float* norm_w, float eps,
                  uint16_t* y_norm, hipStream_t stream) {
  constexpr int P = kWaves / TW;
  // One workgroup per group of tokens: the dispatcher then balances the
  // tail by itself (a persistent grid of 2048 workgroups left a partial
  // last round: kernel trace at M 8704, K 12288: 66.6 -> 61.8 us, M 30000,
  // K 4096: 80.0 -> 74.8 us).  Without the per-wave token loop the kernel
  // needs 30 fewer registers at C = 4 (same-box A/B, M 8704: K 8192
  // 44.5 -> 40.5 us, K 12288 60.0 -> 57.5 us, K 4096 23.8 -> 23.4 us).
  const int64_t rows_per_launch = (int64_t(1) << 30) * P;
  for (int64_t m0 = 0; m0 < M; m0 += rows_per_launch) {
    const int64_t mc = M - m0 < rows_per_launch ? M - m0 : rows_per_launch;
    hipLaunchKernelGGL((rotate_quant_g256_kernel<C, TW, NORM>), dim3(unsigned((mc + P - 1) / P)), dim3(kThreads), 0,
                       stream, x + m0 * K, mc, int(K), xq + m0 * K, xs + m0, norm_w, eps,
                       y_norm ? y_norm + m0 * K : nullptr);
    if (const hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Workgroups of the walking fused-norm kernel that the current device runs
// at once (compute units x resident workgroups per unit).  A read-only fact
// of the device, worked out once per device (the first call with that
// device current; later calls from any host thread only read it); 0 on
// error.
template <int C>
int walk_slots() {
  constexpr int kDevices = 64;
  static std::once_flag once[kDevices];
  static int slots[kDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  auto query = [](int d) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(rotate_quant_g256_kernel<C, 1, true, true>), kThreads, 0) !=
        hipSuccess)
      return 0;
    return cus * (per_cu > 0 ? per_cu : 1);
  };
  if (dev >= kDevices) return query(dev);  // not memoised
  std::call_once(once[dev], [&] { slots[dev] = query(dev); });
  return slots[dev];
}

// The fused norm pass with one wave per token and no bf16 norm output, on
// the resident grid: each workgroup fills the norm factors once and then
// walks its tokens (same-box A/B, M 8704, K 4096: 26.7 -> 25.0 us, 26.0 ->
// 23.8 us on another box; M 20000: 54.6 -> 51.2 us).  With the norm output
// the walk measured slower at M 20000 (81.2 -> 85.1 us), so that case keeps
// one workgroup per four tokens.
template <int C>
hipError_t launch_walk(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, float* xs, const float* norm_w,
                       float eps, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  const int slots = walk_slots<C>();
  if (slots <= 0) return hipErrorInvalidValue;
  const int64_t need = (M + kWaves - 1) / kWaves;
  const unsigned grid = unsigned(need < slots ? need : slots);
  hipLaunchKernelGGL((rotate_quant_g256_kernel<C, 1, true, true>), dim3(grid), dim3(kThreads), 0, stream, x, M,
                     int(K), xq, xs, norm_w, eps, nullptr);
  return hipGetLastError();
}

template <int C, int TW, bool NORM>
hipError_t launch_split(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, float* xs, const float* norm_w,
                        float eps, uint16_t* y_norm, hipStream_t stream) {
  // Few tokens (under four waves per SIMD with one wave per token): split
  // each token over twice the waves, so the waves are shorter and more of
  // them hide each other's latency (kernel trace, K 4096: M 512 5.96 ->
  // 4.20 us, M 2048 8.40 -> 7.96 us; M 8704 is 4 % faster unsplit).
  if constexpr (C % 2 == 0 && TW < 4) {
    if (M < 4096) return launch<C / 2, 2 * TW, NORM>(x, M, K, xq, xs, norm_w, eps, y_norm, stream);
  }
  if constexpr (NORM && TW == 1) {
    if (M >= 4096 && y_norm == nullptr) return launch_walk<C>(x, M, K, xq, xs, norm_w, eps, stream);
  }
  return launch<C, TW, NORM>(x, M, K, xq, xs, norm_w, eps, y_norm, stream);
}

// Any K = 256 * G up to 16384: the G groups take 4 * C * TW slots, with
// one wave per token up to 16 groups, two up to 32, four up to 64.
template <bool NORM>
hipError_t launch_k(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, float* xs, const float* norm_w, float eps,
                    uint16_t* y_norm, hipStream_t stream) {
  if (K % 256 != 0 || K > 16384) return hipErrorNotSupported;
  const int G = int(K / 256);
  if (G <= 4) return launch_split<1, 1, NORM>(x, M, K, xq, xs, norm_w, eps, y_norm, stream);
  if (G <= 8) return launch_split<2, 1, NORM>(x, M, K, xq, xs, norm_w, eps, y_norm, stream);
  if (G <= 12) return launch_split<3, 1, NORM>(x, M, K, xq, xs, norm_w, eps, y_norm, stream);
  if (G <= 16) {
    // The plain pass at K 4096 runs best with a token over several waves:
    // four below 4096 tokens, two above (sweep of every (C, TW) at K 4096:
    // M 2048 8.01 -> 7.55 us, M 8704 23.0 -> 21.7 us).  The fused norm pass
    // is best as before.
    if constexpr (!NORM) {
      if (M < 4096) return launch<1, 4, false>(x, M, K, xq, xs, norm_w, eps, y_norm, stream);
      return launch<2, 2, false>(x, M, K, xq, xs, norm_w, eps, y_norm, stream);
    }
    return launch_split<4, 1, NORM>(x, M, K, xq, xs, norm_w, eps, y_norm, stream);
  }
  if (G <= 24) return launch_split<3, 2, NORM>(x, M, K, xq, xs, norm_w, eps, y_norm, stream);
  if (G <= 32) return launch_split<4, 2, NORM>(x, M, K, xq, xs, norm_w, eps, y_norm, stream);
  if (G <= 48) return launch_split<3, 4, NORM>(x, M, K, xq, xs, norm_w, eps, y_norm, stream);
  return launch_split<4, 4, NORM>(x, M, K, xq, xs, norm_w, eps, y_norm, stream);
}

// ---------------------------------------------------------------------------
// Small groups (G = 16, the group size of ConvRot vision layers whose widths,
// 1152 and 4304, are not multiples of 256: "qwen3vl_8b_int8_convrot", "Layer
// and group selection"; and G = 1, plain row-wise int8).  A group is one
// lane's chunk of 16 values, so the transform never leaves the lane: the
// bit-0 butterfly fused with the unpack, then bits 1..3.  A row spreads over
// L = 64 / RPW lanes of a wave (RPW rows per wave), lane l taking chunks
// l, l + L, ..., so any multiple of 16 fits; RPW is chosen per K to waste
// the fewest chunk slots.  Quantization is the group-256 kernel's (one fma
// and a byte pick, ties away from zero, tiny-row lift); 1/sqrt(16) = 1/4 is
// folded into the scale.
template <int G, int C, int RPW>
__global__ __launch_bounds__(kThreads) void rotate_quant_small_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                                      int K, int8_t* __restrict__ xq,
                                                                      float* __restrict__ x_scale) {
  static_assert(G == 1 || G == 16, "group");
  constexpr int L = 64 / RPW;               // lanes per row
  constexpr int P = kWaves * RPW;           // rows per workgroup iteration
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l = lane % L;
  const int slot = wave * RPW + lane / L;   // this lane's row within the iteration
  const int nchunks = K / 16;

  u32x4 raw[C][2];
  auto load = [&](int64_t tok) {
    if (tok < M) {
      const uint16_t* row = x + tok * K;
#pragma unroll
      for (int j = 0; j < C; ++j) {
        const int c = l + L * j;
        if (c < nchunks) {
          const u32x4* p = reinterpret_cast<const u32x4*>(row + c * 16);
          raw[j][0] = __builtin_nontemporal_load(p);
          raw[j][1] = __builtin_nontemporal_load(p + 1);
        } else {
          raw[j][0] = u32x4{0u, 0u, 0u, 0u};
          raw[j][1] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };

  {
    const int64_t tok = int64_t(blockIdx.x) * P + slot;
    load(tok);
    float v[C][16];
#pragma unroll
    for (int j = 0; j < C; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t w = raw[j][i / 4][i % 4];
        const float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xffff0000u);
        v[j][2 * i] = G == 16 ? lo + hi : lo;
        v[j][2 * i + 1] = G == 16 ? lo - hi : hi;
      }

    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      if constexpr (G == 16) fwht16_rest(v[j]);
#pragma unroll
      for (int i = 0; i < 16; i += 2) max3_abs(amax, v[j][i], v[j][i + 1]);
    }
#pragma unroll
    for (int off = L / 2; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    float s = amax / 127.0f;                      // scale of the unnormalised values
    float out_mul = G == 16 ? 0.25f : 1.0f;       // 1/sqrt(G), exact
    if (s < kTinyScale && s > 0.f) {
      // Tiny row (uniform over the row's lanes): lift by 2^64 as in the
      // group-256 kernel so 1/s stays finite and the quotient identity holds.
#pragma unroll
      for (int j = 0; j < C; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) v[j][i] *= 0x1p64f;
      s = (amax * 0x1p64f) / 127.0f;
      out_mul *= 0x1p-64f;
    }
    const float rb = code_rcp(s);
    if (tok < M) {
      if (l == 0) x_scale[tok] = s * out_mul;
      int8_t* out = xq + tok * K;
#pragma unroll
      for (int j = 0; j < C; ++j) {
        const int c = l + L * j;
        if (c < nchunks) {
          uint32_t q[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) q[i] = code_bits(v[j][i], rb);
          const u32x4 o = {pack4_lo(q[0], q[1], q[2], q[3]), pack4_lo(q[4], q[5], q[6], q[7]),
                           pack4_lo(q[8], q[9], q[10], q[11]), pack4_lo(q[12], q[13], q[14], q[15])};
          __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(out + c * 16));
        }
      }
    }
  }
}

template <int G, int C, int RPW>
hipError_t launch_small(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, float* xs, hipStream_t stream) {
  constexpr int P = kWaves * RPW;
  const int64_t rows_per_launch = (int64_t(1) << 30) * P;  // one workgroup per group, as above
  for (int64_t m0 = 0; m0 < M; m0 += rows_per_launch) {
    const int64_t mc = M - m0 < rows_per_launch ? M - m0 : rows_per_launch;
    hipLaunchKernelGGL((rotate_quant_small_kernel<G, C, RPW>), dim3(unsigned((mc + P - 1) / P)), dim3(kThreads), 0,
                       stream, x + m0 * K, mc, int(K), xq + m0 * K, xs + m0);
    if (const hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Rows per wave and chunks per lane for K: the fewest empty chunk slots
// (ties to more lanes per row), up to 8 chunks per lane (K <= 8192).  The
// kernel times of the three choices differ by at most ~25 % (kernel trace,
// K 1152 and 4304, M 1024 to 16384).
template <int G>
hipError_t launch_small_k(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, float* xs, hipStream_t stream) {
  const int64_t nch = K / 16;
  int best_rpw = 0, best_c = 0;
  int64_t best_waste = 0;
  for (int rpw = 1; rpw <= 4; rpw *= 2) {
    const int64_t lanes = 64 / rpw, c = (nch + lanes - 1) / lanes;
    if (c > 8) continue;
    const int64_t waste = (c * lanes - nch) * rpw;  // empty chunk slots per wave
    if (best_rpw == 0 || waste < best_waste) {
      best_waste = waste;
      best_rpw = rpw;
      best_c = int(c);
    }
  }
  if (best_rpw == 0) return hipErrorNotSupported;
  // Few rows: fewer rows per wave gives more, shorter waves (measured at
  // K 1152: M 1024 3.9 against 5.0 us, M 4096 6.0 against 6.2 us); keep at
  // least two waves per SIMD before packing rows.
  while (best_rpw > 1 && M / best_rpw < 2048) {
    const int rpw = best_rpw / 2;
    const int64_t lanes = 64 / rpw, c = (nch + lanes - 1) / lanes;
    if (c > 8) break;
    best_rpw = rpw;
    best_c = int(c);
  }
#ifdef CONVROT_TUNING
  // Tuning builds only: CONVROT_RQ_SMALL_RPW=<1|2|4> forces the rows per wave
  // when it fits, for sweeps (every choice gives identical results).
  static const int forced_rpw = [] {
    const char* e = getenv("CONVROT_RQ_SMALL_RPW");
    return e ? atoi(e) : 0;
  }();
  if (forced_rpw == 1 || forced_rpw == 2 || forced_rpw == 4) {
    const int64_t lanes = 64 / forced_rpw, c = (nch + lanes - 1) / lanes;
    if (c <= 8) {
      best_rpw = forced_rpw;
      best_c = int(c);
    }
  }
#endif
#define CONVROT_SMALL(RPW_)                                                        \
  switch (best_c) {                                                                \
    case 1: return launch_small<G, 1, RPW_>(x, M, K, xq, xs, stream);              \
    case 2: return launch_small<G, 2, RPW_>(x, M, K, xq, xs, stream);              \
    case 3: return launch_small<G, 3, RPW_>(x, M, K, xq, xs, stream);              \
    case 4: return launch_small<G, 4, RPW_>(x, M, K, xq, xs, stream);              \
    case 5: return launch_small<G, 5, RPW_>(x, M, K, xq, xs, stream);              \
    case 6: return launch_small<G, 6, RPW_>(x, M, K, xq, xs, stream);              \
    case 7: return launch_small<G, 7, RPW_>(x, M, K, xq, xs, stream);              \
    default: return launch_small<G, 8, RPW_>(x, M, K, xq, xs, stream);             \
  }
  if (best_rpw == 1) CONVROT_SMALL(1)
  if (best_rpw == 2) CONVROT_SMALL(2)
  CONVROT_SMALL(4)
#undef CONVROT_SMALL
}

// ---------------------------------------------------------------------------
// Weight-only path, group 256: undo the rotation of stored codes.  A group
// of 256 codes is one DPP row of 16 lanes, lane i holding chunk u(i) as in
// the rotate-quant kernel, so the same butterflies give the transform t of
// the codes (integers below 2^15 in magnitude, exact in fp32 in any order)
// with the lane's known sign; the value s_w * (t * 2^-4) is rounded to bf16.
// t * 2^-4 is formed as fma(v, sign * 2^-4, +0), exact, which also turns a
// zero t into +0 as the plain transform gives it (a bare sign flip would
// leave -0 there); the scale is applied as fma(s, ., +0) for the same
// reason (a zero scale times a negative t would otherwise give -0, where
// the dense product sums to +0).  Groups never straddle rows (K is a
// multiple of 256), so the matrix is walked as a flat list of groups.
// ("MOSS-Image Qwen3.5-9B text encoder, INT8 (W8A8, ConvRot)", file table
// row "Matmul": its weight-only mode expands the codes into a bf16 weight.)
template <bool W4>
__global__ __launch_bounds__(kThreads) void dequant_g256_kernel(const void* __restrict__ wq,
                                                                const float* __restrict__ w_scale, int64_t ngroups,
                                                                int groups_per_row, uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int g = lane & 15;
  const int u = g ^ ((g & 4) ? 3 : 0);
  const float c0 = (u & 1) ? -1.f : 1.f;
  const float c1 = (u & 2) ? -1.f : 1.f;
  const float c2 = (u & 4) ? -1.f : 1.f;
  const float c3 = (u & 8) ? -1.f : 1.f;
  const float sgn = c0 * c1 * c2 * c3;
  // One group per 16 lanes; uniform over a DPP row, so a row that is past
  // the end leaves together and the others' row-local DPP is unaffected.
  const int64_t grp = (int64_t(blockIdx.x) * kThreads + threadIdx.x) >> 4;
  if (grp >= ngroups) return;
  float v[16];
  if constexpr (W4) {
    const uint2 b = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(wq) + grp * 128 + u * 8);
    const uint32_t w[2] = {b.x, b.y};
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // low nibble first; the bit-0 butterfly on each pair
      const uint32_t byte = w[i / 4] >> (8 * (i % 4));
      const float lo = float(int((byte & 0xfu) ^ 8u) - 8), hi = float(int(((byte >> 4) & 0xfu) ^ 8u) - 8);
      v[2 * i] = lo + hi;
      v[2 * i + 1] = lo - hi;
    }
  } else {
    const uint4 b = *reinterpret_cast<const uint4*>(static_cast<const int8_t*>(wq) + grp * 256 + u * 16);
    const uint32_t w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float lo = float(int8_t(w[i / 2] >> (16 * (i % 2)))), hi = float(int8_t(w[i / 2] >> (16 * (i % 2) + 8)));
      v[2 * i] = lo + hi;
      v[2 * i + 1] = lo - hi;
    }
  }
  fwht16_rest(v);
  stage_xor1(v, c0);
  stage_xor2(v, c1);
  stage_xor7(v, c2);
  stage_xor8(v, c3);
  const float s = w_scale[grp / groups_per_row];
  const float sg = sgn * 0.0625f;
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    o[i] = pack_bf16x2(__builtin_fmaf(s, __builtin_fmaf(v[2 * i], sg, 0.0f), 0.0f),
                       __builtin_fmaf(s, __builtin_fmaf(v[2 * i + 1], sg, 0.0f), 0.0f));
  u32x4* dst = reinterpret_cast<u32x4*>(out + grp * 256 + u * 16);
  dst[0] = u32x4{o[0], o[1], o[2], o[3]};
  dst[1] = u32x4{o[4], o[5], o[6], o[7]};
}

}  // namespace

// Group 16 or 1 (log2g 4 or 0), bf16 activations, K <= 8192; otherwise
// hipErrorNotSupported without launching.
hipError_t launch_rotate_quant_small(const uint16_t* x, int64_t M, int64_t K, int log2g, int8_t* xq, float* xs,
                                     hipStream_t stream) {
  if (log2g == 4) return launch_small_k<16>(x, M, K, xq, xs, stream);
  if (log2g == 0) return launch_small_k<1>(x, M, K, xq, xs, stream);
  return hipErrorNotSupported;
}

// Return hipErrorNotSupported (without launching) for shapes this path does
// not cover; the caller then uses the general kernel.
hipError_t launch_rotate_quant_g256(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, float* xs,
                                    hipStream_t stream) {
  return launch_k<false>(x, M, K, xq, xs, nullptr, 0.f, nullptr, stream);
}

// Group 256 (any K that is a multiple of 256); hipErrorNotSupported
// without launching otherwise.
hipError_t launch_dequantize_g256(const void* wq, int wbits, const float* w_scale, int64_t rows, int64_t K,
                                  uint16_t* out, hipStream_t stream) {
  if (K % 256 != 0 || K / 256 > INT32_MAX) return hipErrorNotSupported;
  const int64_t ngroups = rows * (K / 256);
  const int64_t blocks = (ngroups * 16 + kThreads - 1) / kThreads;
  if (blocks > INT32_MAX) return hipErrorNotSupported;
  if (wbits == 4)
    hipLaunchKernelGGL(dequant_g256_kernel<true>, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, wq, w_scale,
                       ngroups, int(K / 256), out);
  else
    hipLaunchKernelGGL(dequant_g256_kernel<false>, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, wq, w_scale,
                       ngroups, int(K / 256), out);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_rotate_quant_g256(const uint16_t* x, const float* norm_w, float eps, int64_t M,
                                            int64_t K, int8_t* xq, float* xs, uint16_t* y_norm,
                                            hipStream_t stream) {
  return launch_k<true>(x, M, K, xq, xs, norm_w, eps, y_norm, stream);
}

}  // namespace convrot
