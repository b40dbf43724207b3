// int8 x int8 -> int32 GEMM on CDNA4 matrix cores with a fused dequant
// epilogue to bf16 (the matmul of the ConvRot W8A8 linear: "MOSS-Image
// Qwen3.5-9B text encoder, INT8 (W8A8, ConvRot)", intro and file table row
// "Matmul"; the int4-weight variant reads two signed nibbles per byte,
// "MossInt4", "Format").
//
//   acc[m][n] = sum_k xq[m][k] * wq[n][k]           (both operands K-major)
//   y[m][n]   = bf16_rne(((float)acc * x_scale[m]) * w_scale[n])
//
// Tiling: a 256-thread workgroup (4 waves, 2 x 2) computes a BM x BN output
// tile; each wave owns a (BM/2) x (BN/2) sub-tile made of 32x32 blocks, each
// accumulated by v_mfma_i32_32x32x32_i8.  K advances in steps of BK = 128
// bytes through two LDS buffers (load of step s+1 overlaps the MFMAs of step
// s; one barrier per step).  LDS rows are 128 bytes; 16-byte chunk c of row r
// is stored at chunk c ^ h(r), h(r) = (r & 7) ^ ((r >> 3) & 1), so that the
// 16-byte operand reads of 8 or 16 consecutive rows hit distinct banks.
//
// int4 weights are unpacked while being staged into LDS: a nibble q becomes
// the byte 16*q (a mask, no shifts), so the accumulator holds 16*acc exactly
// and is shifted back by 4 before the epilogue.
#include "convrot_internal.h"

namespace convrot {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int BK = 128;

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// 16 packed bytes (32 nibbles, k = 0..31) -> two 16-byte chunks of 16*q bytes
// in natural k order.
__device__ __forceinline__ void unpack_nibbles(uint4 p, uint4& c0, uint4& c1) {
  uint32_t w[4] = {p.x, p.y, p.z, p.w};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t lo = (w[i] << 4) & 0xf0f0f0f0u;  // even k, times 16
    uint32_t hi = w[i] & 0xf0f0f0f0u;          // odd k, times 16
    o[2 * i] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    o[2 * i + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
  }
  c0 = make_uint4(o[0], o[1], o[2], o[3]);
  c1 = make_uint4(o[4], o[5], o[6], o[7]);
}

template <int BM, int BN, bool W4>
__global__ __launch_bounds__(kThreads) void gemm_i8_kernel(const int8_t* __restrict__ A,
                                                           const float* __restrict__ sa,
                                                           const uint8_t* __restrict__ B,
                                                           const float* __restrict__ sb, int M, int N, int K,
                                                           int tiles_n, int32_t* __restrict__ acc_out,
                                                           uint16_t* __restrict__ y) {
  constexpr int WM = BM / 2, WN = BN / 2;  // wave tile
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int A_CHUNKS = BM * BK / 16;
  constexpr int B_CHUNKS = BN * BK / 16;
  constexpr int A_PER_T = A_CHUNKS / kThreads;
  constexpr int B_PER_T = W4 ? (BN * BK / 32) / kThreads : B_CHUNKS / kThreads;
  static_assert(A_PER_T >= 1 && B_PER_T >= 1, "tile too small for the thread count");

  __shared__ __attribute__((aligned(16))) int8_t lds[2][(BM + BN) * BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tile_m = blockIdx.x / tiles_n;
  const int tile_n = blockIdx.x % tiles_n;
  const int m0 = tile_m * BM, n0 = tile_n * BN;
  const int64_t Kb = W4 ? K / 2 : K;  // bytes per weight row

  uint4 ra[A_PER_T];
  uint4 rb[B_PER_T];

  auto load_global = [&](int k0) {
#pragma unroll
    for (int j = 0; j < A_PER_T; ++j) {
      const int id = tid + j * kThreads;
      const int r = id / (BK / 16), c = id % (BK / 16);
      const int gm = m0 + r, gk = k0 + c * 16;
      ra[j] = (gm < M && gk < K) ? *reinterpret_cast<const uint4*>(A + int64_t(gm) * K + gk)
                                 : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < B_PER_T; ++j) {
      const int id = tid + j * kThreads;
      if constexpr (W4) {
        const int r = id / (BK / 32), pc = id % (BK / 32);
        const int gn = n0 + r, gk = k0 + pc * 32;
        rb[j] = (gn < N && gk < K) ? *reinterpret_cast<const uint4*>(B + int64_t(gn) * Kb + gk / 2)
                                   : make_uint4(0, 0, 0, 0);
      } else {
        const int r = id / (BK / 16), c = id % (BK / 16);
        const int gn = n0 + r, gk = k0 + c * 16;
        rb[j] = (gn < N && gk < K) ? *reinterpret_cast<const uint4*>(B + int64_t(gn) * Kb + gk)
                                   : make_uint4(0, 0, 0, 0);
      }
    }
  };

  auto store_lds = [&](int buf) {
    int8_t* sA = lds[buf];
    int8_t* sB = lds[buf] + BM * BK;
#pragma unroll
    for (int j = 0; j < A_PER_T; ++j) {
      const int id = tid + j * kThreads;
      const int r = id / (BK / 16), c = id % (BK / 16);
      *reinterpret_cast<uint4*>(sA + r * BK + 16 * (c ^ swz(r))) = ra[j];
    }
#pragma unroll
    for (int j = 0; j < B_PER_T; ++j) {
      const int id = tid + j * kThreads;
      if constexpr (W4) {
        const int r = id / (BK / 32), pc = id % (BK / 32);
        uint4 c0, c1;
        unpack_nibbles(rb[j], c0, c1);
        *reinterpret_cast<uint4*>(sB + r * BK + 16 * ((2 * pc) ^ swz(r))) = c0;
        *reinterpret_cast<uint4*>(sB + r * BK + 16 * ((2 * pc + 1) ^ swz(r))) = c1;
      } else {
        const int r = id / (BK / 16), c = id % (BK / 16);
        *reinterpret_cast<uint4*>(sB + r * BK + 16 * (c ^ swz(r))) = rb[j];
      }
    }
  };

  v16i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  const int ktiles = (K + BK - 1) / BK;
  load_global(0);
  store_lds(0);
  __syncthreads();

  for (int kt = 0; kt < ktiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ktiles) load_global((kt + 1) * BK);
    const int8_t* sA = lds[buf];
    const int8_t* sB = lds[buf] + BM * BK;
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      const int c = 2 * kk + (lane >> 5);
      v4i a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * WM + i * 32 + (lane & 31);
        a[i] = *reinterpret_cast<const v4i*>(sA + r * BK + 16 * (c ^ swz(r)));
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * WN + j * 32 + (lane & 31);
        b[j] = *reinterpret_cast<const v4i*>(sB + r * BK + 16 * (c ^ swz(r)));
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < ktiles) store_lds(buf ^ 1);
    __syncthreads();
  }

  // Epilogue.  32x32 block layout: lane holds column (lane & 31) and rows
  // 8*(e/4) + 4*(lane/32) + (e%4) for e = 0..15.
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + wn * WN + j * 32 + (lane & 31);
      const float swn = (y && n < N) ? sb[n] : 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * WM + i * 32 + 8 * (e / 4) + 4 * (lane >> 5) + (e % 4);
        if (m < M && n < N) {
          int a = acc[i][j][e];
          if constexpr (W4) a >>= 4;
          if (acc_out) acc_out[int64_t(m) * N + n] = a;
          if (y) y[int64_t(m) * N + n] = f32_to_bf16_rne((float(a) * sa[m]) * swn);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(const int8_t* xq, const float* x_scale, const void* wq, int wbits, const float* w_scale,
                       int64_t M, int64_t N, int64_t K, int32_t* acc_out, uint16_t* y, hipStream_t stream) {
  constexpr int BM = 128, BN = 128;
  const int tiles_m = int((M + BM - 1) / BM);
  const int tiles_n = int((N + BN - 1) / BN);
  const dim3 grid(unsigned(tiles_m) * unsigned(tiles_n));
  const uint8_t* B = static_cast<const uint8_t*>(wq);
  if (wbits == 4) {
    hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, true>), grid, dim3(kThreads), 0, stream, xq, x_scale, B, w_scale,
                       int(M), int(N), int(K), tiles_n, acc_out, y);
  } else {
    hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, false>), grid, dim3(kThreads), 0, stream, xq, x_scale, B, w_scale,
                       int(M), int(N), int(K), tiles_n, acc_out, y);
  }
  return hipGetLastError();
}

}  // namespace convrot
