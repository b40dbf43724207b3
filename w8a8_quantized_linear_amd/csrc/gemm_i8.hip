// int8 x int8 -> int32 GEMM on CDNA4 matrix cores with a fused dequant
// epilogue to bf16 (the matmul of the ConvRot W8A8 linear: "MOSS-Image
// Qwen3.5-9B text encoder, INT8 (W8A8, ConvRot)", intro and file table row
// "Matmul"; the int4-weight variant reads two signed nibbles per byte,
// "MossInt4", "Format").
//
//   acc[m][n] = sum_k xq[m][k] * wq[n][k]           (both operands K-major)
//   y[m][n]   = bf16_rne(((float)acc * x_scale[m]) * w_scale[n])
//
// Tiling.  A 256-thread workgroup (4 waves, 2 x 2) computes a BM x BN output
// tile (BM tokens x BN weight rows); each wave owns a (BM/2) x (BN/2)
// sub-tile of 32x32 blocks accumulated by v_mfma_i32_32x32x32_i8.  The MFMA's
// first operand is the weight tile and its second the token tile, so a lane's
// 16 accumulators of a block cover one token and four runs of four
// consecutive weight rows; the epilogue regroups them through LDS into
// 16-byte row-contiguous bf16 stores.
//
// Pipeline.  K advances 64 at a time through a ring of 4 LDS stages filled
// by buffer_load_dwordx4 ... lds (global -> LDS without registers; each wave
// instruction moves a 1 KB block).  Rows past M / N and the K tail read as
// zero through the buffer descriptor's range check.  A step has two phases
// split by one workgroup barrier:
//   phase 1: slice-0 MFMAs (K 0..31 of the step), interleaved with the
//            LDS reads of slice 1 and the token-tile loads of stage kt+3;
//   wait until stage kt+1 has landed (vmcnt), barrier;
//   phase 2: slice-1 MFMAs, interleaved with the weight-tile loads of
//            stage kt+4 (into the buffer just consumed) and the LDS reads of
//            the next step's slice 0.
// Loads and LDS reads are spread one per MFMA: the load path moves about
// 64 B/clk per CU and a wave stalled behind a burst of loads would let the
// matrix pipe drain within one MFMA.  The step count is padded to a multiple
// of 4 and the body has no conditionals (steps past the end of K read zeros),
// so the compiler's count of outstanding loads stays exact.
//
// LDS rows are 64 bytes (4 chunks of 16 B); chunk c of row r is stored at
// chunk c ^ h(r), h(r) = ((r >> 2) ^ (r >> 3)) & 3.  Packed int4 weight rows
// are 32 bytes (2 chunks), swizzled by ((r >> 2) ^ (r >> 3)) & 1.  Both were
// chosen by measuring ds_read_b128 throughput for these exact fragment
// access patterns on gfx950 (about 240 B/clk per CU, against about 140 for
// swizzles that leave two-way bank conflicts).
//
// int4 weights: a lane reads the 16 packed bytes covering both 32-wide K
// slices of the step and unpacks them in registers; a nibble q becomes the
// byte 16*q (masks and byte permutes), so the accumulator holds 16*acc exactly
// and is shifted back by 4 before the epilogue.  For this the K order inside
// a step is permuted identically for both operands (lane half h, slice s
// takes k = 32h + 16s .. +16), which leaves the dot products unchanged.
//
// Tiles are assigned so that each of the 8 XCDs (workgroups are dispatched to
// them round-robin) works on a contiguous block of tiles that share weight
// and token rows in its L2.
#include "convrot_internal.h"

#include <cstdio>
#include <cstdlib>
#include <type_traits>

namespace convrot {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kThreads = 256;
constexpr int kStages = 4;
constexpr int BK = 64;
constexpr unsigned kOOB = 0x7ffffff0u;  // buffer offset beyond every range: reads as zero
constexpr int kBufFlags = 0x00020000;   // raw buffer descriptor word 3 (gfx9 family)

__device__ __forceinline__ int swz64(int r) { return ((r >> 2) ^ (r >> 3)) & 3; }
__device__ __forceinline__ int swz32(int r) { return ((r >> 2) ^ (r >> 3)) & 1; }

// Two fp32 -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// 4 packed bytes (8 nibbles, k = 0..7) -> 8 bytes of 16*q in natural k order.
__device__ __forceinline__ void unpack4(uint32_t w, uint32_t& o0, uint32_t& o1) {
  const uint32_t lo = (w << 4) & 0xf0f0f0f0u;  // even k, times 16
  const uint32_t hi = w & 0xf0f0f0f0u;          // odd k, times 16
  o0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  o1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

// s_waitcnt vmcnt(n), other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | (0x7 << 4) | (0xf << 8) | ((N >> 4) << 14));
}

// Scheduling pattern for one phase: NM MFMAs; the ND LDS reads go one per
// MFMA from the start of the phase (so they have completed by the wait that
// ends it), the NV buffer loads are spread evenly over the whole phase (so
// the load path never sees a burst); a full scheduling barrier closes it.
template <int NM, int NV, int ND>
__device__ __forceinline__ void interleave_phase() {
  int nv = 0;
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i < ND) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    const int v_due = ((i + 1) * NV) / NM;  // loads due after MFMA i
    if (nv < v_due) {
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      ++nv;
    }
  }
  for (int i = NM; i < ND; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  for (; nv < NV; ++nv) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  __builtin_amdgcn_sched_barrier(0);
}

template <int BM, int BN, bool W4>
struct Cfg {
  static constexpr int WM = BM / 2, WN = BN / 2;    // wave extent: tokens, weight rows
  static constexpr int TI = WN / 32, TJ = WM / 32;  // 32x32 blocks along n and m
  static constexpr int WROW = W4 ? 32 : 64;         // weight bytes per row per stage
  static constexpr int W_BYTES = BN * WROW;
  static constexpr int X_BYTES = BM * 64;
  static constexpr int W_LOADS = W_BYTES / 4096;    // 1 KB per wave instruction, 4 waves
  static constexpr int X_LOADS = X_BYTES / 4096;
  static constexpr int LOADS = W_LOADS + X_LOADS;   // per wave per stage
  static_assert(W_LOADS * 4096 == W_BYTES && X_LOADS * 4096 == X_BYTES, "tile must split into 4 KB");
  static_assert(3 * LOADS < 64, "vmcnt budget");
};

template <int BM, int BN, bool W4>
__global__ __launch_bounds__(kThreads, 1) void gemm_i8_kernel(const int8_t* __restrict__ X,
                                                              const float* __restrict__ sx,
                                                              const uint8_t* __restrict__ W,
                                                              const float* __restrict__ sw, int M, int N, int K,
                                                              int tiles_m, int tiles_n,
                                                              int32_t* __restrict__ acc_out,
                                                              uint16_t* __restrict__ y) {
  using C = Cfg<BM, BN, W4>;
  constexpr int WM = C::WM, WN = C::WN, TI = C::TI, TJ = C::TJ, L = C::LOADS;
  __shared__ __attribute__((aligned(1024))) int8_t sW0[C::W_BYTES], sW1[C::W_BYTES], sW2[C::W_BYTES],
      sW3[C::W_BYTES];
  __shared__ __attribute__((aligned(1024))) int8_t sX0[C::X_BYTES], sX1[C::X_BYTES], sX2[C::X_BYTES],
      sX3[C::X_BYTES];
  int8_t* const sWs[kStages] = {sW0, sW1, sW2, sW3};
  int8_t* const sXs[kStages] = {sX0, sX1, sX2, sX3};

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int row = lane & 31, half = lane >> 5;

  // XCD-aware tile order: block b runs on XCD b % 8; XCD x takes the x-th
  // contiguous slice of tiles (token tiles vary fastest).
  const int T = tiles_m * tiles_n;
  int t = blockIdx.x;
  if ((T & 7) == 0) t = (t & 7) * (T >> 3) + (t >> 3);
  const int tile_m = t % tiles_m, tile_n = t / tiles_m;
  const int m0 = tile_m * BM, n0 = tile_n * BN;
  const int Kb = W4 ? K / 2 : K;  // bytes per weight row

  // Buffer descriptors over this tile's rows only; rows past M / N fall
  // outside num_records and read as zero.
  const int rows_x = min(BM, M - m0), rows_w = min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t rsx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(X + int64_t(m0) * K), short(0), rows_x * K, kBufFlags);
  const __amdgpu_buffer_rsrc_t rsw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(W + int64_t(n0) * Kb), short(0), rows_w * Kb, kBufFlags);

  // Per-lane byte offsets (at k0 = 0) of this wave's load blocks, and the k
  // each lane's chunk starts at.  Lane i's chunk lands at byte 16 i of the
  // block, so the swizzle is applied through the choice of source chunk.
  unsigned offw[C::W_LOADS], offx[C::X_LOADS];
  int kw[C::W_LOADS], kx[C::X_LOADS];
#pragma unroll
  for (int j = 0; j < C::W_LOADS; ++j) {
    const int b = wave * C::W_LOADS + j;
    if constexpr (W4) {
      const int r = b * 32 + (lane >> 1);
      const int h = (lane & 1) ^ swz32(r);
      kw[j] = 32 * h;
      offw[j] = unsigned(r * Kb + 16 * h);
    } else {
      const int r = b * 16 + (lane >> 2);
      const int c = (lane & 3) ^ swz64(r);
      kw[j] = 16 * c;
      offw[j] = unsigned(r * Kb + 16 * c);
    }
  }
#pragma unroll
  for (int j = 0; j < C::X_LOADS; ++j) {
    const int b = wave * C::X_LOADS + j;
    const int r = b * 16 + (lane >> 2);
    const int c = (lane & 3) ^ swz64(r);
    kx[j] = 16 * c;
    offx[j] = unsigned(r * K + 16 * c);
  }

  auto issue_w = [&](int s, int k0) {
    const unsigned kw_bytes = W4 ? unsigned(k0 / 2) : unsigned(k0);
#pragma unroll
    for (int j = 0; j < C::W_LOADS; ++j) {
      const unsigned off = (k0 + kw[j] < K) ? offw[j] + kw_bytes : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, (lds_ptr_t)(sWs[s] + (wave * C::W_LOADS + j) * 1024), 16,
                                               off, 0, 0, 0);
    }
  };
  auto issue_x = [&](int s, int k0) {
#pragma unroll
    for (int j = 0; j < C::X_LOADS; ++j) {
      const unsigned off = (k0 + kx[j] < K) ? offx[j] + unsigned(k0) : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsx, (lds_ptr_t)(sXs[s] + (wave * C::X_LOADS + j) * 1024), 16,
                                               off, 0, 0, 0);
    }
  };

  // Fragment row offsets inside a stage (constant over K).
  int wrow_off[TI], xrow_off[TJ], wsw[TI], xsw[TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int r = wn * WN + i * 32 + row;
    wrow_off[i] = r * C::WROW;
    wsw[i] = W4 ? swz32(r) : swz64(r);
  }
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int r = wm * WM + j * 32 + row;
    xrow_off[j] = r * 64;
    xsw[j] = swz64(r);
  }

  // fa[s][i]: weight fragments for K-slice s; fb[s][j]: token fragments.
  v4i fa[2][TI], fb[2][TJ];
  uint2 pw_hi[TI];  // int4 weights: packed bytes of slice 1, unpacked late

  auto read_x = [&](int s, int slice) {
    const int8_t* sX = sXs[s];
    const int c = W4 ? 2 * half + slice : 2 * slice + half;
#pragma unroll
    for (int j = 0; j < TJ; ++j)
      fb[slice][j] = *reinterpret_cast<const v4i*>(sX + xrow_off[j] + 16 * (c ^ xsw[j]));
  };
  // W8: one 16-byte read per fragment and slice.  W4: the slice-0 read
  // fetches the 16 packed bytes of both slices, unpacks slice 0 and keeps the
  // packed slice-1 half until the slice-1 call unpacks it (the current
  // step's slice-1 fragments are still in use when the next step's slice 0
  // is read).
  auto read_w = [&](int s, int slice) {
    const int8_t* sW = sWs[s];
    if constexpr (W4) {
      if (slice == 0) {
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          const uint4 p = *reinterpret_cast<const uint4*>(sW + wrow_off[i] + 16 * (half ^ wsw[i]));
          uint32_t o[4];
          unpack4(p.x, o[0], o[1]);
          unpack4(p.y, o[2], o[3]);
          fa[0][i] = v4i{int(o[0]), int(o[1]), int(o[2]), int(o[3])};
          pw_hi[i] = make_uint2(p.z, p.w);
        }
      } else {
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          uint32_t o[4];
          unpack4(pw_hi[i].x, o[0], o[1]);
          unpack4(pw_hi[i].y, o[2], o[3]);
          fa[1][i] = v4i{int(o[0]), int(o[1]), int(o[2]), int(o[3])};
        }
      }
    } else {
      const int c = 2 * slice + half;
#pragma unroll
      for (int i = 0; i < TI; ++i)
        fa[slice][i] = *reinterpret_cast<const v4i*>(sW + wrow_off[i] + 16 * (c ^ wsw[i]));
    }
  };

  v16i acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  auto mfma_slice = [&](int slice) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[slice][i], fb[slice][j], acc[i][j], 0, 0, 0);
  };

  // Barrier between the phases.  This wave's LDS reads of the consumed
  // stage must be complete (lgkmcnt 0) before other waves refill it; the
  // asynchronous LDS writes are covered by the explicit vmcnt wait that
  // precedes this call.  The empty asm statements keep the compiler from
  // moving LDS accesses across.
  auto sync_stage = [&]() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0), vmcnt/expcnt untouched
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // LDS reads per phase, for the interleaving pattern.
  constexpr int R1 = (W4 ? 0 : TI) + TJ;  // phase 1: slice-1 reads
  constexpr int R2 = TI + TJ;             // phase 2: next slice-0 reads

  const int ksteps = ((K + BK - 1) / BK + kStages - 1) / kStages * kStages;

  // Prologue: stages 0..2 and the weight half of stage 3 are issued; stage 0
  // has landed once at most 2 L + W_LOADS newer loads are outstanding.
  issue_w(0, 0);
  issue_x(0, 0);
  issue_w(1, BK);
  issue_x(1, BK);
  issue_w(2, 2 * BK);
  issue_x(2, 2 * BK);
  issue_w(3, 3 * BK);
  wait_vmcnt<2 * L + C::W_LOADS>();
  sync_stage();
  read_w(0, 0);
  read_x(0, 0);

  // Step kt issues the token loads of stage kt+3 in phase 1 and the weight
  // loads of stage kt+4 in phase 2.  Before the barrier of step kt, stage
  // kt+1 must be complete; the loads issued after its last one are those of
  // stages kt+2 and kt+3, i.e. 2 L.
  for (int kb = 0; kb < ksteps; kb += kStages) {
#pragma unroll
    for (int s = 0; s < kStages; ++s) {
      const int kt = kb + s;
      read_w(s, 1);
      read_x(s, 1);
      mfma_slice(0);
      issue_x((s + 3) % kStages, (kt + 3) * BK);
      interleave_phase<TI * TJ, C::X_LOADS, R1>();
      wait_vmcnt<2 * L>();
      sync_stage();
      __builtin_amdgcn_sched_barrier(0);
      issue_w(s, (kt + 4) * BK);
      read_w((s + 1) % kStages, 0);
      read_x((s + 1) % kStages, 0);
      mfma_slice(1);
      interleave_phase<TI * TJ, C::W_LOADS, R2>();
    }
  }
  wait_vmcnt<0>();

  // Epilogue.  Block (i, j): lane holds token m = ... + (lane & 31) and weight
  // rows n = ... + 8*g + 4*(lane >> 5) + (0..3) in accumulators 4g..4g+3.
  // All scales this lane needs are fetched in one batch first, so their
  // latency is paid once.  The bf16 results of one 32-token block at a time
  // are staged in LDS (wave w uses token stage buffer w, free once every
  // wave has left the main loop) and leave as 16-byte row-contiguous stores;
  // writing straight from the accumulator layout would scatter 8-byte pieces
  // over 32 rows per instruction.
  float swv[TI][4][4];
  float sxv[TJ];
  if (y) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int n = n0 + wn * WN + i * 32 + 8 * g + 4 * half + e;
          swv[i][g][e] = n < N ? sw[n] : 0.f;
        }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int m = m0 + wm * WM + j * 32 + row;
      sxv[j] = m < M ? sx[m] : 0.f;
    }
  }
  if (acc_out) {
    const bool vec_ok = (N & 3) == 0;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int m = m0 + wm * WM + j * 32 + row;
      if (m >= M) continue;
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * WN + i * 32 + 8 * g + 4 * half;
          int a[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a[e] = acc[i][j][4 * g + e];
            if constexpr (W4) a[e] >>= 4;
          }
          if (vec_ok && n + 3 < N) {
            *reinterpret_cast<int4*>(acc_out + int64_t(m) * N + n) = make_int4(a[0], a[1], a[2], a[3]);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < N) acc_out[int64_t(m) * N + n + e] = a[e];
          }
        }
    }
  }
  if (!y) return;
  // Staging layout for a 32 x WN bf16 block: 16-byte chunk q of row r at
  // r * P + 16 * (q ^ f(r)) with a pitch and row hash that keep the 8-byte
  // writes of 16 consecutive rows in distinct banks.
  constexpr int NQ = WN / 8;                       // 16-byte chunks per row
  constexpr int P = (NQ == 12) ? 208 : WN * 2;     // 96 columns: padded pitch
  auto chunk_of = [&](int r, int q) {
    if constexpr (NQ == 16) return q ^ (r & 15);
    else if constexpr (NQ == 8) return q ^ ((r >> 1) & 7);
    else return q;
  };
  static_assert(32 * P <= C::X_BYTES, "epilogue block must fit one token stage buffer");
  int8_t* stage_buf = wave == 0 ? sX0 : wave == 1 ? sX1 : wave == 2 ? sX2 : sX3;
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  const bool full_rows = (N & 7) == 0;
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float f[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          int a = acc[i][j][4 * g + e];
          if constexpr (W4) a >>= 4;
          f[e] = (float(a) * sxv[j]) * swv[i][g][e];
        }
        const int q = i * 4 + g;  // 16-byte chunk holding columns 8q .. 8q+7
        *reinterpret_cast<uint2*>(stage_buf + row * P + 16 * chunk_of(row, q) + 8 * half) =
            make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
      }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // this wave's LDS writes done
    asm volatile("" ::: "memory");
#pragma unroll
    for (int k = 0; k < 32 * NQ / 64; ++k) {
      const int id = lane + 64 * k;
      const int r = id / NQ, q = id % NQ;
      const int m = m0 + wm * WM + j * 32 + r;
      const int n = n0 + wn * WN + 8 * q;
      const uint4 v = *reinterpret_cast<const uint4*>(stage_buf + r * P + 16 * chunk_of(r, q));
      if (m < M) {
        if (full_rows && n + 7 < N) {
          *reinterpret_cast<uint4*>(y + int64_t(m) * N + n) = v;
        } else {
          const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (n + e < N) y[int64_t(m) * N + n + e] = uint16_t(w[e / 2] >> (16 * (e & 1)));
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the next block overwrites
    asm volatile("" ::: "memory");
  }
}

// ---------------------------------------------------------------------------
// int8-weight kernel with 128-byte K stages.  Each row chunk of a stage is a
// whole 128-byte cache line, which the global->LDS load path serves about
// 1.6x faster than half lines (measured on gfx950: ~69 against ~44 B/clk
// per CU).  Two LDS stages; per 128-K step one barrier:
//   phase 1: K-slices 0..2 of stage kt, each slice's MFMAs interleaved with
//            the LDS reads of the next slice (the first group also issues
//            the tail of stage kt+1's loads); then wait for stage kt+1 and
//            barrier;
//   phase 2: slice 3 of stage kt (its fragments are already in registers),
//            interleaved with the reads of stage kt+1's slice 0 and the
//            loads of stage kt+2 into the buffer stage kt has just freed.
// LDS rows are 128 bytes (8 chunks of 16 B); chunk c of row r is stored at
// c ^ ((r >> 1) & 7), conflict-free for the fragment reads (measured).
__device__ __forceinline__ int swz128(int r) { return (r >> 1) & 7; }

template <int BM, int BN>
struct Cfg8 {
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int TI = WN / 32, TJ = WM / 32;
  static constexpr int KB = 128;                                   // K bytes per stage
  static constexpr int W_BYTES = BN * KB, X_BYTES = BM * KB;
  static constexpr int W_LOADS = W_BYTES / 4096, X_LOADS = X_BYTES / 4096;  // per wave
  static constexpr int LOADS = W_LOADS + X_LOADS;
  static constexpr int NM = TI * TJ;                               // MFMAs per slice
  // The next-but-one stage's loads are spread over three slices of MFMAs:
  // phase 2 (P2 loads), then the first two slices of the next phase 1
  // (G0 and G1 loads), so the load path never sees more than about one
  // wave-load per MFMA across the CU and the last load still has a slice
  // of MFMAs before the wait.
#ifndef CONVROT_SPLIT_DEN
#define CONVROT_SPLIT_DEN 3
#endif
  static constexpr int P2 = (LOADS + CONVROT_SPLIT_DEN - 1) / CONVROT_SPLIT_DEN;
  static constexpr int G0 = CONVROT_SPLIT_DEN == 1 ? 0 : (LOADS - P2 + CONVROT_SPLIT_DEN - 2) / (CONVROT_SPLIT_DEN - 1);
  static constexpr int G1 = LOADS - P2 - G0;
  static_assert(P2 <= NM && G0 <= NM && G1 <= NM && G1 >= 0, "at most one load per MFMA");
  static constexpr int STAGE = W_BYTES + X_BYTES;
  static_assert(W_LOADS * 4096 == W_BYTES && X_LOADS * 4096 == X_BYTES, "tile must split into 4 KB");
  static_assert(LOADS < 64, "vmcnt budget");
};

template <int BM, int BN, bool EVEN>
__device__ __forceinline__ void gemm_k128_body(const int8_t* __restrict__ X, const float* __restrict__ sx,
                                               const int8_t* __restrict__ W, const float* __restrict__ sw, int M,
                                               int N, int K, int tiles_m, int tiles_n, int ldy,
                                               int32_t* __restrict__ acc_out, uint16_t* __restrict__ y) {
  using C = Cfg8<BM, BN>;
  constexpr int WM = C::WM, WN = C::WN, TI = C::TI, TJ = C::TJ, L = C::LOADS, P2 = C::P2;
  // Separate arrays per stage buffer: the compiler then knows that the
  // global->LDS writes into one buffer do not alias reads of the other and
  // keeps them interleaved.
  __shared__ __attribute__((aligned(1024))) int8_t sW0[C::W_BYTES], sW1[C::W_BYTES];
  __shared__ __attribute__((aligned(1024))) int8_t sX0[C::X_BYTES], sX1[C::X_BYTES];
  // This tile's weight-row and token scales (rows past N / M read as zero).
  __shared__ __attribute__((aligned(1024))) float sSw[256], sSx[256];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS targets stay scalar
  const int wm = wave >> 1, wn = wave & 1;
  const int row = lane & 31, half = lane >> 5;

  const int T = tiles_m * tiles_n;
  int t = blockIdx.x;
  if ((T & 7) == 0) t = (t & 7) * (T >> 3) + (t >> 3);
  const int tile_m = t % tiles_m, tile_n = t / tiles_m;
  const int m0 = tile_m * BM, n0 = tile_n * BN;

  const int rows_x = min(BM, M - m0), rows_w = min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t rsx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(X + int64_t(m0) * K), short(0), rows_x * K, kBufFlags);
  const __amdgpu_buffer_rsrc_t rsw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(W + int64_t(n0) * K), short(0), rows_w * K, kBufFlags);
  // EVEN (K a multiple of 256, so the steps pair up with no partial stage):
  // the stage's K offset goes into the instruction's scalar offset and each
  // load is one scalar M0 update plus the load itself.  The prefetches of the
  // two stages past K read the next rows or out-of-range zeros into buffers
  // that are never consumed.  Otherwise every 16-byte chunk is range-checked
  // per lane.

  // Load block b (1 KB) holds rows 8b..8b+7; lane i writes LDS byte 16 i of
  // the block, i.e. position i & 7 of row 8b + (i >> 3), which holds source
  // chunk (i & 7) ^ swz128(row).
  unsigned offw[C::W_LOADS], offx[C::X_LOADS];
  int kw[C::W_LOADS], kx[C::X_LOADS];
#pragma unroll
  for (int j = 0; j < C::W_LOADS; ++j) {
    const int r = (wave * C::W_LOADS + j) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz128(r);
    kw[j] = 16 * c;
    offw[j] = unsigned(r * K + 16 * c);
  }
#pragma unroll
  for (int j = 0; j < C::X_LOADS; ++j) {
    const int r = (wave * C::X_LOADS + j) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz128(r);
    kx[j] = 16 * c;
    offx[j] = unsigned(r * K + 16 * c);
  }
  // Loads of one stage in a fixed order (token blocks, then weight blocks);
  // q selects which of them: [Q0, Q1).
  auto issue = [&](int s, int k0, auto q0, auto q1) {
    constexpr int Q0 = decltype(q0)::value, Q1 = decltype(q1)::value;
    int8_t* const sW = s ? sW1 : sW0;
    int8_t* const sX = s ? sX1 : sX0;
#pragma unroll
    for (int q = Q0; q < Q1; ++q) {
      if (q < C::X_LOADS) {
        const int j = q;
        lds_ptr_t dst = (lds_ptr_t)(sX + (wave * C::X_LOADS + j) * 1024);
        if constexpr (EVEN) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsx, dst, 16, offx[j], k0, 0, 0);
        } else {
          const unsigned off = (k0 + kx[j] < K) ? offx[j] + unsigned(k0) : kOOB;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsx, dst, 16, off, 0, 0, 0);
        }
      } else {
        const int j = q - C::X_LOADS;
        lds_ptr_t dst = (lds_ptr_t)(sW + (wave * C::W_LOADS + j) * 1024);
        if constexpr (EVEN) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, dst, 16, offw[j], k0, 0, 0);
        } else {
          const unsigned off = (k0 + kw[j] < K) ? offw[j] + unsigned(k0) : kOOB;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, dst, 16, off, 0, 0, 0);
        }
      }
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using IP2 = std::integral_constant<int, P2>;
  using IG0 = std::integral_constant<int, P2 + C::G0>;
  using IL = std::integral_constant<int, L>;

  // Fragment addresses inside a stage for slice 0; slice sl is at addr ^ 32 sl.
  int wadr[TI], xadr[TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int r = wn * WN + i * 32 + row;
    wadr[i] = r * 128 + 16 * (half ^ swz128(r));
  }
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int r = wm * WM + j * 32 + row;
    xadr[j] = r * 128 + 16 * (half ^ swz128(r));
  }

  v4i fa[2][TI], fb[2][TJ];
  auto read = [&](int s, int sl, int b) {
    const int8_t* bw = s ? sW1 : sW0;
    const int8_t* bx = s ? sX1 : sX0;
#pragma unroll
    for (int i = 0; i < TI; ++i) fa[b][i] = *reinterpret_cast<const v4i*>(bw + (wadr[i] ^ (32 * sl)));
#pragma unroll
    for (int j = 0; j < TJ; ++j) fb[b][j] = *reinterpret_cast<const v4i*>(bx + (xadr[j] ^ (32 * sl)));
  };

  v16i acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  auto mfma = [&](int b) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[b][i], fb[b][j], acc[i][j], 0, 0, 0);
  };
  auto sync_stage = [&]() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0), vmcnt/expcnt untouched
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  constexpr int NM = C::NM, ND = TI + TJ;
  const int ksteps = EVEN ? K / 128 : ((K + 127) / 128 + 1) & ~1;  // even: the loop body covers two steps

  // Prologue: the scales (one 1 KB load each, by waves 0 and 1; first
  // used in the epilogue, long after the main loop's waits), all of stage
  // 0, the phase-2 share of stage 1.
  if (y && wave < 2) {
    const float* src = wave == 0 ? sw + n0 : sx + m0;
    const int nrec = 4 * (wave == 0 ? rows_w : rows_x);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(src), short(0), nrec,
                                                                        kBufFlags);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(wave == 0 ? sSw : sSx), 16, unsigned(lane * 16), 0,
                                             0, 0);
  }
  issue(0, 0, I0{}, IL{});
  issue(1, 128, I0{}, IP2{});
  wait_vmcnt<P2>();
  sync_stage();
  read(0, 0, 0);

  for (int kb = 0; kb < ksteps; kb += 2) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int kt = kb + s;
      // phase 1
      read(s, 1, 1);
      mfma(0);
      issue(s ^ 1, (kt + 1) * 128, IP2{}, IG0{});
      interleave_phase<NM, C::G0, ND>();
      read(s, 2, 0);
      mfma(1);
      issue(s ^ 1, (kt + 1) * 128, IG0{}, IL{});
      interleave_phase<NM, C::G1, ND>();
      read(s, 3, 1);
      mfma(0);
      interleave_phase<NM, 0, ND>();
      wait_vmcnt<0>();
      sync_stage();
      __builtin_amdgcn_sched_barrier(0);
      // phase 2
      issue(s, (kt + 2) * 128, I0{}, IP2{});
      read(s ^ 1, 0, 0);
      mfma(1);
      interleave_phase<NM, P2, ND>();
    }
  }
  wait_vmcnt<0>();

  // Epilogue.  Block (i, j): lane holds token m = ... + (lane & 31) and
  // weight rows n = ... + 8 g + 4 (lane >> 5) + (0..3) in accumulators
  // 4g..4g+3.  The bf16 results of one 32-token block at a time are staged
  // in LDS and leave as 16-byte row-contiguous stores (from the accumulator
  // layout a store would scatter 8-byte pieces over 32 rows).  Scales come
  // from LDS, four weight scales per read.
  if (acc_out) {
    const bool vec_ok = (N & 3) == 0;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int m = m0 + wm * WM + j * 32 + row;
      if (m >= M) continue;
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * WN + i * 32 + 8 * g + 4 * half;
          const int a[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
          if (vec_ok && n + 3 < N) {
            *reinterpret_cast<int4*>(acc_out + int64_t(m) * ldy + n) = make_int4(a[0], a[1], a[2], a[3]);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < N) acc_out[int64_t(m) * ldy + n + e] = a[e];
          }
        }
    }
  }
  if (!y) return;
  constexpr int NQ = WN / 8;
  constexpr int P = (NQ == 12) ? 208 : WN * 2;
  constexpr int STG = (32 * P + 1023) / 1024 * 1024;
  static_assert(4 * STG <= (C::X_BYTES > C::W_BYTES ? C::X_BYTES : C::W_BYTES),
                "epilogue staging must fit one stage buffer");
  auto chunk_of = [&](int r, int q) {
    if constexpr (NQ == 16) return q ^ (r & 15);
    else if constexpr (NQ == 8) return q ^ ((r >> 1) & 7);
    else return q;
  };
  int8_t* stage_buf = (C::X_BYTES >= C::W_BYTES ? sX0 : sW0) + wave * STG;
  __builtin_amdgcn_s_waitcnt(0xc07f);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  // Interior tiles (and N a multiple of 8) store without per-element checks.
  const bool interior = m0 + BM <= M && n0 + BN <= N && (N & 7) == 0;
  const float* swt = sSw + wn * WN + 4 * half;
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const float sxj = sSx[wm * WM + j * 32 + row];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 sw4 = *reinterpret_cast<const float4*>(swt + i * 32 + 8 * g);
        const float f0 = (float(acc[i][j][4 * g + 0]) * sxj) * sw4.x;
        const float f1 = (float(acc[i][j][4 * g + 1]) * sxj) * sw4.y;
        const float f2 = (float(acc[i][j][4 * g + 2]) * sxj) * sw4.z;
        const float f3 = (float(acc[i][j][4 * g + 3]) * sxj) * sw4.w;
        const int q = i * 4 + g;
        *reinterpret_cast<uint2*>(stage_buf + row * P + 16 * chunk_of(row, q) + 8 * half) =
            make_uint2(pack_bf16x2(f0, f1), pack_bf16x2(f2, f3));
      }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    asm volatile("" ::: "memory");
    if (interior) {
#pragma unroll
      for (int k = 0; k < 32 * NQ / 64; ++k) {
        const int id = lane + 64 * k;
        const int r = id / NQ, q = id % NQ;
        const uint4 v = *reinterpret_cast<const uint4*>(stage_buf + r * P + 16 * chunk_of(r, q));
        *reinterpret_cast<uint4*>(y + int64_t(m0 + wm * WM + j * 32 + r) * ldy + (n0 + wn * WN + 8 * q)) = v;
      }
    } else {
#pragma unroll
      for (int k = 0; k < 32 * NQ / 64; ++k) {
        const int id = lane + 64 * k;
        const int r = id / NQ, q = id % NQ;
        const int m = m0 + wm * WM + j * 32 + r;
        const int n = n0 + wn * WN + 8 * q;
        const uint4 v = *reinterpret_cast<const uint4*>(stage_buf + r * P + 16 * chunk_of(r, q));
        if (m < M) {
          if ((N & 7) == 0 && n + 7 < N) {
            *reinterpret_cast<uint4*>(y + int64_t(m) * ldy + n) = v;
          } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (n + e < N) y[int64_t(m) * ldy + n + e] = uint16_t(w[e / 2] >> (16 * (e & 1)));
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    asm volatile("" ::: "memory");
  }
}

// K a multiple of 256 (every group-256 linear): unchecked scalar-offset loads.
template <int BM, int BN>
__global__ __launch_bounds__(kThreads, 1) void gemm_i8_k128_kernel(const int8_t* __restrict__ X,
                                                                   const float* __restrict__ sx,
                                                                   const int8_t* __restrict__ W,
                                                                   const float* __restrict__ sw, int M, int N, int K,
                                                                   int tiles_m, int tiles_n, int ldy,
                                                                   int32_t* __restrict__ acc_out,
                                                                   uint16_t* __restrict__ y) {
  gemm_k128_body<BM, BN, true>(X, sx, W, sw, M, N, K, tiles_m, tiles_n, ldy, acc_out, y);
}

// Any K (a multiple of 16): every 16-byte chunk range-checked.
template <int BM, int BN>
__global__ __launch_bounds__(kThreads, 1) void gemm_i8_k128_tail_kernel(const int8_t* __restrict__ X,
                                                                        const float* __restrict__ sx,
                                                                        const int8_t* __restrict__ W,
                                                                        const float* __restrict__ sw, int M, int N,
                                                                        int K, int tiles_m, int tiles_n, int ldy,
                                                                        int32_t* __restrict__ acc_out,
                                                                        uint16_t* __restrict__ y) {
  gemm_k128_body<BM, BN, false>(X, sx, W, sw, M, N, K, tiles_m, tiles_n, ldy, acc_out, y);
}

// One band of output columns: y and acc_out have row stride ldy; wq,
// w_scale, acc_out and y already point at the band's first column.
template <int BM, int BN>
hipError_t launch_k128(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale, int M, int N,
                       int K, int ldy, int32_t* acc_out, uint16_t* y, hipStream_t stream) {
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + BN - 1) / BN;
  const dim3 grid(unsigned(tiles_m) * unsigned(tiles_n));
  void (*kernel)(const int8_t*, const float*, const int8_t*, const float*, int, int, int, int, int, int, int32_t*,
                 uint16_t*) = gemm_i8_k128_tail_kernel<BM, BN>;
  if (K % 256 == 0) kernel = gemm_i8_k128_kernel<BM, BN>;
  hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, xq, x_scale, wq, w_scale, M, N, K, tiles_m, tiles_n,
                     ldy, acc_out, y);
  return hipGetLastError();
}

template <int BM, int BN, bool W4>
hipError_t launch_cfg(const int8_t* xq, const float* x_scale, const uint8_t* wq, const float* w_scale, int M,
                      int N, int K, int32_t* acc_out, uint16_t* y, hipStream_t stream) {
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + BN - 1) / BN;
  const dim3 grid(unsigned(tiles_m) * unsigned(tiles_n));
  hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, W4>), grid, dim3(kThreads), 0, stream, xq, x_scale, wq, w_scale, M,
                     N, K, tiles_m, tiles_n, acc_out, y);
  return hipGetLastError();
}

struct TileChoice {
  int bm, bn;
};

// Pick the macro tile: fewest rounds of tiles over the 256 CUs, weighted by
// how efficiently each tile size runs (larger tiles reuse LDS operands more).
TileChoice choose_tile(int64_t M, int64_t N, bool w4) {
  static const TileChoice cands[] = {{256, 256}, {256, 192}, {256, 128}, {128, 256}, {128, 128}};
  static const double eff[] = {1.0, 0.97, 0.85, 0.85, 0.6};
  const int cus = 256;
  double best = 1e300;
  TileChoice pick = cands[4];
  for (int c = 0; c < 5; ++c) {
    if (w4 && cands[c].bn == 192) continue;  // packed weight tile must split into 4 KB loads
    const int64_t tiles = ((M + cands[c].bm - 1) / cands[c].bm) * ((N + cands[c].bn - 1) / cands[c].bn);
    const int64_t rounds = (tiles + cus - 1) / cus;
    const double cost = double(rounds) * cands[c].bm * cands[c].bn / eff[c];
    if (cost < best * 0.999) {
      best = cost;
      pick = cands[c];
    }
  }
  return pick;
}

// CONVROT_GEMM_TILE=<BM>x<BN> forces one of the tile shapes above (a tuning
// override for sweeps; every tile gives bit-identical results).
TileChoice tile_override() {
  static const TileChoice forced = [] {
    TileChoice t{0, 0};
    if (const char* s = getenv("CONVROT_GEMM_TILE")) {
      if (sscanf(s, "%dx%d", &t.bm, &t.bn) != 2) t = {0, 0};
    }
    return t;
  }();
  return forced;
}

// A plan for int8 weights: up to two bands of output columns, each with its
// own tile shape (launched back to back on the stream; the chooser below
// uses one band, the override can ask for two).
struct Band {
  int n_cols;  // 0 = the rest of N
  TileChoice tc;
};
struct Plan {
  int nb;
  Band b[2];
};

// Tile plan for int8 weights, from measurements on MI355X under sustained
// load.  The chip runs this GEMM below its top clock, and the clock rises
// when less data moves per MFMA, so the largest tile (256x256: fewest
// L2->LDS bytes per operation) wins once it fills several whole rounds of
// the 256 CUs; otherwise 256x192 when it fills at least three quarters of a
// round, and 128x128 for small problems (more CUs busy).  Splitting N into
// bands of different tiles to even out a partial round measured no faster
// than a single 256x192 launch (the second launch waits for the first).
Plan choose_plan(int64_t M, int64_t N) {
  const int cus = 256;
  auto tiles = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  if (N % 256 == 0 && tiles(256, 256) >= 3 * cus) return {1, {{0, {256, 256}}, {0, {0, 0}}}};
  if (4 * tiles(256, 192) >= 3 * cus) return {1, {{0, {256, 192}}, {0, {0, 0}}}};
  return {1, {{0, {128, 128}}, {0, {0, 0}}}};
}

// CONVROT_GEMM_PLAN=<BM>x<BN>[:<cols>][,<BM>x<BN>] forces a plan (a tuning
// override for sweeps; every plan gives bit-identical results).
bool plan_override(Plan& out) {
  static const Plan forced = [] {
    Plan p{0, {{0, {0, 0}}, {0, {0, 0}}}};
    const char* s = getenv("CONVROT_GEMM_PLAN");
    if (!s) return p;
    int bm0, bn0, cols = 0, bm1, bn1;
    if (sscanf(s, "%dx%d:%d,%dx%d", &bm0, &bn0, &cols, &bm1, &bn1) == 5) return Plan{2, {{cols, {bm0, bn0}}, {0, {bm1, bn1}}}};
    if (sscanf(s, "%dx%d", &bm0, &bn0) == 2) return Plan{1, {{0, {bm0, bn0}}, {0, {0, 0}}}};
    return p;
  }();
  if (forced.nb == 0) return false;
  out = forced;
  return true;
}

hipError_t launch_band8(TileChoice tc, const int8_t* xq, const float* x_scale, const int8_t* wq,
                        const float* w_scale, int M, int N, int K, int ldy, int32_t* acc_out, uint16_t* y,
                        hipStream_t stream) {
  if (tc.bm == 256 && tc.bn == 256) return launch_k128<256, 256>(xq, x_scale, wq, w_scale, M, N, K, ldy, acc_out, y, stream);
  if (tc.bm == 256 && tc.bn == 192) return launch_k128<256, 192>(xq, x_scale, wq, w_scale, M, N, K, ldy, acc_out, y, stream);
  if (tc.bm == 256 && tc.bn == 128) return launch_k128<256, 128>(xq, x_scale, wq, w_scale, M, N, K, ldy, acc_out, y, stream);
  if (tc.bm == 128 && tc.bn == 256) return launch_k128<128, 256>(xq, x_scale, wq, w_scale, M, N, K, ldy, acc_out, y, stream);
  return launch_k128<128, 128>(xq, x_scale, wq, w_scale, M, N, K, ldy, acc_out, y, stream);
}

hipError_t launch_w8(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale, int M, int N,
                     int K, int32_t* acc_out, uint16_t* y, hipStream_t stream) {
  Plan plan;
  const TileChoice forced = tile_override();
  if (!plan_override(plan)) plan = forced.bm ? Plan{1, {{0, forced}, {0, {0, 0}}}} : choose_plan(M, N);
  int n_begin = 0;
  for (int i = 0; i < plan.nb && n_begin < N; ++i) {
    const int cols = (plan.b[i].n_cols > 0 && n_begin + plan.b[i].n_cols < N) ? plan.b[i].n_cols : N - n_begin;
    const hipError_t e = launch_band8(plan.b[i].tc, xq, x_scale, wq + int64_t(n_begin) * K,
                                      w_scale ? w_scale + n_begin : nullptr, M, cols, K, N,
                                      acc_out ? acc_out + n_begin : nullptr, y ? y + n_begin : nullptr, stream);
    if (e != hipSuccess) return e;
    n_begin += cols;
  }
  return hipSuccess;
}

hipError_t launch_w4(const int8_t* xq, const float* x_scale, const uint8_t* wq, const float* w_scale, int M, int N,
                     int K, int32_t* acc_out, uint16_t* y, hipStream_t stream) {
  TileChoice tc = tile_override();
  if (tc.bm == 0 || tc.bn == 192) tc = choose_tile(M, N, true);
  if (tc.bm == 256 && tc.bn == 256) return launch_cfg<256, 256, true>(xq, x_scale, wq, w_scale, M, N, K, acc_out, y, stream);
  if (tc.bm == 256 && tc.bn == 128) return launch_cfg<256, 128, true>(xq, x_scale, wq, w_scale, M, N, K, acc_out, y, stream);
  if (tc.bm == 128 && tc.bn == 256) return launch_cfg<128, 256, true>(xq, x_scale, wq, w_scale, M, N, K, acc_out, y, stream);
  return launch_cfg<128, 128, true>(xq, x_scale, wq, w_scale, M, N, K, acc_out, y, stream);
}

}  // namespace

hipError_t launch_gemm(const int8_t* xq, const float* x_scale, const void* wq, int wbits, const float* w_scale,
                       int64_t M, int64_t N, int64_t K, int32_t* acc_out, uint16_t* y, hipStream_t stream) {
  if (wbits == 4)
    return launch_w4(xq, x_scale, static_cast<const uint8_t*>(wq), w_scale, int(M), int(N), int(K), acc_out, y,
                     stream);
  return launch_w8(xq, x_scale, static_cast<const int8_t*>(wq), w_scale, int(M), int(N), int(K), acc_out, y,
                   stream);
}

}  // namespace convrot
