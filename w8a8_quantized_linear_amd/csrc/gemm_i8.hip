// int8 x int8 -> int32 GEMM on CDNA4 matrix cores with a fused dequant
// epilogue to bf16 (the matmul of the ConvRot W8A8 linear: "MOSS-Image
// Qwen3.5-9B text encoder, INT8 (W8A8, ConvRot)", intro and file table row
// "Matmul"; the int4-weight variant reads two signed nibbles per byte,
// "MossInt4", "Format").
//
//   acc[m][n] = sum_k xq[m][k] * wq[n][k]           (both operands K-major)
//   y[m][n]   = bf16_rne(((float)acc * x_scale[m]) * w_scale[n])
//
// The same body also serves (template flags) several weight matrices that
// share one quantized input in one launch (MULTI), and the bf16 x bf16
// matmul of the weight-only path (BF: v_mfma_f32_32x32x16_bf16, fp32
// accumulators, y = bf16(acc)); the pipeline moves bytes, so both reuse it
// unchanged.
//
// Tiling.  A 256-thread workgroup (4 waves, 2 x 2) computes a BM x BN output
// tile (BM tokens x BN weight rows); each wave owns a (BM/2) x (BN/2)
// sub-tile of 32x32 blocks accumulated by v_mfma_i32_32x32x32_i8.  The MFMA's
// first operand is the weight tile and its second the token tile, so a lane's
// 16 accumulators of a block cover one token and four runs of four
// consecutive weight rows; the epilogue regroups them through LDS into
// 16-byte row-contiguous bf16 stores.
//
// Pipeline.  K advances 128 values per step through two LDS stages filled by
// buffer_load_dwordx4 ... lds (global -> LDS without registers; each wave
// instruction moves a 1 KB block).  A token row chunk of a stage is a whole
// 128-byte cache line: the load path serves whole lines about 1.6x faster
// than half lines (measured on gfx950, ~69 against ~44 B/clk per CU).  One
// barrier per step; the MFMAs of the step's last K-slice run after it, while
// the next stage's first slice is read and the loads of the stage after next
// go out into the buffer just freed (a full step of lead time).  LDS reads and
// loads are interleaved one per MFMA (sched_group_barrier), the loop body has
// no conditionals, and for K a multiple of 256 each load is one scalar M0
// update: the stage's K offset rides in the instruction's scalar offset.
// A tile alone on its CU (few tiles) has nothing else on the CU to hide the
// load latency, and a small tile's step is too short to cover it with one
// stage in flight: such tiles run three stages (256x128) or four (128x128,
// 64x128), each sent two or three steps ahead (template parameter NS).
//
// Why these choices: under sustained load the device holds a shader clock
// well below its 2.4 GHz peak, about 1.75 GHz under a loop of nothing but
// MFMAs and about 1.45-1.50 GHz under this GEMM's main loop, where the MFMA
// pipe is busy 85-91 % of the cycles (rocprofv3 counters).  Feeding the MFMAs
// costs clock more than it costs cycles, so the largest tile that fills the
// machine (the fewest bytes moved per MFMA) wins (see choose_tile), and
// per-load instruction overhead matters as much as bandwidth.
//
// LDS layouts, chosen by measuring ds_read_b128 throughput for these exact
// fragment patterns (about 240 B/clk per CU conflict-free, against about 140
// with two-way conflicts): 128-byte rows with chunk c of row r at
// c ^ ((r >> 1) & 7); 64-byte packed int4 weight rows with chunk c at
// c ^ (((r >> 2) ^ (r >> 3)) & 3).
//
// int4 weights: a lane reads 16 packed bytes (two K-slices' worth) and turns
// each nibble q into the byte 16*q (masks and byte permutes), so the
// accumulator holds 16*acc exactly and is shifted back by 4 before the
// epilogue; the K order inside a stage is permuted identically for both
// operands, which leaves the dot products unchanged.
//
// Tiles are assigned so that each of the 8 XCDs (workgroups are dispatched to
// them round-robin) works on a contiguous block of tiles that share weight
// and token rows in its L2.
#include "convrot_internal.h"

#include <climits>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <type_traits>

namespace convrot {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// 16-byte output store marked nontemporal: the rows are streamed out and
// not read again by this kernel, and keeping them out of the caches' way
// measured 7-12 % faster on the large shapes (same-box A/B: M 2048 K 4096
// N 12288 99.2 -> 92.2 us, M 8704 K 4096 N 12288 434.6 -> 384.6 us).
__device__ __forceinline__ void store_nt(uint16_t* dst, const uint4& v) {
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(dst));
}
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kThreads = 256;
constexpr int kGroupM = 4;  // M-tiles per block of the tile order
constexpr unsigned kOOB = 0x7ffffff0u;  // buffer offset beyond every range: reads as zero
constexpr int kBufFlags = 0x00020000;   // raw buffer descriptor word 3 (gfx9 family)

__device__ __forceinline__ int swz64(int r) { return ((r >> 2) ^ (r >> 3)) & 3; }


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
template <int NM, int NV, int ND, int NA = 0>
__device__ __forceinline__ void interleave_phase() {
  int nv = 0;
  // NA > 0: that many VALU instructions (the unpack of int4 weight
  // fragments read in this phase) go after the second half of the MFMAs,
  // when their LDS reads have landed; placed by the compiler they sat right
  // after the reads and stalled the MFMA issue on the LDS latency (same-box
  // A/B, bit-identical output: M 4096, N 12288, K 4096 163.7 -> 160.5 us,
  // M 2048, N 12288, K 4096 85.1 -> 83.9 us; the deeper-pipeline small tiles
  // measured no gain and keep NA = 0).
  constexpr int H = NM / 2;
  constexpr int PER = NA > 0 ? (NA + (NM - H) - 1) / (NM - H) : 0;
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i < ND) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    const int v_due = ((i + 1) * NV) / NM;  // loads due after MFMA i
    if (nv < v_due) {
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      ++nv;
    }
    if (NA > 0 && i >= H) __builtin_amdgcn_sched_group_barrier(0x002, PER, 0);
  }
  for (int i = NM; i < ND; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  for (; nv < NV; ++nv) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  if (NA > 0) __builtin_amdgcn_sched_group_barrier(0x002, NA, 0);
  __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------------------
// The kernel body, for int8 (W4 = false) or packed int4 (W4 = true) weights.
// Per 128-K step:
//   phase 1: K-slices 0..2 of stage kt, each slice's MFMAs interleaved with
//            the LDS reads of the next slice (the first slice also issues the
//            rest of stage kt+1's loads); then wait for stage kt+1 and
//            barrier;
//   phase 2: slice 3 of stage kt (its fragments are already in registers),
//            interleaved with the reads of stage kt+1's slice 0 and the
//            first half of stage kt+2's loads into the buffer stage kt has
//            just freed.
__device__ __forceinline__ int swz128(int r) { return (r >> 1) & 7; }

// The weight matrices of one launch.  They share the token operand (one
// quantized activation feeding several linears); their column tiles are
// concatenated, output o owning column tiles [tn0[o], tn0[o + 1]).  With a
// single output (MULTI = false) only entry 0 is read, at fixed offsets that
// the kernel fetches with its other arguments; the multi-output kernels
// search tn0 and fetch the tile's entry.
constexpr int kMaxOuts = 8;
struct GemmOut {
  const uint8_t* W;  // [N, K] int8 or [N, K/2] packed int4
  const float* sw;   // [N]
  int32_t* acc;      // [M, ldy] or null (null for every output, or for none)
  uint16_t* y;       // [M, ldy] or null (likewise)
  int N, ldy;
};
struct GemmOuts {
  GemmOut o[kMaxOuts];
  int tn0[kMaxOuts];  // first column tile of each output (unused entries: INT_MAX)
  int n;
};

template <int BM, int BN, bool W4, int NS = 2>
struct CfgK {
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int TI = WN / 32, TJ = WM / 32;
  static constexpr int KB = 128;                                   // K values per stage
  static constexpr int WROW = W4 ? KB / 2 : KB;                    // weight bytes per row and stage
  static constexpr int W_BYTES = BN * WROW, X_BYTES = BM * KB;
  static constexpr int W_LOADS = W_BYTES / 4096, X_LOADS = X_BYTES / 4096;  // per wave
  static constexpr int LOADS = W_LOADS + X_LOADS;
  static constexpr int NM = TI * TJ;                               // MFMAs per slice
  // The next-but-one stage's loads go out in phase 2 (P2) and the first
  // slice of the next phase 1 (G0): at most one wave-load per MFMA, and the
  // last one still has two slices of MFMAs before the wait.
  static constexpr int P2 = (LOADS + 1) / 2;
  static constexpr int G0 = LOADS - P2;
  static_assert(NS > 2 || (P2 <= NM && G0 <= NM), "at most one load per MFMA");
  static_assert(W_LOADS * 4096 == W_BYTES && X_LOADS * 4096 == X_BYTES, "tile must split into 4 KB");
  static_assert(LOADS < 64, "vmcnt budget");
  // Persistent tile walk (the next tile's first loads overlap this tile's
  // epilogue).  Not for 256x256: 256 accumulators per lane leave no room to
  // keep the loop-invariant load offsets live across the epilogue, and the
  // spills cost more than the overlap gains (measured).
  static constexpr bool PERSIST = NS == 2 && !(BM == 256 && BN == 256);
  // Deeper pipelines (NS stages, NS - 1 of them in flight) take one tile
  // per workgroup; every stage's loads go out in phase 1, at most one per
  // MFMA over its three slices.
  static_assert(NS == 2 || (NS <= 4 && LOADS <= 3 * NM), "stages");
  static constexpr int Q1 = LOADS < NM ? LOADS : NM;
  static constexpr int Q2 = LOADS - Q1 < NM ? LOADS - Q1 : NM;
  static constexpr int Q3 = LOADS - Q1 - Q2;
};

template <int BM, int BN, bool W4, bool EVEN, bool MULTI, bool BF, int NS = 2>
__device__ __forceinline__ void gemm_k128_body(const int8_t* __restrict__ X, const float* __restrict__ sx, int M,
                                               int K, int tiles_m, int tiles_n, const GemmOuts& outs) {
  using C = CfgK<BM, BN, W4, NS>;
  constexpr int WM = C::WM, WN = C::WN, TI = C::TI, TJ = C::TJ, L = C::LOADS, P2 = C::P2;
  // K counts bytes of a token row (a bf16 row of k values is 2k bytes);
  // Kb is the bytes of a weight row.
  const int Kb = W4 ? K / 2 : K;
  // Separate arrays per stage buffer: the compiler then knows that the
  // global->LDS writes into one buffer do not alias reads of the other and
  // keeps them interleaved.
  __shared__ __attribute__((aligned(1024))) int8_t sW0[C::W_BYTES], sW1[C::W_BYTES];
  __shared__ __attribute__((aligned(1024))) int8_t sX0[C::X_BYTES], sX1[C::X_BYTES];
  __shared__ __attribute__((aligned(1024))) int8_t sW2[NS > 2 ? C::W_BYTES : 16], sX2[NS > 2 ? C::X_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) int8_t sW3[NS > 3 ? C::W_BYTES : 16], sX3[NS > 3 ? C::X_BYTES : 16];
  // Stage buffer s (s is a constant wherever this is used: the loops over
  // stages are unrolled).
  auto bufw = [&](int s) -> int8_t* { return s == 0 ? sW0 : s == 1 ? sW1 : s == 2 ? sW2 : sW3; };
  auto bufx = [&](int s) -> int8_t* { return s == 0 ? sX0 : s == 1 ? sX1 : s == 2 ? sX2 : sX3; };
  // This tile's weight-row and token scales (rows past N / M read as zero).
  __shared__ __attribute__((aligned(1024))) float sSw[256], sSx[256];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS targets stay scalar
  const int wm = wave >> 1, wn = wave & 1;
  const int row = lane & 31, half = lane >> 5;

  // Persistent tiles: workgroup b takes tiles v = b, b + G, ... in an
  // XCD-aware order (the initial dispatch puts workgroup b on XCD b % 8, so
  // for G a multiple of 8 every tile of b lies in XCD b % 8's contiguous
  // block of tiles, which share weight and token rows in its L2).
  const int T = tiles_m * tiles_n;
  const int G = gridDim.x;
  auto tile_of = [&](int v) { return (T & 7) == 0 ? (v & 7) * (T >> 3) + (v >> 3) : v; };

  // Output of column tile tn (uniform): the number of later outputs whose
  // first tile it has reached.
  auto out_of = [&](int tn) {
    int o = 0;
    if constexpr (MULTI) {
#pragma unroll
      for (int i = 1; i < kMaxOuts; ++i) o += tn >= outs.tn0[i] ? 1 : 0;
    }
    return o;
  };
  const bool has_acc = outs.o[0].acc != nullptr, has_y = outs.o[0].y != nullptr;

  int m0 = 0, n0 = 0, rows_x = 0, rows_w = 0, cur = 0;
  const uint8_t* W = outs.o[0].W;
  const float* sw = outs.o[0].sw;
  __amdgpu_buffer_rsrc_t rsx, rsw;
  auto set_tile = [&](int v) {
    const int t = tile_of(v);
    // Tile t in blocks of kGroupM M-tiles walked N-tile by N-tile, so an
    // XCD's contiguous run of tiles (see tile_of) covers fewer token rows
    // and re-reads less of X (same-box A/B against plain N-major order:
    // M 8704 N 12288 -3.0 %, M 2048 K 12288 -1.9 %, others -0.2..-1.3 %).
    int tm, tn;
    {
      const int nb = tiles_m / kGroupM, per_block = kGroupM * tiles_n, b = t / per_block;
      if (b < nb) {
        const int w = t - b * per_block;
        tm = b * kGroupM + w % kGroupM;
        tn = w / kGroupM;
      } else {  // the last rows of M-tiles, fewer than kGroupM
        const int h = tiles_m - nb * kGroupM, w = t - nb * per_block;
        tm = nb * kGroupM + w % h;
        tn = w / h;
      }
    }
    const int o = out_of(tn);
    cur = o;
    W = outs.o[o].W;
    sw = outs.o[o].sw;
    m0 = tm * BM;
    n0 = (tn - (MULTI ? outs.tn0[o] : 0)) * BN;
    rows_x = min(BM, M - m0);
    rows_w = min(BN, outs.o[o].N - n0);
    rsx = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(X + int64_t(m0) * K), short(0), rows_x * K,
                                            kBufFlags);
    rsw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(W + int64_t(n0) * Kb), short(0), rows_w * Kb,
                                            kBufFlags);
  };
  // EVEN (K a multiple of 256, so the steps pair up with no partial stage):
  // the stage's K offset goes into the instruction's scalar offset and each
  // load is one scalar M0 update plus the load itself.  Otherwise every
  // 16-byte chunk is range-checked per lane.

  // Load block b (1 KB) holds rows 8b..8b+7 of 128-byte rows (16b..16b+15
  // of 64-byte packed int4 rows); lane i writes LDS byte 16 i of the block,
  // i.e. a fixed position of one row, which holds the source chunk that the
  // row's swizzle puts there.  kw/kx: first K value of the lane's chunk.
  unsigned offw[C::W_LOADS], offx[C::X_LOADS];
  int kw[C::W_LOADS], kx[C::X_LOADS];
#pragma unroll
  for (int j = 0; j < C::W_LOADS; ++j) {
    if constexpr (W4) {
      const int r = (wave * C::W_LOADS + j) * 16 + (lane >> 2);
      const int c = (lane & 3) ^ swz64(r);
      kw[j] = 32 * c;
      offw[j] = unsigned(r * Kb + 16 * c);
    } else {
      const int r = (wave * C::W_LOADS + j) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz128(r);
      kw[j] = 16 * c;
      offw[j] = unsigned(r * K + 16 * c);
    }
  }
#pragma unroll
  for (int j = 0; j < C::X_LOADS; ++j) {
    const int r = (wave * C::X_LOADS + j) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz128(r);
    kx[j] = 16 * c;
    offx[j] = unsigned(r * K + 16 * c);
  }
  // Descriptors with no records: the loop's prefetches of the stages past
  // the end of K go through them, so they read zeros without touching memory.
  const __amdgpu_buffer_rsrc_t rsx0 = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(X), short(0), 0,
                                                                        kBufFlags);
  const __amdgpu_buffer_rsrc_t rsw0 = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(W), short(0), 0,
                                                                        kBufFlags);
  // Loads of one stage in a fixed order (token blocks, then weight blocks);
  // q selects which of them: [Q0, Q1).
  auto issue = [&](int s, int k0, auto q0, auto q1) {
    constexpr int Q0 = decltype(q0)::value, Q1 = decltype(q1)::value;
    int8_t* const sW = bufw(s);
    int8_t* const sX = bufx(s);
    const bool live = k0 < K;  // uniform
    const __amdgpu_buffer_rsrc_t rx = live ? rsx : rsx0;
    const __amdgpu_buffer_rsrc_t rw = live ? rsw : rsw0;
#pragma unroll
    for (int q = Q0; q < Q1; ++q) {
      if (q < C::X_LOADS) {
        const int j = q;
        lds_ptr_t dst = (lds_ptr_t)(sX + (wave * C::X_LOADS + j) * 1024);
        if constexpr (EVEN) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, dst, 16, offx[j], k0, 0, 0);
        } else {
          const unsigned off = (k0 + kx[j] < K) ? offx[j] + unsigned(k0) : kOOB;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsx, dst, 16, off, 0, 0, 0);
        }
      } else {
        const int j = q - C::X_LOADS;
        lds_ptr_t dst = (lds_ptr_t)(sW + (wave * C::W_LOADS + j) * 1024);
        const int kwb = W4 ? k0 / 2 : k0;  // byte offset of the stage in a weight row
        if constexpr (EVEN) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, dst, 16, offw[j], kwb, 0, 0);
        } else {
          const unsigned off = (k0 + kw[j] < K) ? offw[j] + unsigned(kwb) : kOOB;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, dst, 16, off, 0, 0, 0);
        }
      }
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using IP2 = std::integral_constant<int, P2>;
  using IL = std::integral_constant<int, L>;

  // K order inside a stage.  int8 weights: slice sl, lane half h takes the
  // 16 K values of chunk 2 sl + h.  int4 weights: a lane reads 16 packed
  // bytes (32 K values) per pair of slices, so slice sl = 2 p + s', half h
  // takes K values 64 p + 32 h + 16 s' .. +16 (token chunk 4 p + 2 h + s',
  // weight chunk 2 p + h of the 64-byte packed row).  Both operands use the
  // same order, which leaves every dot product unchanged.  Addresses below
  // are for slice 0; the slice is applied by XOR (it only flips chunk bits).
  int wadr[TI], xadr[TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int r = wn * WN + i * 32 + row;
    wadr[i] = W4 ? r * 64 + 16 * (half ^ swz64(r)) : r * 128 + 16 * (half ^ swz128(r));
  }
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int r = wm * WM + j * 32 + row;
    xadr[j] = r * 128 + 16 * ((W4 ? 2 * half : half) ^ swz128(r));
  }
  auto xslice = [](int sl) { return W4 ? 16 * (sl & 1) + 64 * (sl >> 1) : 32 * sl; };

  v4i fa[2][TI], fb[2][TJ];
  uint4 pw[TI];  // int4 weights: packed bytes of the current slice pair
  auto read = [&](int s, int sl, int b) {
    const int8_t* bw = bufw(s);
    const int8_t* bx = bufx(s);
    if constexpr (W4) {
      if ((sl & 1) == 0) {
#pragma unroll
        for (int i = 0; i < TI; ++i) pw[i] = *reinterpret_cast<const uint4*>(bw + (wadr[i] ^ (16 * sl)));
      }
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        uint32_t o[4];
        unpack4((sl & 1) ? pw[i].z : pw[i].x, o[0], o[1]);
        unpack4((sl & 1) ? pw[i].w : pw[i].y, o[2], o[3]);
        fa[b][i] = v4i{int(o[0]), int(o[1]), int(o[2]), int(o[3])};
      }
    } else {
#pragma unroll
      for (int i = 0; i < TI; ++i) fa[b][i] = *reinterpret_cast<const v4i*>(bw + (wadr[i] ^ (32 * sl)));
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) fb[b][j] = *reinterpret_cast<const v4i*>(bx + (xadr[j] ^ xslice(sl)));
  };

  using AccT = std::conditional_t<BF, v16f, v16i>;
  AccT acc[TI][TJ];
  auto mfma = [&](int b) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        if constexpr (BF)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, fa[b][i]),
                                                              __builtin_bit_cast(v8bf, fb[b][j]), acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[b][i], fb[b][j], acc[i][j], 0, 0, 0);
  };
  auto sync_stage = [&]() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0), vmcnt/expcnt untouched
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // LDS reads when fetching an even / odd slice (int4 weights are read once
  // per slice pair).
  constexpr int NM = C::NM, ND0 = TI + TJ, ND1 = W4 ? TJ : TI + TJ;
  constexpr int NA = W4 ? 10 * TI : 0;  // unpack VALU per slice of int4 weights (two-stage loop)
  const int ksteps = EVEN ? K / 128 : ((K + 127) / 128 + 1) & ~1;  // even: the loop body covers two steps

  // Epilogue staging: a dedicated LDS area when it fits beside the stage
  // buffers (then both of the next tile's first loads can go out before the
  // epilogue), else the stage-1 arrays (then only stage 0's).
  constexpr int NQ = WN / 8;
  constexpr int P = (NQ == 12) ? 208 : WN * 2;
  constexpr int STG = (32 * P + 1023) / 1024 * 1024;
  constexpr bool DEDICATED = NS == 2 && BM == 256 && 2 * (C::W_BYTES + C::X_BYTES) + 2048 + 4 * STG <= 160 * 1024;
  __shared__ __attribute__((aligned(1024))) int8_t sStg[DEDICATED ? 4 * STG : 16];
  static_assert(DEDICATED || 2 * STG <= C::X_BYTES, "two staging blocks must fit the stage-1 token array");
  static_assert(DEDICATED || 2 * STG <= C::W_BYTES, "two staging blocks must fit the stage-1 weight array");
  int8_t* const stage_buf = DEDICATED ? sStg + wave * STG : (wave < 2 ? sX1 : sW1) + (wave & 1) * STG;

  // The tile's weight-row and token scales go to LDS with one 1 KB load each
  // (waves 0 and 1); they are first read in the epilogue.
  auto load_scales = [&]() {
    if (!BF && has_y && wave < 2) {
      const float* src = wave == 0 ? sw + n0 : sx + m0;
      const int nrec = 4 * (wave == 0 ? rows_w : rows_x);
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(src), short(0), nrec,
                                                                          kBufFlags);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(wave == 0 ? sSw : sSx), 16, unsigned(lane * 16), 0,
                                               0, 0);
    }
  };

  // First tile: scales, all of stage 0, the phase-2 share of stage 1 (two
  // stages); or all of stages 0 .. NS - 2 (deeper pipelines).
  int v = blockIdx.x;
  set_tile(v);
  load_scales();
  if constexpr (NS == 2) {
    issue(0, 0, I0{}, IL{});
    issue(1, 128, I0{}, IP2{});
    wait_vmcnt<P2>();
  } else {
#pragma unroll
    for (int st = 0; st < NS - 1; ++st) issue(st, st * 128, I0{}, IL{});
    wait_vmcnt<(NS - 2) * L>();
  }
  sync_stage();

  for (;;) {
    read(0, 0, 0);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

    if constexpr (NS > 2) {
      // Step kt reads stage kt from buffer kt % NS and sends stage
      // kt + NS - 1 into the buffer step kt - 1 has freed; at its end stage
      // kt + 1 must have landed, the NS - 2 stages after it may still be in
      // flight.  Steps past the end of K read zeros.
      using IQ1 = std::integral_constant<int, C::Q1>;
      using IQ2 = std::integral_constant<int, C::Q1 + C::Q2>;
      const int ksteps_ns = (K + 128 * NS - 1) / (128 * NS) * NS;
      for (int kb = 0; kb < ksteps_ns; kb += NS) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int kt = kb + s;
          const int sf = (s + NS - 1) % NS, sn = (s + 1) % NS;
          const int kf = (kt + NS - 1) * 128;
          read(s, 1, 1);
          mfma(0);
          issue(sf, kf, I0{}, IQ1{});
          interleave_phase<NM, C::Q1, ND1>();
          read(s, 2, 0);
          mfma(1);
          issue(sf, kf, IQ1{}, IQ2{});
          interleave_phase<NM, C::Q2, ND0>();
          read(s, 3, 1);
          mfma(0);
          issue(sf, kf, IQ2{}, IL{});
          interleave_phase<NM, C::Q3, ND1>();
          wait_vmcnt<(NS - 2) * L>();
          sync_stage();
          __builtin_amdgcn_sched_barrier(0);
          read(sn, 0, 0);
          mfma(1);
          interleave_phase<NM, 0, ND0>();
        }
      }
    } else
    for (int kb = 0; kb < ksteps; kb += 2) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int kt = kb + s;
        // phase 1
        read(s, 1, 1);
        mfma(0);
        issue(s ^ 1, (kt + 1) * 128, IP2{}, IL{});
        interleave_phase<NM, C::G0, ND1, NA>();
        read(s, 2, 0);
        mfma(1);
        interleave_phase<NM, 0, ND0, NA>();
        read(s, 3, 1);
        mfma(0);
        interleave_phase<NM, 0, ND1, NA>();
        wait_vmcnt<0>();
        sync_stage();
        __builtin_amdgcn_sched_barrier(0);
        // phase 2
        issue(s, (kt + 2) * 128, I0{}, IP2{});
        read(s ^ 1, 0, 0);
        mfma(1);
        interleave_phase<NM, P2, ND0, NA>();
      }
    }
    wait_vmcnt<0>();
    sync_stage();  // every wave is done with both stage buffers

    // Start the next tile's loads so that they land during this epilogue.
    const int em0 = m0, en0 = n0, eo = cur;
    const int vn = v + G;
    const bool more = C::PERSIST && vn < T;
    if (more) {
      set_tile(vn);
      issue(0, 0, I0{}, IL{});
      if constexpr (DEDICATED) issue(1, 128, I0{}, IP2{});
    }

    // Epilogue.  Block (i, j): lane holds token m = ... + (lane & 31) and
    // weight rows n = ... + 8 g + 4 (lane >> 5) + (0..3) in accumulators
    // 4g..4g+3.  The bf16 results of one 32-token block at a time are staged
    // in LDS and leave as 16-byte row-contiguous stores (from the accumulator
    // layout a store would scatter 8-byte pieces over 32 rows).  Scales come
    // from LDS, four weight scales per read.  Each wave stages in its own
    // region and a wave's LDS operations execute in order, so no wait is
    // needed between a block's staging writes and its reads, nor before the
    // next block overwrites the region: the next block's arithmetic overlaps
    // this block's LDS round trip and stores.
    bool stores_counted = false;  // this epilogue issued exactly S_INT stores per wave
    {
      const int m0 = em0, n0 = en0;
      // This tile's output (set_tile above has moved on to the next tile).
      const int N = outs.o[eo].N, ldy = outs.o[eo].ldy;
      int32_t* const acc_out = outs.o[eo].acc;
      uint16_t* const y = outs.o[eo].y;
    if constexpr (!BF) if (has_acc) {
      const bool vec_ok = ((N | ldy) & 3) == 0;
  #pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int m = m0 + wm * WM + j * 32 + row;
        if (m >= M) continue;
  #pragma unroll
        for (int i = 0; i < TI; ++i)
  #pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int n = n0 + wn * WN + i * 32 + 8 * g + 4 * half;
            constexpr int sh = W4 ? 4 : 0;  // int4 weights accumulate 16 x the product
            const int a[4] = {acc[i][j][4 * g] >> sh, acc[i][j][4 * g + 1] >> sh, acc[i][j][4 * g + 2] >> sh,
                              acc[i][j][4 * g + 3] >> sh};
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
      if (has_y) {
        auto chunk_of = [&](int r, int q) {
          if constexpr (NQ == 16) return q ^ (r & 15);
          else if constexpr (NQ == 8) return q ^ ((r >> 1) & 7);
          else return q;
        };
        // Interior tiles (and N a multiple of 8) store without per-element checks.
        const bool interior = m0 + BM <= M && n0 + BN <= N && ((N | ldy) & 7) == 0;
        stores_counted = interior && !has_acc;
        // All scales this lane needs, read once: the staging writes below go
        // through a per-wave pointer the compiler cannot separate from the
        // scale arrays, so reads inside the block loop would be repeated.
        // (The bf16 product has no scales.)
        float4 sw4s[TI][4];
        float sxv[TJ];
        if constexpr (!BF) {
#pragma unroll
          for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g)
              sw4s[i][g] = *reinterpret_cast<const float4*>(sSw + wn * WN + 4 * half + i * 32 + 8 * g);
#pragma unroll
          for (int j = 0; j < TJ; ++j) sxv[j] = sSx[wm * WM + j * 32 + row];
        }
    #pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const float sxj = BF ? 0.f : sxv[j];
    #pragma unroll
        for (int i = 0; i < TI; ++i)
    #pragma unroll
          for (int g = 0; g < 4; ++g) {
            float f0, f1, f2, f3;
            if constexpr (BF) {
              f0 = acc[i][j][4 * g + 0];
              f1 = acc[i][j][4 * g + 1];
              f2 = acc[i][j][4 * g + 2];
              f3 = acc[i][j][4 * g + 3];
            } else {
              const float4 sw4 = sw4s[i][g];
              constexpr int sh = W4 ? 4 : 0;
              f0 = (float(acc[i][j][4 * g + 0] >> sh) * sxj) * sw4.x;
              f1 = (float(acc[i][j][4 * g + 1] >> sh) * sxj) * sw4.y;
              f2 = (float(acc[i][j][4 * g + 2] >> sh) * sxj) * sw4.z;
              f3 = (float(acc[i][j][4 * g + 3] >> sh) * sxj) * sw4.w;
            }
            const int q = i * 4 + g;
            *reinterpret_cast<uint2*>(stage_buf + row * P + 16 * chunk_of(row, q) + 8 * half) =
                make_uint2(pack_bf16x2(f0, f1), pack_bf16x2(f2, f3));
          }
        if (interior) {
    #pragma unroll
          for (int k = 0; k < 32 * NQ / 64; ++k) {
            const int id = lane + 64 * k;
            const int r = id / NQ, q = id % NQ;
            const uint4 v = *reinterpret_cast<const uint4*>(stage_buf + r * P + 16 * chunk_of(r, q));
            store_nt(y + int64_t(m0 + wm * WM + j * 32 + r) * ldy + (n0 + wn * WN + 8 * q), v);
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
              if (((N | ldy) & 7) == 0 && n + 7 < N) {
                store_nt(y + int64_t(m) * ldy + n, v);
              } else {
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    #pragma unroll
                for (int e = 0; e < 8; ++e)
                  if (n + e < N) y[int64_t(m) * ldy + n + e] = uint16_t(w[e / 2] >> (16 * (e & 1)));
              }
            }
          }
        }
      }
      }
    }
    if (!more) break;

    // Next tile: its scales (this epilogue has finished reading the old ones),
    // the rest of its first loads, then wait until stage 0 has landed.
    // Vector memory operations retire in issue order, so it is enough that
    // no more than the operations issued after stage 0 remain.  After an
    // interior epilogue those are exactly its S_INT row stores (plus the
    // stage-1 share), which need not drain before the next tile starts;
    // after an edge tile (predicated stores) everything but the stage-1
    // share is waited for.
    constexpr int S_INT = TJ * (32 * NQ / 64);
    static_assert(P2 + S_INT < 64, "vmcnt range");
    v = vn;
    sync_stage();
    load_scales();
    if constexpr (DEDICATED) {
      if (stores_counted)
        wait_vmcnt<P2 + S_INT>();
      else
        wait_vmcnt<1>();
    } else {
      issue(1, 128, I0{}, IP2{});
      if (stores_counted)
        wait_vmcnt<P2 + S_INT>();
      else
        wait_vmcnt<P2>();
    }
    sync_stage();
  }
}

// K a multiple of 256 (every group-256 linear): unchecked scalar-offset loads.
template <int BM, int BN, bool W4, bool MULTI, int NS = 2>
__global__ __launch_bounds__(kThreads, 1) void gemm_i8_k128_kernel(const int8_t* __restrict__ X,
                                                                   const float* __restrict__ sx, int M, int K,
                                                                   int tiles_m, int tiles_n, GemmOuts outs) {
  gemm_k128_body<BM, BN, W4, true, MULTI, false, NS>(X, sx, M, K, tiles_m, tiles_n, outs);
}

// Any K (a multiple of 16, of 32 for int4 weights): every chunk range-checked.
template <int BM, int BN, bool W4, bool MULTI, int NS = 2>
__global__ __launch_bounds__(kThreads, 1) void gemm_i8_k128_tail_kernel(const int8_t* __restrict__ X,
                                                                        const float* __restrict__ sx, int M, int K,
                                                                        int tiles_m, int tiles_n, GemmOuts outs) {
  gemm_k128_body<BM, BN, W4, false, MULTI, false, NS>(X, sx, M, K, tiles_m, tiles_n, outs);
}

// bf16 x bf16 -> fp32 on the same pipeline (the weight-only path's matmul):
// a stage still moves 128 bytes of every row, i.e. 64 K values, and each
// MFMA (v_mfma_f32_32x32x16_bf16) takes the same 16 bytes per lane per
// operand as the int8 one.  K here counts row BYTES.
template <int BM, int BN, bool EVEN, int NS = 2>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_k64_kernel(const int8_t* __restrict__ X, int M, int K,
                                                                    int tiles_m, int tiles_n, GemmOuts outs) {
  gemm_k128_body<BM, BN, false, EVEN, false, true, NS>(X, nullptr, M, K, tiles_m, tiles_n, outs);
}

// ---------------------------------------------------------------------------
// Eight-wave 256x384 tiles: int8 weights with one output, or the bf16 matmul
// of the weight-only path (BF: K counts row bytes, fp32 accumulators,
// y = bf16(acc)); K a multiple of 256 bytes, N a multiple of 384.  Two
// groups of four waves share the 256-token tile; group g owns weight rows
// [192 g, 192 g + 192), and inside a group the waves form the 2 x 2 grid of
// 128x96 blocks used above.  Per MFMA this asks a third fewer lines of L2
// than 256x192 (the main loop's cost follows the lines its loads request).
// The two 80 KB stages take all of LDS.
//
// With two waves per SIMD each wave reads one K-slice's fragments at a time
// (one register set: 192 accumulators leave no room for a second), and the
// other wave's MFMAs cover the LDS latency.  One barrier per 128-K step: the
// loads of stage kt + 1 go out during step kt, right after its first LDS
// reads, into the buffer the previous barrier freed, and are waited for at
// its end; the prologue sends stages 0 and 1.  The last step is peeled:
// instead of a stage it loads the tile's scales (int8 only) into the
// buffer it does not read, where the epilogue finds them.  One workgroup
// per tile; the plan is chosen where such tiles fill whole rounds of the
// CUs.  Under sustained load the main loop runs at the device's power
// limit: a schedule with fewer idle MFMA cycles runs at a lower clock
// (rocprofv3 counters: MFMA-busy times clock stays at 1.32-1.34 GHz), so
// what pays is less work around each tile and fewer bytes per MFMA.
constexpr int kW8Threads = 512;
constexpr int kW8BM = 256, kW8BN = 384;
constexpr int kW8GroupM = 8;  // M-tiles per block of the tile order

template <bool BF>
__device__ __forceinline__ void gemm_w8_body(const int8_t* __restrict__ X, const float* __restrict__ sx, int M,
                                             int K, int tiles_m, int tiles_n, const GemmOut& out) {
  constexpr int BM = kW8BM, BN = kW8BN;
  constexpr int W_BYTES = BN * 128, X_BYTES = BM * 128;  // one 128-K stage
  constexpr int WL = W_BYTES / 1024 / 8, XL = X_BYTES / 1024 / 8;  // 1 KB loads per wave and stage
  constexpr int TI = 3, TJ = 4;                                   // 128 tokens x 96 weight rows per wave
  __shared__ __attribute__((aligned(1024))) int8_t sW0[W_BYTES], sW1[W_BYTES];
  __shared__ __attribute__((aligned(1024))) int8_t sX0[X_BYTES], sX1[X_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wm = (wave >> 1) & 1, wn = wave & 1;
  const int row = lane & 31, half = lane >> 5;

  // Tile: the XCD-aware order of the kernel above, in blocks of kW8GroupM
  // M-tiles (a round of 32 tiles per XCD then spans 8 token tiles and 4
  // weight tiles).
  int tm, tn;
  {
    const int T = tiles_m * tiles_n, v = blockIdx.x;
    const int t = (T & 7) == 0 ? (v & 7) * (T >> 3) + (v >> 3) : v;
    const int nb = tiles_m / kW8GroupM, per_block = kW8GroupM * tiles_n, b = t / per_block;
    if (b < nb) {
      const int w = t - b * per_block;
      tm = b * kW8GroupM + w % kW8GroupM;
      tn = w / kW8GroupM;
    } else {
      const int h = tiles_m - nb * kW8GroupM, w = t - nb * per_block;
      tm = nb * kW8GroupM + w % h;
      tn = w / h;
    }
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int rows_x = min(BM, M - m0);  // N is a multiple of BN: weight tiles are whole
  const __amdgpu_buffer_rsrc_t rsx = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(X + int64_t(m0) * K),
                                                                       short(0), rows_x * K, kBufFlags);
  const __amdgpu_buffer_rsrc_t rsw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(out.W + int64_t(n0) * K), short(0), BN * K, kBufFlags);

  // Load block b (1 KB: rows 8b..8b+7, lane i writing LDS byte 16 i, which
  // holds the chunk the row's swizzle puts there).  The swizzle of row r
  // depends on bits 1..3 of r, so the lane offset of block b is that of
  // block b & 1 plus (b >> 1) * 16 rows, which rides in the scalar offset.
  unsigned off[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int r = 8 * p + (lane >> 3);
    off[p] = unsigned(r * K + 16 * ((lane & 7) ^ swz128(r)));
  }
  auto issue = [&](int s, int k0) {
    int8_t* const sX = s ? sX1 : sX0;
    int8_t* const sW = s ? sW1 : sW0;
#pragma unroll
    for (int j = 0; j < XL; ++j) {
      const int b = wave * XL + j;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsx, (lds_ptr_t)(sX + b * 1024), 16, off[b & 1],
                                               (b >> 1) * 16 * K + k0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < WL; ++j) {
      const int b = wave * WL + j;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, (lds_ptr_t)(sW + b * 1024), 16, off[b & 1],
                                               (b >> 1) * 16 * K + k0, 0, 0);
    }
  };
  // Weight scales (384 floats, waves 0 and 1) at byte 0 of sW0 and token
  // scales (256 floats, wave 2; rows past M read as zero) at byte 2048.
  // Only the bf16 output needs them: a call for the int32 accumulators
  // alone may pass no scales (null pointers), so nothing is read then.
  auto load_scales = [&]() {
    if (out.y && wave < 3) {
      const float* src = wave < 2 ? out.sw + n0 + 256 * wave : sx + m0;
      const int nrec = wave == 0 ? 1024 : (wave == 1 ? 4 * (BN - 256) : 4 * rows_x);
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(src), short(0), nrec,
                                                                          kBufFlags);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(sW0 + 1024 * wave), 16, unsigned(lane * 16), 0, 0,
                                               0);
    }
  };

  int wadr[TI], xadr[TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int r = grp * (BN / 2) + wn * 96 + i * 32 + row;
    wadr[i] = r * 128 + 16 * (half ^ swz128(r));
  }
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int r = wm * 128 + j * 32 + row;
    xadr[j] = r * 128 + 16 * (half ^ swz128(r));
  }
  v4i fa[TI], fb[TJ];
  using AccT = std::conditional_t<BF, v16f, v16i>;
  AccT acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  // Step kt: multiply stage kt (buffer kt & 1, K-slice by K-slice) while
  // stage kt + 1 (or, on the last step, the scales) lands in the other.
  // The step's first LDS reads go out before its loads, so the first MFMAs
  // do not wait behind the load issue; the compiler then spreads the loads
  // over the first slice's MFMAs (same-box A/B, bit-identical output:
  // M 2048 N 12288 K 4096 86.8 -> 85.5 us, M 4096 164.9 -> 162.3 us; one
  // cluster of loads after the reads, or the loads a slice later, measured
  // no gain or slower).  Stage 1 goes out in the prologue (FIRST: step 0
  // sends nothing).
  auto step = [&](int kt, auto last_c, auto first_c) {
    constexpr bool LAST = decltype(last_c)::value;
    constexpr bool FIRST = decltype(first_c)::value;
    const int s = kt & 1;
    const int8_t* const bw = s ? sW1 : sW0;
    const int8_t* const bx = s ? sX1 : sX0;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
#pragma unroll
      for (int i = 0; i < TI; ++i) fa[i] = *reinterpret_cast<const v4i*>(bw + (wadr[i] ^ (32 * sl)));
#pragma unroll
      for (int j = 0; j < TJ; ++j) fb[j] = *reinterpret_cast<const v4i*>(bx + (xadr[j] ^ (32 * sl)));
      if (sl == 0) {
        if constexpr (LAST) {
          if constexpr (!BF) load_scales();
        } else if constexpr (!FIRST) {
          issue(s ^ 1, (kt + 1) * 128);
        }
      }
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          if constexpr (BF)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, fa[i]),
                                                                __builtin_bit_cast(v8bf, fb[j]), acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // K / 128 steps, an even number: the last step reads buffer 1, so the
  // scales go to buffer 0.
  const int ksteps = K / 128;
  // The prologue sends stages 0 and 1 and waits for stage 0 only (its 10
  // loads per wave are the older half: vmcnt counts loads in order), so
  // stage 1 has all of step 0 and the prologue's wait to land (same-box A/B,
  // bit-identical output: M 2048 N 12288 K 4096 85.6 -> 84.4 us, M 4096
  // 162.3 -> 161.1 us).
  static_assert(XL + WL == 10, "loads per wave and stage");
  issue(0, 0);
  issue(1, 128);
  wait_vmcnt<XL + WL>();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  step(0, std::false_type{}, std::true_type{});
  for (int kt = 1; kt < ksteps - 1; ++kt) step(kt, std::false_type{}, std::false_type{});
  step(ksteps - 1, std::true_type{}, std::false_type{});

  // Epilogue (as above): scales from sW0, each wave's 32-token blocks staged
  // in buffer 1 (waves 0-5 in sW1, 6-7 in sX1) for 16-byte row stores.
  const float* const sSw = reinterpret_cast<const float*>(sW0);
  const float* const sSx = reinterpret_cast<const float*>(sW0 + 2048);
  const int N = out.N, ldy = out.ldy;
  const int wrow0 = n0 + grp * (BN / 2) + wn * 96;  // this wave's first weight row
  if (!BF && out.acc) {
    const bool vec_ok = ((N | ldy) & 3) == 0;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int m = m0 + wm * 128 + j * 32 + row;
      if (m >= M) continue;
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = wrow0 + i * 32 + 8 * g + 4 * half;
          int32_t* const dst = out.acc + int64_t(m) * ldy + n;
          if (vec_ok) {
            *reinterpret_cast<int4*>(dst) = make_int4(int(acc[i][j][4 * g]), int(acc[i][j][4 * g + 1]),
                                                      int(acc[i][j][4 * g + 2]), int(acc[i][j][4 * g + 3]));
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[e] = int(acc[i][j][4 * g + e]);
          }
        }
    }
  }
  if (out.y) {
    constexpr int NQ = 12, P = 208, STG = 7 * 1024;  // 96 bf16 per row: 12 chunks, padded rows
    static_assert(6 * STG <= W_BYTES && 2 * STG <= X_BYTES, "staging blocks");
    int8_t* const stage_buf = wave < 6 ? sW1 + wave * STG : sX1 + (wave - 6) * STG;
    const bool interior = m0 + BM <= M && ((N | ldy) & 7) == 0;
    float4 sw4s[TI][4];  // (the bf16 product has no scales)
    float sxv[TJ];
    if constexpr (!BF) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          sw4s[i][g] = *reinterpret_cast<const float4*>(sSw + (wrow0 - n0) + 4 * half + i * 32 + 8 * g);
#pragma unroll
      for (int j = 0; j < TJ; ++j) sxv[j] = sSx[wm * 128 + j * 32 + row];
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float f0, f1, f2, f3;
          if constexpr (BF) {
            f0 = acc[i][j][4 * g + 0];
            f1 = acc[i][j][4 * g + 1];
            f2 = acc[i][j][4 * g + 2];
            f3 = acc[i][j][4 * g + 3];
          } else {
            const float4 sw4 = sw4s[i][g];
            f0 = (float(acc[i][j][4 * g + 0]) * sxv[j]) * sw4.x;
            f1 = (float(acc[i][j][4 * g + 1]) * sxv[j]) * sw4.y;
            f2 = (float(acc[i][j][4 * g + 2]) * sxv[j]) * sw4.z;
            f3 = (float(acc[i][j][4 * g + 3]) * sxv[j]) * sw4.w;
          }
          *reinterpret_cast<uint2*>(stage_buf + row * P + 16 * (i * 4 + g) + 8 * half) =
              make_uint2(pack_bf16x2(f0, f1), pack_bf16x2(f2, f3));
        }
#pragma unroll
      for (int k = 0; k < 32 * NQ / 64; ++k) {
        const int id = lane + 64 * k;
        const int r = id / NQ, q = id % NQ;
        const int m = m0 + wm * 128 + j * 32 + r;
        const int n = wrow0 + 8 * q;
        const uint4 v = *reinterpret_cast<const uint4*>(stage_buf + r * P + 16 * q);
        if (interior) {
          store_nt(out.y + int64_t(m) * ldy + n, v);
        } else if (m < M) {
          if (((N | ldy) & 7) == 0) {
            store_nt(out.y + int64_t(m) * ldy + n, v);
          } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) out.y[int64_t(m) * ldy + n + e] = uint16_t(w[e / 2] >> (16 * (e & 1)));
          }
        }
      }
    }
  }
}

__global__ __launch_bounds__(kW8Threads, 1) void gemm_i8_w8_kernel(const int8_t* __restrict__ X,
                                                                   const float* __restrict__ sx, int M, int K,
                                                                   int tiles_m, int tiles_n, GemmOut out) {
  gemm_w8_body<false>(X, sx, M, K, tiles_m, tiles_n, out);
}

// The bf16 matmul on the same tiles (K counts row bytes).
__global__ __launch_bounds__(kW8Threads, 1) void gemm_bf16_w8_kernel(const int8_t* __restrict__ X, int M, int K,
                                                                     int tiles_m, int tiles_n, GemmOut out) {
  gemm_w8_body<true>(X, nullptr, M, K, tiles_m, tiles_n, out);
}

// Workgroups of kernel K the current device runs at once: compute units x
// resident workgroups per unit, a multiple of 8 on MI355X (256 units, one or
// two per unit), so the persistent tile order stays XCD-aware.  A read-only
// fact of the device, worked out once per device and kernel (the first call
// with that device current; later calls from any host thread only read it);
// 0 on error.
template <auto K>
int resident_slots() {
  constexpr int kDevices = 64;
  static std::once_flag once[kDevices];
  static int slots[kDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  auto query = [](int d) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(K), kThreads, 0) !=
        hipSuccess)
      return 0;
    return cus * (per_cu > 0 ? per_cu : 1);
  };
  if (dev >= kDevices) return query(dev);  // not memoised
  std::call_once(once[dev], [&] { slots[dev] = query(dev); });
  return slots[dev];
}

// One launch over the outputs in `d` (each a weight matrix with its
// outputs; all share xq).  Column tiles of the outputs are concatenated.
template <int BM, int BN, bool W4, int NS = 2>
hipError_t launch_k128(const int8_t* xq, const float* x_scale, int M, int K, const GemmOutDesc* d, int n,
                       hipStream_t stream) {
  GemmOuts outs{};
  outs.n = n;
  int tiles_n = 0;
  for (int o = 0; o < kMaxOuts; ++o) {
    outs.tn0[o] = o < n ? tiles_n : INT_MAX;
    if (o < n) {
      outs.o[o] = {static_cast<const uint8_t*>(d[o].wq), d[o].w_scale, d[o].acc, d[o].y, d[o].N, d[o].ldy};
      tiles_n += (d[o].N + BN - 1) / BN;
    }
  }
  const int tiles_m = (M + BM - 1) / BM;
  using Kernel = void (*)(const int8_t*, const float*, int, int, int, int, GemmOuts);
  constexpr Kernel k_multi = gemm_i8_k128_kernel<BM, BN, W4, true, NS>;
  constexpr Kernel k_multi_tail = gemm_i8_k128_tail_kernel<BM, BN, W4, true, NS>;
  constexpr Kernel k_one = gemm_i8_k128_kernel<BM, BN, W4, false, NS>;
  constexpr Kernel k_one_tail = gemm_i8_k128_tail_kernel<BM, BN, W4, false, NS>;
  const bool even = K % 256 == 0;
  const Kernel kernel = n > 1 ? (even ? k_multi : k_multi_tail) : (even ? k_one : k_one_tail);
  // Persistent configurations: as many workgroups as the device holds at
  // once (never more than there are tiles), each walking its tiles in turn;
  // otherwise one workgroup per tile.
  const int64_t tiles = int64_t(tiles_m) * tiles_n;
  int64_t slots = tiles;
  if (CfgK<BM, BN, W4, NS>::PERSIST) {
    slots = n > 1 ? (even ? resident_slots<k_multi>() : resident_slots<k_multi_tail>())
                  : (even ? resident_slots<k_one>() : resident_slots<k_one_tail>());
    if (slots <= 0) return hipErrorInvalidDeviceFunction;
  }
  const dim3 grid(unsigned(tiles < slots ? tiles : slots));
  hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, xq, x_scale, M, K, tiles_m, tiles_n, outs);
  return hipGetLastError();
}

// One launch of the eight-wave 256x384 kernel (int8 weights, one output,
// K % 256 == 0, N % 384 == 0): one workgroup per tile.
hipError_t launch_w8(const int8_t* xq, const float* x_scale, int M, int K, const GemmOutDesc& d,
                     hipStream_t stream) {
  const GemmOut o{static_cast<const uint8_t*>(d.wq), d.w_scale, d.acc, d.y, d.N, d.ldy};
  const int tiles_m = (M + kW8BM - 1) / kW8BM, tiles_n = d.N / kW8BN;
  hipLaunchKernelGGL(gemm_i8_w8_kernel, dim3(unsigned(int64_t(tiles_m) * tiles_n)), dim3(kW8Threads), 0, stream,
                     xq, x_scale, M, K, tiles_m, tiles_n, o);
  return hipGetLastError();
}

bool w8_fits(int64_t K, const GemmOutDesc* d, int n) {
  return n == 1 && K % 256 == 0 && d[0].N % kW8BN == 0;
}

struct TileChoice {
  int bm, bn;
  int ns = 2;  // pipeline stages
};

// Tuning builds only (-DCONVROT_TUNING): CONVROT_GEMM_TILE=<BM>x<BN>[x<stages>]
// forces one of the tile shapes above (the deeper pipelines: 256x128x3,
// 128x256x3, 128x128x3, 128x128x4, 64x128x4, 128x64x4 for int8 and int4
// weights, the first, fourth and fifth for bf16; 256x384, the eight-wave
// tiles, for int8 weights with N % 384 == 0 and K % 256 == 0), for sweeps:
// every choice gives bit-identical results.  The library as built reads no
// environment.
TileChoice tile_override() {
#ifdef CONVROT_TUNING
  static const TileChoice forced = [] {
    TileChoice t{0, 0};
    if (const char* s = getenv("CONVROT_GEMM_TILE")) {
      const int got = sscanf(s, "%dx%dx%d", &t.bm, &t.bn, &t.ns);
      if (got < 2) t = {0, 0};
      if (got == 2) t.ns = 2;
    }
    return t;
  }();
  return forced;
#else
  return TileChoice{0, 0};
#endif
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

// Tile plan, from measurements on MI355X under sustained load.  The device
// holds a lower clock under this GEMM than under MFMAs alone (feeding them
// costs power), so the largest tile (256x256: fewest L2->LDS bytes per
// operation, its main loop 87-91 % MFMA-busy against 85-86 % for 256x192) wins
// once it fills several whole rounds of the CUs;
// otherwise 256x192 when it fills at least three quarters of a round, and
// 128x128 for small problems (more CUs busy).  With a short K (fewer than 16
// stages of 128 bytes per token row) a tile's set-up and epilogue weigh as
// much as its main loop, and 128x128 wins below the 256x256 case: two of its
// workgroups share a CU and hide each other's (M 4096, K 1152, N 3456:
// 31.6 -> 26.4 us against 256x192).  Splitting N into bands of
// different tiles to even out a partial round measured no faster than a
// single 256x192 launch (the second launch waits for the first).  With
// several outputs the tiles of all of them count, and 256x256 needs every
// output's N to be a multiple of 256.
// Compute units of the current device (256 on MI355X; fewer on a
// partitioned device), queried once per device; 256 if the query fails.
int device_cus() {
  constexpr int kDevices = 64;
  static std::once_flag once[kDevices];
  static int cus[kDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevices) return 256;
  std::call_once(once[dev], [dev] {
    int c = 0;
    cus[dev] = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0 ? c : 256;
  });
  return cus[dev];
}

TileChoice choose_tile(int64_t M, int64_t ksteps, const GemmOutDesc* d, int n) {
  const int cus = device_cus();
  auto tiles = [&](int bm, int bn) {
    int64_t t = 0;
    for (int o = 0; o < n; ++o) t += (d[o].N + bn - 1) / bn;
    return ((M + bm - 1) / bm) * t;
  };
  bool n256 = true;
  for (int o = 0; o < n; ++o) n256 = n256 && d[o].N % 256 == 0;
  if (n256 && tiles(256, 256) >= 3 * cus) return {256, 256};
  if (ksteps >= 16 && 4 * tiles(256, 192) >= 3 * cus) return {256, 192};
  // Deeper pipelines (int8, int4 and bf16 operands) for tiles that sit
  // alone on their CU, where nothing else hides the load latency (int4,
  // M 512, K 4096, N 4096: 26.9 -> 15.4 us; bf16, same shape: 54.1 ->
  // 26.5 us): 256x128 with three
  // stages when its tiles fill between three quarters of the CUs and all of
  // them (M 2048, K 12288, N 4096: 256 tiles, 120.5 -> 99.8 us against
  // two-stage 128x128); for small problems the smallest tile that still
  // leaves at most one per CU, with four stages (M 512, K 4096, N 4096:
  // 64x128, 31.4 -> 17.0 us; M 1024, K 4096, N 4096: 128x128, 23.2 us
  // against 32.9 for 64x128 in two rounds).  With more tiles two two-stage
  // 128x128 workgroups share each CU and are as fast or faster.
  if (ksteps >= 16 && 4 * tiles(256, 128) >= 3 * cus && tiles(256, 128) <= cus) return {256, 128, 3};
  if (tiles(64, 128) <= cus) return {64, 128, 4};
  if (tiles(128, 128) <= cus) return {128, 128, 4};
  return {128, 128};
}

// Rows of M that one output gives to the eight-wave 256x384 tiles (int8
// weights; the bf16 matmul with K in bytes), which take one tile per
// workgroup and need K to have at least 16 stages: all of them where the
// tiles make whole rounds of the CUs; otherwise, where two or more whole
// rounds fit, the longest run of whole token tiles whose tiles fill whole
// rounds, the remaining rows (less than a round's worth of tiles) planned
// as a GEMM of their own in a second launch; else none.  Same box,
// interleaved, bit-identical outputs: M 2048, K 4096, N 12288 (one round)
// 95.7 -> 87.2 us against 256x192; M 4096 (two rounds) 176.2 -> 173.8 us
// and M 6144 (three) 252 -> 232 us against 256x256.  A partial round, with
// no second tile per CU to overlap the last tiles' epilogues, gains
// nothing: M 8704 (4.25 rounds) 361 us in one launch, 355-361 us on 256x256
// tiles, 338 us with 8192 rows on these tiles and 512 on the ordinary plan.
int64_t w8_rows(int64_t M, int64_t K, const GemmOutDesc& d) {
  if (K % 256 != 0 || d.N % kW8BN != 0 || K / 128 < 16) return 0;
  const int64_t cus = device_cus(), tn = d.N / kW8BN, tm = (M + kW8BM - 1) / kW8BM;
  if ((tm * tn) % cus == 0) return M;
  int64_t per_round = 1;  // token tiles whose tiles fill whole rounds
  while ((per_round * tn) % cus != 0) ++per_round;
  const int64_t m0 = (M / kW8BM) / per_round * per_round;
  return m0 * tn >= 2 * cus ? m0 * kW8BM : 0;
}

// Tuning builds only (-DCONVROT_TUNING):
// CONVROT_GEMM_PLAN=<BM>x<BN>[:<cols>][,<BM>x<BN>] forces a plan for a single
// output, for sweeps (every plan gives bit-identical results).
bool plan_override(Plan& out) {
#ifdef CONVROT_TUNING
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
#else
  (void)out;
  return false;
#endif
}

template <bool W4>
hipError_t launch_tile(TileChoice tc, const int8_t* xq, const float* x_scale, int M, int K, const GemmOutDesc* d,
                       int n, hipStream_t stream) {
  // Eight-wave 256x384 tiles (int8 weights; others take 256x192).
  if (tc.bm == 256 && tc.bn == 384) {
    if (!W4 && w8_fits(K, d, n)) return launch_w8(xq, x_scale, M, K, d[0], stream);
    tc = {256, 192};
  }
  // Deeper pipelines (one tile per workgroup).
  if (tc.ns == 3 && tc.bm == 256 && tc.bn == 128) return launch_k128<256, 128, W4, 3>(xq, x_scale, M, K, d, n, stream);
  if (tc.ns == 3 && tc.bm == 128 && tc.bn == 256) return launch_k128<128, 256, W4, 3>(xq, x_scale, M, K, d, n, stream);
  if (tc.ns == 4 && tc.bm == 128 && tc.bn == 128) return launch_k128<128, 128, W4, 4>(xq, x_scale, M, K, d, n, stream);
  if (tc.ns == 3 && tc.bm == 128 && tc.bn == 128) return launch_k128<128, 128, W4, 3>(xq, x_scale, M, K, d, n, stream);
  if (tc.ns == 4 && tc.bm == 64 && tc.bn == 128) return launch_k128<64, 128, W4, 4>(xq, x_scale, M, K, d, n, stream);
  if (tc.ns == 4 && tc.bm == 128 && tc.bn == 64) return launch_k128<128, 64, W4, 4>(xq, x_scale, M, K, d, n, stream);
  if (tc.bm == 256 && tc.bn == 256) return launch_k128<256, 256, W4>(xq, x_scale, M, K, d, n, stream);
  if (tc.bm == 256 && tc.bn == 192) return launch_k128<256, 192, W4>(xq, x_scale, M, K, d, n, stream);
  if (tc.bm == 256 && tc.bn == 128) return launch_k128<256, 128, W4>(xq, x_scale, M, K, d, n, stream);
  if (tc.bm == 128 && tc.bn == 256) return launch_k128<128, 256, W4>(xq, x_scale, M, K, d, n, stream);
  return launch_k128<128, 128, W4>(xq, x_scale, M, K, d, n, stream);
}

template <bool W4>
hipError_t launch_plan(const int8_t* xq, const float* x_scale, int M, int K, const GemmOutDesc* d, int n,
                       hipStream_t stream) {
  Plan plan;
  if (n == 1 && plan_override(plan)) {
    // Bands of one output's columns, each its own launch (row stride N).
    const GemmOutDesc& o = d[0];
    const int64_t row_bytes = W4 ? K / 2 : K;
    int n_begin = 0;
    for (int i = 0; i < plan.nb && n_begin < o.N; ++i) {
      const int cols = (plan.b[i].n_cols > 0 && n_begin + plan.b[i].n_cols < o.N) ? plan.b[i].n_cols : o.N - n_begin;
      const GemmOutDesc band{static_cast<const uint8_t*>(o.wq) + n_begin * row_bytes,
                             o.w_scale ? o.w_scale + n_begin : nullptr, cols, o.ldy,
                             o.acc ? o.acc + n_begin : nullptr, o.y ? o.y + n_begin : nullptr};
      const hipError_t e = launch_tile<W4>(plan.b[i].tc, xq, x_scale, M, K, &band, 1, stream);
      if (e != hipSuccess) return e;
      n_begin += cols;
    }
    return hipSuccess;
  }
  const TileChoice forced = tile_override();
  if (!W4 && !forced.bm) {
    // Eight-wave tiles (w8_rows) for every output, or for none: outputs
    // that all qualify run one after the other, each in its own launches.
    int64_t rows[kMaxOuts];
    bool all = true;
    for (int o = 0; o < n; ++o) all = all && (rows[o] = w8_rows(M, K, d[o])) > 0;
    if (all) {
      for (int o = 0; o < n; ++o) {
        const int r = int(rows[o]);
        hipError_t e = launch_w8(xq, x_scale, r, K, d[o], stream);
        if (e == hipSuccess && r < M) {
          const GemmOutDesc rest{d[o].wq, d[o].w_scale, d[o].N, d[o].ldy,
                                 d[o].acc ? d[o].acc + int64_t(r) * d[o].ldy : nullptr,
                                 d[o].y ? d[o].y + int64_t(r) * d[o].ldy : nullptr};
          const TileChoice tc = choose_tile(M - r, (int64_t(K) + 127) / 128, &rest, 1);
          e = launch_tile<W4>(tc, xq + int64_t(r) * K, x_scale ? x_scale + r : nullptr, M - r, K, &rest, 1, stream);
        }
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    }
  }
  const TileChoice tc = forced.bm ? forced : choose_tile(M, (int64_t(K) + 127) / 128, d, n);
  // Where the planner takes persistent 256x192 tiles for int8 weights and
  // 256x256 tiles would fill two or more whole rounds of the CUs on the
  // first rows, those rows take 256x256 tiles and the rest are planned as
  // a GEMM of their own (same-box A/B, bit-identical output, M 8704, N 4096:
  // K 12288 393-398 -> 364 us, K 4096 141 -> 131 us; 256x256 tiles fill
  // 2.1 rounds there).
  if (!W4 && !forced.bm && n == 1 && tc.bm == 256 && tc.bn == 192 && d[0].N % 256 == 0 && K / 128 >= 16) {
    const int64_t cus = device_cus(), tn = d[0].N / 256;
    int64_t per_round = 1;  // token tiles whose tiles fill whole rounds
    while ((per_round * tn) % cus != 0) ++per_round;
    const int64_t m0 = (M / 256) / per_round * per_round;
    if (m0 * tn >= 2 * cus) {
      const int r = int(m0 * 256);
      const hipError_t e = launch_tile<W4>(TileChoice{256, 256}, xq, x_scale, r, K, d, 1, stream);
      if (e != hipSuccess || r == M) return e;
      const GemmOutDesc rest{d[0].wq, d[0].w_scale, d[0].N, d[0].ldy,
                             d[0].acc ? d[0].acc + int64_t(r) * d[0].ldy : nullptr,
                             d[0].y ? d[0].y + int64_t(r) * d[0].ldy : nullptr};
      const TileChoice tr = choose_tile(M - r, (int64_t(K) + 127) / 128, &rest, 1);
      return launch_tile<W4>(tr, xq + int64_t(r) * K, x_scale ? x_scale + r : nullptr, M - r, K, &rest, 1, stream);
    }
  }
  return launch_tile<W4>(tc, xq, x_scale, M, K, d, n, stream);
}

template <int BM, int BN, int NS = 2>
hipError_t launch_bf16(const uint16_t* x, const uint16_t* w, int M, int N, int K, uint16_t* y, hipStream_t stream) {
  GemmOuts outs{};
  outs.n = 1;
  outs.o[0] = {reinterpret_cast<const uint8_t*>(w), nullptr, nullptr, y, N, N};
  for (int o = 0; o < kMaxOuts; ++o) outs.tn0[o] = o ? INT_MAX : 0;
  const int kbytes = 2 * K;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  using Kernel = void (*)(const int8_t*, int, int, int, int, GemmOuts);
  constexpr Kernel k_even = gemm_bf16_k64_kernel<BM, BN, true, NS>;
  constexpr Kernel k_any = gemm_bf16_k64_kernel<BM, BN, false, NS>;
  const bool even = kbytes % 256 == 0;
  const Kernel kernel = even ? k_even : k_any;
  const int64_t tiles = int64_t(tiles_m) * tiles_n;
  int64_t slots = tiles;
  if (CfgK<BM, BN, false, NS>::PERSIST) {
    slots = even ? resident_slots<k_even>() : resident_slots<k_any>();
    if (slots <= 0) return hipErrorInvalidDeviceFunction;
  }
  const dim3 grid(unsigned(tiles < slots ? tiles : slots));
  hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, reinterpret_cast<const int8_t*>(x), M, kbytes,
                     tiles_m, tiles_n, outs);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const uint16_t* x, const uint16_t* w, int64_t M, int64_t N, int64_t K, uint16_t* y,
                            hipStream_t stream) {
  const GemmOutDesc d{w, nullptr, int(N), int(N), nullptr, y};
  const TileChoice forced = tile_override();
  // Eight-wave 256x384 tiles on the rows w8_rows gives them (K in bytes),
  // the rest planned as a GEMM of its own.  Same box, interleaved,
  // identical outputs: M 2048, K 4096, N 12288 (one round) 174.8 -> 161.2 us
  // against 256x192; M 6144 (three rounds) 471.8 -> 454.2 us against
  // 256x256; M 4096 and M 8704 within 0.4 % of 256x256.
  const int64_t w8r = forced.bm ? 0 : w8_rows(M, 2 * K, d);
  if (w8r > 0) {
    const GemmOut o{reinterpret_cast<const uint8_t*>(w), nullptr, nullptr, y, int(N), int(N)};
    const int tiles_m = int((w8r + kW8BM - 1) / kW8BM), tiles_n = int(N / kW8BN);
    hipLaunchKernelGGL(gemm_bf16_w8_kernel, dim3(unsigned(int64_t(tiles_m) * tiles_n)), dim3(kW8Threads), 0, stream,
                       reinterpret_cast<const int8_t*>(x), int(w8r), int(2 * K), tiles_m, tiles_n, o);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || w8r == M) return e;
    return launch_gemm_bf16(x + w8r * K, w, M - w8r, N, K, y + w8r * N, stream);
  }
  const TileChoice tc = forced.bm ? forced : choose_tile(M, (2 * K + 127) / 128, &d, 1);
  if (tc.ns == 3 && tc.bm == 256 && tc.bn == 128) return launch_bf16<256, 128, 3>(x, w, int(M), int(N), int(K), y, stream);
  if (tc.ns == 4 && tc.bm == 128 && tc.bn == 128) return launch_bf16<128, 128, 4>(x, w, int(M), int(N), int(K), y, stream);
  if (tc.ns == 4 && tc.bm == 64 && tc.bn == 128) return launch_bf16<64, 128, 4>(x, w, int(M), int(N), int(K), y, stream);
  if (tc.bm == 256 && tc.bn == 256) return launch_bf16<256, 256>(x, w, int(M), int(N), int(K), y, stream);
  if (tc.bm == 256 && tc.bn == 192) return launch_bf16<256, 192>(x, w, int(M), int(N), int(K), y, stream);
  if (tc.bm == 256 && tc.bn == 128) return launch_bf16<256, 128>(x, w, int(M), int(N), int(K), y, stream);
  if (tc.bm == 128 && tc.bn == 256) return launch_bf16<128, 256>(x, w, int(M), int(N), int(K), y, stream);
  return launch_bf16<128, 128>(x, w, int(M), int(N), int(K), y, stream);
}

hipError_t launch_gemm(const int8_t* xq, const float* x_scale, const void* wq, int wbits, const float* w_scale,
                       int64_t M, int64_t N, int64_t K, int32_t* acc_out, uint16_t* y, hipStream_t stream) {
  const GemmOutDesc d{wq, w_scale, int(N), int(N), acc_out, y};
  return launch_gemm_multi(xq, x_scale, wbits, M, K, &d, 1, stream);
}

hipError_t launch_gemm_multi(const int8_t* xq, const float* x_scale, int wbits, int64_t M, int64_t K,
                             const GemmOutDesc* outs, int n_outs, hipStream_t stream) {
  if (n_outs < 1 || n_outs > kMaxOuts) return hipErrorInvalidValue;
  if (wbits == 4) return launch_plan<true>(xq, x_scale, int(M), int(K), outs, n_outs, stream);
  return launch_plan<false>(xq, x_scale, int(M), int(K), outs, n_outs, stream);
}

}  // namespace convrot
