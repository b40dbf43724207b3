// Measurement helper (not part of the library): a streaming pass that moves
// exactly the bytes of a group-256 rotate-quantize pass, with none of its
// arithmetic.  It reads a bf16 [M, K] matrix, writes one byte per value
// (the high byte of each bf16 word: a data-dependent result, so no load can
// be dropped) and one fp32 per row: 3K + 4 bytes per row, the quantizer's
// algorithmic traffic.  Each lane moves 16 consecutive values (two 16-byte
// nontemporal loads, one 16-byte nontemporal store), as the quantizer's
// lanes do.  The bench times it beside each graded pass: the rate a plain
// streaming kernel reaches when it moves that pass's bytes.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void move_chunk(const u32x4* __restrict__ in, u32x4* __restrict__ out, int64_t c) {
  const u32x4 a = __builtin_nontemporal_load(in + 2 * c);
  const u32x4 b = __builtin_nontemporal_load(in + 2 * c + 1);
  // high byte of each of the 16 bf16 words, in order
  const u32x4 o = {__builtin_amdgcn_perm(a.y, a.x, 0x07050301u), __builtin_amdgcn_perm(a.w, a.z, 0x07050301u),
                   __builtin_amdgcn_perm(b.y, b.x, 0x07050301u), __builtin_amdgcn_perm(b.w, b.z, 0x07050301u)};
  __builtin_nontemporal_store(o, out + c);
}

// One chunk of 16 values per thread (mode 0), or a grid-stride walk over
// the chunks by a grid of `blocks` workgroups (mode 1).  The first lane of
// each row also writes the row's fp32 word.
__global__ __launch_bounds__(256) void stream_rq_kernel(const u32x4* __restrict__ in, u32x4* __restrict__ out,
                                                        float* __restrict__ rowv, int64_t chunks,
                                                        int64_t chunks_per_row) {
  const int64_t stride = int64_t(gridDim.x) * 256;
  for (int64_t c = int64_t(blockIdx.x) * 256 + threadIdx.x; c < chunks; c += stride) {
    move_chunk(in, out, c);
    if (c % chunks_per_row == 0) __builtin_nontemporal_store(1.0f, rowv + c / chunks_per_row);
  }
}

}  // namespace

// x: bf16 bits [M, K] (16-byte aligned), q: bytes [M, K], v: fp32 [M];
// K a multiple of 16.  mode 0: one 16-value chunk per thread; mode 1: a
// grid of `blocks` workgroups walks the chunks.  Returns 0, or 1 for bad
// arguments, 6 for a launch error.
extern "C" int stream_rq_launch(const void* x, void* q, float* v, int64_t M, int64_t K, int mode, int blocks,
                                hipStream_t stream) {
  if (!x || !q || !v || M <= 0 || K <= 0 || K % 16 != 0 || (mode != 0 && mode != 1)) return 1;
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(q)) % 16 != 0) return 1;
  const int64_t chunks = M * (K / 16);
  const int64_t grid = mode == 0 ? (chunks + 255) / 256 : blocks;
  if (grid <= 0 || grid > (int64_t(1) << 31) - 1) return 1;
  hipLaunchKernelGGL(stream_rq_kernel, dim3(unsigned(grid)), dim3(256), 0, stream, static_cast<const u32x4*>(x),
                     static_cast<u32x4*>(q), v, chunks, K / 16);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}
