// C-ABI layer: argument validation, workspace layout and kernel launches.
// Validation runs on the host before anything is enqueued, so a non-zero
// status means nothing was written.
#include "../../include/convrot.h"

#include "convrot_internal.h"

#include <mutex>

// Scratch area of the allocation-free linear (convrot_w8a8_linear_noalloc):
// the quantized activations and token scales.  Each GPU the library runs on
// holds its own copy for the life of the process.  In host code this name
// stands for the array but is not its device address: host code uses only
// the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[CONVROT_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int log2_group(int group) {
  if (group < 1 || group > 256 || (group & (group - 1)) != 0) return -1;
  int l = 0;
  while ((1 << l) < group) ++l;
  return l;
}

// Shape rules shared by every call that rotates or multiplies along K.
int check_k(int64_t K, int group, bool int4) {
  if (log2_group(group) < 0) return CONVROT_ERR_GROUP;
  if (K <= 0 || K % 16 != 0 || K % group != 0 || K > CONVROT_MAX_K) return CONVROT_ERR_SHAPE;
  if (int4 && K % 32 != 0) return CONVROT_ERR_SHAPE;
  return CONVROT_OK;
}

int device_status(hipError_t e) { return e == hipSuccess ? CONVROT_OK : CONVROT_ERR_DEVICE; }

// The GEMM indexes tiles, rows and columns with 32-bit integers.
constexpr int64_t kMaxRows = int64_t(1) << 30;

// Output tiles of the smallest tile shape (128 x 128) must count below 2^31.
bool tiles_fit(int64_t M, int64_t col_tiles) { return ((M + 127) / 128) * col_tiles < (int64_t(1) << 31); }

// Checks shared by the multi-output calls (shapes, then pointers, then
// alignment; the pointer checks are skipped for M == 0).
int check_outs(int64_t M, const convrot_linear_out* outs, int n_outs, bool linear) {
  if (n_outs < 1 || n_outs > CONVROT_MAX_OUTS) return CONVROT_ERR_ARG;
  if (!outs) return CONVROT_ERR_NULL;
  int64_t col_tiles = 0;
  for (int o = 0; o < n_outs; ++o) {
    if (outs[o].N <= 0 || outs[o].N > kMaxRows) return CONVROT_ERR_SHAPE;
    col_tiles += (outs[o].N + 127) / 128;
  }
  if (!tiles_fit(M, col_tiles)) return CONVROT_ERR_SHAPE;
  if (M == 0) return CONVROT_OK;
  const bool has_y = outs[0].y != nullptr, has_acc = outs[0].acc_out != nullptr;
  if (linear && !has_y) return CONVROT_ERR_NULL;
  if (!has_y && !has_acc) return CONVROT_ERR_NULL;
  for (int o = 0; o < n_outs; ++o) {
    const convrot_linear_out& d = outs[o];
    if (!d.wq || (d.y != nullptr) != has_y || (d.acc_out != nullptr) != has_acc) return CONVROT_ERR_NULL;
    if (has_y && !d.w_scale) return CONVROT_ERR_NULL;
  }
  for (int o = 0; o < n_outs; ++o) {
    const convrot_linear_out& d = outs[o];
    if (!aligned(d.wq, 16) || (d.y && !aligned(d.y, 16)) || (d.acc_out && !aligned(d.acc_out, 16)) ||
        (d.w_scale && !aligned(d.w_scale, 4)))
      return CONVROT_ERR_ALIGN;
  }
  return CONVROT_OK;
}

hipError_t launch_outs(const int8_t* xq, const float* xs, int wbits, int64_t M, int64_t K,
                       const convrot_linear_out* outs, int n_outs, hipStream_t stream) {
  convrot::GemmOutDesc d[CONVROT_MAX_OUTS];
  for (int o = 0; o < n_outs; ++o)
    d[o] = {outs[o].wq, outs[o].w_scale, int(outs[o].N), int(outs[o].N), outs[o].acc_out, outs[o].y};
  return convrot::launch_gemm_multi(xq, xs, wbits, M, K, d, n_outs, stream);
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; nullptr if the lookup failed.
constexpr int kScratchDevices = 64;
std::once_flag scratch_once[kScratchDevices];
void* scratch_ptr[kScratchDevices];

void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return nullptr;
  std::call_once(scratch_once[dev], [dev] {
    void* p = nullptr;
    scratch_ptr[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess ? p : nullptr;
  });
  return scratch_ptr[dev];
}

}  // namespace

extern "C" {

int convrot_version(void) { return 103; }

const char* convrot_status_string(int status) {
  switch (status) {
    case CONVROT_OK: return "ok";
    case CONVROT_ERR_NULL: return "a required pointer is NULL";
    case CONVROT_ERR_SHAPE: return "invalid shape (need M >= 0, N > 0, K > 0, K % 16 == 0, K % group == 0, "
                                   "K <= 32768, K % 32 == 0 for int4 weights, and M, N <= 2^30 for the "
                                   "product)";
    case CONVROT_ERR_GROUP: return "group must be a power of two in [1, 256]";
    case CONVROT_ERR_ALIGN: return "tensor pointers must be 16-byte aligned (scales 4-byte aligned)";
    case CONVROT_ERR_WORKSPACE: return "workspace smaller than the call's workspace size";
    case CONVROT_ERR_DEVICE: return "the HIP runtime reported an error";
    case CONVROT_ERR_DTYPE: return "unsupported weight dtype or bit width";
    case CONVROT_ERR_ARG: return "a scalar argument is out of range (eps negative or not finite, or n_outs "
                                 "outside [1, 8])";
    case CONVROT_ERR_SCRATCH: return "input too large for the allocation-free call: convrot_workspace_size(M, K) "
                                     "exceeds CONVROT_NOALLOC_SCRATCH_BYTES (64 MiB)";
    default: return "unknown convrot status";
  }
}

size_t convrot_workspace_size(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0) return 0;
  return round_up(size_t(M) * size_t(K), kAlign) + round_up(size_t(M) * sizeof(float), kAlign);
}

int convrot_quantize_weight(const void* w, int w_dtype, int64_t N, int64_t K, int group, int bits, void* wq,
                            float* w_scale, hipStream_t stream) {
  if (w_dtype != CONVROT_W_F32 && w_dtype != CONVROT_W_BF16) return CONVROT_ERR_DTYPE;
  if (bits != 8 && bits != 4) return CONVROT_ERR_DTYPE;
  if (int rc = check_k(K, group, bits == 4)) return rc;
  if (N < 0) return CONVROT_ERR_SHAPE;
  if (N == 0) return CONVROT_OK;
  if (!w || !wq || !w_scale) return CONVROT_ERR_NULL;
  if (!aligned(w, 16) || !aligned(wq, 16) || !aligned(w_scale, 4)) return CONVROT_ERR_ALIGN;
  const int lg = log2_group(group);
  if (bits == 8)
    return device_status(convrot::launch_rotate_quant(w, w_dtype, N, K, lg, static_cast<int8_t*>(wq), w_scale,
                                                      stream));
  return device_status(convrot::launch_quantize_weight_i4(w, w_dtype, N, K, lg, static_cast<uint8_t*>(wq),
                                                          w_scale, nullptr, stream));
}

// Same as convrot_quantize_weight(bits = 4) but also reports the winning clip
// candidate per row (c = 1 - index/100); used by the tests.
int convrot_quantize_weight_i4_clip(const void* w, int w_dtype, int64_t N, int64_t K, int group, uint8_t* wq4,
                                    float* w_scale, int32_t* clip_index, hipStream_t stream) {
  if (w_dtype != CONVROT_W_F32 && w_dtype != CONVROT_W_BF16) return CONVROT_ERR_DTYPE;
  if (int rc = check_k(K, group, true)) return rc;
  if (N < 0) return CONVROT_ERR_SHAPE;
  if (N == 0) return CONVROT_OK;
  if (!w || !wq4 || !w_scale || !clip_index) return CONVROT_ERR_NULL;
  if (!aligned(w, 16) || !aligned(wq4, 16) || !aligned(w_scale, 4) || !aligned(clip_index, 4))
    return CONVROT_ERR_ALIGN;
  return device_status(convrot::launch_quantize_weight_i4(w, w_dtype, N, K, log2_group(group), wq4, w_scale,
                                                          clip_index, stream));
}

int convrot_rotate_quant(const uint16_t* x, int64_t M, int64_t K, int group, int8_t* xq, float* x_scale,
                         hipStream_t stream) {
  if (int rc = check_k(K, group, false)) return rc;
  if (M < 0) return CONVROT_ERR_SHAPE;
  if (M == 0) return CONVROT_OK;
  if (!x || !xq || !x_scale) return CONVROT_ERR_NULL;
  if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(x_scale, 4)) return CONVROT_ERR_ALIGN;
  return device_status(
      convrot::launch_rotate_quant(x, CONVROT_W_BF16, M, K, log2_group(group), xq, x_scale, stream));
}

int convrot_rmsnorm_rotate_quant(const uint16_t* x, const float* norm_w, float eps, int64_t M, int64_t K,
                                 int group, int8_t* xq, float* x_scale, uint16_t* y_norm, hipStream_t stream) {
  if (int rc = check_k(K, group, false)) return rc;
  if (M < 0) return CONVROT_ERR_SHAPE;
  if (!(eps >= 0.0f) || !(eps <= 3.4028234663852886e38f)) return CONVROT_ERR_ARG;
  if (M == 0) return CONVROT_OK;
  if (!x || !norm_w || !xq || !x_scale) return CONVROT_ERR_NULL;
  if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(x_scale, 4) || !aligned(norm_w, 16) ||
      (y_norm && !aligned(y_norm, 16)))
    return CONVROT_ERR_ALIGN;
  return device_status(convrot::launch_rmsnorm_rotate_quant(x, norm_w, eps, M, K, log2_group(group), xq, x_scale,
                                                            y_norm, stream));
}

int convrot_gemm_i8(const int8_t* xq, const float* x_scale, const void* wq, int wbits, const float* w_scale,
                    int64_t M, int64_t N, int64_t K, int32_t* acc_out, uint16_t* y, hipStream_t stream) {
  if (wbits != 8 && wbits != 4) return CONVROT_ERR_DTYPE;
  if (M < 0 || N <= 0 || K <= 0 || K % 16 != 0 || K > CONVROT_MAX_K || (wbits == 4 && K % 32 != 0))
    return CONVROT_ERR_SHAPE;
  if (M > kMaxRows || N > kMaxRows || !tiles_fit(M, (N + 127) / 128)) return CONVROT_ERR_SHAPE;
  if (M == 0) return CONVROT_OK;
  if (!xq || !wq || (!acc_out && !y)) return CONVROT_ERR_NULL;
  if (y && (!x_scale || !w_scale)) return CONVROT_ERR_NULL;
  if (!aligned(xq, 16) || !aligned(wq, 16) || (acc_out && !aligned(acc_out, 16)) || (y && !aligned(y, 16)) ||
      (x_scale && !aligned(x_scale, 4)) || (w_scale && !aligned(w_scale, 4)))
    return CONVROT_ERR_ALIGN;
  return device_status(convrot::launch_gemm(xq, x_scale, wq, wbits, w_scale, M, N, K, acc_out, y, stream));
}

static int linear_impl(const uint16_t* x, int64_t M, int64_t K, const void* wq, int wbits, const float* w_scale,
                       int64_t N, int group, uint16_t* y, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  if (int rc = check_k(K, group, wbits == 4)) return rc;
  if (M < 0 || N <= 0 || M > kMaxRows || N > kMaxRows || !tiles_fit(M, (N + 127) / 128))
    return CONVROT_ERR_SHAPE;
  if (M == 0) return CONVROT_OK;
  if (!x || !wq || !w_scale || !y || !workspace) return CONVROT_ERR_NULL;
  if (!aligned(x, 16) || !aligned(wq, 16) || !aligned(y, 16) || !aligned(w_scale, 4)) return CONVROT_ERR_ALIGN;
  if (!aligned(workspace, 16)) return CONVROT_ERR_ALIGN;
  if (workspace_bytes < convrot_workspace_size(M, K)) return CONVROT_ERR_WORKSPACE;
  int8_t* xq = static_cast<int8_t*>(workspace);
  float* xs = reinterpret_cast<float*>(static_cast<char*>(workspace) + round_up(size_t(M) * size_t(K), kAlign));
  hipError_t e = convrot::launch_rotate_quant(x, CONVROT_W_BF16, M, K, log2_group(group), xq, xs, stream);
  if (e != hipSuccess) return CONVROT_ERR_DEVICE;
  return device_status(convrot::launch_gemm(xq, xs, wq, wbits, w_scale, M, N, K, nullptr, y, stream));
}

int convrot_w8a8_linear(const uint16_t* x, int64_t M, int64_t K, const int8_t* wq, const float* w_scale,
                        int64_t N, int group, uint16_t* y, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  return linear_impl(x, M, K, wq, 8, w_scale, N, group, y, workspace, workspace_bytes, stream);
}

int convrot_w8a8_linear_noalloc(const uint16_t* x, int64_t M, int64_t K, const int8_t* wq, const float* w_scale,
                                int64_t N, int group, uint16_t* y, hipStream_t stream) {
  // Host checks first, in the order the other linears use; the size limit
  // is checked before any HIP call.
  if (int rc = check_k(K, group, false)) return rc;
  if (M < 0 || N <= 0 || M > kMaxRows || N > kMaxRows || !tiles_fit(M, (N + 127) / 128))
    return CONVROT_ERR_SHAPE;
  if (M == 0) return CONVROT_OK;
  if (!x || !wq || !w_scale || !y) return CONVROT_ERR_NULL;
  if (!aligned(x, 16) || !aligned(wq, 16) || !aligned(y, 16) || !aligned(w_scale, 4)) return CONVROT_ERR_ALIGN;
  if (convrot_workspace_size(M, K) > CONVROT_NOALLOC_SCRATCH_BYTES) return CONVROT_ERR_SCRATCH;
  void* ws = scratch_address();
  if (!ws) return CONVROT_ERR_DEVICE;
  return linear_impl(x, M, K, wq, 8, w_scale, N, group, y, ws, CONVROT_NOALLOC_SCRATCH_BYTES, stream);
}

int convrot_w4a8_linear(const uint16_t* x, int64_t M, int64_t K, const uint8_t* wq4, const float* w_scale,
                        int64_t N, int group, uint16_t* y, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  return linear_impl(x, M, K, wq4, 4, w_scale, N, group, y, workspace, workspace_bytes, stream);
}

int convrot_dequantize_weight(const void* wq, int wbits, const float* w_scale, int64_t N, int64_t K, int group,
                              uint16_t* w_out, hipStream_t stream) {
  if (wbits != 8 && wbits != 4) return CONVROT_ERR_DTYPE;
  if (int rc = check_k(K, group, wbits == 4)) return rc;
  if (N < 0) return CONVROT_ERR_SHAPE;
  if (N == 0) return CONVROT_OK;
  if (!wq || !w_scale || !w_out) return CONVROT_ERR_NULL;
  if (!aligned(wq, 16) || !aligned(w_out, 16) || !aligned(w_scale, 4)) return CONVROT_ERR_ALIGN;
  return device_status(convrot::launch_dequantize_weight(wq, wbits, w_scale, N, K, log2_group(group), w_out, stream));
}

int convrot_gemm_bf16(const uint16_t* x, const uint16_t* w, int64_t M, int64_t N, int64_t K, uint16_t* y,
                      hipStream_t stream) {
  if (M < 0 || N <= 0 || K <= 0 || K % 16 != 0 || K > CONVROT_MAX_K) return CONVROT_ERR_SHAPE;
  if (M > kMaxRows || N > kMaxRows || !tiles_fit(M, (N + 127) / 128)) return CONVROT_ERR_SHAPE;
  if (M == 0) return CONVROT_OK;
  if (!x || !w || !y) return CONVROT_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16)) return CONVROT_ERR_ALIGN;
  return device_status(convrot::launch_gemm_bf16(x, w, M, N, K, y, stream));
}

size_t convrot_dequant_workspace_size(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0) return 0;
  return round_up(size_t(N) * size_t(K) * 2, kAlign);
}

int convrot_dequant_linear(const uint16_t* x, int64_t M, int64_t K, const void* wq, int wbits,
                           const float* w_scale, int64_t N, int group, uint16_t* y, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  if (wbits != 8 && wbits != 4) return CONVROT_ERR_DTYPE;
  if (int rc = check_k(K, group, wbits == 4)) return rc;
  if (M < 0 || N <= 0 || M > kMaxRows || N > kMaxRows || !tiles_fit(M, (N + 127) / 128))
    return CONVROT_ERR_SHAPE;
  if (M == 0) return CONVROT_OK;
  if (!x || !wq || !w_scale || !y || !workspace) return CONVROT_ERR_NULL;
  if (!aligned(x, 16) || !aligned(wq, 16) || !aligned(y, 16) || !aligned(w_scale, 4) || !aligned(workspace, 16))
    return CONVROT_ERR_ALIGN;
  if (workspace_bytes < convrot_dequant_workspace_size(N, K)) return CONVROT_ERR_WORKSPACE;
  uint16_t* w_hat = static_cast<uint16_t*>(workspace);
  const hipError_t e = convrot::launch_dequantize_weight(wq, wbits, w_scale, N, K, log2_group(group), w_hat, stream);
  if (e != hipSuccess) return CONVROT_ERR_DEVICE;
  return device_status(convrot::launch_gemm_bf16(x, w_hat, M, N, K, y, stream));
}

int convrot_gemm_i8_multi(const int8_t* xq, const float* x_scale, int wbits, int64_t M, int64_t K,
                          const convrot_linear_out* outs, int n_outs, hipStream_t stream) {
  if (wbits != 8 && wbits != 4) return CONVROT_ERR_DTYPE;
  if (M < 0 || M > kMaxRows || K <= 0 || K % 16 != 0 || K > CONVROT_MAX_K || (wbits == 4 && K % 32 != 0))
    return CONVROT_ERR_SHAPE;
  if (int rc = check_outs(M, outs, n_outs, false)) return rc;
  if (M == 0) return CONVROT_OK;
  if (!xq) return CONVROT_ERR_NULL;
  if (outs[0].y && !x_scale) return CONVROT_ERR_NULL;
  if (!aligned(xq, 16) || (x_scale && !aligned(x_scale, 4))) return CONVROT_ERR_ALIGN;
  return device_status(launch_outs(xq, x_scale, wbits, M, K, outs, n_outs, stream));
}

int convrot_linear_multi(const uint16_t* x, int64_t M, int64_t K, int group, int wbits,
                         const convrot_linear_out* outs, int n_outs, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  if (wbits != 8 && wbits != 4) return CONVROT_ERR_DTYPE;
  if (int rc = check_k(K, group, wbits == 4)) return rc;
  if (M < 0 || M > kMaxRows) return CONVROT_ERR_SHAPE;
  if (int rc = check_outs(M, outs, n_outs, true)) return rc;
  if (M == 0) return CONVROT_OK;
  if (!x || !workspace) return CONVROT_ERR_NULL;
  if (!aligned(x, 16) || !aligned(workspace, 16)) return CONVROT_ERR_ALIGN;
  if (workspace_bytes < convrot_workspace_size(M, K)) return CONVROT_ERR_WORKSPACE;
  int8_t* xq = static_cast<int8_t*>(workspace);
  float* xs = reinterpret_cast<float*>(static_cast<char*>(workspace) + round_up(size_t(M) * size_t(K), kAlign));
  hipError_t e = convrot::launch_rotate_quant(x, CONVROT_W_BF16, M, K, log2_group(group), xq, xs, stream);
  if (e != hipSuccess) return CONVROT_ERR_DEVICE;
  return device_status(launch_outs(xq, xs, wbits, M, K, outs, n_outs, stream));
}

}  // extern "C"
