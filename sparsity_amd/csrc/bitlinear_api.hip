// C ABI of libbitlinear: host-side validation, then launches on the caller's stream.
// Every check runs before anything is enqueued, so every error path is testable without a GPU.
#include <errno.h>
#include <stdint.h>

#include "bitlinear.h"
#include "launch.hpp"

namespace {

bool aligned16(const void* p) { return p && ((uintptr_t)p & 15u) == 0; }

// Shape rules of the packed layout; returns BL_OK and the packed K axis, or a status.
int check_shape(int64_t n, int64_t K, int N, int M, int layout, int64_t* keff) {
  if (layout != BL_LAYOUT_SPARSE && layout != BL_LAYOUT_DENSE2) return BL_ENOTSUP;
  if (layout == BL_LAYOUT_SPARSE) {
    if (!((N == 2 && M == 4) || (N == 6 && M == 8))) return BL_ENOTSUP;
  } else {
    if (!(M == 4 || M == 8) || N < 1 || N > M) return BL_ENOTSUP;
  }
  if (n < 1 || K < 1) return BL_EINVAL;
  const int64_t kq = layout == BL_LAYOUT_DENSE2 ? 32 : (M == 4 ? 64 : 128);
  if (K % kq != 0) return BL_EINVAL;
  if (n > INT32_MAX || K > INT32_MAX) return BL_EINVAL;
  if ((uint64_t)n * (uint64_t)K >= (1ull << 32)) return BL_EINVAL;
  const int64_t ke = (layout == BL_LAYOUT_SPARSE && M == 8) ? K / 2 * 3 : K;
  if (ke * 127 >= (int64_t)INT32_MAX) return BL_EINVAL;
  *keff = ke;
  return BL_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? BL_OK : BL_EIO; }

}  // namespace

extern "C" {

int bitlinear_layout_version(void) { return BL_LAYOUT_VERSION; }

const char* bitlinear_strerror(int status) {
  switch (status) {
    case BL_OK: return "ok";
    case BL_EINVAL: return "invalid argument, shape, alignment or NULL pointer";
    case BL_ENOTSUP: return "unsupported N:M, layout or dtype";
    case BL_ENOSPC: return "workspace too small";
    case BL_EIO: return "HIP runtime or launch error";
    default: return "unknown status";
  }
}

int bitlinear_packed_bytes(int64_t n, int64_t K, int N, int M, int layout, size_t* codes_bytes,
                           size_t* meta_bytes, int64_t* K_eff, size_t* ws_bytes) {
  int64_t ke = 0;
  const int st = check_shape(n, K, N, M, layout, &ke);
  if (st != BL_OK) return st;
  const uint64_t n_pad = (uint64_t)((n + 31) / 32) * 32;
  const uint64_t slots = layout == BL_LAYOUT_SPARSE ? (uint64_t)ke / 2 : (uint64_t)ke;
  if (codes_bytes) *codes_bytes = (size_t)(n_pad * slots / 4);
  if (meta_bytes) *meta_bytes = layout == BL_LAYOUT_SPARSE ? (size_t)(n_pad * slots / 4) : 0;
  if (K_eff) *K_eff = ke;
  if (ws_bytes) *ws_bytes = bl::kPackWsBytes;
  return BL_OK;
}

int bitlinear_pack(const float* W, int64_t n, int64_t K, int N, int M, int layout, uint8_t* codes,
                   uint8_t* meta, float* gamma, void* ws, size_t ws_bytes, void* stream) {
  int64_t ke = 0;
  const int st = check_shape(n, K, N, M, layout, &ke);
  if (st != BL_OK) return st;
  if (!aligned16(W) || !aligned16(codes) || !aligned16(gamma) || !aligned16(ws)) return BL_EINVAL;
  if (layout == BL_LAYOUT_SPARSE ? !aligned16(meta) : meta != nullptr) return BL_EINVAL;
  if (ws_bytes < bl::kPackWsBytes) return BL_ENOSPC;
  return status_of(bl::launch_pack(W, n, K, N, M, layout, (uint32_t*)codes, (uint32_t*)meta, gamma,
                                   ws, (hipStream_t)stream));
}

int act_quant_i8(const void* x, int x_dtype, int64_t T, int64_t K, int lift_M, int8_t* xq,
                 float* x_scale, void* stream) {
  if (x_dtype != BL_DTYPE_F32 && x_dtype != BL_DTYPE_BF16) return BL_ENOTSUP;
  if (lift_M != 0 && lift_M != 8) return BL_EINVAL;
  if (T < 0 || T > INT32_MAX || K < 8 || K % 8 != 0 || K > (int64_t)1 << 24) return BL_EINVAL;
  if (T == 0) return BL_OK;  // nothing is read or written; pointers may be NULL
  if (!aligned16(x) || !aligned16(xq) || !aligned16(x_scale)) return BL_EINVAL;
  return status_of(bl::launch_act_quant(x, x_dtype == BL_DTYPE_BF16, T, K, lift_M, xq, x_scale,
                                        (hipStream_t)stream));
}

int bitlinear_fwd(const int8_t* xq, const float* x_scale, int64_t T, int64_t K,
                  const uint8_t* codes, const uint8_t* meta, const float* gamma, int N, int M,
                  int layout, int64_t n, float* y, int32_t* acc_opt, void* stream) {
  int64_t ke = 0;
  const int st = check_shape(n, K, N, M, layout, &ke);
  if (st != BL_OK) return st;
  if (T < 0 || T > INT32_MAX || (uint64_t)T * (uint64_t)n >= (1ull << 40)) return BL_EINVAL;
  if ((uint64_t)T * (uint64_t)ke >= (1ull << 31)) return BL_EINVAL;  // 32-bit activation offsets
  if (T == 0) return BL_OK;  // nothing is read or written; pointers may be NULL
  if (!aligned16(xq) || !aligned16(x_scale) || !aligned16(codes) || !aligned16(gamma) ||
      !aligned16(y))
    return BL_EINVAL;
  if (layout == BL_LAYOUT_SPARSE ? !aligned16(meta) : meta != nullptr) return BL_EINVAL;
  if (acc_opt && ((uintptr_t)acc_opt & 3u)) return BL_EINVAL;
  return status_of(bl::launch_fwd(xq, x_scale, T, ke, (const uint32_t*)codes, (const uint32_t*)meta,
                                  gamma, layout, n, y, acc_opt, (hipStream_t)stream));
}

}  // extern "C"
