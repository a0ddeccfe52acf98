// Host-side launchers of the BitLinear kernels.  Arguments are validated by the C ABI layer
// (bitlinear_api.hip) before any of these is called; each returns the hipError_t of its launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

// Workspace of bitlinear_pack: per-block fp64 partial sums of |W|, then the ternary threshold.
constexpr int kGammaBlocks = 1024;
constexpr int kGammaThreads = 256;
constexpr size_t kPackWsBytes = kGammaBlocks * sizeof(double) + 64;

hipError_t launch_pack(const float* W, int64_t n, int64_t K, int N, int M, int layout,
                       uint32_t* codes, uint32_t* meta, float* gamma, void* ws, hipStream_t s);

hipError_t launch_act_quant(const void* x, int x_is_bf16, int64_t T, int64_t K, int lift_M,
                            int8_t* xq, float* x_scale, hipStream_t s);

hipError_t launch_fwd(const int8_t* xq, const float* x_scale, int64_t T, int64_t Keff,
                      const uint32_t* codes, const uint32_t* meta, const float* gamma, int layout,
                      int64_t n, float* y, int32_t* acc_opt, hipStream_t s);

}  // namespace bl
