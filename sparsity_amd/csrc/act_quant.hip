// Per-token absmax int8 activation quantization, optionally with 6:8 or 14:16 activation lifting.
//
// Each token's activations are scaled symmetrically onto [-127, 127] with no zero point
// (BitNet b1.58 page, "The mechanism", Activations).  For 6:8 weights decomposed into three
// overlapping 2:4 windows, the activations are rearranged to match the windows inside the same
// pass (SlideSparse abstract, Activation Lifting): group g of 8 becomes 12 values
// [x0 x1 x2 x3 | x2 x3 x4 x5 | x4 x5 x6 x7], a group of 16 becomes 28 (seven windows).
//
// One block per token: pass 1 takes absmax as the maximum of |x| bit patterns (exact, order
// free); pass 2 re-reads the row (L2 resident) and writes int8 with round-half-even.
#include "device_common.hpp"
#include "launch.hpp"

namespace bl {

template <bool BF16>
__device__ __forceinline__ void load8(const void* __restrict__ x, size_t off, float v[8]) {
  if constexpr (BF16) {
    const uint4 u = *(const uint4*)((const uint16_t*)x + off);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(w[j] << 16);
      v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *(const float4*)((const float*)x + off);
    const float4 b = *(const float4*)((const float*)x + off + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// LM = 0: plain.  LM = 8 or 16: (LM-2):LM activation lifting, each LM-group becomes LM/2 - 1
// windows of four values, window w = x[2w .. 2w+3] (2LM - 4 bytes per group).
template <bool BF16, int LM>
__global__ __launch_bounds__(256) void act_quant_kernel(const void* __restrict__ x, int K,
                                                        int8_t* __restrict__ xq,
                                                        float* __restrict__ xs) {
  constexpr int CH = LM ? LM : 8;         // elements per chunk
  const int t = blockIdx.x;
  const int nchunk = K / CH;
  const size_t row = (size_t)t * K;
  uint32_t mx = 0;
  for (int c = threadIdx.x; c < nchunk; c += 256) {
#pragma unroll
    for (int h = 0; h < CH / 8; ++h) {
      float v[8];
      load8<BF16>(x, row + CH * (size_t)c + 8 * h, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) mx = max(mx, __float_as_uint(v[j]) & 0x7FFFFFFFu);
    }
  }
  mx = wave_max_u32(mx);
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = max(max(red[0], red[1]), max(red[2], red[3]));
  const float amax = __uint_as_float(mx);
  const float s = amax > 0.f ? 127.f / amax : 0.f;
  for (int c = threadIdx.x; c < nchunk; c += 256) {
    uint32_t q[CH];
#pragma unroll
    for (int h = 0; h < CH / 8; ++h) {
      float v[8];
      load8<BF16>(x, row + CH * (size_t)c + 8 * h, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) q[8 * h + j] = q8(v[j], s);
    }
    if constexpr (LM != 0) {
      constexpr int NW = LM / 2 - 1;
      const size_t keff = (size_t)K / LM * (2 * LM - 4);
      uint32_t* o = (uint32_t*)(xq + (size_t)t * keff + (size_t)(2 * LM - 4) * c);
#pragma unroll
      for (int w = 0; w < NW; ++w)
        o[w] = q[2 * w] | (q[2 * w + 1] << 8) | (q[2 * w + 2] << 16) | (q[2 * w + 3] << 24);
    } else {
      const uint32_t lo = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
      const uint32_t hi = q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24);
      *(uint2*)(xq + row + 8 * (size_t)c) = make_uint2(lo, hi);
    }
  }
  if (threadIdx.x == 0) xs[t] = amax / 127.f;
}

hipError_t launch_act_quant(const void* x, int x_is_bf16, int64_t T, int64_t K, int lift_M,
                            int8_t* xq, float* x_scale, hipStream_t s) {
  const dim3 grid((unsigned)T);
  auto run = [&](auto kern) { kern<<<grid, 256, 0, s>>>(x, (int)K, xq, x_scale); };
  if (x_is_bf16) {
    if (lift_M == 8) run(act_quant_kernel<true, 8>);
    else if (lift_M == 16) run(act_quant_kernel<true, 16>);
    else run(act_quant_kernel<true, 0>);
  } else {
    if (lift_M == 8) run(act_quant_kernel<false, 8>);
    else if (lift_M == 16) run(act_quant_kernel<false, 16>);
    else run(act_quant_kernel<false, 0>);
  }
  return hipGetLastError();
}

}  // namespace bl
