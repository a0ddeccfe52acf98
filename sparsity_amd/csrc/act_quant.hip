// Per-token absmax int8 activation quantization, optionally with (M-2):M activation lifting.
//
// Each token's activations are scaled symmetrically onto [-127, 127] with no zero point
// (BitNet b1.58 page, "The mechanism", Activations).  For (M-2):M weights decomposed into M/2 - 1
// overlapping 2:4 windows, the activations are rearranged to match the windows inside the same
// pass (SlideSparse abstract, Activation Lifting): a group of 8 becomes 12 values
// [x0 x1 x2 x3 | x2 x3 x4 x5 | x4 x5 x6 x7], a group of M becomes 2M - 4 (M = 6, 8, ..., 16).
//
// absmax is the maximum of the |x| bit patterns (exact, order free); the int8 values are written
// with round-half-even.  Rows of up to 16384 elements (bf16; 8192 fp32) go to act_quant_row_kernel:
// one wave per token, holding its share of the row in registers, so the row is read from memory
// once and the token needs no block barrier.  Longer rows fall back to act_quant_kernel: one block
// per token, the row read twice (the second pass from L2).
#include <algorithm>
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"
#include "quant_group.hpp"

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

// LM = 0: plain.  LM = 6, 8, ..., 16: (LM-2):LM activation lifting, each LM-group becomes
// LM/2 - 1 windows of four values, window w = x[2w .. 2w+3] (2LM - 4 bytes per group).  A chunk
// is lcm(LM, 8) elements (whole 8-element loads and whole groups).
template <int LM>
constexpr int chunk_elems() { return LM ? lcm_i(LM, 8) : 8; }

// Lifted output of one chunk (CH quantized bytes q, CH / LM groups) at o (4-byte aligned).
template <int LM, int CH>
__device__ __forceinline__ void store_lifted(uint32_t* __restrict__ o, const uint32_t (&q)[CH]) {
  constexpr int NW = LM / 2 - 1;
#pragma unroll
  for (int g = 0; g < CH / LM; ++g)
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int b = g * LM + 2 * w;
      o[g * NW + w] = q[b] | (q[b + 1] << 8) | (q[b + 2] << 16) | (q[b + 3] << 24);
    }
}
template <bool BF16, int LM>
__global__ __launch_bounds__(256) void act_quant_kernel(const void* __restrict__ x, int K,
                                                        int8_t* __restrict__ xq,
                                                        float* __restrict__ xs) {
  constexpr int CH = chunk_elems<LM>();   // elements per chunk
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
      const size_t keff = (size_t)K / LM * (2 * LM - 4);
      store_lifted<LM, CH>((uint32_t*)(xq + (size_t)t * keff + (size_t)(CH / LM) * (2 * LM - 4) * c), q);
    } else {
      const uint32_t lo = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
      const uint32_t hi = q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24);
      *(uint2*)(xq + row + 8 * (size_t)c) = make_uint2(lo, hi);
    }
  }
  if (threadIdx.x == 0) xs[t] = amax / 127.f;
}

// Raw bits of one 8-element piece: 4 dwords of bf16 pairs, or 8 fp32.
template <bool BF16>
struct Piece {
  uint32_t w[BF16 ? 4 : 8];
};

template <bool BF16>
__device__ __forceinline__ void load_piece(const void* __restrict__ x, size_t off, Piece<BF16>& p) {
  if constexpr (BF16) {
    const uint4 u = *(const uint4*)((const uint16_t*)x + off);
    p.w[0] = u.x; p.w[1] = u.y; p.w[2] = u.z; p.w[3] = u.w;
  } else {
    const uint4 a = *(const uint4*)((const float*)x + off);
    const uint4 b = *(const uint4*)((const float*)x + off + 4);
    p.w[0] = a.x; p.w[1] = a.y; p.w[2] = a.z; p.w[3] = a.w;
    p.w[4] = b.x; p.w[5] = b.y; p.w[6] = b.z; p.w[7] = b.w;
  }
}

template <bool BF16>
__device__ __forceinline__ float piece_value(const Piece<BF16>& p, int j) {
  if constexpr (BF16) return __uint_as_float(j & 1 ? p.w[j / 2] & 0xFFFF0000u : p.w[j / 2] << 16);
  else return __uint_as_float(p.w[j]);
}

// One wave per token.  Lane l holds chunks l, l + 64, ... of its token's row (the first `cpl` of
// the CPL register slots; cpl is uniform), CH elements each (8, or lcm(LM, 8) for lifting),
// loaded before the absmax so all of a lane's loads are in flight at once; the quantized chunks
// are written from the registers.
template <bool BF16, int LM, int CPL>
__device__ __forceinline__ void quant_row(const void* __restrict__ x, int K, int8_t* __restrict__ xq,
                                          float* __restrict__ xs, int t, int lane, int cpl) {
  constexpr int CH = chunk_elems<LM>();
  constexpr int PPC = CH / 8;             // pieces per chunk
  const int nchunk = K / CH;
  const size_t row = (size_t)t * K;
  Piece<BF16> p[CPL][PPC];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    if (i < cpl) {
      const int c = min(lane + 64 * i, nchunk - 1);   // past the end: reload the last chunk
#pragma unroll
      for (int h = 0; h < PPC; ++h) load_piece<BF16>(x, row + (size_t)CH * c + 8 * h, p[i][h]);
    }
  }
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    if (i < cpl) {
#pragma unroll
      for (int h = 0; h < PPC; ++h)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          mx = max(mx, __float_as_uint(piece_value<BF16>(p[i][h], j)) & 0x7FFFFFFFu);
    }
  }
  // the raw words pass through opaque copies: without them the compiler keeps every element's
  // unpacked value from the absmax loop alive for the quantization (twice the registers)
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    if (i < cpl) {
#pragma unroll
      for (int h = 0; h < PPC; ++h)
#pragma unroll
        for (int k = 0; k < (BF16 ? 4 : 8); ++k) asm volatile("" : "+v"(p[i][h].w[k]));
    }
  }
  mx = wave_max_u32(mx);
  const float amax = __uint_as_float(mx);
  const float s = amax > 0.f ? 127.f / amax : 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + 64 * i;
    if (c >= nchunk) break;
    uint32_t q[CH];
#pragma unroll
    for (int h = 0; h < PPC; ++h)
#pragma unroll
      for (int j = 0; j < 8; ++j) q[8 * h + j] = q8(piece_value<BF16>(p[i][h], j), s);
    if constexpr (LM != 0) {
      const size_t keff = (size_t)K / LM * (2 * LM - 4);
      store_lifted<LM, CH>((uint32_t*)(xq + (size_t)t * keff + (size_t)(CH / LM) * (2 * LM - 4) * c), q);
    } else {
      const uint32_t lo = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
      const uint32_t hi = q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24);
      *(uint2*)(xq + row + 8 * (size_t)c) = make_uint2(lo, hi);
    }
  }
  if (lane == 0) xs[t] = amax / 127.f;
}

// Four tokens per block, CPL register slots per lane for every row.
template <bool BF16, int LM, int CPL>
__global__ __launch_bounds__(256) void act_quant_row_kernel(const void* __restrict__ x, int T,
                                                            int K, int8_t* __restrict__ xq,
                                                            float* __restrict__ xs) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;                     // the whole wave
  quant_row<BF16, LM, CPL>(x, K, xq, xs, t, threadIdx.x & 63, CPL);
}

// Grouped: the rows of several matrices in one launch.  Block b belongs to the last matrix whose
// first block is at most b (matrices without tokens own no blocks); every wave loads only the
// chunks of its own row, so a short-row matrix in a group with long rows reads nothing extra.
template <bool BF16, int LM, int CPL>
__global__ __launch_bounds__(256) void act_quant_group_kernel(QuantGroupArgs a) {
  constexpr int CH = chunk_elems<LM>();
  const int b = blockIdx.x;
  int m = 0;
  for (int i = 1; i < a.count; ++i)
    if (b >= a.block0[i]) m = i;
  const int t = (b - a.block0[m]) * 4 + (threadIdx.x >> 6);
  if (t >= a.T[m]) return;                // the whole wave
  const int K = a.K[m];
  quant_row<BF16, LM, CPL>(a.x[m], K, a.xq[m], a.xs[m], t, threadIdx.x & 63, (K / CH + 63) / 64);
}

// Calls f(std::integral_constant<int, CPL>) with the smallest CPL instantiation that holds cpl
// chunks per lane within the register budget (raw registers per lane: CPL * CH / 2 for bf16,
// CPL * CH for fp32; at most 128); false if the rows are too long for it.
template <bool BF16, int LM, class F>
static bool with_cpl(int64_t cpl, F&& f) {
  constexpr int CH = chunk_elems<LM>();
  constexpr int MAXR = 128 / (BF16 ? CH / 2 : CH);
  bool done = false;
  auto pick = [&](auto c) {
    constexpr int C = decltype(c)::value;
    if constexpr (C <= MAXR) {
      if (!done && cpl <= C) { f(c); done = true; }
    }
  };
  pick(std::integral_constant<int, 1>{});
  pick(std::integral_constant<int, 2>{});
  pick(std::integral_constant<int, 4>{});
  pick(std::integral_constant<int, 8>{});
  pick(std::integral_constant<int, 12>{});
  pick(std::integral_constant<int, 16>{});
  pick(std::integral_constant<int, 24>{});
  pick(std::integral_constant<int, 32>{});
  return done;
}

template <bool BF16, int LM>
static bool launch_rows(const void* x, int64_t T, int64_t K, int8_t* xq, float* xs,
                        hipStream_t s) {
  constexpr int CH = chunk_elems<LM>();
  const dim3 grid((unsigned)((T + 3) / 4));
  return with_cpl<BF16, LM>((K / CH + 63) / 64, [&](auto c) {
    act_quant_row_kernel<BF16, LM, decltype(c)::value><<<grid, 256, 0, s>>>(x, (int)T, (int)K, xq, xs);
  });
}

template <bool BF16, int LM>
static bool launch_group_rows(const QuantGroupArgs& a, hipStream_t s) {
  constexpr int CH = chunk_elems<LM>();
  int64_t cpl = 0;
  for (int i = 0; i < a.count; ++i) cpl = std::max<int64_t>(cpl, (a.K[i] / CH + 63) / 64);
  const dim3 grid((unsigned)a.block0[a.count]);
  return with_cpl<BF16, LM>(cpl, [&](auto c) {
    act_quant_group_kernel<BF16, LM, decltype(c)::value><<<grid, 256, 0, s>>>(a);
  });
}

// Calls f(std::integral_constant<int, LM>{}) for lift_M (0: no lifting).
template <class F>
static void with_lift(int lift_M, F&& f) {
  if (lift_M == 0) f(std::integral_constant<int, 0>{});
  else dispatch_m(lift_M, f);
}

hipError_t launch_act_quant(const void* x, int x_is_bf16, int64_t T, int64_t K, int lift_M,
                            int8_t* xq, float* x_scale, hipStream_t s) {
  bool done = false;
  with_lift(lift_M, [&](auto lm) {
    constexpr int LM = decltype(lm)::value;
    done = x_is_bf16 ? launch_rows<true, LM>(x, T, K, xq, x_scale, s)
                     : launch_rows<false, LM>(x, T, K, xq, x_scale, s);
  });
  if (done) return hipGetLastError();
  const dim3 grid((unsigned)T);
  with_lift(lift_M, [&](auto lm) {
    constexpr int LM = decltype(lm)::value;
    if (x_is_bf16) act_quant_kernel<true, LM><<<grid, 256, 0, s>>>(x, (int)K, xq, x_scale);
    else act_quant_kernel<false, LM><<<grid, 256, 0, s>>>(x, (int)K, xq, x_scale);
  });
  return hipGetLastError();
}

hipError_t launch_act_quant_group(const QuantGroupArgs& a, int x_is_bf16, int lift_M,
                                  hipStream_t s) {
  if (a.count < 1 || a.block0[a.count] < 1) return hipSuccess;
  bool done = false;
  with_lift(lift_M, [&](auto lm) {
    constexpr int LM = decltype(lm)::value;
    done = x_is_bf16 ? launch_group_rows<true, LM>(a, s) : launch_group_rows<false, LM>(a, s);
  });
  if (done) return hipGetLastError();
  // a row too long for the register budget: the matrices one launch each
  for (int i = 0; i < a.count; ++i) {
    const hipError_t e = launch_act_quant(a.x[i], x_is_bf16, a.T[i], a.K[i], lift_M, a.xq[i],
                                          a.xs[i], s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bl
