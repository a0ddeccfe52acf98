// Absmean scale, N:M mask, ternarization and 2-bit packing of fp32 master weights.
//
// gamma is the mean |W| over the whole dense master (BitNet b1.58 page, "The mechanism",
// absmean quantization), taken before the mask (Sparse-BitNet technical summary, section 2,
// Forward Pass: quantize, then mask).  The mask keeps the N largest |w| of the continuous master
// in each M-group (same summary, Maskering) and (2N-2):2N groups -- 6:8, 14:16 -- are rewritten
// as N-1 overlapping 2:4 windows (SlideSparse abstract, Sliding Window Decomposition).
//
// Two launches, both on the caller's stream:
//   1. gamma_partial_kernel   fp64 partial sums of |w| (HBM-bound read of W)
//   2. pack_kernel            every block first derives gamma from the partials (same data, same
//                             order, so every block gets the same bits): it certifies the fp32
//                             rounding of the exact mean with a rigorous error bound, and only
//                             when the bound cannot decide falls back to an exact exponent-binned
//                             integer sum over W; then the ternary threshold tau.  Its tile of W
//                             (mostly from the 256 MB last-level cache) is already in flight
//                             meanwhile.  Mask, codes by |w| >= tau, slots assembled in LDS,
//                             coalesced dword stores.
#include "device_common.hpp"
#include "launch.hpp"
#include "pack_group.hpp"

namespace bl {

struct PackWs {
  double partial[kGammaBlocks];
  uint32_t exact_used;  // 1 when the exact fallback decided gamma (diagnostic, written by block 0)
};
static_assert(sizeof(PackWs) <= kPackWsBytes, "pack workspace");

__device__ __forceinline__ void gamma_partial_block(const float4* __restrict__ W4, int64_t n4,
                                                    double* __restrict__ partial, int blk) {
  // Four independent fp64 chains per thread keep four 16-byte loads in flight.  Every |w| still
  // passes through at most 4 * ceil(n4 / threads) + 2 additions before the wave sum, inside the
  // depth the finalize step assumes for its error bound.
  const int64_t stride = (int64_t)kGammaBlocks * kGammaThreads;
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
  int64_t i = (int64_t)blk * kGammaThreads + threadIdx.x;
  for (; i + 3 * stride < n4; i += 4 * stride) {
    const float4 v0 = W4[i], v1 = W4[i + stride], v2 = W4[i + 2 * stride], v3 = W4[i + 3 * stride];
    a0 += fabs((double)v0.x); a0 += fabs((double)v0.y); a0 += fabs((double)v0.z); a0 += fabs((double)v0.w);
    a1 += fabs((double)v1.x); a1 += fabs((double)v1.y); a1 += fabs((double)v1.z); a1 += fabs((double)v1.w);
    a2 += fabs((double)v2.x); a2 += fabs((double)v2.y); a2 += fabs((double)v2.z); a2 += fabs((double)v2.w);
    a3 += fabs((double)v3.x); a3 += fabs((double)v3.y); a3 += fabs((double)v3.z); a3 += fabs((double)v3.w);
  }
  for (; i < n4; i += stride) {
    const float4 v = W4[i];
    a0 += fabs((double)v.x); a0 += fabs((double)v.y); a0 += fabs((double)v.z); a0 += fabs((double)v.w);
  }
  double acc = (a0 + a1) + (a2 + a3);
  acc = wave_sum_f64(acc);
  __shared__ double red[kGammaThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double s = 0.0;
    for (int w = 0; w < kGammaThreads / 64; ++w) s += red[w];
    partial[blk] = s;
  }
}

__global__ __launch_bounds__(kGammaThreads) void gamma_partial_kernel(const float4* __restrict__ W4,
                                                                      int64_t n4,
                                                                      double* __restrict__ partial) {
  gamma_partial_block(W4, n4, partial, blockIdx.x);
}

// Round (sum_e bins[e] * 2^(max(e,1)-150)) / count to the nearest fp32, ties to even, exactly.
// bins[e] is the integer sum of the 24-bit significands of the magnitudes with biased exponent e.
__device__ float exact_mean_from_bins(const unsigned long long* bins, uint64_t count) {
  constexpr int L = 10;  // 320-bit integer in units of 2^-149 (sum < 2^310)
  uint32_t lim[L];
  for (int i = 0; i < L; ++i) lim[i] = 0;
  for (int e = 0; e < 255; ++e) {
    unsigned long long v = bins[e];
    if (!v) continue;
    const int sh = (e > 0 ? e : 1) - 1;
    int w = sh >> 5;
    const int b = sh & 31;
    // v << b spans at most 88 bits: three 32-bit words starting at limb w
    uint32_t part[3];
    part[0] = (uint32_t)(v << b);
    part[1] = (uint32_t)((b ? (v >> (32 - b)) : (v >> 32)) & 0xFFFFFFFFull);
    part[2] = (uint32_t)(b ? (v >> (64 - b)) : 0ull);
    uint64_t carry = 0;
    for (int k = 0; w + k < L; ++k) {
      uint64_t add = (k < 3 ? part[k] : 0u) + carry + (uint64_t)lim[w + k];
      lim[w + k] = (uint32_t)add;
      carry = add >> 32;
      if (k >= 2 && carry == 0) break;
    }
  }
  // long division by count (< 2^32)
  uint32_t q[L];
  uint64_t rem = 0;
  for (int i = L - 1; i >= 0; --i) {
    const uint64_t cur = (rem << 32) | lim[i];
    q[i] = (uint32_t)(cur / count);
    rem = cur % count;
  }
  // bit length of the quotient
  int len = 0;
  for (int i = L - 1; i >= 0; --i)
    if (q[i]) { len = 32 * i + (32 - __clz(q[i])); break; }
  const int shift = len > 24 ? len - 24 : 0;
  auto bit = [&](int pos) -> uint32_t { return (q[pos >> 5] >> (pos & 31)) & 1u; };
  uint32_t sig = 0;
  for (int k = 23; k >= 0; --k) sig = (sig << 1) | (shift + k < 32 * L ? bit(shift + k) : 0u);
  bool up;
  if (shift == 0) {
    up = (2 * rem > count) || (2 * rem == count && (sig & 1));
  } else {
    const uint32_t half = bit(shift - 1);
    bool lower = rem != 0;
    for (int pos = 0; pos < shift - 1 && !lower; ++pos) lower = bit(pos) != 0;
    up = half && (lower || (sig & 1));
  }
  int sh = shift;
  sig += up ? 1u : 0u;
  if (sig == (1u << 24)) { sig = 1u << 23; sh += 1; }
  const uint32_t out = sig >= (1u << 23) ? (((uint32_t)(sh + 1) << 23) | (sig & 0x7FFFFFu)) : sig;
  return __uint_as_float(out);
}

// Smallest fp32 tau with fl32(tau / gamma) > 0.5.  Under round-to-nearest-even the fp32 quotient
// exceeds 0.5 exactly when the real quotient exceeds 0.5 + 2^-25 (the spacing above 0.5 is
// 2^-24), i.e. when x > gamma * (2^24 + 1) * 2^-25; that product is exact in fp64.
__device__ float ternary_threshold(float gamma) {
  if (!(gamma > 0.f)) return __int_as_float(0x7f800000);
  const double t = (double)gamma * 16777217.0 * 0x1p-25;
  float f = (float)t;
  if ((double)f <= t) f = __int_as_float(__float_as_int(f) + 1);
  while (true) {
    const float prev = __int_as_float(__float_as_int(f) - 1);
    if ((double)prev > t) f = prev; else break;
  }
  return f;
}

// gamma and tau from the partial sums, computed by one whole block (every pack block runs it and
// gets the same bits).  Returns through LDS: *g_sh, *tau_sh, *exact_sh.
// `v` is this thread's sum of partials threadIdx.x + i * NT (loaded by the caller, ahead of its
// own tile loads, so waiting for them does not wait for the tile).
// Rare path of block_gamma: the exact mean of |W| by the whole block (exponent-binned integer
// sums in LDS), kept out of line so the common path stays small.  Every thread of the block calls
// it; thread 0 writes *g_sh.
template <int NT>
__device__ __noinline__ void exact_gamma_block(const float* __restrict__ W, int64_t count,
                                               float* g_sh, unsigned long long* bins_sh) {
  for (int i = threadIdx.x; i < 256; i += NT) bins_sh[i] = 0ull;
  __syncthreads();
  for (int64_t i = threadIdx.x; i < count; i += NT) {
    const uint32_t b = __float_as_uint(W[i]) & 0x7FFFFFFFu;
    const uint32_t e = b >> 23;
    const uint32_t m = (b & 0x7FFFFFu) | (e ? 0x800000u : 0u);
    atomicAdd(&bins_sh[e], (unsigned long long)m);
  }
  __syncthreads();
  if (threadIdx.x == 0) *g_sh = exact_mean_from_bins(bins_sh, (uint64_t)count);
}

template <int NT>
__device__ __forceinline__ void block_gamma(double v, const float* __restrict__ W, int64_t count, float* g_sh,
                            float* tau_sh, int* exact_sh, double* red_sh,
                            unsigned long long* bins_sh) {
  static_assert(kGammaBlocks % NT == 0 && NT % 64 == 0, "partials split evenly");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_f64(v);
  if (lane == 0) red_sh[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    double S = 0.0;
    for (int w = 0; w < NT / 64; ++w) S += red_sh[w];
    // longest chain of fp64 additions any |w| goes through: the partial kernel's per-thread
    // chains (at most 4 per float4 it reads, plus 2 to join its four chains), its wave butterfly
    // (6) and block sum (4), then here the per-thread sum (kGammaBlocks / NT), the butterfly (6)
    // and the block sum (NT / 64); 64 covers every fixed term
    const int64_t n4 = count / 4;
    const int64_t per_thread = (n4 + (int64_t)kGammaBlocks * kGammaThreads - 1) / ((int64_t)kGammaBlocks * kGammaThreads);
    const double depth = 4.0 * (double)per_thread + 64.0;
    const double u = 0x1p-53;
    const double err = 2.0 * depth * u * S;  // >= ((1+u)^depth - 1) * S for nonnegative terms
    const double cnt = (double)count;
    const double lo = (S - err) / cnt * (1.0 - 4.0 * u);
    const double hi = (S + err) / cnt * (1.0 + 4.0 * u);
    const float glo = (float)lo, ghi = (float)hi;
    if (S == 0.0) { *exact_sh = 0; *g_sh = 0.f; }
    else if (glo == ghi) { *exact_sh = 0; *g_sh = glo; }
    else *exact_sh = 1;
  }
  __syncthreads();
  if (*exact_sh)   // uniform; rare: the bound straddles an fp32 rounding boundary
    exact_gamma_block<NT>(W, count, g_sh, bins_sh);
  if (threadIdx.x == 0) *tau_sh = ternary_threshold(*g_sh);
  __syncthreads();
}

constexpr int kPackKB = 256;  // dense K columns per pack tile

// One block packs one 32-row panel x 256 dense columns.  Phase 1 stages the fp32 tile in LDS with
// coalesced 1 KB row reads; phase 2 turns each M-group into slot bytes (code | index << 2);
// phase 3 assembles 16-slot units into code/meta dwords, which land contiguously in the tiled
// layout (unit v = 32*u + r of the tile is dword base + v).
template <int LAYOUT, int M>
__device__ __forceinline__ void pack_tile(const float* __restrict__ W, int n, int K, int N,
                                          int k_tiles, PackWs* __restrict__ ws,
                                          float* __restrict__ gamma_out,
                                          uint32_t* __restrict__ codes,
                                          uint32_t* __restrict__ meta, int blk) {
  constexpr bool SP = LAYOUT == kLayoutSparse;
  constexpr int WS = kPackKB + 4;                                      // padded fp32 row
  constexpr int NKEEP = M == 4 ? 2 : M - 2;                           // SPARSE: 2:4, 6:8, 14:16
  constexpr int SLOTS = SP ? kPackKB * NKEEP / M : kPackKB;
  constexpr int SS = SLOTS + 16;                                       // padded slot row
  constexpr int GPR = kPackKB / M;                                     // groups per tile row
  constexpr int UPR = SLOTS / 16;                                      // units per tile row
  __shared__ __attribute__((aligned(16))) float tile[32 * WS];
  __shared__ __attribute__((aligned(16))) uint8_t slots[32 * SS];
  __shared__ double red_sh[4];
  __shared__ unsigned long long bins_sh[256];
  __shared__ float g_sh, tau_sh;
  __shared__ int exact_sh;

  const int P = blk / k_tiles;
  const int kb = blk % k_tiles;
  const int k0 = kb * kPackKB;
  const int r0 = P * kPanel;
  const int kw = min(kPackKB, K - k0);

  // this thread's share of the gamma partial sums first (L2 hits), then all eight 16-byte tile
  // loads before its first LDS store (addresses clamped into the matrix; out-of-range rows and
  // columns are zeroed after the load)
  double pv = 0.0;
#pragma unroll
  for (int i = 0; i < kGammaBlocks / 256; ++i) pv += ws->partial[threadIdx.x + i * 256];
  asm volatile("" ::: "memory");
  {
    const int c4 = threadIdx.x & 63;
    const bool col_ok = 4 * c4 < kw;
    const int col = k0 + min(4 * c4, kw - 4);
    float4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = i * 4 + (threadIdx.x >> 6);
      v[i] = *(const float4*)(W + (size_t)min(r0 + row, n - 1) * K + col);
    }
    // gamma while the tile is in flight
    block_gamma<256>(pv, W, (int64_t)n * K, &g_sh, &tau_sh, &exact_sh, red_sh, bins_sh);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = i * 4 + (threadIdx.x >> 6);
      if (!(col_ok && r0 + row < n)) v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      *(float4*)&tile[row * WS + 4 * c4] = v[i];
    }
  }
  if (blk == 0 && threadIdx.x == 0) {
    gamma_out[0] = g_sh;
    ws->exact_used = (uint32_t)exact_sh;
  }
  const float tau = tau_sh;
  __syncthreads();

  const int nkeep = SP ? NKEEP : N;
  for (int gid = threadIdx.x; gid < 32 * GPR; gid += 256) {
    const int row = gid / GPR, g = gid % GPR;
    float w[M];
    uint32_t a[M];
#pragma unroll
    for (int j = 0; j < M; ++j) {
      w[j] = tile[row * WS + g * M + j];
      a[j] = __float_as_uint(w[j]) & 0x7FFFFFFFu;
    }
    uint32_t keep = 0;
#pragma unroll
    for (int i = 0; i < M; ++i) {
      int rank = 0;
#pragma unroll
      for (int j = 0; j < M; ++j)
        if (j != i) rank += (a[j] > a[i]) || (a[j] == a[i] && j < i);
      if (rank < nkeep) keep |= 1u << i;
    }
    // 00 = 0, 01 = +1, 10 = -1
    auto code = [&](int j) -> uint32_t { return fabsf(w[j]) >= tau ? (w[j] < 0.f ? 2u : 1u) : 0u; };
    uint8_t* out = &slots[row * SS];
    if constexpr (SP && M == 4) {
      int s = 0;
#pragma unroll
      for (int p = 0; p < 4; ++p)
        if (keep >> p & 1u) { out[2 * g + s] = (uint8_t)(code(p) | (p << 2)); ++s; }
    } else if constexpr (SP) {
      // (M-2):M into M/2 - 1 windows covering positions 2w..2w+3: kept positions in ascending
      // order, each to the lowest window that covers it and holds fewer than two (position p
      // is covered by windows (p - 2) / 2 and p / 2, clipped to the window range)
      constexpr int NWIN = M / 2 - 1;
      int cnt[NWIN];
#pragma unroll
      for (int w = 0; w < NWIN; ++w) cnt[w] = 0;
#pragma unroll
      for (int p = 0; p < M; ++p) {
        if (!(keep >> p & 1u)) continue;
        const int wlo = p >= 2 ? (p - 2) >> 1 : 0;                     // constants after unrolling
        const int whi = (p >> 1) < NWIN - 1 ? (p >> 1) : NWIN - 1;
        int wdw, slot;
        if (cnt[wlo] < 2) { wdw = wlo; slot = 2 * wlo + cnt[wlo]; ++cnt[wlo]; }
        else { wdw = whi; slot = 2 * whi + cnt[whi]; ++cnt[whi]; }
        out[NKEEP * g + slot] = (uint8_t)(code(p) | ((p - 2 * wdw) << 2));
      }
    } else {
#pragma unroll
      for (int j = 0; j < M; ++j) out[g * M + j] = (uint8_t)((keep >> j & 1u) ? code(j) : 0u);
    }
  }
  __syncthreads();

  const int valid_slots = SP ? kw * NKEEP / M : kw;
  const int units_valid = valid_slots / 16;
  const int nfrag = SP ? (M == 4 ? K : K / M * (2 * M - 4)) / 64 : K / 32;   // fragments per panel
  const size_t base = ((size_t)P * nfrag + (size_t)kb * (UPR / 2)) * 64;
  for (int v = threadIdx.x; v < 32 * UPR; v += 256) {
    const int u = v >> 5, r = v & 31;
    if (u >= units_valid) continue;
    const uint4 sb = *(const uint4*)&slots[r * SS + 16 * u];
    const uint32_t wd[4] = {sb.x, sb.y, sb.z, sb.w};
    uint32_t cw = 0, mw = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t b = (wd[i >> 2] >> (8 * (i & 3))) & 0xFFu;
      cw |= (b & 3u) << (8 * (i & 3) + 2 * (i >> 2));
      mw |= (b >> 2) << (2 * i);
    }
    codes[base + v] = cw;
    if constexpr (SP) meta[base + v] = mw;
  }
}

template <int LAYOUT, int M>
__global__ __launch_bounds__(256) void pack_kernel(const float* __restrict__ W, int n, int K, int N,
                                                   int k_tiles, PackWs* __restrict__ ws,
                                                   float* __restrict__ gamma_out,
                                                   uint32_t* __restrict__ codes,
                                                   uint32_t* __restrict__ meta) {
  pack_tile<LAYOUT, M>(W, n, K, N, k_tiles, ws, gamma_out, codes, meta, blockIdx.x);
}

// ---------------------------------------------------------------------------------------------
// Grouped pack: the bitlinear_pack calls of several masters in two launches, each tensor's blocks
// running exactly the single call's arithmetic (so gamma, codes and meta are the same bits).
// The partial-sum launch walks the tensors in table order and the pack launch in reverse, so
// the tensors read last by the first launch -- still in the last-level cache -- are packed first.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kGammaThreads) void gamma_partial_group_kernel(
    const uint8_t* __restrict__ table) {
  const PackGroupHeader* hd = (const PackGroupHeader*)table;
  if (hd->magic != kPackGroupMagic) return;
  const int b = blockIdx.x;
  if (b >= hd->count * kGammaBlocks) return;
  const PackGroupItem it = ((const PackGroupItem*)(table + sizeof(PackGroupHeader)))[b / kGammaBlocks];
  gamma_partial_block((const float4*)it.W, (int64_t)it.n * it.K / 4, ((PackWs*)it.ws)->partial,
                      b % kGammaBlocks);
}

template <int LAYOUT, int M>
__global__ __launch_bounds__(256) void pack_group_kernel(const uint8_t* __restrict__ table) {
  const PackGroupHeader* hd = (const PackGroupHeader*)table;
  if (hd->magic != kPackGroupMagic || hd->layout != LAYOUT || hd->M != M) return;
  const int b = blockIdx.x;
  if (b >= hd->pack_blocks) return;
  const PackGroupItem* items = (const PackGroupItem*)(table + sizeof(PackGroupHeader));
  // items[count - 1] owns the first blocks: find the last r with items[count - 1 - r].block0 <= b
  int lo = 0, hi = hd->count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (items[hd->count - 1 - mid].block0 <= b) lo = mid; else hi = mid - 1;
  }
  const PackGroupItem it = items[hd->count - 1 - lo];
  pack_tile<LAYOUT, M>(it.W, it.n, it.K, hd->N, it.k_tiles, (PackWs*)it.ws, it.gamma, it.codes,
                       it.meta, b - it.block0);
}

hipError_t launch_pack(const float* W, int64_t n, int64_t K, int N, int M, int layout,
                       uint32_t* codes, uint32_t* meta, float* gamma, void* ws_raw, hipStream_t s) {
  PackWs* ws = (PackWs*)ws_raw;
  const int64_t count = n * K;
  gamma_partial_kernel<<<kGammaBlocks, kGammaThreads, 0, s>>>((const float4*)W, count / 4, ws->partial);
  const int panels = (int)((n + kPanel - 1) / kPanel);
  const int k_tiles = (int)((K + kPackKB - 1) / kPackKB);
  const dim3 grid((unsigned)(panels * k_tiles));
  auto run = [&](auto kern, uint32_t* mt) {
    kern<<<grid, 256, 0, s>>>(W, (int)n, (int)K, N, k_tiles, ws, gamma, codes, mt);
  };
  if (layout == kLayoutSparse) {
    if (M == 4) run(pack_kernel<kLayoutSparse, 4>, meta);
    else if (M == 8) run(pack_kernel<kLayoutSparse, 8>, meta);
    else run(pack_kernel<kLayoutSparse, 16>, meta);
  } else {
    if (M == 4) run(pack_kernel<kLayoutDense2, 4>, nullptr);
    else if (M == 8) run(pack_kernel<kLayoutDense2, 8>, nullptr);
    else run(pack_kernel<kLayoutDense2, 16>, nullptr);
  }
  return hipGetLastError();
}

hipError_t launch_pack_group(const void* table, int64_t count, int64_t pack_blocks, int layout,
                             int M, hipStream_t s) {
  const uint8_t* t = (const uint8_t*)table;
  gamma_partial_group_kernel<<<(unsigned)(count * kGammaBlocks), kGammaThreads, 0, s>>>(t);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned g = (unsigned)pack_blocks;
  if (layout == kLayoutSparse) {
    if (M == 4) pack_group_kernel<kLayoutSparse, 4><<<g, 256, 0, s>>>(t);
    else if (M == 8) pack_group_kernel<kLayoutSparse, 8><<<g, 256, 0, s>>>(t);
    else pack_group_kernel<kLayoutSparse, 16><<<g, 256, 0, s>>>(t);
  } else {
    if (M == 4) pack_group_kernel<kLayoutDense2, 4><<<g, 256, 0, s>>>(t);
    else if (M == 8) pack_group_kernel<kLayoutDense2, 8><<<g, 256, 0, s>>>(t);
    else pack_group_kernel<kLayoutDense2, 16><<<g, 256, 0, s>>>(t);
  }
  return hipGetLastError();
}

}  // namespace bl
