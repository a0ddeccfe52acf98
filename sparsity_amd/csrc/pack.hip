// Absmean scale, N:M mask, ternarization and 2-bit packing of fp32 master weights.
//
// gamma is the mean |W| over the whole dense master (BitNet b1.58 page, "The mechanism",
// absmean quantization), taken before the mask (Sparse-BitNet technical summary, section 2,
// Forward Pass: quantize, then mask).  The mask keeps the N largest |w| of the continuous master
// in each M-group (same summary, Maskering) and (2N-2):2N groups -- 6:8, 14:16 -- are rewritten
// as N-1 overlapping 2:4 windows (SlideSparse abstract, Sliding Window Decomposition).
//
// Five launches, all on the caller's stream, one HBM pass over W in the common case:
//   1. gamma_sample_kernel  a fixed share of W (1 chunk of 4 KB in S, S = 1..32 by size) spread
//                           over the matrix: per-block sums of |w|; block 0 also clears the
//                           accumulators of launches 3-4
//   2. band_kernel          one block: the sample's estimate of mean |W| and its standard error
//                           give a band [tau_lo, tau_hi] that holds the exact threshold tau unless
//                           the sample misleads
//   3. pack_spec_kernel     the pass over W: per 32-row tile, the fp64 sums of |w| (added into one
//                           of kGammaBlocks slots), the mask and meta (final: they do not depend on
//                           gamma) and the codes against the band -- |w| >= tau_hi codes +-1,
//                           |w| < tau_lo codes 0, and a kept weight in between codes 0 and is
//                           listed in the tile's own region of the workspace with its code
//                           position and |w|
//   4. gamma_exact_kernel   every block sums the slots in one fixed order and certifies the fp32
//                           rounding of the exact mean with a rigorous error bound.  Certified
//                           (the common case): block 0 stores gamma and the ternary threshold tau,
//                           and every block exits.  Otherwise the blocks sum |W| exactly as
//                           integers (24-bit significands shifted to a 2^-149 fixed point, kept as
//                           carry-free 32-bit words in 64-bit accumulators), each block stores its
//                           word sums in a line of its own, and the last block to arrive rounds
//                           the exact mean to fp32 and stores gamma and tau
//   5. pack_fix_kernel      tau inside the band and no region overflowed: the listed codes with
//                           |w| >= tau are set.  Otherwise (tau outside the band, a tile listed
//                           more than its region holds, no band) every tile is packed again
//                           against tau: a second pass over W.
// The codes therefore follow |w| >= tau for the exact tau whatever the sample says; the sample
// only decides how much work the fix-up has.
#include <mutex>

#include "device_common.hpp"
#include "launch.hpp"
#include "pack_ws.hpp"
#include "pack_group.hpp"

namespace bl {

static_assert(sizeof(PackWs) <= kPackWsFixed, "pack workspace");
static_assert(kSampleBlocks <= kGammaThreads, "one sampling block per thread of a pack block");

// Sampling stride: about 2^19 sampled weights, at least a 32nd of the master, all of a small one.
__host__ __device__ __forceinline__ int64_t sample_stride(int64_t count) {
  int64_t S = 1;
  while (S < 32 && (count >> 19) >= 2 * S) S *= 2;
  return S;
}

// The sampled chunks: 1024 floats (4 KB) each, chunk j = S j + (7 j mod S) for j < count / (1024
// S), dealt to the blocks round-robin.  Thread t reads float4 t of each of its block's chunks and
// keeps the sum s of their |w| and their number c; the block stores the sums of s, s^2, s c, c
// and c^2 over its threads.  Threads are the sampling units: each one's elements lie in chunks
// far apart in the matrix.
__device__ __forceinline__ void gamma_sample_block(const float4* __restrict__ W4, int64_t count,
                                                   PackWs* __restrict__ ws, int blk) {
  const int64_t S = sample_stride(count);
  const int64_t ns = count / (1024 * S);
  constexpr int U = 8;   // chunks in flight per block (a 2^19-weight sample is ~4-8 per block)
  double s = 0.0, c = 0.0;
  for (int64_t j = blk; j < ns; j += U * kSampleBlocks) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t jj = min(j + u * kSampleBlocks, ns - 1);
      v[u] = W4[(S * jj + ((7 * jj) & (S - 1))) * 256 + threadIdx.x];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (j + u * kSampleBlocks < ns) {
        s += (fabs((double)v[u].x) + fabs((double)v[u].y)) + (fabs((double)v[u].z) + fabs((double)v[u].w));
        c += 4.0;
      }
  }
  double st[kSampleStats] = {s, s * s, s * c, c, c * c};
  __shared__ double red[kGammaThreads / 64][kSampleStats];
#pragma unroll
  for (int i = 0; i < kSampleStats; ++i) {
    st[i] = wave_sum_f64(st[i]);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6][i] = st[i];
  }
  __syncthreads();
  if (threadIdx.x < kSampleStats) {
    double t = 0.0;
    for (int w = 0; w < kGammaThreads / 64; ++w) t += red[w][threadIdx.x];
    ws->sample[threadIdx.x][blk] = t;
  }
}

// Block 0 of the sampling launch clears what launches 3-4 accumulate into: the sum slots, the
// overflow flag and the exact pass's arrival counters.  (The exact pass's per-block word slots
// and the tiles' regions are overwritten, not added to.)
__device__ __forceinline__ void clear_pack_state(PackWs* __restrict__ ws, int blk) {
  if (blk != 0) return;
  for (int i = threadIdx.x; i < kGammaBlocks; i += kGammaThreads) ws->partial[i] = 0.0;
  if (threadIdx.x < kExactGroups) ws->done_grp[threadIdx.x][0] = 0u;
  if (threadIdx.x == 0) {
    ws->done_all = 0u;
    ws->overflow = 0u;
  }
}

__global__ __launch_bounds__(kGammaThreads) void gamma_sample_kernel(const float4* __restrict__ W4,
                                                                     int64_t count,
                                                                     PackWs* __restrict__ ws) {
  clear_pack_state(ws, blockIdx.x);
  gamma_sample_block(W4, count, ws, blockIdx.x);
}

// Round (sum_i words[i] * 2^(32 i - 149)) / count to the nearest fp32, ties to even, exactly.
// Each word is a 64-bit sum of 32-bit pieces (carry-free form); the carries are taken here.
__device__ float exact_mean_from_words(const unsigned long long* words, uint64_t count) {
  constexpr int L = 11;  // 352-bit integer in units of 2^-149
  uint32_t lim[L];
  uint64_t carry = 0;
  for (int i = 0; i < L; ++i) {
    const unsigned long long w = i < kExactWords ? words[i] : 0ull;
    // lim[i] = low word of (w + high word of the previous column + carry)
    const uint64_t lo = (uint64_t)(uint32_t)w + carry;
    lim[i] = (uint32_t)lo;
    carry = (lo >> 32) + (w >> 32);
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
  // word w of the quotient (0 past the top), as a select chain over the unrolled digits
  auto word = [&](int w) -> uint32_t {
    uint32_t r = 0;
#pragma unroll
    for (int i = 0; i < L; ++i) r = i == w ? q[i] : r;
    return r;
  };
  // the 24 significant bits: quotient bits shift .. shift + 23
  const uint64_t two = (uint64_t)word(shift >> 5) | ((uint64_t)word((shift >> 5) + 1) << 32);
  const uint32_t sig0 = (uint32_t)(two >> (shift & 31)) & 0xFFFFFFu;
  uint32_t sig = sig0;
  bool up;
  if (shift == 0) {
    up = (2 * rem > count) || (2 * rem == count && (sig & 1));
  } else {
    const int hb = shift - 1;                                   // the first bit below sig
    const uint32_t half = (word(hb >> 5) >> (hb & 31)) & 1u;
    bool lower = rem != 0;                                      // anything below the half bit
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int below = hb - 32 * i;                            // bits of word i under hb
      const uint32_t mask = below >= 32 ? 0xFFFFFFFFu : (below > 0 ? (1u << below) - 1u : 0u);
      lower = lower || (q[i] & mask) != 0u;
    }
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

constexpr int kExactThreads = 1024;  // 16 waves: four per SIMD for the rare exact pass
constexpr int kExactLoads = 2;       // float4 loads per thread per iteration of the exact pass

// Certified fp32 rounding of mean |W| from the fp64 slot sums, computed by one wave in one fixed
// order (every wave that certifies a master gets the same bits).  Returns 1 and *g when the
// rigorous error bound of the fp64 sum decides the rounding (or the sum is 0), else 0; the result
// is uniform across the wave.
__device__ __forceinline__ int wave_certify(const PackWs* __restrict__ ws, int64_t count,
                                            int64_t tiles, float* __restrict__ g) {
  static_assert(kGammaBlocks % 64 == 0, "slots split evenly over a wave");
  const int lane = threadIdx.x & 63;
  double v = 0.0;
#pragma unroll
  for (int i = 0; i < kGammaBlocks / 64; ++i) v += ws->partial[lane + 64 * i];
  v = wave_sum_f64(v);
  const double S = __shfl(v, 0, 64);
  // longest chain of fp64 additions any |w| goes through: in its pack tile the thread's 32
  // terms and the wave butterfly (6); its slot's chain (one hardware atomic addition per wave of
  // each tile that shares the slot, four per tile, counted twice in case the atomic unit rounds
  // faithfully rather than to nearest); here the lane's 16 slots and the butterfly (6).  128
  // covers every fixed term.
  const double depth = 128.0 + 8.0 * (double)((tiles + kGammaBlocks - 1) / kGammaBlocks);
  const double u = 0x1p-53;
  const double err = 2.0 * depth * u * S;  // >= ((1+u)^depth - 1) * S for nonnegative terms
  const double cnt = (double)count;
  const double lo = (S - err) / cnt * (1.0 - 4.0 * u);
  const double hi = (S + err) / cnt * (1.0 + 4.0 * u);
  const float glo = (float)lo, ghi = (float)hi;
  if (S == 0.0) { *g = 0.f; return 1; }
  if (glo == ghi) { *g = glo; return 1; }
  return 0;
}

// The exact pass of launch 4, for a master whose gamma the bound did not decide: the exact sum of
// |W| over this block's share (float4 i4 = blk * NT + tid, strided by the launch's blocks), the
// last block to finish rounding the exact mean.
// Each element's m << (max(e,1) - 1) is split into 32-bit pieces p0 (word w) and p1 (word w + 1);
// a lane keeps one 64-bit sum per word, so no carry is taken until the end (every word sum stays
// below count * 2^32 < 2^64).  Words no lane of the wave touches in an iteration are skipped.
__device__ __forceinline__ void gamma_exact_pass(const float* __restrict__ W, int64_t count,
                                                 PackWs* __restrict__ ws,
                                                 float* __restrict__ gamma_out, int blk, int nblk) {
  unsigned long long acc[kExactWords];
#pragma unroll
  for (int i = 0; i < kExactWords; ++i) acc[i] = 0ull;
  typedef __attribute__((address_space(1))) const v4f g_v4f;
  g_v4f* W4 = (g_v4f*)W;
  const int64_t n4 = count / 4;
  const int64_t stride = (int64_t)nblk * kExactThreads;
  // kExactLoads float4 loads per thread per iteration, issued one iteration ahead (the next
  // iteration's loads fly while this one's elements are summed); then, per word that some lane of
  // the wave touches, every element's piece for that word in one select chain
  constexpr int U = kExactLoads;
  auto load = [&](int64_t b, v4f (&dst)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i4 = b + u * stride + threadIdx.x;
      dst[u] = W4[min(i4, n4 - 1)];
      if (i4 >= n4) dst[u] = v4f{0.f, 0.f, 0.f, 0.f};   // past the end: adds nothing
    }
  };
  v4f nxt[U];
  load((int64_t)blk * kExactThreads, nxt);
  for (int64_t base = (int64_t)blk * kExactThreads; base < n4; base += U * stride) {
    v4f v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = nxt[u];
    load(base + U * stride, nxt);
    constexpr int E = 4 * U;
    uint32_t wd[E], p0[E], p1[E];
    uint32_t wmask = 0u;                  // words this lane's elements touch
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const uint32_t b = __float_as_uint(v[j / 4][j % 4]) & 0x7FFFFFFFu;
      const uint32_t e = b >> 23;
      const uint32_t m = (b & 0x7FFFFFu) | (e ? 0x800000u : 0u);
      const uint32_t sh = (e ? e : 1u) - 1u;
      const uint64_t piece = (uint64_t)m << (sh & 31u);   // p0 in word sh / 32, p1 in the next
      wd[j] = sh >> 5;
      p0[j] = (uint32_t)piece;
      p1[j] = (uint32_t)(piece >> 32);
      wmask |= m ? 3u << wd[j] : 0u;
    }
#pragma unroll
    for (int i = 0; i < kExactWords; ++i) {
      if (__ballot((wmask >> i) & 1u) == 0ull) continue;   // uniform: no lane touches word i
      uint64_t add = 0;
#pragma unroll
      for (int j = 0; j < E; ++j)
        add += wd[j] == (uint32_t)i ? p0[j] : (wd[j] + 1u == (uint32_t)i ? p1[j] : 0u);
      acc[i] += add;
    }
  }
  // block sums per word into this block's slot (plain stores); then the arrival counters
  __shared__ unsigned long long red[kExactThreads / 64][kExactWords];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < kExactWords; ++i) {
    unsigned long long x = acc[i];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    if (lane == 0) red[wave][i] = x;
  }
  __syncthreads();
  if (threadIdx.x < kExactWords) {
    unsigned long long x = 0ull;
    for (int w = 0; w < kExactThreads / 64; ++w) x += red[w][threadIdx.x];
    ws->slot[blk][threadIdx.x] = x;
  }
  // Release / acquire at agent scope: the slot stores of every block of a group happen before
  // its counter reaches the group's size; the last block of a group then counts in done_all,
  // and the block that completes done_all sees every slot.
  __shared__ int last_sh;
  __shared__ unsigned long long words_sh[kExactWords];
  // the barrier completes the slot stores (into this XCD's L2); thread 0's agent-scope release
  // below then writes them back for the other XCDs -- one L2 write-back per block, not one per
  // wave (a fence in every thread made this phase longer than the pass over W)
  __syncthreads();
  if (threadIdx.x == 0) {
    int last = 0;
    const int grp = blk % kExactGroups;
    const uint32_t gsize = (uint32_t)((nblk - 1 - grp) / kExactGroups + 1);
    if (__hip_atomic_fetch_add(&ws->done_grp[grp][0], 1u, __ATOMIC_ACQ_REL,
                               __HIP_MEMORY_SCOPE_AGENT) == gsize - 1u) {
      const uint32_t ngroups = (uint32_t)(nblk < kExactGroups ? nblk : kExactGroups);
      last = __hip_atomic_fetch_add(&ws->done_all, 1u, __ATOMIC_ACQ_REL,
                                    __HIP_MEMORY_SCOPE_AGENT) == ngroups - 1u;
    }
    last_sh = last;
  }
  __syncthreads();
  if (last_sh) {
    // sum the blocks' slots per word: wave w < kExactWords takes word w (no carry beyond 64 bits:
    // every word sum stays below count * 2^32 < 2^64)
    if (wave < kExactWords) {
      unsigned long long x = 0ull;
      for (int b = lane; b < nblk; b += 64)
        x += __hip_atomic_load(&ws->slot[b][wave], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
      if (lane == 0) words_sh[wave] = x;
    }
    __syncthreads();
  }
  if (last_sh && threadIdx.x == 0) {
    unsigned long long words[kExactWords];
    for (int i = 0; i < kExactWords; ++i) words[i] = words_sh[i];
    const float ge = exact_mean_from_words(words, (uint64_t)count);
    ws->gamma = ge;
    ws->tau = ternary_threshold(ge);
    ws->exact_used = 1u;
    gamma_out[0] = ge;
  }
}

// Launch 4 over `nm` masters (kExactBlocks blocks): wave w of every block certifies masters w,
// w + 16, ... (the same bits in every block, so the decisions are uniform), block 0 stores each
// certified master's gamma and tau, and then all blocks run the exact pass of each master the
// bound did not decide, in order.  item(m) gives master m's (W, count, tiles, ws, gamma).
template <typename Item>
__device__ __forceinline__ void gamma_masters(int nm, Item item) {
  constexpr int NW = kExactThreads / 64;
  __shared__ int need_sh[NW];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int m0 = 0; m0 < nm; m0 += NW) {
    if (m0 + wave < nm) {
      const float* W; int64_t count, tiles; PackWs* ws; float* gout;
      item(m0 + wave, &W, &count, &tiles, &ws, &gout);
      float g = 0.f;
      const int ok = wave_certify(ws, count, tiles, &g);
      if (lane == 0) need_sh[wave] = !ok;
      if (ok && blockIdx.x == 0 && lane == 0) {
        ws->gamma = g;
        ws->tau = ternary_threshold(g);
        ws->exact_used = 0u;
        gout[0] = g;
      }
    }
    __syncthreads();
    for (int w = 0; w < NW && m0 + w < nm; ++w) {
      if (!need_sh[w]) continue;   // uniform
      const float* W; int64_t count, tiles; PackWs* ws; float* gout;
      item(m0 + w, &W, &count, &tiles, &ws, &gout);
      gamma_exact_pass(W, count, ws, gout, blockIdx.x, gridDim.x);
      __syncthreads();
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kExactThreads) void gamma_exact_kernel(const float* __restrict__ W,
                                                                    int64_t count, int64_t tiles,
                                                                    PackWs* __restrict__ ws,
                                                                    float* __restrict__ gamma_out) {
  gamma_masters(1, [&](int, const float** w, int64_t* c, int64_t* t, PackWs** p, float** g) {
    *w = W; *c = count; *t = tiles; *p = ws; *g = gamma_out;
  });
}

constexpr int kPackWidth = 256;  // dense columns of a pack tile at most (one float4 per lane)

// fp32 neighbours of a positive fp64 value: the largest fp32 <= x and the smallest fp32 >= x.
__device__ __forceinline__ float f32_down(double x) {
  float f = (float)x;
  if ((double)f > x) f = __int_as_float(__float_as_int(f) - 1);
  return f;
}
__device__ __forceinline__ float f32_up(double x) {
  float f = (float)x;
  if ((double)f < x) f = __int_as_float(__float_as_int(f) + 1);
  return f;
}

// The band regions: tile t's kTileEntries entries at (uint2) entries[t * kTileEntries + e], each
// (code position word, |w| bits); unused entries hold kNoEntry, whose NaN never passes |w| >= tau.
constexpr uint32_t kNoEntryPos = 0xFFFFFFFFu, kNoEntryAbs = 0x7FFFFFFFu;
__device__ __forceinline__ uint2* ws_entries(PackWs* ws) {
  return (uint2*)((uint8_t*)ws + pack_ws_entries_off());
}

// The coding band, from the sampling launch's sums (one block per master, before the pass).  The
// sample mean mu estimates mean |W|; its standard error comes from the spread of the per-thread
// sums (ratio estimator).  gamma is taken to lie within mu (1 +- d), d = 6 standard errors +
// 2^-20, rounded outward to fp32, and the band is the two thresholds of those bounds: whatever
// gamma turns out to be inside it, a weight below tau_lo codes 0 and one at or above tau_hi codes
// +-1.  Not usable (band_ok 0, both bounds +inf: every weight codes 0 and nothing is listed, so
// the fix-up repacks) when the sample is empty, not finite, wider than a quarter of mu, the
// workspace has no region for every tile, or the code positions do not fit the entries' 27 bits.
__device__ __forceinline__ void band_block(PackWs* __restrict__ ws, uint64_t code_dwords,
                                           bool regions) {
  __shared__ double red[kSampleBlocks / 64][kSampleStats];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave < kSampleBlocks / 64) {
#pragma unroll
    for (int i = 0; i < kSampleStats; ++i) {
      const double t = wave_sum_f64(ws->sample[i][threadIdx.x]);
      if (lane == 0) red[wave][i] = t;
    }
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  double st[kSampleStats];
#pragma unroll
  for (int i = 0; i < kSampleStats; ++i) {
    st[i] = 0.0;
    for (int w = 0; w < kSampleBlocks / 64; ++w) st[i] += red[w][i];
  }
  float lo = __int_as_float(0x7f800000), hi = lo;
  uint32_t ok = 0u;
  const double c1 = st[3];
  const double mu = c1 > 0.0 ? st[0] / c1 : 0.0;
  // sum over threads of (s - mu c)^2
  const double v = fmax(st[1] - 2.0 * mu * st[2] + mu * mu * st[4], 0.0);
  const double d = 6.0 * sqrt(v) / c1 / mu + 0x1p-20;
  if (regions && c1 > 0.0 && mu > 0.0 && isfinite(mu) && d < 0.25 && code_dwords < (1ull << 27)) {
    const float glo = f32_down(mu * (1.0 - d)), ghi = f32_up(mu * (1.0 + d));
    if (glo > 0.f && ghi < 3.0e38f) {
      lo = ternary_threshold(glo);
      hi = ternary_threshold(ghi);
      ok = 1u;
    }
  }
  ws->tau_lo = lo;
  ws->tau_hi = hi;
  ws->band_ok = ok;
}

// Code dwords of a master (32-row panels x packed fragments x 64) and its pack tiles.
__host__ __device__ __forceinline__ uint64_t pack_code_dwords(int64_t n, int64_t K, int layout, int M) {
  const int64_t nfrag = layout == kLayoutSparse ? (M == 4 ? K : K / M * (2 * M - 4)) / 64 : K / 32;
  return (uint64_t)((n + kPanel - 1) / kPanel) * (uint64_t)nfrag * 64u;
}

__global__ __launch_bounds__(kGammaThreads) void band_kernel(PackWs* __restrict__ ws,
                                                             uint64_t code_dwords, int regions) {
  band_block(ws, code_dwords, regions != 0);
}

// One block packs one 32-row panel x KB dense columns (KB = pack_cols: whole M-groups and whole
// 32-slot fragments, at most 256).  Every lane loads one float4 of eight rows.  M = 4: that
// float4 is one whole group, masked and coded in registers; otherwise the fp32 tile is staged in
// LDS and each thread takes whole groups from it.  Either way a group becomes slot bytes
// (code | index << 2) in LDS, and 16-slot units are assembled into code/meta dwords, which land
// contiguously in the tiled layout (unit v = 32*u + r of the tile is dword base + v, slot i of it
// at bits 8 (i % 4) + 2 (i / 4)).
// SPEC (the one-pass pack): codes against the band; each wave's fp64 sum of |w| goes into slot
// blk % kGammaBlocks and the tile's band entries into its region.  Otherwise (the fix-up's
// repack) codes against the exact tau.
template <int LAYOUT, int M, bool SPEC>
__device__ __forceinline__ void pack_tile(const float* __restrict__ W, int n, int K, int N,
                                          int k_tiles, PackWs* __restrict__ ws,
                                          uint32_t* __restrict__ codes,
                                          uint32_t* __restrict__ meta, int blk) {
  constexpr bool SP = LAYOUT == kLayoutSparse;
  constexpr bool REG = M == 4;                                         // one group per float4
  constexpr int KB = pack_cols(LAYOUT, M);
  constexpr int WS = kPackWidth + 4;                                   // padded fp32 row
  constexpr int NKEEP = M == 4 ? 2 : M - 2;                           // SPARSE: 2:4, (M-2):M
  constexpr int SLOTS = SP ? KB * NKEEP / M : KB;
  constexpr int SS = SLOTS + 16;                                       // padded slot row
  constexpr int GPR = KB / M;                                          // groups per tile row
  constexpr int UPR = SLOTS / 16;                                      // units per tile row
  static_assert(!REG || GPR == 64, "a lane's float4 is group c4 of its rows");
  __shared__ __attribute__((aligned(16))) float tile[REG ? 1 : 32 * WS];
  __shared__ __attribute__((aligned(16))) uint8_t slots[32 * SS];
  __shared__ uint2 lst[SPEC ? kTileEntries : 1];
  __shared__ int nl_sh;

  const int P = blk / k_tiles;
  const int kb = blk % k_tiles;
  const int k0 = kb * KB;
  const int r0 = P * kPanel;
  const int kw = min(KB, K - k0);
  const int nfrag = SP ? (M == 4 ? K : K / M * (2 * M - 4)) / 64 : K / 32;   // fragments per panel
  const size_t base = ((size_t)P * nfrag + (size_t)kb * (UPR / 2)) * 64;

  // all eight 16-byte tile loads before anything else (addresses clamped into the matrix;
  // out-of-range rows and columns are zeroed after the load); non-temporal: the pass reads each
  // weight once
  const int c4 = threadIdx.x & 63, wv = threadIdx.x >> 6;
  float4 v[8];
  {
    typedef float f4v __attribute__((ext_vector_type(4)));
    const int col = k0 + min(4 * c4, kw - 4);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f4v t = __builtin_nontemporal_load(
          (const f4v*)(W + (size_t)min(r0 + i * 4 + wv, n - 1) * K + col));
      v[i] = make_float4(t.x, t.y, t.z, t.w);
    }
  }
  // codes: |w| >= hi is +-1, |w| < lo is 0, between (SPEC only) listed
  const float lo = SPEC ? ws->tau_lo : ws->tau, hi = SPEC ? ws->tau_hi : ws->tau;
  const uint32_t band_ok = SPEC ? ws->band_ok : 0u;
  if (SPEC && threadIdx.x == 0) nl_sh = 0;
  {
    const bool col_ok = 4 * c4 < kw;
    double ts = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = i * 4 + wv;
      if (!(col_ok && r0 + row < n)) v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (!REG) *(float4*)&tile[row * WS + 4 * c4] = v[i];
      if constexpr (SPEC) {
        ts += fabs((double)v[i].x); ts += fabs((double)v[i].y);
        ts += fabs((double)v[i].z); ts += fabs((double)v[i].w);
      }
    }
    if constexpr (SPEC) {
      // each wave adds its sum into the tile's slot; no return value is waited for
      ts = wave_sum_f64(ts);
      if (c4 == 0) unsafeAtomicAdd(&ws->partial[blk % kGammaBlocks], ts);
    }
  }
  // the LDS tile is complete and the entry counter is clear before any group reads or appends
  if constexpr (!REG || SPEC) __syncthreads();

  const int nkeep = SP ? NKEEP : N;
  // One M-group at (row, g) with values w: mask, codes, slot bytes.
  auto group = [&](int row, int g, const float (&w)[M]) {
    uint32_t a[M];
#pragma unroll
    for (int j = 0; j < M; ++j) a[j] = __float_as_uint(w[j]) & 0x7FFFFFFFu;
    uint32_t keep = 0;
#pragma unroll
    for (int i = 0; i < M; ++i) {
      int rank = 0;
#pragma unroll
      for (int j = 0; j < M; ++j)
        if (j != i) rank += (a[j] > a[i]) || (a[j] == a[i] && j < i);
      if (rank < nkeep) keep |= 1u << i;
    }
    // 00 = 0, 01 = +1, 10 = -1.  A kept weight of the band codes 0 here and is listed with its
    // code position (dword, slot i of the unit, sign) and |w|, for the fix-up.
    auto code = [&](int j, int sp) -> uint32_t {
      const float aj = __uint_as_float(a[j]);
      if (SPEC && aj >= lo && aj < hi) {
        const int i = sp & 15;
        const uint32_t x = (uint32_t)(base + 32 * (sp >> 4) + row) |
                           ((uint32_t)(4 * (i & 3) + (i >> 2)) << 27) | (w[j] < 0.f ? 1u << 31 : 0u);
        const int e = atomicAdd(&nl_sh, 1);
        if (e < kTileEntries) lst[e] = make_uint2(x, a[j]);
        return 0u;
      }
      return aj >= hi ? (w[j] < 0.f ? 2u : 1u) : 0u;
    };
    uint8_t* out = &slots[row * SS];
    if constexpr (SP && M == 4) {
      int s = 0;
#pragma unroll
      for (int p = 0; p < 4; ++p)
        if (keep >> p & 1u) { out[2 * g + s] = (uint8_t)(code(p, 2 * g + s) | (p << 2)); ++s; }
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
        out[NKEEP * g + slot] = (uint8_t)(code(p, NKEEP * g + slot) | ((p - 2 * wdw) << 2));
      }
    } else {
#pragma unroll
      for (int j = 0; j < M; ++j) out[g * M + j] = (uint8_t)((keep >> j & 1u) ? code(j, g * M + j) : 0u);
    }
  };
  if constexpr (REG) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float w[M];
      w[0] = v[i].x; w[1] = v[i].y; w[2] = v[i].z; w[3] = v[i].w;
      group(i * 4 + wv, c4, w);
    }
  } else {
    for (int gid = threadIdx.x; gid < 32 * GPR; gid += 256) {
      const int row = gid / GPR, g = gid % GPR;
      float w[M];
#pragma unroll
      for (int j = 0; j < M; ++j) w[j] = tile[row * WS + g * M + j];
      group(row, g, w);
    }
  }
  __syncthreads();

  const int valid_slots = SP ? kw * NKEEP / M : kw;
  const int units_valid = valid_slots / 16;
  for (int u4 = threadIdx.x; u4 < 32 * UPR; u4 += 256) {
    const int u = u4 >> 5, r = u4 & 31;
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
    codes[base + u4] = cw;
    if constexpr (SP) meta[base + u4] = mw;
  }
  if constexpr (SPEC) {
    // the tile's region: its band entries, then kNoEntry (no counter shared between tiles)
    if (!band_ok) return;
    const int nl = nl_sh;   // final: every append happened before the barrier above
    int e = threadIdx.x;
    asm volatile("" : "+v"(e));   // derive the entry's addresses here, not at the top
    if (nl > kTileEntries && e == 0) ws->overflow = 1u;
    if (e < kTileEntries)
      ws_entries(ws)[(size_t)blk * kTileEntries + e] =
          e < nl && nl <= kTileEntries ? lst[e] : make_uint2(kNoEntryPos, kNoEntryAbs);
  }
}

template <int LAYOUT, int M>
__global__ __launch_bounds__(256, 7) void pack_spec_kernel(const float* __restrict__ W, int n, int K,
                                                        int N, int k_tiles,
                                                        PackWs* __restrict__ ws,
                                                        uint32_t* __restrict__ codes,
                                                        uint32_t* __restrict__ meta) {
  pack_tile<LAYOUT, M, true>(W, n, K, N, k_tiles, ws, codes, meta, blockIdx.x);
}

// Sets the listed codes with |w| >= tau: entries start, start + stride, ... of the master's
// tiles * kTileEntries, four loads in flight per thread.
__device__ __forceinline__ void patch_codes(PackWs* __restrict__ ws, int64_t tiles,
                                            uint32_t* __restrict__ codes, float tau,
                                            int64_t start, int64_t stride) {
  constexpr int U = 4;
  const uint2* ent = ws_entries(ws);
  const int64_t total = tiles * kTileEntries;
  for (int64_t b = start; b < total; b += U * stride) {
    uint2 e[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      e[u] = b + u * stride < total ? ent[b + u * stride] : make_uint2(kNoEntryPos, kNoEntryAbs);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (__uint_as_float(e[u].y) >= tau)
        atomicOr(&codes[e[u].x & 0x7FFFFFFu], ((e[u].x >> 31) ? 2u : 1u) << (2 * ((e[u].x >> 27) & 15u)));
  }
}

// Launch 5 for one master (block blk of nblk): the listed codes are set when tau lies inside the
// band and no region overflowed; otherwise every tile is packed again (block blk takes tiles blk,
// blk + nblk, ...).  Uniform across the launch.
template <int LAYOUT, int M>
__device__ __forceinline__ void pack_fix_block(const float* __restrict__ W, int n, int K, int N,
                                               int k_tiles, PackWs* __restrict__ ws,
                                               uint32_t* __restrict__ codes,
                                               uint32_t* __restrict__ meta, int blk, int nblk) {
  const float tau = ws->tau;
  const bool patch = ws->band_ok && !ws->overflow && ws->tau_lo <= tau && tau <= ws->tau_hi;
  if (blk == 0 && threadIdx.x == 0) ws->fix_mode = patch ? 0u : 1u;
  const int64_t tiles = (int64_t)((n + kPanel - 1) / kPanel) * k_tiles;
  if (patch) {
    patch_codes(ws, tiles, codes, tau, (int64_t)blk * 256 + threadIdx.x, (int64_t)nblk * 256);
    return;
  }
  for (int64_t t = blk; t < tiles; t += nblk) {
    __syncthreads();   // the previous tile's LDS reads are done
    pack_tile<LAYOUT, M, false>(W, n, K, N, k_tiles, ws, codes, meta, (int)t);
  }
}

template <int LAYOUT, int M>
__global__ __launch_bounds__(256) void pack_fix_kernel(const float* __restrict__ W, int n, int K,
                                                       int N, int k_tiles, PackWs* __restrict__ ws,
                                                       uint32_t* __restrict__ codes,
                                                       uint32_t* __restrict__ meta) {
  pack_fix_block<LAYOUT, M>(W, n, K, N, k_tiles, ws, codes, meta, blockIdx.x, gridDim.x);
}

// ---------------------------------------------------------------------------------------------
// Grouped pack: the bitlinear_pack calls of several masters in five launches, each tensor's
// blocks running exactly the single call's arithmetic (so gamma, codes and meta are the same
// bits).  Every master's workspace slice holds a band region per tile of that master.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ PackGroupItem group_item(const uint8_t* __restrict__ table, int i) {
  return ((const PackGroupItem*)(table + sizeof(PackGroupHeader)))[i];
}

__device__ __forceinline__ int64_t item_tiles(const PackGroupItem& it) {
  return (int64_t)((it.n + kPanel - 1) / kPanel) * it.k_tiles;
}

// kSampleBlocks blocks per master, in table order.
__global__ __launch_bounds__(kGammaThreads) void gamma_sample_group_kernel(
    const uint8_t* __restrict__ table) {
  const PackGroupHeader* hd = (const PackGroupHeader*)table;
  if (hd->magic != kPackGroupMagic) return;
  const int b = blockIdx.x;
  if (b >= hd->count * kSampleBlocks) return;
  const PackGroupItem it = group_item(table, b / kSampleBlocks);
  clear_pack_state((PackWs*)it.ws, b % kSampleBlocks);
  gamma_sample_block((const float4*)it.W, (int64_t)it.n * it.K, (PackWs*)it.ws, b % kSampleBlocks);
}

// One block per master (every slice holds a region for each of its master's tiles).
__global__ __launch_bounds__(kGammaThreads) void band_group_kernel(const uint8_t* __restrict__ table) {
  const PackGroupHeader* hd = (const PackGroupHeader*)table;
  if (hd->magic != kPackGroupMagic || (int)blockIdx.x >= hd->count) return;
  const PackGroupItem it = group_item(table, blockIdx.x);
  band_block((PackWs*)it.ws, pack_code_dwords(it.n, it.K, hd->layout, hd->M), true);
}

template <int LAYOUT, int M>
__global__ __launch_bounds__(256, 7) void pack_group_kernel(const uint8_t* __restrict__ table) {
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
  pack_tile<LAYOUT, M, true>(it.W, it.n, it.K, hd->N, it.k_tiles, (PackWs*)it.ws, it.codes,
                             it.meta, b - it.block0);
}

// kExactBlocks blocks for the whole group.
__global__ __launch_bounds__(kExactThreads) void gamma_exact_group_kernel(
    const uint8_t* __restrict__ table) {
  const PackGroupHeader* hd = (const PackGroupHeader*)table;
  if (hd->magic != kPackGroupMagic) return;
  gamma_masters(hd->count, [&](int m, const float** w, int64_t* c, int64_t* t, PackWs** p, float** g) {
    const PackGroupItem it = group_item(table, m);
    *w = it.W; *c = (int64_t)it.n * it.K; *t = item_tiles(it); *p = (PackWs*)it.ws; *g = it.gamma;
  });
}

// kFixBlocks blocks per master, in table order.
template <int LAYOUT, int M>
__global__ __launch_bounds__(256) void pack_fix_group_kernel(const uint8_t* __restrict__ table) {
  const PackGroupHeader* hd = (const PackGroupHeader*)table;
  if (hd->magic != kPackGroupMagic || hd->layout != LAYOUT || hd->M != M) return;
  const int b = blockIdx.x;
  if (b >= hd->count * kFixBlocks) return;
  const PackGroupItem it = group_item(table, b / kFixBlocks);
  pack_fix_block<LAYOUT, M>(it.W, it.n, it.K, hd->N, it.k_tiles, (PackWs*)it.ws, it.codes,
                            it.meta, b % kFixBlocks, kFixBlocks);
}

hipError_t launch_pack(const float* W, int64_t n, int64_t K, int N, int M, int layout,
                       uint32_t* codes, uint32_t* meta, float* gamma, void* ws_raw,
                       int64_t tiles_cap, hipStream_t s) {
  PackWs* ws = (PackWs*)ws_raw;
  const int64_t count = n * K;
  const int panels = (int)((n + kPanel - 1) / kPanel);
  const int k_tiles = (int)((K + pack_cols(layout, M) - 1) / pack_cols(layout, M));
  const int64_t tiles = (int64_t)panels * k_tiles;
  gamma_sample_kernel<<<kSampleBlocks, kGammaThreads, 0, s>>>((const float4*)W, count, ws);
  band_kernel<<<1, kGammaThreads, 0, s>>>(ws, pack_code_dwords(n, K, layout, M), tiles <= tiles_cap);
  bool ok = dispatch_m(M, [&](auto m) {
    constexpr int MM = decltype(m)::value;
    if (layout == kLayoutSparse)
      pack_spec_kernel<kLayoutSparse, MM><<<(unsigned)tiles, 256, 0, s>>>(W, (int)n, (int)K, N, k_tiles, ws, codes, meta);
    else
      pack_spec_kernel<kLayoutDense2, MM><<<(unsigned)tiles, 256, 0, s>>>(W, (int)n, (int)K, N, k_tiles, ws, codes, nullptr);
  });
  if (!ok) return hipErrorInvalidValue;
  gamma_exact_kernel<<<kExactBlocks, kExactThreads, 0, s>>>(W, count, tiles, ws, gamma);
  ok = dispatch_m(M, [&](auto m) {
    constexpr int MM = decltype(m)::value;
    if (layout == kLayoutSparse)
      pack_fix_kernel<kLayoutSparse, MM><<<kFixBlocks, 256, 0, s>>>(W, (int)n, (int)K, N, k_tiles, ws, codes, meta);
    else
      pack_fix_kernel<kLayoutDense2, MM><<<kFixBlocks, 256, 0, s>>>(W, (int)n, (int)K, N, k_tiles, ws, codes, nullptr);
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Allocation-free pack, for callers that cannot allocate (code under graph capture, serving loops,
// harnesses that forbid allocation): bitlinear_pack with its workspace in this file's static
// device array instead of a caller buffer.  The array holds one pack workspace (kPackWsBytes,
// the same for every shape); each GPU the library runs on holds its own copy until the process
// ends, and every call on that GPU shares it, so calls that overlap on one GPU race.  The
// sampling launch clears the state the later launches accumulate into (sum slots, list counters,
// overflow flag, arrival counters), so a call never depends on what the previous one left there.
// ---------------------------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[kPackWsBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device, once looked up
}  // namespace

size_t pack_noalloc_capacity() { return sizeof(scratch); }

// The array's device address on the current device (looked up on the first call there).  In
// host code `scratch` names a host-side stand-in, never the device memory itself.
static hipError_t scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_pack_noalloc(const float* W, int64_t n, int64_t K, int N, int M, int layout,
                               uint32_t* codes, uint32_t* meta, float* gamma, hipStream_t s) {
  void* ws = nullptr;
  const hipError_t e = scratch_on_current_device(&ws);
  if (e != hipSuccess) return e;
  // band regions for at most kNoallocTiles tiles: a larger master is packed in two passes
  const int64_t tiles = (n + kPanel - 1) / kPanel * ((K + pack_cols(layout, M) - 1) / pack_cols(layout, M));
  return launch_pack(W, n, K, N, M, layout, codes, meta, gamma, ws,
                     tiles <= kNoallocTiles ? tiles : 0, s);
}

hipError_t launch_pack_group(const void* table, int64_t count, int64_t pack_blocks, int layout,
                             int M, hipStream_t s) {
  const uint8_t* t = (const uint8_t*)table;
  gamma_sample_group_kernel<<<(unsigned)(count * kSampleBlocks), kGammaThreads, 0, s>>>(t);
  band_group_kernel<<<(unsigned)count, kGammaThreads, 0, s>>>(t);
  const unsigned g = (unsigned)pack_blocks;
  bool ok = dispatch_m(M, [&](auto m) {
    constexpr int MM = decltype(m)::value;
    if (layout == kLayoutSparse) pack_group_kernel<kLayoutSparse, MM><<<g, 256, 0, s>>>(t);
    else pack_group_kernel<kLayoutDense2, MM><<<g, 256, 0, s>>>(t);
  });
  if (!ok) return hipErrorInvalidValue;
  gamma_exact_group_kernel<<<kExactBlocks, kExactThreads, 0, s>>>(t);
  const unsigned gf = (unsigned)(count * kFixBlocks);
  ok = dispatch_m(M, [&](auto m) {
    constexpr int MM = decltype(m)::value;
    if (layout == kLayoutSparse) pack_fix_group_kernel<kLayoutSparse, MM><<<gf, 256, 0, s>>>(t);
    else pack_fix_group_kernel<kLayoutDense2, MM><<<gf, 256, 0, s>>>(t);
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace bl
