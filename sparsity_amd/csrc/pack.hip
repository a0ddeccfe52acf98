// Absmean scale, N:M mask, ternarization and 2-bit packing of fp32 master weights.
//
// gamma is the mean |W| over the whole dense master (BitNet b1.58 page, "The mechanism",
// absmean quantization), taken before the mask (Sparse-BitNet technical summary, section 2,
// Forward Pass: quantize, then mask).  The mask keeps the N largest |w| of the continuous master
// in each M-group (same summary, Maskering) and (2N-2):2N groups -- 6:8, 14:16 -- are rewritten
// as N-1 overlapping 2:4 windows (SlideSparse abstract, Sliding Window Decomposition).
//
// Three launches, all on the caller's stream:
//   1. gamma_partial_kernel   fp64 partial sums of |w| (HBM-bound read of W); it also clears the
//                             arrival counters of launch 2
//   2. gamma_exact_kernel     every block sums the partials in one fixed order (all get the same
//                             bits) and certifies the fp32 rounding of the exact mean with a
//                             rigorous error bound.  Certified (the common case): block 0 stores
//                             gamma and the ternary threshold tau, and every block exits.
//                             Otherwise the blocks sum |W| exactly as integers (24-bit
//                             significands shifted to a 2^-149 fixed point, kept as carry-free
//                             32-bit words in 64-bit accumulators), each block stores its word
//                             sums in a line of its own, and the last block to arrive sums them,
//                             rounds the exact mean to fp32 and stores gamma and tau: one extra
//                             pass over W, once per master
//   3. pack_kernel            reads tau; mask, codes by |w| >= tau, slots assembled in LDS,
//                             coalesced dword stores.
#include <mutex>

#include "device_common.hpp"
#include "launch.hpp"
#include "pack_group.hpp"

namespace bl {


// The exact fixed-point sum: |w| = m * 2^(max(e,1) - 150) with a 24-bit significand m is
// m << (max(e,1) - 1) units of 2^-149, at most 24 + 253 bits, so word kExactWords - 1 = 8 is the
// highest a piece reaches.
struct PackWs {
  double partial[kGammaBlocks];      // fp64 partial sums of |w|, one per partial-sum block
  // exact fallback: block b's word sums (sum_i slot[b][i] * 2^(32 i) units of 2^-149), one
  // 128-byte line per block, written with plain stores: no two blocks touch one line
  unsigned long long slot[kExactBlocks][16];
  // arrival counters, one line each: block b counts in group b % kExactGroups; the last block of
  // a group counts in done_all (at most kExactBlocks / kExactGroups atomics queue on one line)
  uint32_t done_grp[kExactGroups][32];
  uint32_t done_all, pad[31];
  float gamma, tau;                  // gamma and the ternary threshold, read by every pack block
  uint32_t exact_used;               // 1 when the exact fallback decided gamma (diagnostic)
  uint32_t pad2;
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

// Block 0 also clears the exact pass's arrival counters: the exact launch counts in them, and
// this launch has completed before it starts.  (The per-block word slots are overwritten, not
// added to.)
__device__ __forceinline__ void clear_exact_state(PackWs* __restrict__ ws, int blk) {
  if (blk == 0 && threadIdx.x < kExactGroups) ws->done_grp[threadIdx.x][0] = 0u;
  if (blk == 0 && threadIdx.x == kExactGroups) ws->done_all = 0u;
}

__global__ __launch_bounds__(kGammaThreads) void gamma_partial_kernel(const float4* __restrict__ W4,
                                                                      int64_t n4,
                                                                      PackWs* __restrict__ ws) {
  clear_exact_state(ws, blockIdx.x);
  gamma_partial_block(W4, n4, ws->partial, blockIdx.x);
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

// Certified fp32 rounding of mean |W| from the fp64 partial sums, computed by a whole block in one
// fixed order (every block gets the same bits).  Returns 1 and *g when the rigorous error bound of
// the fp64 sum decides the rounding (or the sum is 0), else 0.
__device__ __forceinline__ int block_certify(const PackWs* __restrict__ ws, int64_t count,
                                             float* __restrict__ g) {
  static_assert(kGammaBlocks % kExactThreads == 0, "partials split evenly");
  __shared__ double red_sh[kExactThreads / 64];
  __shared__ float g_sh;
  __shared__ int ok_sh;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double v = 0.0;
#pragma unroll
  for (int i = 0; i < kGammaBlocks / kExactThreads; ++i) v += ws->partial[threadIdx.x + i * kExactThreads];
  v = wave_sum_f64(v);
  if (lane == 0) red_sh[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    double S = 0.0;
    for (int w = 0; w < kExactThreads / 64; ++w) S += red_sh[w];
    // longest chain of fp64 additions any |w| goes through: the partial kernel's per-thread
    // chains (at most 4 per float4 it reads, plus 2 to join its four chains), its wave butterfly
    // (6) and block sum (4), then here the per-thread sum (kGammaBlocks / kExactThreads = 1),
    // the butterfly (6) and the block sum (kExactThreads / 64 = 16); 64 covers every fixed term
    const int64_t n4 = count / 4;
    const int64_t per_thread = (n4 + (int64_t)kGammaBlocks * kGammaThreads - 1) / ((int64_t)kGammaBlocks * kGammaThreads);
    const double depth = 4.0 * (double)per_thread + 64.0;
    const double u = 0x1p-53;
    const double err = 2.0 * depth * u * S;  // >= ((1+u)^depth - 1) * S for nonnegative terms
    const double cnt = (double)count;
    const double lo = (S - err) / cnt * (1.0 - 4.0 * u);
    const double hi = (S + err) / cnt * (1.0 + 4.0 * u);
    const float glo = (float)lo, ghi = (float)hi;
    if (S == 0.0) { ok_sh = 1; g_sh = 0.f; }
    else if (glo == ghi) { ok_sh = 1; g_sh = glo; }
    else ok_sh = 0;
  }
  __syncthreads();
  *g = g_sh;
  return ok_sh;
}

// The exact sum of |W| over this block's share (float4 i4 = blk * NT + tid, strided by the
// master's blocks), added to ws->words; the last block to finish rounds the exact mean.
// Each element's m << (max(e,1) - 1) is split into 32-bit pieces p0 (word w) and p1 (word w + 1);
// a lane keeps one 64-bit sum per word, so no carry is taken until the end (every word sum stays
// below count * 2^32 < 2^64).  Words no lane of the wave touches in an iteration are skipped.
__device__ __forceinline__ void gamma_exact_block(const float* __restrict__ W, int64_t count, PackWs* __restrict__ ws,
                                  float* __restrict__ gamma_out, int blk, int nblk) {
  float g = 0.f;
  if (block_certify(ws, count, &g)) {   // uniform across the block and the launch
    if (blk == 0 && threadIdx.x == 0) {
      ws->gamma = g;
      ws->tau = ternary_threshold(g);
      ws->exact_used = 0u;
      gamma_out[0] = g;
    }
    return;
  }
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

__global__ __launch_bounds__(kExactThreads) void gamma_exact_kernel(const float* __restrict__ W,
                                                                    int64_t count,
                                                                    PackWs* __restrict__ ws,
                                                                    float* __restrict__ gamma_out) {
  gamma_exact_block(W, count, ws, gamma_out, blockIdx.x, gridDim.x);
}

constexpr int kPackWidth = 256;  // LDS width of a pack tile (fp32 columns)

// One block packs one 32-row panel x KB dense columns (KB = pack_cols: whole M-groups and whole
// 32-slot fragments, at most 256).  Phase 1 stages the fp32 tile in LDS with
// coalesced 1 KB row reads; phase 2 turns each M-group into slot bytes (code | index << 2);
// phase 3 assembles 16-slot units into code/meta dwords, which land contiguously in the tiled
// layout (unit v = 32*u + r of the tile is dword base + v).
template <int LAYOUT, int M>
__device__ __forceinline__ void pack_tile(const float* __restrict__ W, int n, int K, int N,
                                          int k_tiles, const PackWs* __restrict__ ws,
                                          uint32_t* __restrict__ codes,
                                          uint32_t* __restrict__ meta, int blk) {
  constexpr bool SP = LAYOUT == kLayoutSparse;
  constexpr int KB = pack_cols(LAYOUT, M);
  constexpr int WS = kPackWidth + 4;                                   // padded fp32 row
  constexpr int NKEEP = M == 4 ? 2 : M - 2;                           // SPARSE: 2:4, (M-2):M
  constexpr int SLOTS = SP ? KB * NKEEP / M : KB;
  constexpr int SS = SLOTS + 16;                                       // padded slot row
  constexpr int GPR = KB / M;                                          // groups per tile row
  constexpr int UPR = SLOTS / 16;                                      // units per tile row
  __shared__ __attribute__((aligned(16))) float tile[32 * WS];
  __shared__ __attribute__((aligned(16))) uint8_t slots[32 * SS];

  const int P = blk / k_tiles;
  const int kb = blk % k_tiles;
  const int k0 = kb * KB;
  const int r0 = P * kPanel;
  const int kw = min(KB, K - k0);

  // all eight 16-byte tile loads before the first LDS store (addresses clamped into the matrix;
  // out-of-range rows and columns are zeroed after the load)
  const float tau = ws->tau;
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
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = i * 4 + (threadIdx.x >> 6);
      if (!(col_ok && r0 + row < n)) v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      *(float4*)&tile[row * WS + 4 * c4] = v[i];
    }
  }
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
                                                   int k_tiles, const PackWs* __restrict__ ws,
                                                   uint32_t* __restrict__ codes,
                                                   uint32_t* __restrict__ meta) {
  pack_tile<LAYOUT, M>(W, n, K, N, k_tiles, ws, codes, meta, blockIdx.x);
}

// ---------------------------------------------------------------------------------------------
// Grouped pack: the bitlinear_pack calls of several masters in three launches, each tensor's
// blocks running exactly the single call's arithmetic (so gamma, codes and meta are the same
// bits).  The partial-sum launch walks the tensors in table order and the pack launch in reverse,
// so the tensors read last by the first launch -- still in the last-level cache -- are packed
// first.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kGammaThreads) void gamma_partial_group_kernel(
    const uint8_t* __restrict__ table) {
  const PackGroupHeader* hd = (const PackGroupHeader*)table;
  if (hd->magic != kPackGroupMagic) return;
  const int b = blockIdx.x;
  if (b >= hd->count * kGammaBlocks) return;
  const PackGroupItem it = ((const PackGroupItem*)(table + sizeof(PackGroupHeader)))[b / kGammaBlocks];
  clear_exact_state((PackWs*)it.ws, b % kGammaBlocks);
  gamma_partial_block((const float4*)it.W, (int64_t)it.n * it.K / 4, ((PackWs*)it.ws)->partial,
                      b % kGammaBlocks);
}

// kExactBlocks blocks per master, in table order (each exits at once unless its master is flagged).
__global__ __launch_bounds__(kExactThreads) void gamma_exact_group_kernel(
    const uint8_t* __restrict__ table) {
  const PackGroupHeader* hd = (const PackGroupHeader*)table;
  if (hd->magic != kPackGroupMagic) return;
  const int b = blockIdx.x;
  if (b >= hd->count * kExactBlocks) return;
  const PackGroupItem it = ((const PackGroupItem*)(table + sizeof(PackGroupHeader)))[b / kExactBlocks];
  gamma_exact_block(it.W, (int64_t)it.n * it.K, (PackWs*)it.ws, it.gamma, b % kExactBlocks,
                    kExactBlocks);
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
  pack_tile<LAYOUT, M>(it.W, it.n, it.K, hd->N, it.k_tiles, (const PackWs*)it.ws, it.codes,
                       it.meta, b - it.block0);
}

hipError_t launch_pack(const float* W, int64_t n, int64_t K, int N, int M, int layout,
                       uint32_t* codes, uint32_t* meta, float* gamma, void* ws_raw, hipStream_t s) {
  PackWs* ws = (PackWs*)ws_raw;
  const int64_t count = n * K;
  gamma_partial_kernel<<<kGammaBlocks, kGammaThreads, 0, s>>>((const float4*)W, count / 4, ws);
  gamma_exact_kernel<<<kExactBlocks, kExactThreads, 0, s>>>(W, count, ws, gamma);
  const int panels = (int)((n + kPanel - 1) / kPanel);
  const int k_tiles = (int)((K + pack_cols(layout, M) - 1) / pack_cols(layout, M));
  const dim3 grid((unsigned)(panels * k_tiles));
  const bool ok = dispatch_m(M, [&](auto m) {
    constexpr int MM = decltype(m)::value;
    if (layout == kLayoutSparse)
      pack_kernel<kLayoutSparse, MM><<<grid, 256, 0, s>>>(W, (int)n, (int)K, N, k_tiles, ws, codes, meta);
    else
      pack_kernel<kLayoutDense2, MM><<<grid, 256, 0, s>>>(W, (int)n, (int)K, N, k_tiles, ws, codes, nullptr);
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
// partial-sum launch clears the state the later launches accumulate into (exact words, block
// counter), so a call never depends on what the previous one left there.
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
  return launch_pack(W, n, K, N, M, layout, codes, meta, gamma, ws, s);
}

hipError_t launch_pack_group(const void* table, int64_t count, int64_t pack_blocks, int layout,
                             int M, hipStream_t s) {
  const uint8_t* t = (const uint8_t*)table;
  gamma_partial_group_kernel<<<(unsigned)(count * kGammaBlocks), kGammaThreads, 0, s>>>(t);
  gamma_exact_group_kernel<<<(unsigned)(count * kExactBlocks), kExactThreads, 0, s>>>(t);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned g = (unsigned)pack_blocks;
  const bool ok = dispatch_m(M, [&](auto m) {
    constexpr int MM = decltype(m)::value;
    if (layout == kLayoutSparse) pack_group_kernel<kLayoutSparse, MM><<<g, 256, 0, s>>>(t);
    else pack_group_kernel<kLayoutDense2, MM><<<g, 256, 0, s>>>(t);
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace bl
