// SPARSE6: the 2:4 ternary weights of a decode projection re-encoded at 6 bits per 4-wide group.
//
// A 2:4 group keeps two of its four positions (Sparse-BitNet summary, section 2, Maskering) and
// holds a ternary value on each (BitNet b1.58 page, "The mechanism"): 6 position pairs x 3 x 3
// values = 54 states, which fit in 6 bits -- 0.1875 bytes per weight against the 0.25 of the 2-bit
// codes plus 2-bit indices.  Decode is bound by weight bytes (BitNet b1.58 page, "Prior limits";
// the Bitnet.cpp abstract on the aitopics "bitnet" tag page argues for ternary formats below 2 bits
// per weight), so a quarter fewer bytes is a quarter less time if decoding stays off the critical
// path.
//
// State s = 9 * pair + 3 * digit(lower) + digit(upper); pairs (0,1) (0,2) (0,3) (1,2) (1,3) (2,3);
// digit(0, +1, -1) = 0, 1, 2 -- which is the 2-bit code of the 2:4 layout, so re-encoding is
// plain integer arithmetic on the packed buffers.
//
// Decoding: a 64-entry LDS table maps a state to the group's four effective int8 weights (one
// dword; state 0..53, zero above), so a 6-bit field costs an extract, a shift and one LDS read.
// Distinct states sit in distinct banks, so a wave's 64 table reads never conflict.  The weights
// are dense int8 after the lookup and feed v_mfma_i32_16x16x64_i8: A = 16 rows x 64 K of the
// panel (lane l: row l % 16, 16 bytes), B = 64 K x 16 tokens (lane l: token l % 16, 16 bytes), so
// the 16-token tile fits decode (T <= 16; two B tiles for T <= 32).  A lane's A and B bytes cover
// the same K positions whatever order the instruction gives them internally.
//
// Stream (per 32-row panel P and step pair c = 128 columns, NC = ceil(K / 128) pairs): lane l holds
// 96 bits in three dwords at dword ((P * NC + c) * 64 + l) * 3; field f = 8 s2 + 4 rt + g' (bits
// 6f..6f+5) is the state of row 32P + 16 rt + l % 16, group 32 c + 16 s2 + 4 (l / 16) + g'.  The
// A operand of row tile rt at step 2c + s2 is fields 8 s2 + 4 rt + 0..3: K 64 (2c + s2) +
// 16 (l / 16) + 0..15 of its row, and the lane's B operand is the 16 activation bytes of token
// l % 16 at the same K.  Rows past n and groups past K hold state 0 (zero weights).
//
// D layout of the 16x16 tile: lane l holds rows 4 (l / 16) + r (r = 0..3) of token l % 16.
#include "device_common.hpp"
#include "launch.hpp"

namespace bl {

namespace {
typedef __attribute__((address_space(1))) const uint32_t g6_u32;
typedef __attribute__((address_space(1))) const v4i g6_v4i;
typedef __attribute__((address_space(3))) const uint32_t lds_u32;

constexpr int kPairDwords = 64 * 3;   // stream dwords of one (panel, step pair)

// The four effective int8 weights of a state (byte k = position k of the group); 0 for 54..63.
__device__ __forceinline__ uint32_t state6_word(int s) {
  if (s >= 54) return 0u;
  const int p = s / 9, r = s % 9;
  const int i = p < 3 ? 0 : (p < 5 ? 1 : 2);
  const int j = p < 3 ? p + 1 : (p < 5 ? p - 1 : 3);
  const uint32_t va = (r / 3) == 0 ? 0u : (r / 3) == 1 ? 0x01u : 0xFFu;
  const uint32_t vb = (r % 3) == 0 ? 0u : (r % 3) == 1 ? 0x01u : 0xFFu;
  return (va << (8 * i)) | (vb << (8 * j));
}

// Field F (0..15) of a lane's 96 bits.
template <int F>
__device__ __forceinline__ uint32_t field6(uint32_t d0, uint32_t d1, uint32_t d2) {
  if constexpr (F < 5) return (d0 >> (6 * F)) & 63u;
  else if constexpr (F == 5) return __builtin_amdgcn_alignbit(d1, d0, 30) & 63u;
  else if constexpr (F < 10) return (d1 >> (6 * F - 32)) & 63u;
  else if constexpr (F == 10) return __builtin_amdgcn_alignbit(d2, d1, 28) & 63u;
  else return (d2 >> (6 * F - 64)) & 63u;
}

// A operand of step half S2, row tile RT: the effective weights of fields 8 S2 + 4 RT + 0..3.
template <int S2, int RT>
__device__ __forceinline__ v4i a6(uint32_t d0, uint32_t d1, uint32_t d2, lds_u32* lut) {
  constexpr int F = 8 * S2 + 4 * RT;
  v4i a;
  a[0] = (int)lut[field6<F>(d0, d1, d2)];
  a[1] = (int)lut[field6<F + 1>(d0, d1, d2)];
  a[2] = (int)lut[field6<F + 2>(d0, d1, d2)];
  a[3] = (int)lut[field6<F + 3>(d0, d1, d2)];
  return a;
}

__device__ __forceinline__ v4i mfma16(const v4i& a, const v4i& b, const v4i& c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// One step pair of one 32-row panel: 2 steps x 2 row tiles x TH token tiles of MFMAs.  b[s2][th]
// are the lane's B operands of the two steps.
template <int TH>
__device__ __forceinline__ void pair6(uint32_t d0, uint32_t d1, uint32_t d2, const v4i (&b)[2][TH],
                                      lds_u32* lut, v4i (&acc)[2][TH]) {
  const v4i a00 = a6<0, 0>(d0, d1, d2, lut), a01 = a6<0, 1>(d0, d1, d2, lut);
#pragma unroll
  for (int th = 0; th < TH; ++th) {
    acc[0][th] = mfma16(a00, b[0][th], acc[0][th]);
    acc[1][th] = mfma16(a01, b[0][th], acc[1][th]);
  }
  const v4i a10 = a6<1, 0>(d0, d1, d2, lut), a11 = a6<1, 1>(d0, d1, d2, lut);
#pragma unroll
  for (int th = 0; th < TH; ++th) {
    acc[0][th] = mfma16(a10, b[1][th], acc[0][th]);
    acc[1][th] = mfma16(a11, b[1][th], acc[1][th]);
  }
}
}  // namespace

// ---------------------------------------------------------------------------------------------
// re-encoding: 2:4 packed codes + meta -> SPARSE6 stream
// ---------------------------------------------------------------------------------------------
// One thread per (panel, step pair, lane): it reads the four (code, meta) unit dwords its 16 fields
// come from and writes its three stream dwords.  The 2:4 unit of row r holding group g is unit
// g / 8 (slots 2 (g % 8), 2 (g % 8) + 1); unit (r, u) is dword ((r / 32) (U / 2) + u / 2) 64 +
// (u % 2) 32 + r % 32 with U = K / 32 units per row.
__global__ __launch_bounds__(256) void transcode6_kernel(const uint32_t* __restrict__ codes,
                                                         const uint32_t* __restrict__ meta,
                                                         int npanels, int K,
                                                         uint32_t* __restrict__ out) {
  const int NC = (K + 127) >> 7;
  const int U = K >> 5;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (int64_t)npanels * NC * 64) return;
  const int l = (int)(id & 63);
  const int c = (int)((id >> 6) % NC);
  const int P = (int)((id >> 6) / NC);
  uint32_t w[3] = {0u, 0u, 0u};
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    const int g0 = 32 * c + 16 * s2 + 4 * (l >> 4);   // first of the lane's four groups
    if (4 * g0 >= K) continue;                         // past K: state 0
    const int u = g0 >> 3, j0 = g0 & 7;                // unit; first window in it (0 or 4)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int r = 16 * rt + (l & 15);                // row within the panel
      const size_t at = ((size_t)P * (U / 2) + u / 2) * 64 + (u % 2) * 32 + r;
      const uint32_t cd = codes[at], md = meta[at];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int a = 2 * (j0 + g), b = a + 1;         // the group's two slots
        const uint32_t ca = (cd >> (8 * (a & 3) + 2 * (a >> 2))) & 3u;
        const uint32_t cb = (cd >> (8 * (b & 3) + 2 * (b >> 2))) & 3u;
        const uint32_t ia = (md >> (2 * a)) & 3u, ib = (md >> (2 * b)) & 3u;
        const uint32_t p = ia == 0 ? ib - 1 : (ia == 1 ? ib + 1 : 5u);
        const uint32_t st = 9 * p + 3 * ca + cb;
        const int f = 8 * s2 + 4 * rt + g, bit = 6 * f;
        w[bit >> 5] |= st << (bit & 31);
        if ((bit & 31) > 26) w[(bit >> 5) + 1] |= st >> (32 - (bit & 31));
      }
    }
  }
  uint32_t* o = out + (size_t)id * 3;
  o[0] = w[0];
  o[1] = w[1];
  o[2] = w[2];
}

hipError_t launch_transcode6(const uint32_t* codes, const uint32_t* meta, int64_t n, int64_t K,
                             uint32_t* out, hipStream_t s) {
  const int npanels = (int)((n + kPanel - 1) / kPanel);
  const int64_t threads = (int64_t)npanels * ((K + 127) / 128) * 64;
  transcode6_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(codes, meta, npanels, (int)K,
                                                                     out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// single projection: one block per 32-row panel, waves split the step pairs
// ---------------------------------------------------------------------------------------------
// The layout of gemv_kernel: each wave issues its stream loads first (at most MAXP pairs, three
// dwords each), the block stages xq[T][K] in LDS (row stride K + 16) when it fits (LDSB), the
// waves' int32 partials are summed through LDS in wave order.  Pairs past a wave's share reload
// the last pair with its fields zeroed (state 0: zero weights); the second step of a half pair
// past K reads the activations of the last full step (clamped), against zero weights.
template <int NW, int MAXP, int TH, bool LDSB>
__global__ __launch_bounds__(64 * NW) void gemv6_kernel(const int8_t* __restrict__ xq,
                                                        const float* __restrict__ xs, int T, int K,
                                                        const uint32_t* __restrict__ stream,
                                                        const float* __restrict__ gamma_p, int n,
                                                        float* __restrict__ y,
                                                        int32_t* __restrict__ acc_out) {
  extern __shared__ __attribute__((aligned(16))) int8_t gsm[];
  __shared__ uint32_t lut[64];
  const int P = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int NC = (K + 127) >> 7, NS = K >> 6;
  const int per = (NC + NW - 1) / NW;              // host guarantees per <= MAXP
  const int c_begin = min(wave * per, NC - 1);
  const int cnt = min(per, NC - wave * per);      // may be <= 0 for trailing waves
  g6_u32* wp = (g6_u32*)stream + ((size_t)P * NC * 64 + lane) * 3;
  uint32_t d[MAXP][3];
#pragma unroll
  for (int u = 0; u < MAXP; ++u) {
    const int c = min(c_begin + u, NC - 1);
#pragma unroll
    for (int k = 0; k < 3; ++k) d[u][k] = __builtin_nontemporal_load(wp + (size_t)c * kPairDwords + k);
  }
  if (threadIdx.x < 64) lut[threadIdx.x] = state6_word(threadIdx.x);

  const int tok = lane & 15, q = lane >> 4;
  const float gamma = *gamma_p;
  const int stride = K + 16;
  if constexpr (LDSB) {
    const int cpr = K / 16;
    const int chunks = T * cpr;
    for (int c0 = 0; c0 < chunks; c0 += 64 * NW * 8) {
      int4 v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int ci = min(c0 + k * 64 * NW + (int)threadIdx.x, chunks - 1);
        v[k] = *(const int4*)(xq + (size_t)(ci / cpr) * K + 16 * (ci % cpr));
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int ci = c0 + k * 64 * NW + (int)threadIdx.x;
        if (ci < chunks) *(int4*)&gsm[(ci / cpr) * stride + 16 * (ci % cpr)] = v[k];
      }
    }
  }
  __syncthreads();

  v4i acc[2][TH];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int th = 0; th < TH; ++th) acc[rt][th] = v4i{0, 0, 0, 0};
#pragma unroll
  for (int u = 0; u < MAXP; ++u) {
    const int c = min(c_begin + u, NC - 1);
    const bool live = u < cnt;
    v4i b[2][TH];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int s = min(2 * c + s2, NS - 1);
#pragma unroll
      for (int th = 0; th < TH; ++th) {
        const int row = min(tok + 16 * th, T - 1);   // dead token lanes read a live row
        if constexpr (LDSB)
          b[s2][th] = *(const v4i*)(gsm + row * stride + 64 * s + 16 * q);
        else
          b[s2][th] = *(g6_v4i*)(xq + (size_t)row * K + 64 * s + 16 * q);
      }
    }
    pair6<TH>(live ? d[u][0] : 0u, live ? d[u][1] : 0u, live ? d[u][2] : 0u, b, (lds_u32*)lut, acc);
  }

  constexpr int R = 2 * TH * 4;                    // accumulator registers per lane
  int* red = (int*)(gsm + (LDSB ? ((size_t)T * stride + 15) / 16 * 16 : 0));
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int th = 0; th < TH; ++th)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(wave * R + (rt * TH + th) * 4 + r) * 64 + lane] = acc[rt][th][r];
  __syncthreads();
  for (int i = threadIdx.x; i < R * 64; i += 64 * NW) {
    const int reg = i >> 6, l = i & 63;
    const int rt = reg / (4 * TH), th = (reg >> 2) % TH, r = reg & 3;
    const int tk = 16 * th + (l & 15);
    const int o = P * kPanel + 16 * rt + 4 * (l >> 4) + r;
    if (tk < T && o < n) {
      int32_t sum = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) sum += red[(w * R + reg) * 64 + l];
      const size_t idx = (size_t)tk * n + o;
      y[idx] = ((float)sum * gamma) * xs[tk];
      if (acc_out) acc_out[idx] = sum;
    }
  }
}

size_t gemv6_smem_bytes(int64_t T, int64_t K, bool ldsb) {
  const size_t stage = ldsb ? ((size_t)T * (K + 16) + 15) / 16 * 16 : 0;
  return stage + (size_t)8 * (2 * 2 * 4) * 64 * 4;
}

hipError_t launch_fwd6(const int8_t* xq, const float* xs, int64_t T, int64_t K,
                       const uint32_t* stream, const float* gamma, int64_t n, float* y,
                       int32_t* acc, hipStream_t s) {
  const int npanels = (int)((n + kPanel - 1) / kPanel);
  const int64_t nc = (K + 127) / 128;
  const bool ldsb = gemv6_smem_bytes(T, K, true) <= 160 * 1024 - 512;
  const size_t smem = gemv6_smem_bytes(T, K, ldsb);
  auto run = [&](auto kern) -> hipError_t {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)smem);
    if (e != hipSuccess) return e;
    kern<<<npanels, 512, smem, s>>>(xq, xs, (int)T, (int)K, stream, gamma, (int)n, y, acc);
    return hipGetLastError();
  };
  auto by_th = [&](auto maxp) -> hipError_t {
    constexpr int MP = decltype(maxp)::value;
    if (T <= 16) return ldsb ? run(gemv6_kernel<8, MP, 1, true>) : run(gemv6_kernel<8, MP, 1, false>);
    return ldsb ? run(gemv6_kernel<8, MP, 2, true>) : run(gemv6_kernel<8, MP, 2, false>);
  };
  // pairs per wave bounded by MAXP (the host checked nc <= 8 * 16)
  if (nc <= 8 * 2) return by_th(std::integral_constant<int, 2>{});
  if (nc <= 8 * 4) return by_th(std::integral_constant<int, 4>{});
  if (nc <= 8 * 8) return by_th(std::integral_constant<int, 8>{});
  return by_th(std::integral_constant<int, 16>{});
}

// ---------------------------------------------------------------------------------------------
// grouped decode over a table of projections (the layout of gemv_group_kernel)
// ---------------------------------------------------------------------------------------------
// Work item = up to 16 consecutive 32-row panels of one projection; wave w owns panels w and
// w + 8 over the whole K axis.  K is walked in chunks of two step pairs (256 columns): each
// wave's stream dwords (two panels x two pairs x three) and the block's token rows for the chunk
// ride a ring of kGD6 register chunks, the rows go to a double-buffered LDS tile one chunk ahead,
// and the MFMAs read B from LDS.  Pairs past the end of K re-read the last pair with their fields
// zeroed.
namespace {
constexpr int kGD6 = 3;        // ring depth in chunks
constexpr int kCB6 = 256;      // token row bytes per chunk
constexpr int kRow6 = kCB6 + 16;

struct Chunk6 {
  uint32_t d[kGroupPanelsPerWave][2][3];   // [panel][pair][dword]
  v4i b;                                   // this thread's 16-byte piece of the token rows
};

template <int TH>
struct Group6 {
  int8_t* bs;                  // LDS: two buffers of 32 rows x kRow6 bytes
  lds_u32* lut;
  g6_u32* wp[kGroupPanelsPerWave];   // this lane's first dword of pair 0 of each panel
  int ws[kGroupPanelsPerWave];       // dwords between pairs: kPairDwords, or 0 past the panels
  __attribute__((address_space(1))) const int8_t* xq;
  int tid, T, K, NC, NS, nch, bpieces, tok, q;
  v4i acc[kGroupPanelsPerWave][2][TH];

  __device__ __forceinline__ void issue(int j, Chunk6& r) const {
#pragma unroll
    for (int p = 0; p < kGroupPanelsPerWave; ++p)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int c = min(2 * j + u, NC - 1);
#pragma unroll
        for (int k = 0; k < 3; ++k)
          r.d[p][u][k] = __builtin_nontemporal_load(wp[p] + (size_t)c * ws[p] + k);
      }
    // token piece tid: row tid / 16, 16 bytes at column 16 (tid % 16) of the chunk (clamped into
    // the matrix; a piece past K only meets zero weights)
    const int row = min(tid >> 4, T - 1), col = min(16 * (tid & 15) + j * kCB6, K - 16);
    r.b = *(g6_v4i*)(xq + (size_t)row * K + col);
  }
  __device__ __forceinline__ void put(int j, const Chunk6& r) const {
    if (tid < bpieces) *(v4i*)&bs[(j & 1) * (32 * kRow6) + (tid >> 4) * kRow6 + 16 * (tid & 15)] = r.b;
  }
  __device__ __forceinline__ void compute(int j, const Chunk6& r) {
    const int8_t* xr = bs + (j & 1) * (32 * kRow6) + 16 * q;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const bool live = 2 * j + u < NC;
      v4i b[2][TH];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int th = 0; th < TH; ++th)
          b[s2][th] = *(const v4i*)(xr + min(tok + 16 * th, T - 1) * kRow6 + 128 * u + 64 * s2);
#pragma unroll
      for (int p = 0; p < kGroupPanelsPerWave; ++p)
        pair6<TH>(live ? r.d[p][u][0] : 0u, live ? r.d[p][u][1] : 0u, live ? r.d[p][u][2] : 0u, b,
                  lut, acc[p]);
    }
  }
  __device__ __forceinline__ void step(int j, Chunk6& cur, const Chunk6& nxt) {
    if (j < nch) compute(j, cur);
    put(j + 1, nxt);
    issue(j + kGD6, cur);
    block_sync_lds();
  }
};

template <int TH>
__device__ __forceinline__ void group6_item(const GroupLayer& L, int panel0, int8_t* bs,
                                            const uint32_t* lut) {
  Group6<TH> k;
  k.tid = threadIdx.x;
  const int lane = k.tid & 63, wave = k.tid >> 6;
  k.T = L.T;
  k.K = L.Keff;
  k.NC = (k.K + 127) >> 7;
  k.NS = k.K >> 6;
  k.nch = (k.NC + 1) >> 1;
  const int n = L.n;
  const int npanels = (n + kPanel - 1) / kPanel;
  int P[kGroupPanelsPerWave];
#pragma unroll
  for (int p = 0; p < kGroupPanelsPerWave; ++p) {
    P[p] = panel0 + p * kGroupWaves + wave;
    const int Pl = min(P[p], npanels - 1);
    k.wp[p] = (g6_u32*)L.codes + ((size_t)Pl * k.NC * 64 + lane) * 3;
    k.ws[p] = P[p] < npanels ? kPairDwords : 0;
  }
  k.xq = (__attribute__((address_space(1))) const int8_t*)L.xq;
  k.bs = bs;
  k.lut = (lds_u32*)lut;
  k.bpieces = k.T * 16;
  k.tok = lane & 15;
  k.q = lane >> 4;
  const float gamma = *(__attribute__((address_space(1))) const float*)L.gamma;

  Chunk6 r[kGD6];
#pragma unroll
  for (int i = 0; i < kGD6; ++i) {
    k.issue(i, r[i]);
    asm volatile("" ::: "memory");
  }
  k.put(0, r[0]);
  block_sync_lds();
#pragma unroll
  for (int p = 0; p < kGroupPanelsPerWave; ++p)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int th = 0; th < TH; ++th) k.acc[p][rt][th] = v4i{0, 0, 0, 0};
  for (int j = 0; j < k.nch; j += kGD6) {
#pragma unroll
    for (int i = 0; i < kGD6; ++i) k.step(j + i, r[i], r[(i + 1) % kGD6]);
  }

  const bool vec = (n & 3) == 0;
#pragma unroll
  for (int th = 0; th < TH; ++th) {
    const int tk = 16 * th + k.tok;
    if (tk >= k.T) continue;
    const float sc = *((__attribute__((address_space(1))) const float*)L.xs + tk);
#pragma unroll
    for (int p = 0; p < kGroupPanelsPerWave; ++p) {
      if (P[p] >= npanels) break;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int o = P[p] * kPanel + 16 * rt + 4 * k.q;
        const size_t idx = (size_t)tk * n + o;
        const v4i a = k.acc[p][rt][th];
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = ((float)a[i] * gamma) * sc;
        if (vec && o + 3 < n) {
          *(float4*)(L.y + idx) = make_float4(v[0], v[1], v[2], v[3]);
          if (L.acc)
#pragma unroll
            for (int i = 0; i < 4; ++i) L.acc[idx + i] = a[i];
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (o + i < n) {
              L.y[idx + i] = v[i];
              if (L.acc) L.acc[idx + i] = a[i];
            }
        }
      }
    }
  }
}
}  // namespace

__global__ __launch_bounds__(64 * kGroupWaves) __attribute__((amdgpu_waves_per_eu(4)))
void gemv6_group_kernel(const uint8_t* __restrict__ table) {
  __shared__ __attribute__((aligned(16))) int8_t bs[2 * 32 * kRow6];
  __shared__ uint32_t lut[64];
  const GroupHeader* hdr = (const GroupHeader*)table;
  const int item = blockIdx.x;
  if (hdr->magic != kGroupMagic || hdr->layout != kLayoutSparse6 || hdr->fused != 0 ||
      item >= hdr->items)
    return;
  const GroupItem it = ((const GroupItem*)(table + sizeof(GroupHeader) +
                                           hdr->count * sizeof(GroupLayer)))[item];
  if (it.layer == kGroupNoItem) return;
  const GroupLayer L = ((const GroupLayer*)(table + sizeof(GroupHeader)))[it.layer];
  if (threadIdx.x < 64) lut[threadIdx.x] = state6_word(threadIdx.x);
  // the table is complete before the first decode: issue() of the ring prologue does not read it,
  // and the block_sync_lds after put(0) orders the table writes before every compute()
  if (L.T > 16) group6_item<2>(L, (int)it.panel0, bs, lut);
  else group6_item<1>(L, (int)it.panel0, bs, lut);
}

hipError_t launch_fwd6_group(const void* table, int64_t items, hipStream_t s) {
  gemv6_group_kernel<<<(unsigned)items, 64 * kGroupWaves, 0, s>>>((const uint8_t*)table);
  return hipGetLastError();
}

}  // namespace bl
