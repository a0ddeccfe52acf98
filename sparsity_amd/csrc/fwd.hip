// Sparse ternary x int8 forward: y[t][o] = gamma * scale[t] * sum_k W_eff[o][k] * xq[t][k].
//
// A ternary multiply-accumulate is an add, a subtract or a skip (BitNet b1.58 page, "The
// mechanism"); on gfx950 the cheapest way to do that at scale is to hand the ternary values to
// the matrix cores as int8.  SPARSE weights feed the int8 sparse MFMA (v_smfmac_i32_32x32x64_i8):
// one packed unit per lane is exactly its A operand -- the code dword expands to the 16
// compressed int8 values with four v_perm_b32 lookups and the meta dword *is* the instruction's
// index operand.  DENSE2 weights feed the dense v_mfma_i32_32x32x32_i8.  Accumulation is int32
// (exact: |acc| <= 127 * K_eff < 2^31); the fp32 rescale is fused into the epilogue.
//
// Operand layouts of the 32x32 tiles (lane l, h = l / 32):
//   A (weights)  row l % 32 of the panel; 32 dense K positions 32h.. (sparse) / 16 (dense)
//   B (tokens)   token l % 32; sparse: K bytes [16h, 16h+16) and [32+16h, 48+16h) of the step;
//                dense: K bytes [16h, 16h+16)
//   D (int32)    token l % 32; rows 8*(r/4) + 4h + r%4 for register r = 0..15
//
// Two kernels:
//   gemv_kernel  decode, T <= 32 tokens: one block per 32-row panel, waves split the K steps,
//                B straight from global/L2 (only lanes of live tokens load), int32 partials
//                reduced through LDS in a fixed order.
//   gemm_kernel  prefill: block tile BM rows x BN tokens; B staged in LDS (double buffered),
//                A loaded per wave straight into registers one step ahead.
#include "device_common.hpp"
#include "launch.hpp"

namespace bl {

template <bool SP>
__device__ __forceinline__ v16i mfma_step(uint32_t code, uint32_t meta, const int4& blo,
                                          const int4& bhi, v16i acc) {
  const v4i a = expand_codes(code);
  if constexpr (SP) {
    v8i b;
    b[0] = blo.x; b[1] = blo.y; b[2] = blo.z; b[3] = blo.w;
    b[4] = bhi.x; b[5] = bhi.y; b[6] = bhi.z; b[7] = bhi.w;
    return __builtin_amdgcn_smfmac_i32_32x32x64_i8(a, b, acc, (int)meta, 0, 0);
  } else {
    v4i b;
    b[0] = blo.x; b[1] = blo.y; b[2] = blo.z; b[3] = blo.w;
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc, 0, 0, 0);
  }
}

__device__ __forceinline__ void store_out(float* __restrict__ y, int32_t* __restrict__ acc_out,
                                          size_t idx, int32_t a, float gamma, float sc) {
  const float v = ((float)a * gamma) * sc;
  y[idx] = v;
  if (acc_out) acc_out[idx] = a;
}

// ---------------------------------------------------------------------------------------------
// decode GEMV
// ---------------------------------------------------------------------------------------------
template <int LAYOUT, int NW, int UNROLL>
__global__ __launch_bounds__(64 * NW) void gemv_kernel(const int8_t* __restrict__ xq,
                                                       const float* __restrict__ xs, int T,
                                                       int Keff, const uint32_t* __restrict__ codes,
                                                       const uint32_t* __restrict__ meta,
                                                       const float* __restrict__ gamma_p, int n,
                                                       float* __restrict__ y,
                                                       int32_t* __restrict__ acc_out) {
  constexpr bool SP = LAYOUT == kLayoutSparse;
  constexpr int KSTEP = SP ? 64 : 32;
  const int P = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int NF = Keff / KSTEP;
  const uint32_t* cp = codes + (size_t)P * NF * 64 + lane;
  const uint32_t* mp = SP ? meta + (size_t)P * NF * 64 + lane : nullptr;
  const int tok = lane & 31, h = lane >> 5;
  const bool live = tok < T;
  const int8_t* xp = xq + (size_t)(live ? tok : 0) * Keff + 16 * h;
  v16i acc = {};
  for (int s0 = wave * UNROLL; s0 < NF; s0 += NW * UNROLL) {
    uint32_t c[UNROLL], m[UNROLL];
    int4 blo[UNROLL], bhi[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int s = s0 + u;
      const bool ok = s < NF;
      c[u] = ok ? __builtin_nontemporal_load(cp + (size_t)s * 64) : 0u;
      m[u] = (SP && ok) ? __builtin_nontemporal_load(mp + (size_t)s * 64) : kPadMeta;
      blo[u] = make_int4(0, 0, 0, 0);
      bhi[u] = make_int4(0, 0, 0, 0);
      if (ok && live) {
        blo[u] = *(const int4*)(xp + (size_t)s * KSTEP);
        if constexpr (SP) bhi[u] = *(const int4*)(xp + (size_t)s * KSTEP + 32);
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc = mfma_step<SP>(c[u], m[u], blo[u], bhi[u], acc);
  }
  __shared__ int red[NW][16][64];
#pragma unroll
  for (int r = 0; r < 16; ++r) red[wave][r][lane] = acc[r];
  __syncthreads();
  const float gamma = *gamma_p;
  for (int i = threadIdx.x; i < 16 * 64; i += 64 * NW) {
    const int r = i >> 6, l = i & 63;
    const int tk = l & 31;
    const int o = P * kPanel + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
    if (tk < T && o < n) {
      int32_t sum = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) sum += red[w][r][l];
      store_out(y, acc_out, (size_t)tk * n + o, sum, gamma, xs[tk]);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// prefill GEMM
// ---------------------------------------------------------------------------------------------
template <int LAYOUT, int WM, int WN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, int T, int Keff,
    const uint32_t* __restrict__ codes, const uint32_t* __restrict__ meta,
    const float* __restrict__ gamma_p, int n, int npanels, float* __restrict__ y,
    int32_t* __restrict__ acc_out, int tiles_m) {
  constexpr bool SP = LAYOUT == kLayoutSparse;
  constexpr int KSTEP = SP ? 64 : 32;
  constexpr int NT = 64 * WAVES_M * WAVES_N;
  constexpr int BM = 32 * WM * WAVES_M;
  constexpr int BN = 32 * WN * WAVES_N;
  constexpr int LSTR = KSTEP + 16;             // padded LDS bytes per token row
  constexpr int CPR = KSTEP / 16;              // 16-byte chunks per token row
  constexpr int CPT = BN * CPR / NT;           // chunks per thread per step
  static_assert((BN * CPR) % NT == 0, "B tile chunks must divide among threads");
  __shared__ __attribute__((aligned(16))) int8_t lds[2][BN * LSTR];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int row0 = tm * BM, tok0 = tn * BN;
  const int NF = Keff / KSTEP;

  const uint32_t* cptr[WM];
  const uint32_t* mptr[WM];
  bool pvalid[WM];
#pragma unroll
  for (int p = 0; p < WM; ++p) {
    const int panel = row0 / kPanel + wm * WM + p;
    pvalid[p] = panel < npanels;
    const size_t off = (size_t)(pvalid[p] ? panel : 0) * NF * 64 + lane;
    cptr[p] = codes + off;
    mptr[p] = SP ? meta + off : nullptr;
  }

  int4 breg[CPT];
  auto load_b = [&](int s) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = threadIdx.x + i * NT;
      const int tk = tok0 + c / CPR;
      breg[i] = tk < T ? *(const int4*)(xq + (size_t)tk * Keff + (size_t)s * KSTEP + 16 * (c % CPR))
                       : make_int4(0, 0, 0, 0);
    }
  };
  auto store_b = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = threadIdx.x + i * NT;
      *(int4*)&lds[buf][(c / CPR) * LSTR + 16 * (c % CPR)] = breg[i];
    }
  };
  uint32_t ac[WM], am[WM];
  auto load_a = [&](int s) {
#pragma unroll
    for (int p = 0; p < WM; ++p) {
      ac[p] = pvalid[p] ? cptr[p][(size_t)s * 64] : 0u;
      am[p] = (SP && pvalid[p]) ? mptr[p][(size_t)s * 64] : kPadMeta;
    }
  };

  v16i acc[WM][WN];
#pragma unroll
  for (int p = 0; p < WM; ++p)
#pragma unroll
    for (int g = 0; g < WN; ++g) acc[p][g] = v16i{};

  load_b(0);
  load_a(0);
  store_b(0);
  __syncthreads();
  const int h = lane >> 5;
  for (int s = 0; s < NF; ++s) {
    const int buf = s & 1;
    uint32_t cc[WM], mm[WM];
#pragma unroll
    for (int p = 0; p < WM; ++p) { cc[p] = ac[p]; mm[p] = am[p]; }
    if (s + 1 < NF) { load_b(s + 1); load_a(s + 1); }
#pragma unroll
    for (int g = 0; g < WN; ++g) {
      const int trow = (wn * WN + g) * 32 + (lane & 31);
      const int8_t* bp = &lds[buf][trow * LSTR + 16 * h];
      const int4 blo = *(const int4*)bp;
      const int4 bhi = SP ? *(const int4*)(bp + 32) : make_int4(0, 0, 0, 0);
#pragma unroll
      for (int p = 0; p < WM; ++p) acc[p][g] = mfma_step<SP>(cc[p], mm[p], blo, bhi, acc[p][g]);
    }
    if (s + 1 < NF) store_b(buf ^ 1);
    __syncthreads();
  }

  const float gamma = *gamma_p;
#pragma unroll
  for (int g = 0; g < WN; ++g) {
    const int tk = tok0 + (wn * WN + g) * 32 + (lane & 31);
    if (tk >= T) continue;
    const float sc = xs[tk];
#pragma unroll
    for (int p = 0; p < WM; ++p) {
      const int obase = row0 + (wm * WM + p) * 32 + 4 * h;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int o = obase + 8 * (r >> 2) + (r & 3);
        if (o < n) store_out(y, acc_out, (size_t)tk * n + o, acc[p][g][r], gamma, sc);
      }
    }
  }
}

template <int LAYOUT>
static hipError_t launch_fwd_layout(const int8_t* xq, const float* xs, int64_t T, int64_t Keff,
                                    const uint32_t* codes, const uint32_t* meta,
                                    const float* gamma, int64_t n, float* y, int32_t* acc,
                                    hipStream_t s) {
  const int npanels = (int)((n + kPanel - 1) / kPanel);
  if (T <= 32) {
    gemv_kernel<LAYOUT, 8, 4><<<npanels, 512, 0, s>>>(xq, xs, (int)T, (int)Keff, codes, meta, gamma,
                                                      (int)n, y, acc);
  } else {
    constexpr int WM = 2, WN = 2, WAM = 2, WAN = 2;
    constexpr int BM = 32 * WM * WAM, BN = 32 * WN * WAN;
    const int tiles_m = (int)((n + BM - 1) / BM);
    const int tiles_n = (int)((T + BN - 1) / BN);
    gemm_kernel<LAYOUT, WM, WN, WAM, WAN><<<tiles_m * tiles_n, 64 * WAM * WAN, 0, s>>>(
        xq, xs, (int)T, (int)Keff, codes, meta, gamma, (int)n, npanels, y, acc, tiles_m);
  }
  return hipGetLastError();
}

hipError_t launch_fwd(const int8_t* xq, const float* x_scale, int64_t T, int64_t Keff,
                      const uint32_t* codes, const uint32_t* meta, const float* gamma, int layout,
                      int64_t n, float* y, int32_t* acc_opt, hipStream_t s) {
  if (layout == kLayoutSparse)
    return launch_fwd_layout<kLayoutSparse>(xq, x_scale, T, Keff, codes, meta, gamma, n, y, acc_opt, s);
  return launch_fwd_layout<kLayoutDense2>(xq, x_scale, T, Keff, codes, meta, gamma, n, y, acc_opt, s);
}

}  // namespace bl
