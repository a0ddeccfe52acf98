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
#include <utility>

#include "device_common.hpp"
#include "gemm_group.hpp"
#include "launch.hpp"

namespace bl {

__device__ __forceinline__ void store_out(float* __restrict__ y, int32_t* __restrict__ acc_out,
                                          size_t idx, int32_t a, float gamma, float sc) {
  const float v = ((float)a * gamma) * sc;
  y[idx] = v;
  if (acc_out) acc_out[idx] = a;
}

// ---------------------------------------------------------------------------------------------
// decode GEMV
// ---------------------------------------------------------------------------------------------
// One block per 32-row panel; wave w owns the K steps [w*per, (w+1)*per).  A decode matrix is only
// a few MB, so the kernel is bound by latency: each wave first issues its weight loads (at most
// MAXU code + MAXU meta dwords, well under the per-wave limit of outstanding vector loads), then
// the block stages the int8 activations xq[T][K_eff] in LDS with wide coalesced loads (row stride
// K_eff + 16 keeps the fragment reads of different tokens on different banks), and the MFMAs read
// their B fragments from LDS.  Partial accumulators of the live tokens are summed across waves
// through LDS in wave order.
template <int LAYOUT, int NW, int MAXU>
__global__ __launch_bounds__(64 * NW) void gemv_kernel(const int8_t* __restrict__ xq,
                                                       const float* __restrict__ xs, int T,
                                                       int Keff, const uint32_t* __restrict__ codes,
                                                       const uint32_t* __restrict__ meta,
                                                       const float* __restrict__ gamma_p, int n,
                                                       float* __restrict__ y,
                                                       int32_t* __restrict__ acc_out) {
  constexpr bool SP = LAYOUT == kLayoutSparse;
  constexpr int KSTEP = SP ? 64 : 32;
  extern __shared__ __attribute__((aligned(16))) int8_t gsm[];
  const int P = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int NF = Keff / KSTEP;
  const int per = (NF + NW - 1) / NW;            // host guarantees per <= MAXU
  const int s_begin = min(wave * per, NF - 1);
  const int cnt = min(per, NF - wave * per);    // may be <= 0 for trailing waves
  const uint32_t* cp = codes + (size_t)P * NF * 64 + lane;
  const uint32_t* mp = SP ? meta + (size_t)P * NF * 64 + lane : nullptr;
  uint32_t c[MAXU], m[MAXU];
#pragma unroll
  for (int u = 0; u < MAXU; ++u) {
    const int s = min(s_begin + u, NF - 1);     // past the end: reload the last step, code zeroed
    c[u] = __builtin_nontemporal_load(cp + (size_t)s * 64);   // read once: streamed past the caches
    m[u] = SP ? __builtin_nontemporal_load(mp + (size_t)s * 64) : kPadMeta;
  }

  // epilogue operands early: their latency hides behind the weight loads
  const int tok = lane & 31, h = lane >> 5;
  const float gamma = *gamma_p;
  const float sc_l = xs[min(tok, T - 1)];

  // activations -> LDS, rows of K_eff bytes at stride K_eff + 16; all of a thread's loads are in
  // flight before its first LDS store (a load-store loop would pay one L2 round trip per chunk)
  const int stride = Keff + 16;
  const int cpr = Keff / 16;
  const int chunks = T * cpr;
  for (int c0 = 0; c0 < chunks; c0 += 64 * NW * 8) {
    int4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int ci = min(c0 + k * 64 * NW + (int)threadIdx.x, chunks - 1);
      v[k] = *(const int4*)(xq + (size_t)(ci / cpr) * Keff + 16 * (ci % cpr));
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int ci = c0 + k * 64 * NW + (int)threadIdx.x;
      if (ci < chunks) *(int4*)&gsm[(ci / cpr) * stride + 16 * (ci % cpr)] = v[k];
    }
  }
  __syncthreads();

  // two accumulators halve the dependent MFMA chain
  const int8_t* xr = gsm + min(tok, T - 1) * stride + 16 * h;   // dead token lanes read row T-1
  v16i acc0 = {}, acc1 = {};
#pragma unroll
  for (int u = 0; u < MAXU; ++u) {
    const int s = min(s_begin + u, NF - 1);
    const int4 blo = *(const int4*)(xr + s * KSTEP);
    const int4 bhi = SP ? *(const int4*)(xr + s * KSTEP + 32) : make_int4(0, 0, 0, 0);
    if (u & 1) acc1 = mfma_step<SP>(u < cnt ? c[u] : 0u, m[u], blo, bhi, acc1);
    else acc0 = mfma_step<SP>(u < cnt ? c[u] : 0u, m[u], blo, bhi, acc0);
  }
  v16i acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = acc0[r] + acc1[r];

  // live tokens only: D column = token = lane % 32
  int* red = (int*)(gsm + ((T * stride + 15) & ~15));
  const bool live = tok < T;
  if (live) {
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(wave * 16 + r) * 64 + lane] = acc[r];
  }
  __syncthreads();
  // thread i sums output (register r, lane l) with l = i % 64: its own token's scale is sc_l
  for (int i = threadIdx.x; i < 16 * 64; i += 64 * NW) {
    const int r = i >> 6, l = i & 63;
    const int tk = l & 31;
    const int o = P * kPanel + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
    if (tk < T && o < n) {
      int32_t sum = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) sum += red[(w * 16 + r) * 64 + l];
      store_out(y, acc_out, (size_t)tk * n + o, sum, gamma, sc_l);
    }
  }
}

template <int NW>
constexpr size_t gemv_red_bytes() { return (size_t)NW * 16 * 64 * 4; }

inline size_t gemv_smem_bytes(int64_t T, int64_t Keff, int nw) {
  return ((size_t)T * (Keff + 16) + 15) / 16 * 16 + (size_t)nw * 16 * 64 * 4;
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

// Large-tile prefill GEMM: block tile 256 rows x 128 tokens, 4 waves stacked along the rows, each
// wave 64 rows x 128 tokens = 2 panels x 4 token groups = 8 MFMA tiles (128 int32 accumulators
// per lane; two blocks per CU, so two waves share a SIMD and hide each other's LDS latency).  A
// code dword expanded once feeds four MFMAs: on this kernel VALU and MFMA issue from one SIMD
// barely overlap, and these wave tiles measured 8-10% faster than 128 x 64 ones.
//
// Operands reach LDS with direct global->LDS loads (global_load_lds_dwordx4: lane l's 16 bytes
// land at the wave-uniform LDS base + 16*l), so no VGPRs stage them, and a ring of NBUF stage
// buffers keeps NBUF - 1 stages in flight while one is multiplied.  A stage is KS MFMA K-steps: B = 128 tokens x 128
// bytes, A = 8 panels x KS fragments of codes (and of meta).  The stage loop is unrolled by NBUF,
// so every access names its buffer statically.  The loads are inline asm the compiler does not track, so
// each wave waits on its own vmcnt (every stage issues exactly LPS loads per wave) and meets the
// others at a bare s_barrier (no fence: a fence would also drain the loads meant to stay in
// flight).  B rows are
// XOR-swizzled in 16-byte chunks: chunk c of token t sits at position c ^ ((t / 2) % 8).  Two
// 128-byte rows fill the 64 four-byte banks once, so the 16 lanes served together (16 consecutive
// tokens, one chunk each) then hit 16 distinct 16-byte bank groups; swizzling by t % 8 instead
// pairs rows t and t+8 on the same banks (measured 1.7x slower reads).
//
// Rows past the last panel, tokens past T and K past the end (a partial last stage) read clamped,
// valid addresses; their codes are zeroed or their results never stored.
//
// Blocks are mapped XCD-major (big_tile_of_block): each XCD owns a slab of token tiles and walks
// them fastest, so its activations stay in its L2 and every weight panel is fetched once per XCD.
constexpr int kBigWaves = 4;
// Three stage buffers (72 KB of LDS) allow two blocks per CU.  A six-deep ring for grids of one
// tile per CU (one block, 144 KB) measured 7% slower on the 2048-token window GEMM: its unrolled
// loop needs more registers than the file holds beside the accumulators.
constexpr int kBigRing = 3;
constexpr int kBigWaveRows = 4, kBigWaveM = 2, kBigWaveN = 4;

template <int LAYOUT, int NWAVE_, int WR_, int WM_, int WN_, int NBUF_ = 3>
struct BigGemm {
  static constexpr bool SP = LAYOUT == kLayoutSparse;
  static constexpr int KSTEP = SP ? 64 : 32;
  static constexpr int KS = SP ? 2 : 4;              // MFMA K-steps per stage: 128 K bytes
  static constexpr int NWAVE = NWAVE_;               // waves as WR (rows) x NWAVE/WR (tokens)
  static constexpr int WR = WR_;
  static constexpr int WM = WM_, WN = WN_;            // 32*WM rows x 32*WN tokens per wave
  static constexpr int BM = 32 * WM * WR, BN = 32 * WN * (NWAVE / WR);
  static constexpr int SK = KS * KSTEP;              // 128 bytes of K per token per stage
  static constexpr int B_BYTES = BN * SK;
  static constexpr int A_PANEL = KS * 256 * (SP ? 2 : 1);
  static constexpr int A_BYTES = (BM / 32) * A_PANEL;
  static constexpr int B_LOADS = B_BYTES / 1024 / NWAVE;
  static constexpr int A_LOADS = A_BYTES / 1024 / NWAVE;
  static constexpr int LPS = B_LOADS + (SP ? 2 : 1) * A_LOADS;   // loads per wave per stage
  static constexpr int STAGE = B_BYTES + A_BYTES;
  static constexpr int NBUF = NBUF_;                 // stage buffers in the LDS ring
  static_assert(NBUF >= 3 && (NBUF - 2) * LPS <= 63, "loads in flight fit the vmcnt field");
  static_assert(SK == 128, "stage layout");
  static_assert(A_LOADS >= 1 && A_BYTES % (1024 * NWAVE) == 0, "A stage splits evenly over waves");

  int8_t* ring;                                      // NBUF stage buffers in LDS
  const int8_t* __restrict__ xq;
  const uint32_t* __restrict__ codes;
  const uint32_t* __restrict__ meta;
  int Keff, NF, NS, lane, wave, wm, wn, h;
  uint32_t m0_b, m0_a;                  // this wave's LDS destinations inside a stage buffer
  uint32_t b_off[B_LOADS], b_off_tail[B_LOADS];   // per-lane byte offsets from xq + st * SK
  uint32_t a_off[A_LOADS], a_off_tail[A_LOADS];   // per-lane byte offsets from codes/meta + st * KS * 256
  v16i acc[WM][WN];

  // Loads of stage st (clamped to the last real stage: the padded stages of the unrolled loop
  // reload valid data that their zeroed codes never use).  The stage advance lives in the scalar
  // base; the one partial stage (K_eff not a multiple of the stage) uses offsets clamped inside
  // each row.  A loads come in a code half (lanes 0-31) and a meta half (lanes 32-63).  Load q of
  // a stage: q < B_LOADS the token rows, then per A load a code and (SPARSE) a meta instruction.
  template <int BUF>
  __device__ __forceinline__ void issue_one(int st_in, int q) {
    const int st = min(st_in, NS - 1);
    const bool partial = (st + 1) * KS > NF;
    const uint32_t m0b = m0_b + BUF * STAGE, m0a = m0_a + BUF * STAGE;
    if (q < B_LOADS) {
      const int8_t* sb = xq + (size_t)st * SK;
      lds_dma16_s(sb, partial ? b_off_tail[q] : b_off[q], m0b + q * 1024);
    } else {
      const int qa = (q - B_LOADS) / (SP ? 2 : 1);
      const bool is_meta = SP && ((q - B_LOADS) & 1);
      const uint8_t* src = (const uint8_t*)(is_meta ? meta : codes) + (size_t)st * (KS * 256);
      const uint32_t off = partial ? a_off_tail[qa] : a_off[qa];
      if (!SP || (lane < 32) != is_meta) lds_dma16_s(src, off, m0a + qa * 1024);
    }
  }

  template <int BUF>
  __device__ __forceinline__ void issue(int st_in) {
#pragma unroll
    for (int q = 0; q < LPS; ++q) issue_one<BUF>(st_in, q);
  }

  // Operands of one MFMA K-step, read from LDS one step ahead of their use.
  struct StepRegs {
    uint32_t code[WM];
    uint32_t meta[WM];
    v8i b[WN];
  };

  __device__ __forceinline__ void read_step(const int8_t* bb, int j, StepRegs& r) const {
    const int8_t* ab = bb + B_BYTES;
#pragma unroll
    for (int p = 0; p < WM; ++p) {
      const int8_t* pa = ab + (wm * WM + p) * A_PANEL + j * 256 + 4 * lane;
      r.code[p] = *(const uint32_t*)pa;
      r.meta[p] = SP ? *(const uint32_t*)(pa + KS * 256) : 0u;
    }
#pragma unroll
    for (int g = 0; g < WN; ++g) {
      const int tt = (wn * WN + g) * 32 + (lane & 31);
      const int8_t* rowp = bb + tt * SK;
      const int c1 = (j * KSTEP) / 16 + h;
      const int sw = (tt >> 1) & 7;
      const int4 blo = *(const int4*)(rowp + 16 * (c1 ^ sw));
      r.b[g][0] = blo.x; r.b[g][1] = blo.y; r.b[g][2] = blo.z; r.b[g][3] = blo.w;
      if constexpr (SP) {
        const int4 bhi = *(const int4*)(rowp + 16 * ((c1 + 2) ^ sw));
        r.b[g][4] = bhi.x; r.b[g][5] = bhi.y; r.b[g][6] = bhi.z; r.b[g][7] = bhi.w;
      }
    }
  }

  // Panel by panel: expand one code dword, then its WN MFMAs, so the matrix core starts after
  // the first expansion instead of after all of them (VALU and MFMA issue from one SIMD barely
  // overlap on this kernel).
  __device__ __forceinline__ void mma_step(const StepRegs& r, bool live) {
#pragma unroll
    for (int p = 0; p < WM; ++p) {
      const v4i ap = expand_codes(live ? r.code[p] : 0u);
#pragma unroll
      for (int g = 0; g < WN; ++g) {
        if constexpr (SP) {
          acc[p][g] = __builtin_amdgcn_smfmac_i32_32x32x64_i8(ap, r.b[g], acc[p][g], (int)r.meta[p], 0, 0);
        } else {
          v4i bd;
          bd[0] = r.b[g][0]; bd[1] = r.b[g][1]; bd[2] = r.b[g][2]; bd[3] = r.b[g][3];
          acc[p][g] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ap, bd, acc[p][g], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int p = 0; p < WM; ++p) {
      __builtin_amdgcn_sched_group_barrier(0x002, 9, 0);    // one code expansion (VALU)
      __builtin_amdgcn_sched_group_barrier(0x008, WN, 0);   // its MFMAs
    }
  }

  // The last step of a stage, with the refill of this stage's buffer spread over it: before each
  // MFMA goes one global->LDS load (LPS <= WM * WN; any rest follows), the next stage's first-step
  // reads go out with the first one.  Issued as a burst, the loads stall the wave behind the memory pipeline while
  // the matrix core idles; spread out, each is accepted while MFMAs run.  The scheduling fences
  // keep exactly this order.
  template <int BUF>
  __device__ __forceinline__ void mma_step_refill(const StepRegs& r, bool live, int st_refill,
                                                  StepRegs& nxt) {
#pragma unroll
    for (int p = 0; p < WM; ++p) {
      __builtin_amdgcn_sched_barrier(0);
      if (p * WN < LPS) issue_one<BUF>(st_refill, p * WN);
      if (p == 0) read_step(ring + ((BUF + 1) % NBUF) * STAGE, 0, nxt);
      const v4i ap = expand_codes(live ? r.code[p] : 0u);
#pragma unroll
      for (int g = 0; g < WN; ++g) {
        if (g > 0) {
          __builtin_amdgcn_sched_barrier(0);
          if (p * WN + g < LPS) issue_one<BUF>(st_refill, p * WN + g);
        }
        if constexpr (SP) {
          acc[p][g] = __builtin_amdgcn_smfmac_i32_32x32x64_i8(ap, r.b[g], acc[p][g], (int)r.meta[p], 0, 0);
        } else {
          v4i bd;
          bd[0] = r.b[g][0]; bd[1] = r.b[g][1]; bd[2] = r.b[g][2]; bd[3] = r.b[g][3];
          acc[p][g] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ap, bd, acc[p][g], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = WM * WN; q < LPS; ++q) issue_one<BUF>(st_refill, q);
  }

  // One stage (buffer BUF) as KS pipelined steps: while step j's MFMAs run, step j+1's operands
  // are read from LDS into the other register set.  At the last step the next stage's buffer is
  // needed, so the wave first waits for its own loads of that stage (the loads of the NBUF - 2
  // stages after it stay outstanding) and for its outstanding LDS reads, meets the other waves at a
  // bare s_barrier (after which no wave reads this stage's buffer again), then refills this buffer
  // with stage st + NBUF and reads the next stage's first step while the step's MFMAs run.
  // ALL_LIVE: every step of the stage is real.  Stages past the last real one (the padding of the
  // last group of NBUF) do nothing: every wave skips them alike, and the loads still in flight
  // into their buffers are drained before the epilogue.
  template <int BUF, bool ALL_LIVE>
  __device__ __forceinline__ void stage(int st, StepRegs& R0, StepRegs& R1) {
    if (!ALL_LIVE && st >= NS) return;
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      StepRegs& cur = (j % 2 == 0) ? R0 : R1;
      StepRegs& nxt = (j % 2 == 0) ? R1 : R0;
      if (j + 1 < KS) {
        read_step(ring + BUF * STAGE, j + 1, nxt);
        mma_step(cur, ALL_LIVE || st * KS + j < NF);
      } else {
        __builtin_amdgcn_s_waitcnt(waitcnt_imm((NBUF - 2) * LPS, 0));
        block_barrier_nofence();
        mma_step_refill<BUF>(cur, ALL_LIVE || st * KS + j < NF, st + NBUF, nxt);
      }
    }
  }
};

// One 256-row x 128-token output tile at (row0, tok0): the pipelined main loop, then the epilogue.
template <class G, int... I>
__device__ __forceinline__ void big_issue_ring(G& k, std::integer_sequence<int, I...>) {
  (k.template issue<I>(I), ...);
}
template <bool ALL_LIVE, class G, int... I>
__device__ __forceinline__ void big_stage_group(G& k, int st, typename G::StepRegs& R0,
                                                typename G::StepRegs& R1,
                                                std::integer_sequence<int, I...>) {
  (k.template stage<I, ALL_LIVE>(st + I, R0, R1), ...);
}

template <int LAYOUT, int NWAVE, int NBUF>
__device__ __forceinline__ void big_tile(
    int8_t* ring, const int8_t* __restrict__ xq, const float* __restrict__ xs, int T, int Keff,
    const uint32_t* __restrict__ codes, const uint32_t* __restrict__ meta,
    const float* __restrict__ gamma_p, int n, int npanels, float* __restrict__ y,
    int32_t* __restrict__ acc_out, int row0, int tok0) {
  using G = BigGemm<LAYOUT, NWAVE, kBigWaveRows, kBigWaveM, kBigWaveN, NBUF>;
  G k;
  k.ring = ring;
  k.xq = xq; k.codes = codes; k.meta = meta; k.Keff = Keff;
  k.lane = threadIdx.x & 63;
  k.wave = threadIdx.x >> 6;
  k.wm = k.wave % G::WR;
  k.wn = k.wave / G::WR;
  k.h = k.lane >> 5;
  k.NF = Keff / G::KSTEP;
  k.NS = (k.NF + G::KS - 1) / G::KS;

  // B: load i of a wave fills LDS bytes [(wave*B_LOADS + i) * 1024, +1024) of a stage = 8 token
  // rows of SK bytes; lane l covers position l % 8 of token row tt and fetches global chunk
  // (l % 8) ^ ((tt / 2) % 8).  In the partial last stage chunks past K_eff reread the last chunk.
  const int last = k.NS - 1;
#pragma unroll
  for (int i = 0; i < G::B_LOADS; ++i) {
    const int tt = (k.wave * G::B_LOADS + i) * 8 + (k.lane >> 3);
    const int chunk = 16 * ((k.lane & 7) ^ ((tt >> 1) & 7));
    const uint32_t row = (uint32_t)(min(tok0 + tt, T - 1) * Keff);
    k.b_off[i] = row + chunk;
    k.b_off_tail[i] = row + (uint32_t)(min(last * G::SK + chunk, Keff - 16) - last * G::SK);
  }
  // A: load q of a wave fills LDS bytes [(wave*A_LOADS + q) * 1024, +1024) of the A stage, laid
  // out [panel][codes: KS fragments][meta: KS fragments], 256 bytes per fragment; lane l < 32
  // fetches 16 code bytes, lane l >= 32 the matching 16 meta bytes (SPARSE).  In the partial
  // last stage fragments past the last K step reread the last one.
#pragma unroll
  for (int q = 0; q < G::A_LOADS; ++q) {
    const int byte0 = (k.wave * G::A_LOADS + q) * 1024 + k.lane * 16;
    const int pw = byte0 / G::A_PANEL;
    const int inrun = (byte0 % G::A_PANEL) % (G::KS * 256);   // byte inside the codes/meta run
    const int frag = inrun / 256;
    const int panel = min(row0 / kPanel + pw, npanels - 1);
    const uint32_t pbase = (uint32_t)panel * k.NF * 256u + (uint32_t)(inrun % 256);
    k.a_off[q] = pbase + frag * 256;
    k.a_off_tail[q] = pbase + (uint32_t)(min(last * G::KS + frag, k.NF - 1) - last * G::KS) * 256u;
  }
  k.m0_b = __builtin_amdgcn_readfirstlane(lds_offset(ring) + (uint32_t)k.wave * (G::B_LOADS * 1024));
  k.m0_a = __builtin_amdgcn_readfirstlane(lds_offset(ring) + G::B_BYTES + (uint32_t)k.wave * (G::A_LOADS * 1024));
#pragma unroll
  for (int p = 0; p < G::WM; ++p)
#pragma unroll
    for (int g = 0; g < G::WN; ++g) k.acc[p][g] = v16i{};

  // Groups of NBUF stages (one per ring buffer).  Groups made only of full stages skip the
  // per-step liveness select; the last group, which may hold the partial stage and padding up to
  // a multiple of NBUF, keeps it (a partial stage's padded steps have their codes zeroed; whole
  // padded stages are skipped).  Every real stage issues its refill (clamped to real data), so
  // each wave always has exactly LPS loads per stage in flight.
  const int full_stages = k.NF / G::KS;
  const int main_end = full_stages / NBUF * NBUF;
  typename G::StepRegs R0, R1;
  big_issue_ring(k, std::make_integer_sequence<int, NBUF>{});
  __builtin_amdgcn_s_waitcnt(waitcnt_imm((NBUF - 1) * G::LPS));   // stage 0 landed (this wave's part)
  block_barrier_nofence();
  k.read_step(ring, 0, R0);
  for (int st = 0; st < main_end; st += NBUF)
    big_stage_group<true>(k, st, R0, R1, std::make_integer_sequence<int, NBUF>{});
  if (main_end < k.NS)
    big_stage_group<false>(k, main_end, R0, R1, std::make_integer_sequence<int, NBUF>{});
  // No load may still be writing LDS once the ring is reused below or the block ends; after the
  // barrier no wave reads the ring any more.
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0));
  block_barrier_nofence();

  const float gamma = *gamma_p;
  const int lane = k.lane, h = k.h;
  // Lane (token lane % 32) holds rows 8j + 4h + i (i = 0..3) of each 32-row panel: four runs of
  // four consecutive outputs.  Stored as they are, one instruction writes 32-byte pieces of 32
  // token rows, so the tile's output costs four L2 requests per 128-byte line.  A 32-token group
  // whose 64 rows and 32 tokens all lie inside y is therefore first written to a wave-private
  // region of the (now idle) ring, [token][row] with rows padded to 68 floats so that both the
  // 16-byte writes of 16 tokens and the reads of 16 consecutive row pieces hit distinct banks,
  // then read back four tokens at a time: each store instruction then writes 256 contiguous bytes
  // of four token rows.  Other groups (ragged rows or tokens, n not a multiple of 4) store from
  // the registers: one 16-byte store per run where aligned, else element stores.  The staged
  // stores are non-temporal: whole lines that would otherwise evict operand lines from L2 (2-5%
  // faster); the 32-byte pieces of the register path must merge in L2 first (non-temporal, they
  // reached HBM one by one: 1.7x slower for the whole GEMM).
  const bool vec_ok = (n & 3) == 0;
  constexpr int kStgRow = 68;                                  // floats per staged token row
  static_assert(G::NWAVE * 32 * kStgRow * 4 <= NBUF * G::STAGE, "staging fits the ring");
  static_assert(G::WM * 32 == 64, "staged rows: two panels per wave");
  float* stg = (float*)(ring + k.wave * (32 * kStgRow * 4));
  const int orow0 = row0 + k.wm * G::WM * 32;                  // first output row of the wave
#pragma unroll
  for (int g = 0; g < G::WN; ++g) {
    const int tg0 = tok0 + (k.wn * G::WN + g) * 32;
    const int tk = tg0 + (lane & 31);
    if (vec_ok && orow0 + 64 <= n && tg0 + 32 <= T) {
      const float sc = xs[tk];
#pragma unroll
      for (int p = 0; p < G::WM; ++p)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          v4f v;
          v[0] = ((float)k.acc[p][g][4 * jj + 0] * gamma) * sc;
          v[1] = ((float)k.acc[p][g][4 * jj + 1] * gamma) * sc;
          v[2] = ((float)k.acc[p][g][4 * jj + 2] * gamma) * sc;
          v[3] = ((float)k.acc[p][g][4 * jj + 3] * gamma) * sc;
          *(v4f*)&stg[(lane & 31) * kStgRow + p * 32 + 8 * jj + 4 * h] = v;
        }
      // a wave's LDS accesses complete in order; the clobber keeps the compiler from moving the
      // reads above the writes (or the next group's writes above these reads)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int tt = 4 * it + (lane >> 4), r4 = 4 * (lane & 15);
        const v4f v = *(const v4f*)&stg[tt * kStgRow + r4];
        __builtin_nontemporal_store(v, (v4f*)(y + (size_t)(tg0 + tt) * n + orow0 + r4));
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      continue;
    }
    if (tk >= T) continue;
    const float sc = xs[tk];
    float* yrow = y + (size_t)tk * n;
#pragma unroll
    for (int p = 0; p < G::WM; ++p) {
      const int o0 = row0 + (k.wm * G::WM + p) * 32;
      if (vec_ok && o0 + 32 <= n) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int o = o0 + 8 * jj + 4 * h;
          v4f v;
          v[0] = ((float)k.acc[p][g][4 * jj + 0] * gamma) * sc;
          v[1] = ((float)k.acc[p][g][4 * jj + 1] * gamma) * sc;
          v[2] = ((float)k.acc[p][g][4 * jj + 2] * gamma) * sc;
          v[3] = ((float)k.acc[p][g][4 * jj + 3] * gamma) * sc;
          *(v4f*)(yrow + o) = v;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int o = o0 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (o < n) yrow[o] = ((float)k.acc[p][g][r] * gamma) * sc;
        }
      }
    }
  }
  if (acc_out) {
#pragma unroll
    for (int g = 0; g < G::WN; ++g) {
      const int tk = tok0 + (k.wn * G::WN + g) * 32 + (lane & 31);
      if (tk >= T) continue;
#pragma unroll
      for (int p = 0; p < G::WM; ++p)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int o = row0 + (k.wm * G::WM + p) * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (o < n) acc_out[(size_t)tk * n + o] = k.acc[p][g][r];
        }
    }
  }
}

// Tile of block b.  The hardware deals consecutive block ids round-robin to the 8 XCDs, each with
// its own L2.  When the token tiles split evenly over the XCDs, XCD x = b % 8 owns token tiles
// [x * ntn, (x + 1) * ntn) and walks them fastest, row tile by row tile (i = b / 8): its token
// slab (ntn token tiles of activations) stays in its L2 and each packed weight panel is fetched
// once per XCD, instead of once per token tile.  Otherwise each XCD takes a contiguous run of
// tiles in row-tile-fastest order.
__device__ __forceinline__ void big_tile_of_block(int b, int tiles_m, int tiles_n, int* tm, int* tn) {
  const int tiles = tiles_m * tiles_n;
  if ((tiles_n & 7) == 0) {
    const int ntn = tiles_n >> 3, x = b & 7, i = b >> 3;
    *tn = x * ntn + i % ntn;
    *tm = i / ntn;
    return;
  }
  const int full = (tiles / 8) * 8;
  const int t = b < full ? (b % 8) * (tiles / 8) + b / 8 : b;
  *tm = t % tiles_m;
  *tn = t / tiles_m;
}

template <int LAYOUT, int NWAVE, int NBUF>
__global__ __launch_bounds__(64 * NWAVE, 2) void gemm_big_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, int T, int Keff,
    const uint32_t* __restrict__ codes, const uint32_t* __restrict__ meta,
    const float* __restrict__ gamma_p, int n, int npanels, float* __restrict__ y,
    int32_t* __restrict__ acc_out, int tiles_m, int tiles) {
  using G = BigGemm<LAYOUT, NWAVE, kBigWaveRows, kBigWaveM, kBigWaveN, NBUF>;
  __shared__ __attribute__((aligned(16))) int8_t ring[NBUF * G::STAGE];
  int tm, tn;
  big_tile_of_block(blockIdx.x, tiles_m, tiles / tiles_m, &tm, &tn);
  big_tile<LAYOUT, NWAVE, NBUF>(ring, xq, xs, T, Keff, codes, meta, gamma_p, n, npanels, y, acc_out,
                          tm * G::BM, tn * G::BN);
}

// ---------------------------------------------------------------------------------------------
// Grouped prefill: every tile of several projections (the bitlinear_fwd calls of a layer set with
// prefill-sized T) in one launch.  Each job is one gemm_big_kernel tile with its projection's
// arguments, so the results are those of the separate calls bit for bit; the host deals runs of
// tiles that share a token tile to the XCDs longest first, so the grid tails of the separate
// launches become one.
// ---------------------------------------------------------------------------------------------
template <int LAYOUT>
__global__ __launch_bounds__(64 * kBigWaves, 2) void gemm_big_group_kernel(
    const uint8_t* __restrict__ table) {
  using G = BigGemm<LAYOUT, kBigWaves, kBigWaveRows, kBigWaveM, kBigWaveN, kBigRing>;
  __shared__ __attribute__((aligned(16))) int8_t ring[kBigRing * G::STAGE];
  const GemmGroupHeader* hd = (const GemmGroupHeader*)table;
  if (hd->magic != kGemmGroupMagic || hd->layout != LAYOUT || (int)blockIdx.x >= hd->jobs) return;
  const GemmGroupJob jb = ((const GemmGroupJob*)(table + hd->jobs_off))[blockIdx.x];
  if (jb.proj < 0) return;
  const GemmGroupProj P = ((const GemmGroupProj*)(table + sizeof(GemmGroupHeader)))[jb.proj];
  big_tile<LAYOUT, kBigWaves, kBigRing>(ring, P.xq, P.xs, P.T, P.Keff, P.codes, P.meta, P.gamma, P.n,
                              P.npanels, P.y, P.acc, jb.tm * G::BM, jb.tn * G::BN);
}

hipError_t launch_gemm_group(const void* table, int64_t jobs, int layout, hipStream_t s) {
  const uint8_t* t = (const uint8_t*)table;
  if (layout == kLayoutSparse)
    gemm_big_group_kernel<kLayoutSparse><<<(unsigned)jobs, 64 * kBigWaves, 0, s>>>(t);
  else
    gemm_big_group_kernel<kLayoutDense2><<<(unsigned)jobs, 64 * kBigWaves, 0, s>>>(t);
  return hipGetLastError();
}

int gemm_group_tile_rows() { return BigGemm<kLayoutSparse, kBigWaves, kBigWaveRows, kBigWaveM, kBigWaveN>::BM; }
int gemm_group_tile_tokens() { return BigGemm<kLayoutSparse, kBigWaves, kBigWaveRows, kBigWaveM, kBigWaveN>::BN; }

template <int LAYOUT>
static hipError_t launch_fwd_layout(const int8_t* xq, const float* xs, int64_t T, int64_t Keff,
                                    const uint32_t* codes, const uint32_t* meta,
                                    const float* gamma, int64_t n, float* y, int32_t* acc,
                                    hipStream_t s) {
  const int npanels = (int)((n + kPanel - 1) / kPanel);
  constexpr int KSTEP = LAYOUT == kLayoutSparse ? 64 : 32;
  const int64_t nf = Keff / KSTEP;
  if (T <= 32 && nf <= 8 * 16 && gemv_smem_bytes(T, Keff, 8) <= 160 * 1024) {
    const size_t smem = gemv_smem_bytes(T, Keff, 8);
    auto run = [&](auto kern) -> hipError_t {
      hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)smem);
      if (e != hipSuccess) return e;
      kern<<<npanels, 512, smem, s>>>(xq, xs, (int)T, (int)Keff, codes, meta, gamma, (int)n, y, acc);
      return hipGetLastError();
    };
    // steps per wave bounded by MAXU; the smallest MAXU that fits keeps the load count low
    if (nf <= 8 * 4) return run(gemv_kernel<LAYOUT, 8, 4>);
    if (nf <= 8 * 8) return run(gemv_kernel<LAYOUT, 8, 8>);
    return run(gemv_kernel<LAYOUT, 8, 16>);
  } else if (T > 128) {
    using G = BigGemm<LAYOUT, kBigWaves, kBigWaveRows, kBigWaveM, kBigWaveN>;
    const int tiles_m = (int)((n + G::BM - 1) / G::BM);
    const int tiles = tiles_m * (int)((T + G::BN - 1) / G::BN);
    gemm_big_kernel<LAYOUT, kBigWaves, kBigRing><<<tiles, 64 * kBigWaves, 0, s>>>(
        xq, xs, (int)T, (int)Keff, codes, meta, gamma, (int)n, npanels, y, acc, tiles_m, tiles);
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
