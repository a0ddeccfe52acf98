// Straight-through backward of the sparse ternary BitLinear (Sparse-BitNet technical summary,
// Training Strategie: Dual STE -- the rounding, the clip and the Top-N selection pass the gradient
// straight through, and every master weight, masked or kept, receives it).  With W_q = gamma W_eff
// the layer is y = X^ W_q^T, so
//   dX[t][k] = gamma * sum_o dY[t][o] W_eff[o][k]        (reduction over out-features)
//   dW[o][k] = sum_t dY[t][o] X^[t][k],  X^ = bf16(fp32(q * scale_t))   (reduction over tokens)
// Both are dense bf16 products with fp32 accumulation: the ternary values and X^ are exact in
// bfloat16 and so are the products of two bfloat16 values in fp32.  The 2:4 structure runs along
// K, the output axis of dX and of dW, so the sparse matrix instruction (which needs the pattern on
// the reduction axis) does not apply; the kept structure only makes W_eff cheap to expand.
//
// Both products run through one kernel, C[i][j] = alpha * sum_r A[i][r] B[j][r], whose operands
// are row-major with the reduction axis contiguous ("NT").  Three memory-bound prep kernels put
// the operands in that form, in the caller's workspace:
//   Wt[k][o]  = W_eff[o][k] as bf16 (+-1 / 0), expanded from the packed codes   (dX's B)
//   dYt[o][t] = dY[t][o]                                                      (dW's A)
//   Xt[k][t]  = X^[t][k]                                                       (dW's B)
// and dX's A is dY itself (or a zero-padded copy when n is not a multiple of 32).  The reduction
// axis of every operand is zero-padded to a multiple of 32, so the kernel has no reduction tail.
#include "bwd_group.hpp"
#include "device_common.hpp"
#include "launch.hpp"

namespace bl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// bf16 bit pattern of a 2-bit ternary code (01 = +1 -> 0x3F80, 10 = -1 -> 0xBF80, 00 -> 0).
__device__ __forceinline__ uint32_t code_bf16(uint32_t c) {
  return c ? (0x3F80u | ((c & 2u) << 14)) : 0u;
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------------------------
// Wt[k][o] = W_eff[o][k] from the packed layout.  One thread per (row pair, M-group): rows 2p and
// 2p+1 sit in adjacent dwords of the tiled unit layout, so each thread loads two code (and meta)
// dwords per unit at once and writes M dwords, each the bf16 pair of rows (2p, 2p+1) at one K
// position; consecutive threads take consecutive row pairs, so a wave writes 256 contiguous bytes
// per position.  Padded rows (o >= n) have all-zero codes and come out as zeros.
//   SPARSE (windows): the M-group g holds slots g(M-2) .. g(M-2)+M-3 of the row; slot j of the
//     group is in window j/2 and sits at position 2(j/2) + index (index from meta), so the kept
//     positions (all distinct) are scattered into the group.
//   DENSE2: slot s is position s.
// ---------------------------------------------------------------------------------------------
template <int LAYOUT, int M>
__device__ __forceinline__ void wt_expand_one(const uint32_t* __restrict__ codes,
                                              const uint32_t* __restrict__ meta, int U, int groups,
                                              int pairs, uint32_t* __restrict__ wt, int64_t id) {
  if (id >= (int64_t)groups * pairs) return;
  const int p = (int)(id % pairs), g = (int)(id / pairs);
  const int r = 2 * p, panel = r / kPanel, rr = r % kPanel;
  auto unit_at = [&](int c) -> size_t {
    return ((size_t)panel * (U / 2) + c / 2) * 64 + (c % 2) * 32 + rr;
  };
  constexpr int S = LAYOUT == kLayoutSparse ? M - 2 : M;   // slots per group
  const int s0 = g * S;
  const int c0 = s0 / 16, c1 = (s0 + S - 1) / 16;          // at most two units
  // both units are loaded unconditionally (c1 == c0 when the group sits in one unit)
  const uint2 cw0 = *(const uint2*)(codes + unit_at(c0));
  const uint2 cw1 = *(const uint2*)(codes + unit_at(c1));
  uint2 mw0 = make_uint2(0u, 0u), mw1 = make_uint2(0u, 0u);
  if constexpr (LAYOUT == kLayoutSparse) {
    mw0 = *(const uint2*)(meta + unit_at(c0));
    mw1 = *(const uint2*)(meta + unit_at(c1));
  }
  uint32_t out[M];
#pragma unroll
  for (int j = 0; j < M; ++j) out[j] = 0u;
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const int s = s0 + j, i = s % 16;
    const bool second = s / 16 != c0;
    const uint32_t cx = second ? cw1.x : cw0.x, cy = second ? cw1.y : cw0.y;
    const int sh = 8 * (i % 4) + 2 * (i / 4);
    const uint32_t v = code_bf16((cx >> sh) & 3u) | (code_bf16((cy >> sh) & 3u) << 16);
    if constexpr (LAYOUT == kLayoutSparse) {
      const uint32_t mx = second ? mw1.x : mw0.x, my = second ? mw1.y : mw0.y;
      // the two rows of the pair have their own indices: place each half separately
      const int pos0 = 2 * (j / 2) + (int)((mx >> (2 * i)) & 3u);
      const int pos1 = 2 * (j / 2) + (int)((my >> (2 * i)) & 3u);
#pragma unroll
      for (int q = 0; q < M; ++q) {
        if (q == pos0) out[q] |= v & 0xFFFFu;
        if (q == pos1) out[q] |= v & 0xFFFF0000u;
      }
    } else {
      out[j] = v;
    }
  }
  const int64_t row_dwords = (int64_t)pairs;   // Wt row = n_pad bf16 = pairs dwords
#pragma unroll
  for (int j = 0; j < M; ++j) wt[(int64_t)(g * M + j) * row_dwords + p] = out[j];
}

template <int LAYOUT, int M>
__global__ __launch_bounds__(256) void wt_expand_kernel(const uint32_t* __restrict__ codes,
                                                        const uint32_t* __restrict__ meta, int U,
                                                        int groups, int pairs,
                                                        uint32_t* __restrict__ wt) {
  wt_expand_one<LAYOUT, M>(codes, meta, U, groups, pairs, wt,
                           (int64_t)blockIdx.x * 256 + threadIdx.x);
}

// ---------------------------------------------------------------------------------------------
// Transposes to the reduction-contiguous layouts of dW, 64 x 64 element tiles through LDS.
//   Q8:  src = xq int8 [T][C] with scale[T]; dst[c][t] = bf16(fp32(q * scale_t))
//   !Q8: src = bf16 [T][C];                  dst[c][t] = src[t][c]
// dst rows have pitch ld_dst (T rounded up to 32) and are zero for t >= T; only c < C is written.
// Load: thread (t = tid/4, 16 consecutive c).  Store: thread (c = tid/4, 16 consecutive t) as two
// 16-byte stores.  The LDS tile has a row pitch of 66 bf16 (33 dwords): the 16 column reads of a
// store run hit distinct banks.
// ---------------------------------------------------------------------------------------------
constexpr int kTrPitch = 66;

template <bool Q8>
__device__ __forceinline__ void transpose_tile(const void* __restrict__ src,
                                               const float* __restrict__ scale, int T, int C,
                                               int ld_src, uint16_t* __restrict__ dst, int ld_dst,
                                               int tc, int tt, uint16_t* tile) {
  const int tid = threadIdx.x;
  const int t0 = tt * 64, c0 = tc * 64;
  {
    const int t = tid >> 2, cc = (tid & 3) * 16;
    const int tg = t0 + t, cg = c0 + cc;
    uint32_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0u;
    if (tg < T && cg < C) {
      if constexpr (Q8) {
        const int4 raw = *(const int4*)((const int8_t*)src + (int64_t)tg * ld_src + cg);
        const float s = scale[tg];
        const int w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int word = w[e / 2];
          const int b0 = (int)(int8_t)(word >> (16 * (e % 2)));
          const int b1 = (int)(int8_t)(word >> (16 * (e % 2) + 8));
          v[e] = f32_to_bf16_rne((float)b0 * s) | (f32_to_bf16_rne((float)b1 * s) << 16);
        }
      } else {
        const uint16_t* row = (const uint16_t*)src + (int64_t)tg * ld_src;
        if (cg + 16 <= C && (ld_src & 7) == 0) {
          const uint4 a = *(const uint4*)(row + cg);
          const uint4 b = *(const uint4*)(row + cg + 8);
          v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
          v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (cg + e < C) v[e / 2] |= (uint32_t)row[cg + e] << (16 * (e % 2));
        }
      }
    }
    uint32_t* trow = (uint32_t*)(tile + t * kTrPitch + cc);
#pragma unroll
    for (int e = 0; e < 8; ++e) trow[e] = v[e];
  }
  __syncthreads();
  {
    const int c = tid >> 2, tt16 = (tid & 3) * 16;
    const int cg = c0 + c, tg = t0 + tt16;
    if (cg < C && tg < ld_dst) {
      uint32_t w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        w[e] = (uint32_t)tile[(tt16 + 2 * e) * kTrPitch + c] |
               ((uint32_t)tile[(tt16 + 2 * e + 1) * kTrPitch + c] << 16);
      uint4* o = (uint4*)(dst + (int64_t)cg * ld_dst + tg);
      o[0] = make_uint4(w[0], w[1], w[2], w[3]);
      o[1] = make_uint4(w[4], w[5], w[6], w[7]);
    }
  }
}

template <bool Q8>
__global__ __launch_bounds__(256) void transpose_kernel(const void* __restrict__ src,
                                                        const float* __restrict__ scale, int T,
                                                        int C, int ld_src, uint16_t* __restrict__ dst,
                                                        int ld_dst, int tiles_c) {
  __shared__ uint16_t tile[64 * kTrPitch];
  transpose_tile<Q8>(src, scale, T, C, ld_src, dst, ld_dst, (int)(blockIdx.x % tiles_c),
                     (int)(blockIdx.x / tiles_c), tile);
}

// dYp[t][o] = dY[t][o] for o < n, 0 for n <= o < ld (rows padded to a multiple of 32).
__device__ __forceinline__ void pad_rows_one(const uint16_t* __restrict__ src, int64_t T, int n,
                                             int ld, uint16_t* __restrict__ dst, int64_t id) {
  if (id >= T * ld) return;
  const int64_t t = id / ld;
  const int o = (int)(id % ld);
  dst[id] = o < n ? src[t * n + o] : (uint16_t)0;
}

__global__ __launch_bounds__(256) void pad_rows_kernel(const uint16_t* __restrict__ src, int64_t T,
                                                       int n, int ld, uint16_t* __restrict__ dst) {
  pad_rows_one(src, T, n, ld, dst, (int64_t)blockIdx.x * 256 + threadIdx.x);
}

// ---------------------------------------------------------------------------------------------
// C[i][j] = alpha * sum_r A[i][r] B[j][r] (+ C[i][j] when accumulating), bf16 operands, fp32
// accumulation and output.  A: rows_a x R (pitch lda), B: rows_b x R (pitch ldb), R % 32 == 0.
//
// Block tile 256 (i) x 256 (j), four waves as 2 x 2, each wave 128 x 128 outputs = 4 x 4 tiles of
// v_mfma_f32_32x32x16_bf16 (256 fp32 accumulators per lane, one wave per SIMD).  Per 16-wide
// reduction step a wave reads 4 + 4 operand fragments (1 KB each) from LDS for 16 MFMAs.  The
// MFMA's row operand is B (so j runs along the 32 rows of a tile) and its column operand is A: a
// lane then holds one i and four runs of four consecutive j, stored as 16-byte vectors.
//
// Operands reach LDS with direct global->LDS loads (16 bytes per lane, no VGPR staging).  A stage
// is 32 reduction elements (64 bytes) of all 256 A rows and 256 B rows, 32 KB; a ring of five
// stage buffers keeps three stages in flight while one is multiplied and the previous one is
// still being read, and each wave waits on its own vmcnt (every stage issues exactly kNtLoads
// loads per wave) before a bare s_barrier.  Rows
// are stored 64 bytes apart with their 16-byte chunks XOR-swizzled by (row / 4) % 4, so the 16
// lanes served together (16 consecutive rows, one chunk each) hit 16 distinct 16-byte bank groups.
// Rows past rows_a / rows_b load clamped, valid rows whose results are never stored.
// ---------------------------------------------------------------------------------------------
constexpr int kNtWI = 4, kNtWJ = 4;          // 32 x 32 tiles per wave along i and along j
constexpr int kNtBI = 256, kNtBJ = 256;      // block tile (2 x 2 waves)
constexpr int kNtRowBytes = 64;              // bytes of the reduction axis per row per stage
constexpr int kNtHalf = kNtBI * kNtRowBytes; // A part of a stage (B follows)
constexpr int kNtStage = (kNtBI + kNtBJ) * kNtRowBytes;
constexpr int kNtRing = 5;                   // 5 x 32 KB: all of the CU's 160 KB of LDS
constexpr int kNtLoads = kNtStage / 1024 / 4;   // global->LDS loads per wave per stage
constexpr int kNtGroupI = 8;                     // row tiles per group of the tile order
static_assert(kNtLoads == 8, "stage split");

struct NtArgs {
  const uint16_t* a;
  const uint16_t* b;
  const float* alpha;   // device scalar, or NULL for 1
  float* c;
  int rows_a, rows_b, lda, ldb, ldc, R, accumulate, tiles_i, tiles;
};

struct NtGemm {
  uint8_t* ring;
  const uint8_t* a;
  const uint8_t* b;
  int NS, lane, wi, wj, h;
  uint32_t m0;                                 // this wave's LDS destination in stage buffer 0
  uint32_t a_off[kNtLoads / 2], b_off[kNtLoads / 2];
  v16f acc[kNtWI][kNtWJ];

  struct Regs {
    bf16x8 a[kNtWI];
    bf16x8 b[kNtWJ];
  };

  template <int BUF>
  __device__ __forceinline__ void issue(int st_in) {
    const int st = min(st_in, NS - 1);
    const uint8_t* sa = a + (size_t)st * kNtRowBytes;
    const uint8_t* sb = b + (size_t)st * kNtRowBytes;
    const uint32_t base = m0 + BUF * kNtStage;
#pragma unroll
    for (int q = 0; q < kNtLoads / 2; ++q) lds_dma16_s(sa, a_off[q], base + q * 1024);
#pragma unroll
    for (int q = 0; q < kNtLoads / 2; ++q) lds_dma16_s(sb, b_off[q], base + kNtHalf + q * 1024);
  }

  // Fragment f of reduction step j: f = 0..3 the A fragments (rows wi*128 + 32f ..), f = 4..7 the B
  // fragments.  Lane l reads row l % 32 of the fragment, 8 bf16 at reduction offset 16j + 8(l/32).
  __device__ __forceinline__ void read_frag(const uint8_t* buf, int j, int f, Regs& r) const {
    const bool is_a = f < kNtWI;
    const int row = (is_a ? wi : wj) * 128 + (is_a ? f : f - kNtWI) * 32 + (lane & 31);
    const int chunk = (2 * j + h) ^ ((row >> 2) & 3);
    const bf16x8 v = *(const bf16x8*)(buf + (is_a ? 0 : kNtHalf) + row * kNtRowBytes + chunk * 16);
    if (is_a) r.a[f] = v; else r.b[f - kNtWI] = v;
  }

  __device__ __forceinline__ void read_step(const uint8_t* buf, int j, Regs& r) const {
#pragma unroll
    for (int f = 0; f < kNtWI + kNtWJ; ++f) read_frag(buf, j, f, r);
  }

  __device__ __forceinline__ void mma_one(const Regs& r, int fi, int fj) {
    acc[fi][fj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r.b[fj], r.a[fi], acc[fi][fj], 0, 0, 0);
  }

  __device__ __forceinline__ void mma(const Regs& r) {
#pragma unroll
    for (int fi = 0; fi < kNtWI; ++fi)
#pragma unroll
      for (int fj = 0; fj < kNtWJ; ++fj) mma_one(r, fi, fj);
  }

  // The next step's eight LDS reads go out one before each of the first eight MFMAs, so their
  // latency hides under the current step's matrix work (left alone, the scheduler sinks them
  // below all sixteen MFMAs and the next step waits on them).
  __device__ __forceinline__ static void interleave_reads() {
#pragma unroll
    for (int q = 0; q < kNtWI + kNtWJ; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kNtWI * kNtWJ - (kNtWI + kNtWJ), 0);
  }

  // One stage (two reduction steps) from buffer BUF.  On entry R0 holds its first step; on exit
  // R0 holds the next stage's first step.
  //   First half: step 0's sixteen MFMAs, with step 1's reads interleaved.
  //   Then the wave waits for its own loads of the next stage (the two stages after it stay in
  //   flight) and meets the other waves: every wave has consumed its reads of the previous
  //   stage's buffer by now, so the barrier waits on no LDS read.
  //   Second half: step 1's sixteen MFMAs in pairs; before each pair go one global->LDS load of
  //   stage st + 4 into the previous stage's buffer and one read of the next stage's first step.
  //   A burst of eight loads would stall the wave's issue behind the memory pipeline (one wave per
  //   SIMD: the matrix core would idle); spread out, each load is accepted while MFMAs run.  The
  //   scheduling fences keep exactly this order.
  template <int BUF>
  __device__ __forceinline__ void stage(int st, Regs& R0, Regs& R1) {
    read_step(ring + BUF * kNtStage, 1, R1);
    mma(R0);
    interleave_reads();
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * kNtLoads));
    block_barrier_nofence();
    constexpr int REFILL = (BUF + kNtRing - 1) % kNtRing;
    const int stn = min(st + kNtRing - 1, NS - 1);
    const uint8_t* sa = a + (size_t)stn * kNtRowBytes;
    const uint8_t* sb = b + (size_t)stn * kNtRowBytes;
    const uint32_t base = m0 + REFILL * kNtStage;
    const uint8_t* nbuf = ring + ((BUF + 1) % kNtRing) * kNtStage;
    static_assert(kNtLoads == kNtWI + kNtWJ && kNtWI * kNtWJ == 2 * kNtLoads, "pairing");
#pragma unroll
    for (int q = 0; q < kNtLoads; ++q) {
      __builtin_amdgcn_sched_barrier(0);
      if (q < kNtLoads / 2) lds_dma16_s(sa, a_off[q], base + q * 1024);
      else lds_dma16_s(sb, b_off[q - kNtLoads / 2], base + kNtHalf + (q - kNtLoads / 2) * 1024);
      read_frag(nbuf, 0, q, R0);
      mma_one(R1, q / 2, 2 * (q % 2));
      mma_one(R1, q / 2, 2 * (q % 2) + 1);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
};

// One 256 x 256 output tile at (i0, j0): the pipeline over the whole reduction, then the epilogue.
// On entry the ring may still be in use by an earlier tile of the same block only if the caller
// has drained and synchronized it (gemm_nt_group_kernel does before every segment after the
// first).
struct NtTile {
  const uint16_t* a;
  const uint16_t* b;
  const float* alpha;   // device scalar, or NULL for 1
  float* c;
  int rows_a, rows_b, lda, ldb, ldc, R, accumulate, i0, j0;
};

typedef __attribute__((address_space(1))) float g_f32;
typedef __attribute__((address_space(1))) v4f g_v4f;

__device__ __forceinline__ void nt_tile(uint8_t* ring, const NtTile& p, int tid) {
  NtGemm k;
  k.ring = ring;
  k.a = (const uint8_t*)p.a;
  k.b = (const uint8_t*)p.b;
  k.lane = tid & 63;
  const int wave = tid >> 6;
  k.wi = wave & 1;
  k.wj = wave >> 1;
  k.h = k.lane >> 5;
  k.NS = p.R / 32;
  const int i0 = p.i0, j0 = p.j0;

  // Load q of a wave covers rows (wave * 4 + q) * 16 .. +15 of the A (or B) part of a stage: lane
  // l fills position l % 4 of row l / 4 with the global chunk (l % 4) ^ ((row / 4) % 4).
#pragma unroll
  for (int q = 0; q < kNtLoads / 2; ++q) {
    const int row = (wave * 4 + q) * 16 + (k.lane >> 2);
    const int chunk = (k.lane & 3) ^ ((row >> 2) & 3);
    k.a_off[q] = (uint32_t)min(i0 + row, p.rows_a - 1) * (uint32_t)p.lda * 2u + chunk * 16;
    k.b_off[q] = (uint32_t)min(j0 + row, p.rows_b - 1) * (uint32_t)p.ldb * 2u + chunk * 16;
  }
  k.m0 = __builtin_amdgcn_readfirstlane(lds_offset(ring) + (uint32_t)wave * (kNtLoads / 2) * 1024);
#pragma unroll
  for (int fi = 0; fi < kNtWI; ++fi)
#pragma unroll
    for (int fj = 0; fj < kNtWJ; ++fj) k.acc[fi][fj] = v16f{};

  if (k.NS > 0) {
    NtGemm::Regs R0, R1;
    k.issue<0>(0);
    k.issue<1>(1);
    k.issue<2>(2);
    k.issue<3>(3);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(3 * kNtLoads));   // stage 0 landed (this wave's part)
    block_barrier_nofence();
    k.read_step(ring, 0, R0);
    static_assert(kNtRing == 5, "the stage loop is unrolled over the ring");
    for (int st = 0; st < k.NS; st += kNtRing) {
      k.stage<0>(st, R0, R1);
      if (st + 1 < k.NS) k.stage<1>(st + 1, R0, R1);
      if (st + 2 < k.NS) k.stage<2>(st + 2, R0, R1);
      if (st + 3 < k.NS) k.stage<3>(st + 3, R0, R1);
      if (st + 4 < k.NS) k.stage<4>(st + 4, R0, R1);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0));   // no load may still be writing LDS at exit
  }

  const float alpha = p.alpha ? *(const g_f32*)p.alpha : 1.0f;
  const int lane = k.lane, h = k.h;
  const bool vec_ok = (p.rows_b & 3) == 0 && (p.ldc & 3) == 0;
#pragma unroll
  for (int fi = 0; fi < kNtWI; ++fi) {
    const int i = i0 + k.wi * 128 + fi * 32 + (lane & 31);
    if (i >= p.rows_a) continue;
    g_f32* crow = (g_f32*)p.c + (size_t)i * p.ldc;
#pragma unroll
    for (int fj = 0; fj < kNtWJ; ++fj) {
      const int jb = j0 + k.wj * 128 + fj * 32;
      if (vec_ok && jb + 32 <= p.rows_b) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = jb + 8 * jj + 4 * h;
          v4f v;
          v[0] = k.acc[fi][fj][4 * jj + 0] * alpha;
          v[1] = k.acc[fi][fj][4 * jj + 1] * alpha;
          v[2] = k.acc[fi][fj][4 * jj + 2] * alpha;
          v[3] = k.acc[fi][fj][4 * jj + 3] * alpha;
          if (p.accumulate) v += *(const g_v4f*)(crow + j);
          *(g_v4f*)(crow + j) = v;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = jb + 8 * (r >> 2) + 4 * h + (r & 3);
          if (j < p.rows_b) {
            float v = k.acc[fi][fj][r] * alpha;
            if (p.accumulate) v += crow[j];
            crow[j] = v;
          }
        }
      }
    }
  }
}

__global__ __launch_bounds__(256, 1) void gemm_nt_kernel(NtArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kNtRing * kNtStage];
  // XCD-major tile order: block b runs on XCD b % 8 and each XCD takes a contiguous run of tile
  // numbers t.  Tile numbers run through groups of kNtGroupI row tiles (i) by all column tiles
  // (j), i fastest inside a group, so the 32 tiles an XCD's 32 CUs hold at once form an 8 x 4
  // patch: 12 operand tiles per 32 output tiles stay in that XCD's L2, where a run along i alone
  // (32 x 1) streams 33.
  const int full = (p.tiles / 8) * 8;
  const int b = blockIdx.x;
  const int t = b < full ? (b % 8) * (p.tiles / 8) + b / 8 : b;
  const int tiles_j = p.tiles / p.tiles_i;
  const int per_group = kNtGroupI * tiles_j;
  const int first_i = (t / per_group) * kNtGroupI;
  const int gsize = min(p.tiles_i - first_i, kNtGroupI);
  const int ti = first_i + (t % per_group) % gsize, tj = (t % per_group) / gsize;
  NtTile tile;
  tile.a = p.a; tile.b = p.b; tile.alpha = p.alpha; tile.c = p.c;
  tile.rows_a = p.rows_a; tile.rows_b = p.rows_b; tile.lda = p.lda; tile.ldb = p.ldb;
  tile.ldc = p.ldc; tile.R = p.R; tile.accumulate = p.accumulate;
  tile.i0 = ti * kNtBI; tile.j0 = tj * kNtBJ;
  nt_tile(ring, tile, threadIdx.x);
}

// ---------------------------------------------------------------------------------------------
// Grouped backward: every projection of a layer set in two launches.  bwd_prep_kernel runs all
// operand preparations (W_eff^T expansions, dY pads and transposes, one X^^T per distinct
// activation); gemm_nt_group_kernel runs every output tile of every dX and dW product, one job
// per block.  A dX buffer named by several projections is one set of tiles whose segments (one
// per projection, in descriptor order) each finish with the store or accumulate of that
// projection's call, so the result is bit for bit that of the calls one after another.  The host
// orders the jobs longest first and deals 8 x 4 tile patches to the XCDs by load, so the tails of
// the separate launches become one tail.
// ---------------------------------------------------------------------------------------------
template <int LAYOUT, int M>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint8_t* __restrict__ table) {
  __shared__ uint16_t tile[64 * kTrPitch];
  const BwdHeader* hd = (const BwdHeader*)table;
  if (hd->magic != kBwdMagic || hd->layout != LAYOUT || hd->M != M) return;
  const int b = blockIdx.x;
  if (b >= hd->prep_blocks) return;
  const BwdPrep* items = (const BwdPrep*)(table + hd->prep_off);
  int lo = 0, hi = hd->prep_items - 1;   // last item with block0 <= b
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (items[mid].block0 <= b) lo = mid; else hi = mid - 1;
  }
  const BwdPrep it = items[lo];
  const int local = b - it.block0;
  const int T = (int)hd->T;
  switch (it.kind) {
    case kPrepWt:
      wt_expand_one<LAYOUT, M>((const uint32_t*)it.src0, (const uint32_t*)it.src1, it.a0, it.a1,
                               it.a2, (uint32_t*)it.dst, (int64_t)local * 256 + threadIdx.x);
      break;
    case kPrepPad:
      pad_rows_one((const uint16_t*)it.src0, T, it.a0, it.a1, (uint16_t*)it.dst,
                   (int64_t)local * 256 + threadIdx.x);
      break;
    case kPrepTrDy:
      transpose_tile<false>(it.src0, nullptr, T, it.a0, it.a0, (uint16_t*)it.dst, (int)hd->t32,
                            local % it.a1, local / it.a1, tile);
      break;
    default:
      transpose_tile<true>(it.src0, (const float*)it.src1, T, it.a0, it.a0, (uint16_t*)it.dst,
                           (int)hd->t32, local % it.a1, local / it.a1, tile);
      break;
  }
}

__global__ __launch_bounds__(256, 1) void gemm_nt_group_kernel(const uint8_t* __restrict__ table,
                                                                 int layout, int M) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kNtRing * kNtStage];
  const BwdHeader* hd = (const BwdHeader*)table;
  if (hd->magic != kBwdMagic || hd->layout != layout || hd->M != M || (int)blockIdx.x >= hd->jobs)
    return;
  const BwdJob job = ((const BwdJob*)(table + hd->jobs_off))[blockIdx.x];
  const BwdSeg* segs = (const BwdSeg*)(table + hd->segs_off) + job.seg0;
  for (int s = 0; s < job.nseg; ++s) {
    if (s > 0) {
      // the previous segment's LDS reads and loads are done in every wave before the ring refills
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
      block_barrier_nofence();
    }
    const BwdSeg sg = segs[s];
    NtTile t;
    t.a = sg.a; t.b = sg.b; t.alpha = sg.alpha; t.c = job.c;
    t.rows_a = job.rows_a; t.rows_b = job.rows_b; t.lda = sg.lda; t.ldb = sg.ldb;
    t.ldc = job.ldc; t.R = sg.R; t.accumulate = sg.accumulate;
    t.i0 = job.i0; t.j0 = job.j0;
    // Opaque per-segment copies: without them the compiler hoists the tile's address arithmetic
    // out of the segment loop, and the values it keeps live across the main loop spill (the
    // main loop already holds 256 accumulators and all 256 vector registers).
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    asm volatile("" : "+s"(t.c), "+s"(t.rows_a), "+s"(t.rows_b), "+s"(t.ldc), "+s"(t.i0),
                 "+s"(t.j0));
    nt_tile(ring, t, tid);
  }
}

static hipError_t launch_gemm_nt(const uint16_t* a, int rows_a, int lda, const uint16_t* b,
                                 int rows_b, int ldb, int R, const float* alpha, float* c, int ldc,
                                 int accumulate, hipStream_t s) {
  NtArgs p;
  p.a = a; p.b = b; p.alpha = alpha; p.c = c;
  p.rows_a = rows_a; p.rows_b = rows_b; p.lda = lda; p.ldb = ldb; p.ldc = ldc; p.R = R;
  p.accumulate = accumulate;
  p.tiles_i = (rows_a + kNtBI - 1) / kNtBI;
  p.tiles = p.tiles_i * ((rows_b + kNtBJ - 1) / kNtBJ);
  gemm_nt_kernel<<<p.tiles, 256, 0, s>>>(p);
  return hipGetLastError();
}

template <int LAYOUT, int M>
static void launch_wt(const uint32_t* codes, const uint32_t* meta, int U, int groups, int pairs,
                      uint32_t* wt, hipStream_t s) {
  const int64_t threads = (int64_t)groups * pairs;
  wt_expand_kernel<LAYOUT, M><<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(codes, meta, U,
                                                                               groups, pairs, wt);
}

hipError_t launch_bwd(const uint16_t* dy, int64_t T, int64_t n, const int8_t* xq,
                      const float* x_scale, int64_t K, const uint32_t* codes, const uint32_t* meta,
                      const float* gamma, int N, int M, int layout, float* dx, float* dw, int flags,
                      void* ws, hipStream_t s) {
  const BwdWorkspace w = bwd_workspace(T, n, K);
  uint8_t* base = (uint8_t*)ws;
  if (dx && T > 0) {
    uint16_t* wt = (uint16_t*)(base + w.wt_off);
    const int64_t keff = (layout == kLayoutSparse && M > 4) ? K / M * (2 * M - 4) : K;
    const int U = (int)(layout == kLayoutSparse ? keff / 32 : K / 16);
    const int groups = (int)(K / M), pairs = (int)(w.n32 / 2);
    const bool ok = dispatch_m(M, [&](auto m) {
      constexpr int MM = decltype(m)::value;
      if (layout == kLayoutSparse) launch_wt<kLayoutSparse, MM>(codes, meta, U, groups, pairs, (uint32_t*)wt, s);
      else launch_wt<kLayoutDense2, MM>(codes, nullptr, U, groups, pairs, (uint32_t*)wt, s);
    });
    if (!ok) return hipErrorInvalidValue;
    const uint16_t* a = dy;
    if (w.n32 != n) {
      uint16_t* dyp = (uint16_t*)(base + w.dyp_off);
      const int64_t total = T * w.n32;
      pad_rows_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(dy, T, (int)n, (int)w.n32, dyp);
      a = dyp;
    }
    hipError_t e = launch_gemm_nt(a, (int)T, (int)w.n32, wt, (int)K, (int)w.n32, (int)w.n32, gamma,
                                  dx, (int)K, (flags & 1) != 0, s);
    if (e != hipSuccess) return e;
  }
  if (dw) {
    uint16_t* dyt = (uint16_t*)(base + w.dyt_off);
    uint16_t* xt = (uint16_t*)(base + w.xt_off);
    if (T > 0) {
      const int tt = (int)((T + 63) / 64);
      const int tn = (int)((n + 63) / 64), tk = (int)((K + 63) / 64);
      transpose_kernel<false><<<tt * tn, 256, 0, s>>>(dy, nullptr, (int)T, (int)n, (int)n, dyt,
                                                      (int)w.t32, tn);
      transpose_kernel<true><<<tt * tk, 256, 0, s>>>(xq, x_scale, (int)T, (int)K, (int)K, xt,
                                                     (int)w.t32, tk);
    }
    hipError_t e = launch_gemm_nt(dyt, (int)n, (int)w.t32, xt, (int)K, (int)w.t32, (int)w.t32,
                                  nullptr, dw, (int)K, (flags & 2) != 0, s);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_group(const void* table, int64_t prep_blocks, int64_t jobs, int layout,
                            int M, hipStream_t s) {
  const uint8_t* t = (const uint8_t*)table;
  if (prep_blocks > 0) {
    const unsigned g = (unsigned)prep_blocks;
    const bool ok = dispatch_m(M, [&](auto m) {
      constexpr int MM = decltype(m)::value;
      if (layout == kLayoutSparse) bwd_prep_kernel<kLayoutSparse, MM><<<g, 256, 0, s>>>(t);
      else bwd_prep_kernel<kLayoutDense2, MM><<<g, 256, 0, s>>>(t);
    });
    if (!ok) return hipErrorInvalidValue;
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (jobs > 0) gemm_nt_group_kernel<<<(unsigned)jobs, 256, 0, s>>>(t, layout, M);
  return hipGetLastError();
}

}  // namespace bl
