/*
 * bitlinear.h -- C ABI of libbitlinear, the sparse ternary BitLinear forward on MI355X (gfx950).
 *
 * The operation (pages cited by title and section):
 *   - "BitNet b1.58: Ternary Weights for 1.58-bit LLMs", section "The mechanism": weights are
 *     quantized with an absmean scale gamma = mean|W| and RoundClip(W / gamma, -1, 1) to
 *     {-1, 0, +1}; activations are quantized per token to 8 bits on the symmetric grid
 *     [-Qb, Qb]; a ternary multiply-accumulate is an add, a subtract or a skip.
 *   - "Sparse-BitNet: 1.58-bit LLMs are Naturally Friendly to Semi-Structured Sparsity",
 *     technical summary section 2 (Sparse-BitLinear): an N:M mask keeps the N largest |w| of
 *     the continuous master weights in every group of M, recomputed at every training step,
 *     and is applied to the ternary weights (quantize, then mask).
 *   - SlideSparse abstract on "Is 2:4 Sparsity Still Worth It? ...": a 6:8 block is rewritten
 *     losslessly as 3 overlapping 2:4 windows (Sliding Window Decomposition), and the
 *     activations are rearranged to match inside per-token quantization (Activation Lifting).
 *
 * y[t][o] = gamma * scale[t] * sum_k W_eff[o][k] * xq[t][k]   (int32 accumulation, fp32 out)
 * with W_eff = mask(W) * RoundClip(W / gamma) and (xq, scale) the int8 activations.
 *
 * Precise definitions used (the page lost the formulas of the absmean quantizer):
 *   gamma   = the exact mean of |W| over all n*K entries of the dense master, rounded once to
 *             fp32 (ties to even); no epsilon.  gamma == 0 gives all-zero codes.
 *   W~      = clip(rint(fl32(W / gamma)), -1, 1), rint = round half to even.
 *   mask    = per row, per contiguous group of M along K from k = 0, the N largest |w| of the
 *             master; ties to the lower index; exactly N positions kept even if their code is 0.
 *   xq      = clamp(rint(fl32(x * fl32(127 / absmax_t))), -127, 127); scale[t] =
 *             fl32(absmax_t / 127); absmax_t = 0 gives xq = 0 and scale = 0.
 *
 * ---------------------------------------------------------------------------------------------
 * Packed weight layout (layout id BL_LAYOUT_VERSION = 1)
 *   slot    one kept weight.  BL_LAYOUT_SPARSE: each 4-wide window j of a row's packed K axis
 *           holds slots 2j, 2j+1 = its two kept positions in ascending order; 2:4 windows are
 *           the M-groups, 6:8 groups become 3 windows covering positions 0-3, 2-5, 4-7 of the
 *           group (packed K axis K_eff = 3K/2; greedy assignment in ascending position order:
 *           window 0 takes up to 2 kept positions in 0-3, window 1 up to 2 of the rest in 2-5,
 *           window 2 the rest).  BL_LAYOUT_DENSE2: every position is a slot (K_eff = K).
 *   code    2 bits per slot: 00 = 0, 01 = +1, 11 = -1 (10 is never written).
 *   index   2 bits per slot (SPARSE only): the slot's position 0..3 inside its window.
 *   unit    16 consecutive slots of one row = one little-endian code dword (slot i at bits
 *           8*(i%4) + 2*(i/4)) and, for SPARSE, one meta dword (slot i's index at bits 2*i).
 *   tiling  rows are padded to a multiple of 32 (padded rows: codes 0, every window's indices
 *           (0,1), i.e. meta 0x44444444).  With U units per row (K_eff/32 SPARSE, K/16 DENSE2),
 *           unit (r, c) is dword ((r/32) * (U/2) + c/2) * 64 + (c%2) * 32 + r%32 of each buffer.
 *           One 64-dword fragment is the A operand of one int8 sparse-MFMA 32x32x64 (SPARSE)
 *           or dense MFMA 32x32x32 (DENSE2) instruction: lane = (c%2)*32 + r%32.
 *
 * Shapes: n >= 1 (out features), K (in features): SPARSE 2:4 needs K % 64 == 0; SPARSE 6:8
 * needs K % 128 == 0; DENSE2 needs K % 32 == 0 and K % M == 0 with M in {4, 8}, 1 <= N <= M.
 * n * K < 2^32.  K_eff * 127 < 2^31.  T >= 0 tokens (T == 0 enqueues nothing), T * K_eff < 2^31.
 *
 * Conventions for every call:
 *   - All buffers are device memory owned by the caller; the library allocates nothing and keeps
 *     no pointer after a call returns.  Buffers must be 16-byte aligned and non-NULL unless a
 *     parameter says otherwise; with T == 0 the token-sized buffers of act_quant_i8 and
 *     bitlinear_fwd are never touched and may be NULL (the call then enqueues nothing).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls are enqueued asynchronously on
 *     it and are stream-ordered; no call synchronizes the host.  The library has no global
 *     mutable state; calls on different streams with disjoint buffers may run concurrently.
 *   - Every argument is validated on the host before anything is enqueued; on error nothing is
 *     enqueued.  Non-finite inputs (NaN, Inf) are outside the contract.
 *   - Return value: BL_OK, or a negative status (see bitlinear_strerror).
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BL_OK 0
#define BL_EINVAL (-22)   /* bad argument, shape, alignment or NULL pointer */
#define BL_ENOTSUP (-95)  /* unsupported N:M for the layout, or unknown layout / dtype */
#define BL_ENOSPC (-28)   /* workspace smaller than bitlinear_packed_bytes reports */
#define BL_EIO (-5)       /* HIP runtime or launch error */

#define BL_LAYOUT_SPARSE 0
#define BL_LAYOUT_DENSE2 1
#define BL_LAYOUT_VERSION 1

#define BL_DTYPE_F32 0
#define BL_DTYPE_BF16 1

/* Sizes of the packed buffers of an n x K master under (N, M, layout), in bytes, the packed K
 * axis K_eff, and the workspace bytes bitlinear_pack needs.  Any output pointer may be NULL.
 * Host only; enqueues nothing. */
int bitlinear_packed_bytes(int64_t n, int64_t K, int N, int M, int layout, size_t* codes_bytes,
                           size_t* meta_bytes, int64_t* K_eff, size_t* ws_bytes);

/* Mask + ternarize + pack one fp32 master W[n][K] (row-major, nn.Linear out x in).
 * Writes codes[codes_bytes], meta[meta_bytes] (SPARSE; pass NULL for DENSE2) and gamma[1]
 * (device fp32), all in the packed layout above.  ws is scratch of at least ws_bytes (from
 * bitlinear_packed_bytes); its contents on entry do not matter.  W is only read. */
int bitlinear_pack(const float* W, int64_t n, int64_t K, int N, int M, int layout, uint8_t* codes,
                   uint8_t* meta, float* gamma, void* ws, size_t ws_bytes, void* stream);

/* Per-token absmax int8 quantization of x[T][K] (row-major; x_dtype BL_DTYPE_F32 or
 * BL_DTYPE_BF16).  Writes xq[T][K_eff] int8 and x_scale[T] fp32 (absmax/127).
 * lift_M = 0: K_eff = K.  lift_M = 8: activation lifting for 6:8 windows, K_eff = 3K/2,
 * xq[t][12g + 4w + j] = q[t][8g + 2w + j] (w = 0..2, j = 0..3); needs K % 8 == 0. */
int act_quant_i8(const void* x, int x_dtype, int64_t T, int64_t K, int lift_M, int8_t* xq,
                 float* x_scale, void* stream);

/* y[T][n] fp32 = gamma * x_scale[t] * (xq[T][K_eff] . W_eff^T), int32 accumulation.
 * K is the master's in-feature count; (N, M, layout) must be those the weights were packed
 * with, and xq must be on the packed K axis (lifted with lift_M = 8 for SPARSE 6:8).
 * gamma is the device scalar written by bitlinear_pack.  acc_opt, if not NULL, receives the
 * int32 accumulators [T][n] (4-byte alignment suffices for it). */
int bitlinear_fwd(const int8_t* xq, const float* x_scale, int64_t T, int64_t K,
                  const uint8_t* codes, const uint8_t* meta, const float* gamma, int N, int M,
                  int layout, int64_t n, float* y, int32_t* acc_opt, void* stream);

/* Static description of a status code. */
const char* bitlinear_strerror(int status);

/* BL_LAYOUT_VERSION of the packed format this build reads and writes. */
int bitlinear_layout_version(void);

#ifdef __cplusplus
}
#endif
#endif /* BITLINEAR_H */
