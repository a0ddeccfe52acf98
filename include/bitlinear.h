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
 *   - SlideSparse abstract on "Is 2:4 Sparsity Still Worth It? ...": a (2N-2):2N block (6:8,
 *     14:16) is rewritten losslessly as N-1 overlapping 2:4 windows (Sliding Window
 *     Decomposition), and the activations are rearranged to match inside per-token
 *     quantization (Activation Lifting).
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
 * Packed weight layout (layout id BL_LAYOUT_VERSION = 2)
 *   slot    one kept weight.  BL_LAYOUT_SPARSE: each 4-wide window j of a row's packed K axis
 *           holds slots 2j, 2j+1 = its two kept positions in ascending order; 2:4 windows are
 *           the M-groups; an (M-2):M group (6:8, 14:16) becomes M/2 - 1 windows, window w
 *           covering positions 2w..2w+3 of the group (packed K axis K_eff = (2M-4)K/M: 3K/2
 *           for 6:8, 7K/4 for 14:16).  Assignment: kept positions in ascending order, each to
 *           the lowest window that covers it and holds fewer than two (for 6:8: window 0 takes
 *           up to 2 kept positions in 0-3, window 1 up to 2 of the rest in 2-5, window 2 the
 *           rest).  BL_LAYOUT_DENSE2: every position is a slot (K_eff = K).
 *   code    2 bits per slot: 00 = 0, 01 = +1, 10 = -1 (11 is never written).
 *   index   2 bits per slot (SPARSE only): the slot's position 0..3 inside its window.
 *   unit    16 consecutive slots of one row = one little-endian code dword (slot i at bits
 *           8*(i%4) + 2*(i/4)) and, for SPARSE, one meta dword (slot i's index at bits 2*i).
 *   tiling  rows are padded to a multiple of 32 (padded rows: codes 0, every window's indices
 *           (0,1), i.e. meta 0x44444444).  With U units per row (K_eff/32 SPARSE, K/16 DENSE2),
 *           unit (r, c) is dword ((r/32) * (U/2) + c/2) * 64 + (c%2) * 32 + r%32 of each buffer.
 *           One 64-dword fragment is the A operand of one int8 sparse-MFMA 32x32x64 (SPARSE)
 *           or dense MFMA 32x32x32 (DENSE2) instruction: lane = (c%2)*32 + r%32.
 *
 * SPARSE6 (BL_LAYOUT_SPARSE6, decode only): a 2:4 SPARSE matrix re-encoded at 6 bits per 4-wide
 * group, 0.1875 bytes per weight against 0.25 (the Bitnet.cpp abstract on the aitopics "bitnet"
 * tag page argues for ternary formats below 2 bits per weight; the pages fix no format).  A
 * group's 54 states (kept pair (i, j) of 6, one ternary value on each) are numbered
 * state = 9 * pair + 3 * code(lower) + code(upper), pairs in the order (0,1) (0,2) (0,3) (1,2)
 * (1,3) (2,3), code = the 2-bit code above (0, +1, -1 -> 0, 1, 2); 54..63 are never written.
 * Tiling for 16-row MFMA tiles: rows padded to 32, K to whole step pairs of 128 columns
 * (NC = ceil(K/128)); lane l (0..63) of (panel P, pair c) holds 96 bits in three little-endian
 * dwords at dword ((P*NC + c)*64 + l)*3, field f = 8*s2 + 4*rt + g (s2, rt in {0,1}, g in 0..3)
 * at bits 6f..6f+5 = the state of row 32P + 16rt + l%16, group 32c + 16s2 + 4(l/16) + g.
 * Padded rows and groups past K hold state 0 (zero weights).  Written by bitlinear_transcode6
 * from the 2:4 packed buffers; read by bitlinear_fwd (T <= 32) and the decode group.
 *
 * Shapes: n >= 1 (out features), K (in features).  SPARSE 2:4 (and SPARSE6) needs K % 64 == 0.
 * SPARSE (M-2):M for even M = 6..16 needs K to be a multiple of the smallest multiple k of M for
 * which both the packed axis k(2M-4)/M is a multiple of 64 and k is a multiple of lcm(M, 8):
 * 4:6 48, 6:8 128, 8:10 40, 10:12 192, 12:14 112, 14:16 256.  DENSE2 needs even M in 4..16,
 * 1 <= N <= M and K % lcm(32, M) == 0.
 * n * K < 2^32.  K_eff * 127 < 2^31.  T >= 0 tokens (T == 0 enqueues nothing), T * K_eff < 2^31.
 *
 * Conventions for every call:
 *   - All buffers are device memory owned by the caller; the library allocates nothing and keeps
 *     no pointer after a call returns (a group table keeps the pointers it was built with).
 *     Buffers must be 16-byte aligned and non-NULL unless a parameter says otherwise (x_scale
 *     and acc_opt need only 4-byte alignment, so a token slice of a larger buffer qualifies); with T == 0 the token-sized buffers of act_quant_i8 and
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
#define BL_LAYOUT_SPARSE6 2   /* 2:4 re-encoded at 6 bits per group; decode only (see above) */
#define BL_LAYOUT_VERSION 2

#define BL_DTYPE_F32 0
#define BL_DTYPE_BF16 1

/* Sizes of the packed buffers of an n x K master under (N, M, layout), in bytes, the packed K
 * axis K_eff, and the workspace bytes bitlinear_pack needs.  Any output pointer may be NULL.
 * For BL_LAYOUT_SPARSE6 (N:M 2:4 only): codes_bytes is the stream's size, meta_bytes 0, K_eff K,
 * ws_bytes 0.  Host only; enqueues nothing. */
int bitlinear_packed_bytes(int64_t n, int64_t K, int N, int M, int layout, size_t* codes_bytes,
                           size_t* meta_bytes, int64_t* K_eff, size_t* ws_bytes);

/* Mask + ternarize + pack one fp32 master W[n][K] (row-major, nn.Linear out x in).
 * Writes codes[codes_bytes], meta[meta_bytes] (SPARSE; pass NULL for DENSE2) and gamma[1]
 * (device fp32), all in the packed layout above.  ws is scratch of at least ws_bytes (from
 * bitlinear_packed_bytes: a fixed part plus 512 bytes per packing tile of 32 rows x at most 256
 * columns, 1.6% of W's bytes for 2:4); its contents on entry do not matter, and it must be
 * ordinary device memory (hipMalloc or a framework allocator on it: the pass adds into it with
 * device atomics that fine-grained or managed memory does not support).  W is only read.
 * Five launches, one pass over W in the common case: a share of W (all of a small master, at
 * least a 32nd of a large one) sampled to estimate gamma, and a band around the threshold that
 * estimate gives (one small block); the pass that sums |W| in fp64, writes
 * the mask and meta and every code whose weight lies clear of a narrow band around the
 * estimate's threshold (the kept weights inside it are listed); gamma, certified by a rigorous
 * bound of the fp64 sum, with an exact integer pass over W only when the exact mean lies too
 * close to an fp32 rounding boundary for the bound to decide; a fix-up that sets the listed codes
 * -- or, if the exact threshold fell outside the band or a tile listed more weights than its
 * region holds, packs W again.  The results never depend on the sample. */
int bitlinear_pack(const float* W, int64_t n, int64_t K, int N, int M, int layout, uint8_t* codes,
                   uint8_t* meta, float* gamma, void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation): bitlinear_pack without a caller workspace.  Same arguments
 * minus ws / ws_bytes, same shape, alignment and error rules, same results bit for bit.  The
 * workspace is a static device array inside the library, BL_PACK_NOALLOC_WS_BYTES bytes: the
 * workspace of a bitlinear_pack call on up to 8192 tiles (67 M weights).  A larger master is
 * packed without the band, in two passes over W, so every shape bitlinear_pack accepts fits
 * (BL_ENOSPC would report one that did not).  Each GPU the
 * library runs on holds its own copy from the first call there until the process ends; the call
 * allocates nothing.  Every call on one GPU shares that copy: calls that may overlap on one GPU
 * (different streams, or different host threads) race and must be serialized by the caller. */
#define BL_PACK_NOALLOC_WS_BYTES 4241664
int bitlinear_pack_noalloc(const float* W, int64_t n, int64_t K, int N, int M, int layout,
                           uint8_t* codes, uint8_t* meta, float* gamma, void* stream);

/* Per-token absmax int8 quantization of x[T][K] (row-major; x_dtype BL_DTYPE_F32 or
 * BL_DTYPE_BF16).  Writes xq[T][K_eff] int8 and x_scale[T] fp32 (absmax/127).
 * lift_M = 0: K_eff = K.  lift_M = 8 or 16: activation lifting for (M-2):M windows,
 * K_eff = (2M-4)K/M, xq[t][(2M-4)g + 4w + j] = q[t][Mg + 2w + j] (w = 0..M/2-2, j = 0..3);
 * needs K % 8 == 0 (and K % 16 == 0 for lift_M = 16). */
int act_quant_i8(const void* x, int x_dtype, int64_t T, int64_t K, int lift_M, int8_t* xq,
                 float* x_scale, void* stream);

/* act_quant_i8 of several activation matrices in one launch (a decode step quantizes the inputs
 * of its independent projections together; BitNet b1.58 page, "The mechanism", per-token absmax
 * quantization).  descs[i] holds the x, T, K, xq and x_scale of one act_quant_i8 call; all share
 * x_dtype and lift_M.  Each matrix's xq and x_scale are bit-identical to that call's, and each
 * follows its rules (T == 0 entries are skipped and may hold NULL pointers).  Inputs may be
 * shared or overlap; an output (xq, x_scale) may overlap no other output and no input
 * (BL_EINVAL).  1 <= count <= 16.  No table and no build step: the descriptors are copied into
 * the launch's arguments, so the call is asynchronous and capturable like act_quant_i8.  Rows
 * longer than 16384 bf16 (8192 fp32) elements make the group fall back to one launch per
 * matrix. */
typedef struct bl_quant_desc {
  const void* x;         /* [T][K] activations, x_dtype */
  int64_t T, K;
  int8_t* xq;            /* [T][K_eff] int8 */
  float* x_scale;        /* [T] fp32 token scales */
} bl_quant_desc;

int act_quant_i8_group(const bl_quant_desc* descs, int64_t count, int x_dtype, int lift_M,
                       void* stream);

/* y[T][n] fp32 = gamma * x_scale[t] * (xq[T][K_eff] . W_eff^T), int32 accumulation.
 * K is the master's in-feature count; (N, M, layout) must be those the weights were packed
 * with, and xq must be on the packed K axis (lifted with lift_M = M for SPARSE 6:8 and 14:16).
 * gamma is the device scalar written by bitlinear_pack.  acc_opt, if not NULL, receives the
 * int32 accumulators [T][n] (4-byte alignment suffices for it).
 * BL_LAYOUT_SPARSE6: codes is the stream of bitlinear_transcode6, meta must be NULL, N:M 2:4,
 * T <= 32 and K <= 16384 (BL_ENOTSUP otherwise); results equal those of the 2:4 SPARSE buffers
 * the stream was made from, bit for bit. */
int bitlinear_fwd(const int8_t* xq, const float* x_scale, int64_t T, int64_t K,
                  const uint8_t* codes, const uint8_t* meta, const float* gamma, int N, int M,
                  int layout, int64_t n, float* y, int32_t* acc_opt, void* stream);

/* Re-encode the 2:4 SPARSE packed buffers of an n x K master (codes, meta as bitlinear_pack wrote
 * them with N:M 2:4) into the SPARSE6 stream out[codes_bytes of bitlinear_packed_bytes(n, K, 2,
 * 4, BL_LAYOUT_SPARSE6)].  The re-encoding is exact (a group's state is its kept pair and codes);
 * gamma is unchanged and shared.  Buffers not written by bitlinear_pack (an index pair that is not
 * ascending, code 11) give an unspecified stream.  out may not overlap codes or meta (BL_EINVAL).
 * One launch, one thread per three stream dwords. */
int bitlinear_transcode6(const uint8_t* codes, const uint8_t* meta, int64_t n, int64_t K,
                         uint8_t* out, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Grouped pack: the bitlinear_pack calls of several masters (a training step re-packs every
 * master of a layer set; Sparse-BitNet technical summary, the mask is recomputed at each step) in
 * five launches instead of five per master.
 *
 * Each master's gamma, codes and meta are exactly bitlinear_pack's, bit for bit: the five
 * launches are bitlinear_pack's, each over every master (sample, band, pass, gamma, fix-up).  The workspace is the sum of the masters' bitlinear_pack workspaces.  All
 * masters share (N, M, layout); each follows bitlinear_pack's shape and
 * alignment rules.  Masters may be shared or overlap; outputs (codes, meta, gamma) must not
 * overlap each other or any master (BL_EINVAL).  1 <= count <= 4096.
 *
 * Use: bitlinear_pack_group_plan sizes the table and workspace; bitlinear_pack_group_build writes
 * the table (16-byte aligned device memory, caller-owned) for one workspace (256-byte aligned,
 * caller-owned, contents on entry irrelevant) and synchronizes `stream`: build once, outside any
 * graph capture; bitlinear_pack_group enqueues the five launches (asynchronous, stream-ordered,
 * capturable).  The table keeps the descriptors' pointers; masters are read at launch time, so
 * updated masters in the same buffers need no rebuild.  Launches sharing a workspace must be
 * ordered on one stream.  A table of another N:M or layout is ignored (nothing is written).
 */
typedef struct bl_pack_desc {
  const float* W;         /* [n][K] fp32 master */
  int64_t n, K;
  uint8_t* codes;         /* bitlinear_packed_bytes' codes_bytes */
  uint8_t* meta;          /* meta_bytes (SPARSE) or NULL (DENSE2) */
  float* gamma;           /* device scalar */
} bl_pack_desc;

typedef struct bl_pack_group_plan {
  size_t table_bytes;     /* device table */
  size_t ws_bytes;        /* device workspace */
  int64_t count;          /* masters */
  int64_t pack_blocks;    /* workgroups of the pack launch */
  int32_t N, M, layout;
  int32_t reserved;
} bl_pack_group_plan;

int bitlinear_pack_group_plan(const bl_pack_desc* descs, int64_t count, int N, int M, int layout,
                              bl_pack_group_plan* plan);
int bitlinear_pack_group_build(const bl_pack_desc* descs, int64_t count, int N, int M,
                               int layout, void* ws, size_t ws_bytes, void* table,
                               size_t table_bytes, void* stream);
int bitlinear_pack_group(const void* table, const bl_pack_group_plan* plan, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Grouped decode forward: many independent bitlinear_fwd projections in one launch.
 *
 * The operation of each projection is exactly bitlinear_fwd's (same definitions, same packed
 * layout, same results bit for bit).  A decode projection is a few MB of packed weights, so one
 * launch per projection is bound by launch and memory latency, not by HBM bandwidth; a group
 * covers projections that do not depend on each other (the Q/K/V or gate/up projections of a
 * decoder block, the experts of a layer, or a stream of layers whose activations are already
 * quantized) with one grid that streams all of their weights.
 *
 * Each descriptor holds the arguments of one bitlinear_fwd call; all projections of a group share
 * (N, M, layout).  Per projection: 0 <= T <= 32 (T == 0 projections are skipped and may hold NULL
 * token buffers), the bitlinear_fwd shape and alignment rules, acc_opt may be NULL.
 * Projections may share xq / x_scale; their y and acc_opt buffers must not overlap.
 * BL_LAYOUT_SPARSE6 groups (N:M 2:4, codes = bitlinear_transcode6 streams, meta NULL) run the
 * 6-bit decode kernel, with no bound on K beyond the shape rules.
 *
 * Use: bitlinear_group_table_bytes sizes a device table, bitlinear_group_build validates every
 * descriptor on the host and writes the table (it synchronizes `stream`: build once, outside any
 * graph capture), and bitlinear_fwd_group launches the group (asynchronous, stream-ordered,
 * capturable, no host work beyond argument checks).  The table holds the descriptors' pointers:
 * their buffers must stay allocated while the table is used, and their contents are read at launch
 * time, so new activations written into the same xq / x_scale buffers need no rebuild.
 * N, M and layout passed to bitlinear_fwd_group must be the table's, and work_items the count
 * bitlinear_group_table_bytes reported; a table of another layout is ignored (nothing is written).
 */
typedef struct bl_fwd_desc {
  const int8_t* xq;      /* [T][K_eff] int8 activations */
  const float* x_scale;  /* [T] fp32 token scales */
  int64_t T;             /* tokens: 0..32 (decode group), > 128 (prefill group) */
  int64_t K;             /* master in-features */
  const uint8_t* codes;  /* packed codes from bitlinear_pack */
  const uint8_t* meta;   /* packed meta (SPARSE) or NULL (DENSE2) */
  const float* gamma;    /* device scalar from bitlinear_pack */
  int64_t n;             /* out-features */
  float* y;              /* [T][n] fp32 output */
  int32_t* acc_opt;      /* [T][n] int32 accumulators, or NULL */
} bl_fwd_desc;

/* Validates descs[0..count) (host memory) and reports the device table size in bytes and the
 * number of work items of the group.  Output pointers may be NULL.  Enqueues nothing. */
int bitlinear_group_table_bytes(const bl_fwd_desc* descs, int64_t count, int N, int M, int layout,
                                size_t* table_bytes, int64_t* work_items);

/* Validates the group and writes its device table (table: 16-byte aligned device memory of at
 * least table_bytes, caller-owned).  Copies on `stream` and waits for it: returns when the table
 * is in place.  BL_ENOSPC if table_bytes is too small. */
int bitlinear_group_build(const bl_fwd_desc* descs, int64_t count, int N, int M, int layout,
                          void* table, size_t table_bytes, void* stream);

/* Enqueues the grouped forward of a built table on `stream`.  work_items == 0 enqueues nothing. */
int bitlinear_fwd_group(const void* table, int64_t work_items, int N, int M, int layout,
                        void* stream);

/* ---------------------------------------------------------------------------------------------
 * Fused decode: activation quantization inside the grouped forward.
 *
 * The same grouped forward as above, but each projection hands over its activations x[T][K] as
 * bfloat16 (bit patterns, row-major) instead of act_quant_i8's int8 rows and token scales: the
 * kernel takes the per-token absmax and quantizes the rows itself (BitNet b1.58 page, "The
 * mechanism"), with exactly act_quant_i8's expressions, so y (and acc_opt) are bit-identical to
 * act_quant_i8 followed by bitlinear_fwd_group.  A decode step then needs one launch instead of a
 * quantization launch per activation matrix plus the group launch.
 *
 * Layouts without activation lifting only: BL_LAYOUT_SPARSE with N:M = 2:4, or BL_LAYOUT_DENSE2
 * (BL_ENOTSUP otherwise, SPARSE6 included).  Per projection: 0 <= T <= 32, T * K * 2 < 2^31, x 16-byte aligned,
 * the other rules and the build / launch protocol as for the plain group; projections may share
 * x.  A fused table launched through bitlinear_fwd_group (or a plain one through
 * bitlinear_fwd_group_fused) writes nothing.
 */
typedef struct bl_fwd_x_desc {
  const uint16_t* x;     /* [T][K] bf16 activations */
  int64_t T;             /* tokens, 0..32 */
  int64_t K;             /* master in-features */
  const uint8_t* codes;  /* packed codes from bitlinear_pack */
  const uint8_t* meta;   /* packed meta (SPARSE) or NULL (DENSE2) */
  const float* gamma;    /* device scalar from bitlinear_pack */
  int64_t n;             /* out-features */
  float* y;              /* [T][n] fp32 output */
  int32_t* acc_opt;      /* [T][n] int32 accumulators, or NULL */
} bl_fwd_x_desc;

int bitlinear_group_fused_table_bytes(const bl_fwd_x_desc* descs, int64_t count, int N, int M,
                                      int layout, size_t* table_bytes, int64_t* work_items);
int bitlinear_group_fused_build(const bl_fwd_x_desc* descs, int64_t count, int N, int M,
                                int layout, void* table, size_t table_bytes, void* stream);
int bitlinear_fwd_group_fused(const void* table, int64_t work_items, int N, int M, int layout,
                              void* stream);

/* ---------------------------------------------------------------------------------------------
 * Fused decode over a chain of dependent layers: layer l + 1's input is layer l's output y.
 *
 * In a decoder every layer reads the previous layer's output, so its per-token int8 quantization
 * (BitNet b1.58 page, "The mechanism") cannot be batched with the others; separate calls pay an
 * act_quant_i8 launch and a bitlinear_fwd launch per layer.  bitlinear_fwd_chain runs the whole
 * chain in one persistent launch: per layer, the per-token absmax of its input, the int8
 * quantization (act_quant_i8's expressions), the sparse ternary GEMV and the rescale
 * (bitlinear_fwd's), with the next layer's absmax folded in as each layer writes its y.  Every
 * layer's y and acc_opt are bit-identical to act_quant_i8(previous y, fp32) followed by
 * bitlinear_fwd (layer 0: act_quant_i8(x0)).  Each layer's packed weights are loaded before its
 * wait for the previous layer.
 *
 * Layers: 2:4 BL_LAYOUT_SPARSE only (BL_ENOTSUP otherwise); K of layer l + 1 == n of layer l;
 * each n x K follows bitlinear_pack's shape rules with K <= 8192; 1 <= T <= 32 with
 * T * (K + 16) <= 129024 (the layer's int8 input rows stay in LDS); 1 <= L <= 4096.
 * codes, meta, y and x0 16-byte aligned, gamma 4 bytes, acc_opt 4 bytes or NULL.  Outputs (every
 * y and acc_opt) may not overlap each other, x0 or any weight buffer (BL_EINVAL).
 *
 * Use: bitlinear_chain_plan sizes the device table and the workspace; bitlinear_chain_build
 * writes the table (16-byte aligned device memory, caller-owned; synchronizes `stream`: build
 * once, outside graph capture); bitlinear_fwd_chain enqueues a clear of the workspace (a small
 * kernel) and the cooperative chain launch (64 workgroups, all resident).  The workspace
 * (caller-owned device memory, 16-byte aligned, contents on entry irrelevant) holds the grid
 * barrier's counter, an error word, per-workgroup partial absmax of every layer's input and
 * T x 8192 bytes for the int8 input rows of a layer whose fp32 input is larger than 256 KB (such
 * a layer is quantized in slices by all workgroups, one extra grid barrier, then copied into each
 * workgroup's LDS); calls sharing it must be ordered on one stream.  Every wait at the grid barrier is bounded by spin_limit polls
 * (<= 0: a default of about a second); a wait that gives up sets the uint32 error word at byte
 * offset 4 of the workspace to nonzero and its block returns, so the launch always ends -- then
 * the outputs are invalid.  Read that word after the launch completes.
 */
typedef struct bl_chain_layer {
  const uint8_t* codes;   /* packed 2:4 codes of the n x K master */
  const uint8_t* meta;    /* packed meta */
  const float* gamma;     /* device scalar */
  int64_t n, K;           /* out- and in-features; K == previous layer's n */
  float* y;               /* [T][n] fp32 output (the next layer's input) */
  int32_t* acc_opt;       /* [T][n] int32 accumulators, or NULL */
} bl_chain_layer;

typedef struct bl_chain_plan {
  size_t table_bytes;     /* device table */
  size_t ws_bytes;        /* device workspace */
  int64_t L, T;
  int32_t smem;           /* dynamic LDS bytes of the chain launch */
  int32_t reserved;
} bl_chain_plan;

int bitlinear_chain_plan(const bl_chain_layer* layers, int64_t L, int64_t T, int N, int M,
                         int layout, bl_chain_plan* plan);
int bitlinear_chain_build(const bl_chain_layer* layers, int64_t L, int64_t T, int N, int M,
                          int layout, void* table, size_t table_bytes, void* stream);
int bitlinear_fwd_chain(const void* table, const bl_chain_plan* plan, const void* x0, int x_dtype,
                        void* ws, size_t ws_bytes, int64_t spin_limit, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Grouped prefill forward: the bitlinear_fwd calls of a layer set with prefill-sized T in one
 * launch.
 *
 * Same operation and descriptors as the grouped decode forward (bl_fwd_desc; BitNet b1.58 page,
 * "The mechanism"), but for 128 < T per projection: y (and acc_opt) are those of bitlinear_fwd
 * for each descriptor, bit for bit.  Every 256-row x 128-token output tile of every projection
 * is one workgroup of the launch, so the separate launches' partial last waves become one; when
 * every projection's token tiles divide by 8 each XCD takes the same eighth of the token tiles
 * of every projection (projections sharing xq back to back), otherwise runs of tiles are dealt
 * to the XCDs longest first.  All projections share (N, M, layout); each follows
 * bitlinear_fwd's shape and alignment rules with T > 128 (BL_EINVAL otherwise).  Inputs (xq,
 * x_scale, codes, meta, gamma) may be shared or overlap; outputs (y, acc_opt) may overlap
 * nothing (BL_EINVAL).  1 <= count <= 4096.
 *
 * Use: bitlinear_gemm_group_plan validates the group and sizes the table (enqueues nothing);
 * bitlinear_gemm_group_build writes it (table: 16-byte aligned device memory of at least
 * table_bytes, caller-owned; copies on `stream` and waits for it, BL_ENOSPC if too small): build
 * once, outside any graph capture; bitlinear_gemm_group enqueues the launch (asynchronous,
 * stream-ordered, capturable).  The table keeps the descriptors' pointers, and their contents are
 * read at launch time: new activations in the same buffers need no rebuild.  A table of another
 * layout is ignored (nothing is written).
 */
typedef struct bl_gemm_group_plan {
  size_t table_bytes;     /* device table */
  int64_t jobs;           /* workgroups of the launch */
  int32_t N, M, layout;   /* the group's packing */
  int32_t reserved;
} bl_gemm_group_plan;

int bitlinear_gemm_group_plan(const bl_fwd_desc* descs, int64_t count, int N, int M, int layout,
                              bl_gemm_group_plan* plan);
int bitlinear_gemm_group_build(const bl_fwd_desc* descs, int64_t count, int N, int M, int layout,
                               void* table, size_t table_bytes, void* stream);
int bitlinear_gemm_group(const void* table, const bl_gemm_group_plan* plan, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Backward for training (Sparse-BitNet technical summary, Training Strategie: Dual STE).
 *
 * The rounding, the clip and the Top-N selection are passed straight through, and the gradient
 * reaches every master weight, the masked ones included.  With the forward y = X^ (gamma W_eff)^T
 * of bitlinear_fwd (X^ = q * scale_t):
 *   dx[T][K] = gamma * (dY . W_eff)         fp32; W_eff is the masked ternary matrix of the packed
 *                                           weights (any layout and N:M bitlinear_fwd accepts)
 *   dw[n][K] = dY^T . X^                    fp32, the gradient of the dense fp32 master;
 *                                           X^[t][k] = bf16(fp32(q[t][k] * x_scale[t])), both
 *                                           roundings to nearest even
 * dy is the output gradient in bfloat16 (bit patterns, row-major [T][n]).  xq is the plain
 * (never lifted) int8 activation [T][K] of act_quant_i8 with lift_M = 0 and x_scale its token
 * scales.  Products are exact (bf16 x bf16 in fp32) and sums are fp32 in an unspecified order;
 * dx is rounded once more by the gamma product.  No gradient flows to gamma or to the token
 * scales (straight through).
 *
 * flags: BL_BWD_ACCUM_DX adds the result to dx (dx += ...), BL_BWD_ACCUM_DW to dw; otherwise the
 * outputs are overwritten.  dx or dw may be NULL to skip that gradient (not both).  T == 0 leaves
 * dx alone and writes dw = 0 (or leaves it unchanged under BL_BWD_ACCUM_DW); dy, xq and x_scale
 * may then be NULL.
 *
 * Shapes follow bitlinear_fwd (K, N:M and layout as packed; n >= 1); in addition every operand of
 * the two products must stay below 2^31 bytes: T * n32, K * n32, n * T32 and K * T32 bf16
 * elements, where n32 and T32 are n and T rounded up to multiples of 32.  Alignment: dy, xq,
 * codes, meta, dx and dw 16 bytes, x_scale and gamma 4 bytes, ws 256 bytes.
 *
 * ws: caller-owned device workspace of at least bitlinear_bwd_workspace_bytes bytes, used for the
 * transposed bf16 operands; its contents on entry do not matter and are scratch afterwards.
 * Asynchronous and stream-ordered; calls that share a workspace must be ordered on one stream.
 */
#define BL_BWD_ACCUM_DX 1
#define BL_BWD_ACCUM_DW 2

/* Workspace bytes of bitlinear_bwd for T tokens, n out-features and K in-features. */
int bitlinear_bwd_workspace_bytes(int64_t T, int64_t n, int64_t K, size_t* ws_bytes);

int bitlinear_bwd(const uint16_t* dy, int64_t T, int64_t n, const int8_t* xq,
                  const float* x_scale, int64_t K, const uint8_t* codes, const uint8_t* meta,
                  const float* gamma, int N, int M, int layout, float* dx, float* dw, int flags,
                  void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Grouped backward: the bitlinear_bwd calls of a whole layer set in two launches.
 *
 * The operation is exactly that of calling bitlinear_bwd for descs[0], descs[1], ... in order on
 * one stream, bit for bit (same definitions as above).  One launch prepares every operand (the
 * W_eff^T expansions, the dY copies and transposes, and one X^^T per distinct activation: the
 * projections that share xq / x_scale transpose it once); the other runs every 256 x 256 output
 * tile of every dX and dW product as one grid, longest tiles first, so the grid tails of the
 * separate calls become one.  Projections that name the same dx (same pointer and K, e.g. Q/K/V
 * reading one activation) sum into it in descriptor order, each term with its own flags: a
 * descriptor with BL_BWD_ACCUM_DX adds to what the earlier ones left, one without overwrites it.
 *
 * All projections share T and (N, M, layout).  Per projection the rules of bitlinear_bwd apply;
 * in addition outputs must not overlap each other (apart from a shared dx) or any input of the
 * group (dy, xq, x_scale, codes, meta, gamma): BL_EINVAL.
 *
 * Use: bitlinear_bwd_group_plan validates the descriptors and sizes the device table and the
 * workspace; bitlinear_bwd_group_build writes the table (16-byte aligned device memory, caller-
 * owned) for one workspace (256-byte aligned device memory, caller-owned) -- it synchronizes
 * `stream`, so build once, outside any graph capture; bitlinear_bwd_group enqueues the two
 * launches (asynchronous, stream-ordered, capturable).  The table holds the descriptors' pointers
 * and the workspace's: they must stay allocated while it is used, and their contents are read at
 * launch time, so new gradients and activations in the same buffers need no rebuild.  Launches
 * that share a workspace must be ordered on one stream.  The plan passed to bitlinear_bwd_group
 * must be the one reported for the table's descriptors; a table of another N:M or layout is
 * ignored (nothing is written).
 */
typedef struct bl_bwd_desc {
  const uint16_t* dy;     /* [T][n] bf16 output gradient */
  const int8_t* xq;       /* [T][K] int8 activations (act_quant_i8, lift_M = 0) */
  const float* x_scale;   /* [T] token scales */
  int64_t K;              /* master in-features */
  const uint8_t* codes;   /* packed codes from bitlinear_pack */
  const uint8_t* meta;    /* packed meta (SPARSE) or NULL (DENSE2) */
  const float* gamma;     /* device scalar from bitlinear_pack */
  int64_t n;              /* out-features */
  float* dx;              /* [T][K] fp32 input gradient, or NULL */
  float* dw;              /* [n][K] fp32 master-weight gradient, or NULL */
  int32_t flags;          /* BL_BWD_ACCUM_DX | BL_BWD_ACCUM_DW, as for bitlinear_bwd */
  int32_t reserved;
} bl_bwd_desc;

typedef struct bl_bwd_group_plan {
  size_t table_bytes;     /* device table */
  size_t ws_bytes;        /* device workspace */
  int64_t prep_blocks;    /* workgroups of the operand launch */
  int64_t jobs;           /* workgroups of the product launch */
  int32_t N, M, layout;   /* the group's packing */
  int32_t reserved;
} bl_bwd_group_plan;

/* Validates descs[0..count) (host memory, 1 <= count <= 65536) and fills *plan.  Enqueues
 * nothing. */
int bitlinear_bwd_group_plan(const bl_bwd_desc* descs, int64_t count, int64_t T, int N, int M,
                             int layout, bl_bwd_group_plan* plan);

/* Validates the group and writes its device table for workspace ws.  Copies on `stream` and waits
 * for it.  BL_ENOSPC if ws_bytes or table_bytes is below the plan's. */
int bitlinear_bwd_group_build(const bl_bwd_desc* descs, int64_t count, int64_t T, int N, int M,
                              int layout, void* ws, size_t ws_bytes, void* table,
                              size_t table_bytes, void* stream);

/* Enqueues the grouped backward of a built table on `stream`. */
int bitlinear_bwd_group(const void* table, const bl_bwd_group_plan* plan, void* stream);

/* Static description of a status code. */
const char* bitlinear_strerror(int status);

/* BL_LAYOUT_VERSION of the packed format this build reads and writes. */
int bitlinear_layout_version(void);

#ifdef __cplusplus
}
#endif
#endif /* BITLINEAR_H */
