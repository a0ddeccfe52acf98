// Device table of a grouped backward (bitlinear_bwd_group_build writes it, bwd_prep_kernel and
// gemm_nt_group_kernel read it).  Layout from the table's start, every array 16-byte aligned:
//   BwdHeader
//   BwdPrep[prep_items]   operand preparation items, sorted by first block
//   BwdJob[jobs]          one per block of the product launch (padding jobs have nseg == 0)
//   BwdSeg[segs]          reduction segments of the jobs
// All pointers are absolute: the descriptors' buffers and the workspace the table was built with.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

constexpr uint32_t kBwdMagic = 0x42474c42u;   // "BLGB"

// Operand preparation kinds (the prep launch runs them all, one item per range of blocks).
enum BwdPrepKind : int32_t {
  kPrepWt = 0,    // W_eff^T [K][n32] bf16 from codes / meta: a0 = U, a1 = groups, a2 = pairs
  kPrepPad = 1,   // dY [T][n] -> [T][n32] zero-padded rows: a0 = n, a1 = n32
  kPrepTrDy = 2,  // dY^T [n][t32]: a0 = n (columns), a1 = tiles along n
  kPrepTrX = 3,   // X^^T [K][t32] from int8 and token scales: a0 = K, a1 = tiles along K
};

struct BwdHeader {
  uint32_t magic;
  int32_t layout, N, M;
  int64_t T;
  int32_t prep_items, prep_blocks, jobs, segs;
  int64_t prep_off, jobs_off, segs_off;   // byte offsets from the table's start
  int64_t t32;                            // T rounded up to a multiple of 32
  int64_t reserved;
};
static_assert(sizeof(BwdHeader) == 80, "backward table header is 80 bytes");

struct BwdPrep {
  int32_t kind, block0;     // first block of the item in the prep launch
  int32_t a0, a1, a2, a3;
  const void* src0;         // codes | dY | dY | xq
  const void* src1;         // meta (or NULL) | - | - | token scales
  void* dst;                // W_eff^T | padded dY | dY^T | X^^T
};
static_assert(sizeof(BwdPrep) == 48, "prep item is 48 bytes");

// One 256 x 256 tile of C: its segments run in order, each a full reduction whose epilogue
// scales by its alpha and stores into C or adds to it.
struct BwdJob {
  float* c;
  int32_t seg0, nseg;       // nseg == 0: the block does nothing
  int32_t i0, j0;
  int32_t rows_a, rows_b, ldc, reserved;
};
static_assert(sizeof(BwdJob) == 40, "job record is 40 bytes");

struct BwdSeg {
  const uint16_t* a;        // [rows_a][lda] bf16, reduction-contiguous
  const uint16_t* b;        // [rows_b][ldb] bf16, reduction-contiguous
  const float* alpha;       // device scalar, or NULL for 1
  int32_t lda, ldb, R, accumulate;
};
static_assert(sizeof(BwdSeg) == 40, "segment record is 40 bytes");

hipError_t launch_bwd_group(const void* table, int64_t prep_blocks, int64_t jobs, int layout,
                            int M, hipStream_t s);

}  // namespace bl
