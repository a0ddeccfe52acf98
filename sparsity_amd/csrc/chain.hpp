// Device table and workspace of a fused decode over a chain of dependent layers
// (bitlinear_chain_build writes the table, chain_kernel reads it).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

constexpr uint32_t kChainMagic = 0x43474c42u;   // "BLGC"
constexpr int kChainWaves = 8;                   // waves per block
constexpr int kChainMaxSteps = 32;               // K steps per wave of a panel: K / 64 <= 8 * 32
constexpr int kChainMaxT = 32;
constexpr int kChainBlocks = 64;                 // workgroups of a chain launch (at most)

struct ChainHeader {
  uint32_t magic;
  int32_t L, T, smem;       // layers, tokens, dynamic LDS bytes of the launch
  int64_t reserved[6];
};
static_assert(sizeof(ChainHeader) == 64, "chain header is 64 bytes");

struct ChainLayer {
  const uint32_t* codes;    // packed 2:4 codes / meta of the n x K master
  const uint32_t* meta;
  const float* gamma;
  float* y;                 // [T][n] fp32 output; the next layer's input
  int32_t* acc;             // [T][n] int32 accumulators, or NULL
  int32_t n, K;
  int64_t reserved;
};
static_assert(sizeof(ChainLayer) == 56, "chain layer record is 56 bytes");

// Workspace (uint32 words): [0] arrivals at the grid barrier (every block adds 1 per barrier),
// [1] error flag (a bounded barrier wait gave up), [2..63] unused, then
// pmax[(L + 1)][kChainBlocks][T]: each block's max |x| bit pattern per token of each layer's
// input (layer l's input is layer l - 1's y); the layer's absmax is the max over the blocks.
// Then, from the next 256-byte boundary, xq[T][K]: the int8 input rows of a layer quantized in
// slices by all blocks (layers whose fp32 input exceeds kChainSplitBytes), sized for the
// largest K a chain accepts.
constexpr int kChainWsHead = 64;
constexpr int kChainMaxK = 8192;

__host__ __device__ inline size_t chain_xq_offset(int64_t L, int64_t T) {
  return (((size_t)kChainWsHead + (size_t)(L + 1) * kChainBlocks * T) * 4 + 255) / 256 * 256;
}
inline size_t chain_ws_bytes(int64_t L, int64_t T) {
  return chain_xq_offset(L, T) + (size_t)T * kChainMaxK;
}

// A layer whose fp32 input rows (T x K x 4 bytes) exceed this is quantized in two stages: every
// block quantizes a 1/G slice of the rows into xq, a grid barrier, then every block copies the
// int8 rows (a quarter of the bytes) into LDS.  Below it every block quantizes the whole input
// itself, which saves the barrier.
constexpr int64_t kChainSplitBytes = 256 * 1024;

// Dynamic LDS of a layer: its int8 input rows (T x (K + 16)), then the waves' int32 partials.
// A wave's 16 x 64 int32 partials with a row stride of 65 words, so that the reads of 32
// consecutive panel rows of one token fall on distinct banks.
constexpr int kChainRedStride = 65;
constexpr int64_t kChainRedBytes = (int64_t)kChainWaves * 16 * kChainRedStride * 4;

hipError_t launch_chain(const void* table, int64_t L, int64_t T, int smem, const void* x0,
                        int x_is_bf16, void* ws, int64_t spin_limit, hipStream_t s);

}  // namespace bl
