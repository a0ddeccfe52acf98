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

// Workspace (uint32 words): [0] arrivals at the grid barrier (every block adds 1 per phase),
// [1] error flag (a bounded barrier wait gave up), [2..63] unused, then
// pmax[(L + 1)][kChainBlocks][T]: each block's max |x| bit pattern per token of each layer's
// input (layer l's input is layer l - 1's y); the layer's absmax is the max over the blocks.
constexpr int kChainWsHead = 64;

inline size_t chain_ws_bytes(int64_t L, int64_t T) {
  return ((size_t)kChainWsHead + (size_t)(L + 1) * kChainBlocks * T) * 4;
}

// Dynamic LDS of a layer: its int8 input rows (T x (K + 16)), then the waves' int32 partials.
constexpr int64_t kChainRedBytes = (int64_t)kChainWaves * 16 * 64 * 4;

hipError_t launch_chain(const void* table, int64_t L, int64_t T, int smem, const void* x0,
                        int x_is_bf16, void* ws, int64_t spin_limit, hipStream_t s);

}  // namespace bl
