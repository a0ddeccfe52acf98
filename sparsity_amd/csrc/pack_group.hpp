// Device table of a grouped pack (bitlinear_pack_group_build writes it, the five grouped pack
// launches read it): a header, then one item per master in descriptor order.  Sampling block b
// serves item b / kSampleBlocks, band block b item b, fix-up block b item b / kFixBlocks; pass
// blocks are dealt to the items in reverse order, item count - 1 first, and item i owns pass
// blocks [block0, block0 + its tile count).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

constexpr uint32_t kPackGroupMagic = 0x50474c42u;   // "BLGP"

struct PackGroupHeader {
  uint32_t magic;
  int32_t layout, N, M;
  int32_t count, pack_blocks;
  int64_t reserved[5];
};
static_assert(sizeof(PackGroupHeader) == 64, "pack group header is 64 bytes");

struct PackGroupItem {
  const float* W;        // [n][K] fp32 master
  uint32_t* codes;
  uint32_t* meta;        // NULL for DENSE2
  float* gamma;
  void* ws;              // this master's workspace (partial sums), inside the group's workspace
  int32_t n, K, k_tiles, block0;
  int64_t reserved;
};
static_assert(sizeof(PackGroupItem) == 64, "pack group item is 64 bytes");

hipError_t launch_pack_group(const void* table, int64_t count, int64_t pack_blocks, int layout,
                             int M, hipStream_t s);

}  // namespace bl
