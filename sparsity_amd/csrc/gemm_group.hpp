// Device table of a grouped prefill (bitlinear_gemm_group_build writes it, gemm_big_group_kernel
// reads it): a header, one GemmGroupProj per projection, then one GemmGroupJob per block of the
// launch (padding jobs have proj == -1).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

constexpr uint32_t kGemmGroupMagic = 0x46474c42u;   // "BLGF"

struct GemmGroupHeader {
  uint32_t magic;
  int32_t layout, N, M;
  int32_t count, jobs;
  int64_t jobs_off;            // byte offset of the jobs from the table's start
  int64_t reserved[4];
};
static_assert(sizeof(GemmGroupHeader) == 64, "gemm group header is 64 bytes");

struct GemmGroupProj {
  const int8_t* xq;
  const float* xs;
  const uint32_t* codes;
  const uint32_t* meta;
  const float* gamma;
  float* y;
  int32_t* acc;
  int32_t T, Keff, n, npanels;
};
static_assert(sizeof(GemmGroupProj) == 72, "gemm group projection record is 72 bytes");

struct GemmGroupJob {
  int32_t proj, tm, tn, reserved;
};
static_assert(sizeof(GemmGroupJob) == 16, "gemm group job is 16 bytes");

// Tile shape of the prefill kernel (rows x tokens).
int gemm_group_tile_rows();
int gemm_group_tile_tokens();

hipError_t launch_gemm_group(const void* table, int64_t jobs, int layout, hipStream_t s);

}  // namespace bl
