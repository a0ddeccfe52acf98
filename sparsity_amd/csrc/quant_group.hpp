// Grouped activation quantization (act_quant_i8_group): the arguments of up to kQuantGroupMax
// act_quant_i8 calls, passed by value as one kernel argument, so the launch needs no device table.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

constexpr int kQuantGroupMax = 16;

struct QuantGroupArgs {
  const void* x[kQuantGroupMax];     // [T][K] bf16 or fp32 rows
  int8_t* xq[kQuantGroupMax];        // [T][K_eff] int8
  float* xs[kQuantGroupMax];         // [T] token scales
  int32_t T[kQuantGroupMax], K[kQuantGroupMax];
  int32_t block0[kQuantGroupMax + 1];   // first block of each matrix (4 tokens per block); the
                                        // last entry is the grid size
  int32_t count;                     // matrices with tokens, in launch order
};

// One launch for the whole group (matrices whose rows exceed the register budget of the
// one-wave-per-token kernel make it fall back to one launch per matrix).
hipError_t launch_act_quant_group(const QuantGroupArgs& a, int x_is_bf16, int lift_M,
                                  hipStream_t s);

}  // namespace bl
