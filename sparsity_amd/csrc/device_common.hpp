// Device helpers shared by the BitLinear kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kLayoutSparse = 0;
constexpr int kLayoutDense2 = 1;
constexpr int kPanel = 32;       // rows per packed panel (the M side of a 32x32 MFMA tile)
constexpr uint32_t kPadMeta = 0x44444444u;

// Expand one packed code dword (16 two-bit codes, slot i at bits 8*(i%4) + 2*(i/4)) into the
// 16 int8 values of an MFMA A operand: register q, byte p holds slot 4q + p.  Each register is
// one v_perm_b32 lookup: selector byte = code (0, 1 or 3) picks byte 0 (0x00), 1 (0x01) or
// 3 (0xFF) of the table operand.
__device__ __forceinline__ v4i expand_codes(uint32_t c) {
  const uint32_t table = 0xFF000100u;
  v4i r;
  r[0] = (int)__builtin_amdgcn_perm(0u, table, c & 0x03030303u);
  r[1] = (int)__builtin_amdgcn_perm(0u, table, (c >> 2) & 0x03030303u);
  r[2] = (int)__builtin_amdgcn_perm(0u, table, (c >> 4) & 0x03030303u);
  r[3] = (int)__builtin_amdgcn_perm(0u, table, (c >> 6) & 0x03030303u);
  return r;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace bl
