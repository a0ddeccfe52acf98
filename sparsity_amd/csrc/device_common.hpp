// Device helpers shared by the BitLinear kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Group sizes M of the N:M masks: 2:4, and (M-2):M for even M = 6..16 as M/2 - 1 overlapping 2:4
// windows (SlideSparse abstract, Sliding Window Decomposition: (2N-2):2N into N-1 windows).
// Calls f(std::integral_constant<int, M>{}) for a supported M; false otherwise.
template <class F>
inline bool dispatch_m(int M, F&& f) {
  switch (M) {
    case 4: f(std::integral_constant<int, 4>{}); return true;
    case 6: f(std::integral_constant<int, 6>{}); return true;
    case 8: f(std::integral_constant<int, 8>{}); return true;
    case 10: f(std::integral_constant<int, 10>{}); return true;
    case 12: f(std::integral_constant<int, 12>{}); return true;
    case 14: f(std::integral_constant<int, 14>{}); return true;
    case 16: f(std::integral_constant<int, 16>{}); return true;
    default: return false;
  }
}

constexpr int gcd_i(int a, int b) { return b ? gcd_i(b, a % b) : a; }
constexpr int lcm_i(int a, int b) { return a / gcd_i(a, b) * b; }

// Dense K columns of one pack tile (at most 256): whole M-groups, and whole 32-slot fragments of
// the packed row (SPARSE: (M-2)/M slots per column, 2:4 one per two; DENSE2: one per column).
constexpr int pack_cols(int layout, int M) {
  int best = 0;
  for (int kb = M; kb <= 256; kb += M) {
    const int slots = layout == 0 ? (M == 4 ? kb / 2 : kb / M * (M - 2)) : kb;
    if (slots % 32 == 0) best = kb;
  }
  return best;
}

constexpr int kLayoutSparse = 0;
constexpr int kLayoutDense2 = 1;
constexpr int kLayoutSparse6 = 2;   // 2:4 re-encoded at 6 bits per group (decode only)
constexpr int kPanel = 32;       // rows per packed panel (the M side of a 32x32 MFMA tile)
constexpr uint32_t kPadMeta = 0x44444444u;

// Expand one packed code dword (16 two-bit codes, slot i at bits 8*(i%4) + 2*(i/4); 00 = 0,
// 01 = +1, 10 = -1) into the 16 int8 values of an MFMA A operand: register q, byte p holds slot
// 4q + p.  Each register is one v_perm_b32 byte lookup on a masked selector; a selector byte 0..7
// picks a byte of {src0, src1} (0-3 from src1, 4-7 from src0) and 8 replicates bit 15 of src1.
//   q = 0, 2: selector = code (0, 1, 2)      -> src1 bytes 0, 1, 2 = 0x00, 0x01, 0xFF
//   q = 1, 3: selector = code << 2 (0, 4, 8) -> src1 byte 0 (0x00), src0 byte 0 (0x01), or
//             bit 15 of src1 (set: 0xFF)
// Nine VALU instructions per dword: one shift, four masks, four permutes.
__device__ __forceinline__ v4i expand_codes(uint32_t c) {
  const uint32_t t_even = 0x00FF0100u;   // src1 of the q = 0, 2 lookups
  const uint32_t t_odd1 = 0x00008000u;   // src1 of the q = 1, 3 lookups (byte 0 = 0, bit 15 set)
  const uint32_t t_odd0 = 0x00000001u;   // src0 of the q = 1, 3 lookups (byte 0 = +1)
  const uint32_t c4 = c >> 4;
  v4i r;
  r[0] = (int)__builtin_amdgcn_perm(0u, t_even, c & 0x03030303u);
  r[1] = (int)__builtin_amdgcn_perm(t_odd0, t_odd1, c & 0x0C0C0C0Cu);
  r[2] = (int)__builtin_amdgcn_perm(0u, t_even, c4 & 0x03030303u);
  r[3] = (int)__builtin_amdgcn_perm(t_odd0, t_odd1, c4 & 0x0C0C0C0Cu);
  return r;
}

// One 32x32 int8 MFMA step of a panel: A = the expanded code dword (16 int8 per lane), B = the
// token fragment (SPARSE: 32 bytes per lane covering 64 K positions, with `meta` as the sparse
// instruction's index operand; DENSE2: 16 bytes per lane covering 32 K positions).
template <bool SP>
__device__ __forceinline__ v16i mfma_step(uint32_t code, uint32_t meta, const int4& blo,
                                          const int4& bhi, v16i acc) {
  const v4i a = expand_codes(code);
  if constexpr (SP) {
    v8i b;
    b[0] = blo.x; b[1] = blo.y; b[2] = blo.z; b[3] = blo.w;
    b[4] = bhi.x; b[5] = bhi.y; b[6] = bhi.z; b[7] = bhi.w;
    return __builtin_amdgcn_smfmac_i32_32x32x64_i8(a, b, acc, (int)meta, 0, 0);
  } else {
    v4i b;
    b[0] = blo.x; b[1] = blo.y; b[2] = blo.z; b[3] = blo.w;
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc, 0, 0, 0);
  }
}

// One activation onto the int8 grid: clamp(rint(fl32(v * s)), -127, 127) with round-half-even,
// as an unsigned byte.  s = fl32(127 / absmax) of the token (BitNet b1.58 page, "The mechanism",
// per-token absmax quantization to [-Qb, Qb]).
__device__ __forceinline__ uint32_t q8(float v, float s) {
  float r = rintf(v * s);
  r = fminf(fmaxf(r, -127.f), 127.f);
  return (uint32_t)(int32_t)r & 0xFFu;
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

// Workgroup barrier without the memory fence __syncthreads adds: the fence makes the compiler drain
// every outstanding global load (vmcnt(0)), which would empty a prefetch ring at each barrier.
// The "memory" clobber still keeps the compiler from moving memory accesses across it; callers
// wait for their own LDS writes (block_sync_lds) or LDS DMA (explicit vmcnt) first.
__device__ __forceinline__ void block_barrier_nofence() {
  asm volatile("s_barrier" ::: "memory");
}

// s_waitcnt immediate for gfx9: vmcnt in bits 3:0 and 15:14, expcnt 6:4 (7 = no wait), lgkmcnt
// 11:8 (15 = no wait).
constexpr int waitcnt_imm(int vm, int lgkm = 15) {
  return (vm & 0xF) | (((vm >> 4) & 3) << 14) | (7 << 4) | ((lgkm & 0xF) << 8);
}

// Barrier after plain LDS writes: this wave's LDS operations complete, then all waves meet.
// Outstanding global loads stay in flight.
__device__ __forceinline__ void block_sync_lds() {
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  block_barrier_nofence();
}

typedef __attribute__((address_space(3))) int8_t lds_i8;
__device__ __forceinline__ uint32_t lds_offset(const void* p) { return (uint32_t)(uintptr_t)(lds_i8*)p; }

// global_load_lds_dwordx4 issued as inline asm: 16 bytes per lane from `src` to LDS at
// m0 + 16 * lane.  It writes no VGPR, so nothing can consume a register before the data lands;
// completion is tracked by the caller's explicit vmcnt waits.  (Issued through the builtin, the
// compiler cannot prove the in-flight loads miss the buffer being read and drains them all before
// every LDS read, which serializes the pipeline.)  One wait state separates the m0 write from
// its use.
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(m0), "v"(src) : "memory", "m0");
}
// Same, scalar base + per-lane 32-bit byte offset (no VALU address arithmetic per load).
__device__ __forceinline__ void lds_dma16_s(const void* sbase, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(m0), "v"(voff), "s"(sbase) : "memory", "m0");
}

}  // namespace bl
