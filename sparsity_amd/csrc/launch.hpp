// Host-side launchers of the BitLinear kernels.  Arguments are validated by the C ABI layer
// (bitlinear_api.hip) before any of these is called; each returns the hipError_t of its launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

// ws holds band regions for tiles_cap tiles (fewer than the master's tiles: no band, two passes).
hipError_t launch_pack(const float* W, int64_t n, int64_t K, int N, int M, int layout,
                       uint32_t* codes, uint32_t* meta, float* gamma, void* ws, int64_t tiles_cap,
                       hipStream_t s);

// bitlinear_pack with the library's static per-device workspace (no caller workspace).
hipError_t launch_pack_noalloc(const float* W, int64_t n, int64_t K, int N, int M, int layout,
                               uint32_t* codes, uint32_t* meta, float* gamma, hipStream_t s);
size_t pack_noalloc_capacity();   // bytes of that workspace

hipError_t launch_act_quant(const void* x, int x_is_bf16, int64_t T, int64_t K, int lift_M,
                            int8_t* xq, float* x_scale, hipStream_t s);

hipError_t launch_fwd(const int8_t* xq, const float* x_scale, int64_t T, int64_t Keff,
                      const uint32_t* codes, const uint32_t* meta, const float* gamma, int layout,
                      int64_t n, float* y, int32_t* acc_opt, hipStream_t s);

}  // namespace bl

namespace bl {

// Device table of a group of independent decode projections (bitlinear_group_build writes it,
// gemv_group_kernel reads it): a header, one GroupLayer per projection, then one GroupItem per
// work item in launch order.  A work item is up to kGroupPanels consecutive 32-row panels of one
// projection: wave w of the block takes panels w and w + kGroupWaves.
constexpr int kGroupWaves = 8;
constexpr int kGroupPanelsPerWave = 2;
constexpr int kGroupPanels = kGroupWaves * kGroupPanelsPerWave;
constexpr int kXcds = 8;                       // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr uint32_t kGroupMagic = 0x32474c42u;  // "BLG2"
constexpr uint32_t kGroupNoItem = 0xFFFFFFFFu; // padding item: its block does nothing

struct GroupHeader {
  uint32_t magic;
  int32_t layout, N, M;
  int64_t count, items;
  int32_t fused;          // 1: layers hold bf16 activations, quantized inside the kernel
  int32_t pad;
  int64_t reserved[3];
};
static_assert(sizeof(GroupHeader) == 64, "group table header is 64 bytes");

struct GroupLayer {
  const int8_t* xq;       // int8 activations, or (fused) bf16 activations [T][K]
  const float* xs;        // token scales (not used by fused tables)
  const uint32_t* codes;
  const uint32_t* meta;
  const float* gamma;
  float* y;
  int32_t* acc;
  int32_t T, Keff, n, reserved;
};
static_assert(sizeof(GroupLayer) == 72, "group layer record is 72 bytes");

struct GroupItem {
  uint32_t layer;   // projection index, or kGroupNoItem
  uint32_t panel0;  // first 32-row panel of the item
};

hipError_t launch_fwd_group(const void* table, int64_t items, int layout, int fused,
                            hipStream_t s);

// SPARSE6: re-encoding of 2:4 packed buffers, the single-projection decode (T <= 32, K <= 16384)
// and the grouped decode over a table built for layout SPARSE6.
hipError_t launch_transcode6(const uint32_t* codes, const uint32_t* meta, int64_t n, int64_t K,
                             uint32_t* out, hipStream_t s);
hipError_t launch_fwd6(const int8_t* xq, const float* xs, int64_t T, int64_t K,
                       const uint32_t* stream, const float* gamma, int64_t n, float* y,
                       int32_t* acc, hipStream_t s);
hipError_t launch_fwd6_group(const void* table, int64_t items, hipStream_t s);

}  // namespace bl

namespace bl {

// Workspace of bitlinear_bwd, in bytes from its start (segments 256-byte aligned):
//   wt  [K][n32] bf16   W_eff^T (dX only)
//   dyp [T][n32] bf16   dY with rows zero-padded to n32 (dX only, when n % 32 != 0)
//   dyt [n][t32] bf16   dY^T, tokens zero-padded to t32 (dW only)
//   xt  [K][t32] bf16   X^^T (dW only)
// n32 and t32 are n and T rounded up to multiples of 32.
struct BwdWorkspace {
  int64_t n32, t32;
  size_t wt_off, dyp_off, dyt_off, xt_off, total;
};

inline BwdWorkspace bwd_workspace(int64_t T, int64_t n, int64_t K) {
  auto up = [](size_t v, size_t a) { return (v + a - 1) / a * a; };
  BwdWorkspace w;
  w.n32 = (n + 31) / 32 * 32;
  w.t32 = (T + 31) / 32 * 32;
  size_t off = 0;
  w.wt_off = off;  off = up(off + (size_t)K * w.n32 * 2, 256);
  w.dyp_off = off; off = up(off + (w.n32 != n ? (size_t)T * w.n32 * 2 : 0), 256);
  w.dyt_off = off; off = up(off + (size_t)n * w.t32 * 2, 256);
  w.xt_off = off;  off = up(off + (size_t)K * w.t32 * 2, 256);
  w.total = off;
  return w;
}

hipError_t launch_bwd(const uint16_t* dy, int64_t T, int64_t n, const int8_t* xq,
                      const float* x_scale, int64_t K, const uint32_t* codes, const uint32_t* meta,
                      const float* gamma, int N, int M, int layout, float* dx, float* dw, int flags,
                      void* ws, hipStream_t s);

}  // namespace bl
