// Host-side launchers of the BitLinear kernels.  Arguments are validated by the C ABI layer
// (bitlinear_api.hip) before any of these is called; each returns the hipError_t of its launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

// Workspace of bitlinear_pack: a fixed part (PackWs) and, after it, one band region per pack tile
// (kTileEntries entries), so its size grows with the master: 512 bytes per 8192 weights.
constexpr int kGammaBlocks = 1024;    // fp64 sum slots of |W| per master
constexpr int kGammaThreads = 256;
constexpr int kExactWords = 9;
constexpr int kExactBlocks = 256;     // exact-pass blocks per master (one per CU)
constexpr int kExactGroups = 8;       // arrival counter groups (block b counts in group b % 8)
constexpr int kSampleBlocks = 128;    // blocks of the sampling launch per master
constexpr int kSampleStats = 5;       // per sampling block: sums of s, s^2, s*c, c, c^2
constexpr int kTileEntries = 64;      // band entries one pack tile can list
constexpr int kFixBlocks = 256;       // blocks of the fix-up launch per master
constexpr int kNoallocTiles = 8192;   // band regions of the static workspace (67 M weights)

struct PackWs {
  // fp64 sums of |w|: pack tile t adds its tile's sum into partial[t % kGammaBlocks]
  double partial[kGammaBlocks];
  // exact fallback: block b's word sums (sum_i slot[b][i] * 2^(32 i) units of 2^-149), one
  // 128-byte line per block, written with plain stores: no two blocks touch one line
  unsigned long long slot[kExactBlocks][16];
  // arrival counters, one line each: block b counts in group b % kExactGroups; the last block of
  // a group counts in done_all (at most kExactBlocks / kExactGroups atomics queue on one line)
  uint32_t done_grp[kExactGroups][32];
  uint32_t done_all, pad[31];
  float gamma, tau;                  // gamma and the ternary threshold
  uint32_t exact_used;               // 1 when the exact fallback decided gamma (diagnostic)
  uint32_t fix_mode;                 // 0: listed codes set; 1: every tile repacked (diagnostic)
  float tau_lo, tau_hi;              // the coding band of the one-pass pack
  uint32_t band_ok;                  // the band is usable (finite, positive, narrow, regions)
  uint32_t overflow;                 // some tile listed more than kTileEntries weights
  uint32_t pad2[24];
  double sample[kSampleStats][kSampleBlocks];     // the sampling launch's per-block sums
};
constexpr size_t kPackWsFixed = (sizeof(PackWs) + 255) / 256 * 256;

// The band regions follow the fixed part: kTileEntries entries of 8 bytes per tile.
constexpr size_t pack_ws_entries_off() { return kPackWsFixed; }
constexpr size_t pack_ws_bytes_for_tiles(int64_t tiles) {
  return kPackWsFixed + (size_t)tiles * kTileEntries * 8;
}
constexpr size_t kPackWsBytes = pack_ws_bytes_for_tiles(kNoallocTiles);   // the static workspace

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
