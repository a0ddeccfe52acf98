// Workspace of bitlinear_pack (pack.hip writes and reads it; bitlinear_api.hip sizes it).
#pragma once
#include <stddef.h>
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

}  // namespace bl
