// Grouped decode GEMV: many independent sparse ternary projections (T <= 32 tokens each) in one
// launch, y = gamma * scale[t] * (xq . W_eff^T) for every projection of the group.
//
// A single decode projection is a few MB of packed weights, too little to cover the launch and
// memory latency of a kernel of its own; a group streams the weights of all its projections
// through one grid, so the chip sees one long HBM stream.  This is the shape of the independent
// projections of a decoder (Q/K/V, gate/up) and of a stream of layers whose activations are
// already quantized.
//
// Work item = up to 16 consecutive 32-row panels of one projection; wave w of the block owns panels
// w and w + 8 over the whole K axis, so no cross-wave reduction is needed, and every activation
// byte staged in LDS feeds two MFMAs per wave (at T = 16 the item's activation rows are a quarter
// of its weight bytes, read from L2 once per item).  The host lays the items out so
// that each XCD gets a contiguous run of the projections (their activation rows stay in that XCD's
// L2) and starts with its largest items.  K is walked in chunks of kGS MFMA steps:
//   - the wave's packed weights (one code and one meta dword per lane per step) are loaded straight
//     into a ring of kGD register chunks, kGD - 1 chunks ahead of the MFMAs, as non-temporal
//     loads: every weight byte is read once per launch, and marking the stream as such lifts the
//     launch from about 105 to 95 us at T = 1 on the 566 MB decode stream;
//   - the block's token rows for the chunk (T x kGS*KSTEP int8, at most one 16-byte load per
//     thread) ride in the same ring and are written to a double-buffered LDS tile one chunk ahead,
//     so the 8 waves share every activation byte they read from L2;
//   - the MFMAs read their B fragments from LDS (row stride + 16 bytes keeps 16 tokens' 16-byte
//     reads on distinct banks).
// Steps past the end of K re-read the last step with the code forced to 0 (zero weights add 0).
//
// Fused variant (tables built by bitlinear_group_fused_build): the projections hold bf16
// activations instead of int8 ones, and the kernel quantizes them itself (per-token absmax, BitNet
// b1.58 page, "The mechanism"), so a decode step needs no separate quantization launch.  Each work
// item first takes the absmax of its projection's T token rows (the rows are shared by all items
// of the projection and come from L2), then its token pieces ride the ring as bf16 and are
// quantized on their way into LDS with the very expression of act_quant_i8, so results are
// bit-identical to act_quant_i8 + the plain group.  Only unlifted layouts (2:4 SPARSE, DENSE2).
#include "device_common.hpp"
#include "launch.hpp"

namespace bl {

namespace {
constexpr int kGS = 4;  // MFMA steps per chunk
constexpr int kGD = 3;  // register ring depth in chunks (two panels per wave: 121 VGPRs, two
                        // blocks per CU)

typedef __attribute__((address_space(1))) const uint32_t g_u32;
typedef __attribute__((address_space(1))) const v4i g_v4i;
}  // namespace

// One chunk of the register ring: a wave's code/meta dwords for kGS steps and this thread's share
// of the block's token rows for the same K range (a 16-position piece: 16 int8 bytes, or 32 bytes
// of bf16 in the fused variant).
template <int BPT, int VPP>
struct GroupChunk {
  uint32_t c[kGS * kGroupPanelsPerWave], m[kGS * kGroupPanelsPerWave];   // [panel][step]
  v4i b[BPT * VPP];
};

template <int LAYOUT, bool FUSED>
struct GroupGemv {
  static constexpr bool SP = LAYOUT == kLayoutSparse;
  static constexpr int KSTEP = SP ? 64 : 32;           // K positions per MFMA step
  static constexpr int NT = 64 * kGroupWaves;
  static constexpr int CB = kGS * KSTEP;               // bytes of one token row per chunk
  static constexpr int ROW = CB + 16;                  // LDS row stride
  static constexpr int V16 = CB / 16;                  // 16-position pieces per token row per chunk
  static constexpr int BPT = (32 * V16 + NT - 1) / NT; // pieces per thread at T = 32
  static constexpr int VPP = FUSED ? 2 : 1;            // 16-byte loads per piece
  typedef GroupChunk<BPT, VPP> Chunk;

  int8_t* bs;             // LDS: two buffers of 32 rows x ROW bytes
  g_u32* cp[kGroupPanelsPerWave];   // this lane's code dword of step 0 of each of the wave's panels
  g_u32* mp[kGroupPanelsPerWave];
  int cs[kGroupPanelsPerWave];      // dwords between steps: 64, or 0 for a panel past the end
  __attribute__((address_space(1))) const int8_t* xq;   // int8 rows, or bf16 rows (fused)
  int tid, T, Keff, NF, nch, bpieces, brow, h;
  float qs[BPT];          // fused: 127 / absmax of the token row of each of this thread's pieces
  v16i acc[kGroupPanelsPerWave];

  // Every call issues the same number of loads (addresses clamped into the projection), so the
  // compiler waits for one chunk with a fixed vmcnt instead of draining the ring.  Clamped reads
  // past the end of K only meet steps whose code is forced to 0.
  __device__ __forceinline__ void issue(int j, Chunk& r) const {
#pragma unroll
    for (int p = 0; p < kGroupPanelsPerWave; ++p)
#pragma unroll
      for (int u = 0; u < kGS; ++u) {
        const int s = min(j * kGS + u, NF - 1);
        r.c[p * kGS + u] = __builtin_nontemporal_load(cp[p] + (size_t)s * cs[p]);
        r.m[p * kGS + u] = SP ? __builtin_nontemporal_load(mp[p] + (size_t)s * cs[p]) : kPadMeta;
      }
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      const int pc = tid + k * NT;
      const int row = min(pc / V16, T - 1), col = min(16 * (pc % V16) + j * CB, Keff - 16);
      const size_t e = (size_t)row * Keff + col;   // element offset of the piece
#pragma unroll
      for (int v = 0; v < VPP; ++v) r.b[k * VPP + v] = *(g_v4i*)(xq + e * VPP + 16 * v);
    }
  }
  // int8 bytes of one piece: as loaded, or (fused) 16 bf16 values quantized with the token's s
  __device__ __forceinline__ v4i piece(const Chunk& r, int k) const {
    if constexpr (!FUSED) {
      return r.b[k];
    } else {
      v4i out;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t w0 = (uint32_t)r.b[2 * k + d / 2][2 * (d % 2)];
        const uint32_t w1 = (uint32_t)r.b[2 * k + d / 2][2 * (d % 2) + 1];
        out[d] = (int)(q8(__uint_as_float(w0 << 16), qs[k]) |
                       (q8(__uint_as_float(w0 & 0xFFFF0000u), qs[k]) << 8) |
                       (q8(__uint_as_float(w1 << 16), qs[k]) << 16) |
                       (q8(__uint_as_float(w1 & 0xFFFF0000u), qs[k]) << 24));
      }
      return out;
    }
  }
  __device__ __forceinline__ void put(int j, const Chunk& r) const {
    int8_t* dst = bs + (j & 1) * (32 * ROW);
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      const int pc = tid + k * NT;
      if (pc < bpieces) *(v4i*)&dst[(pc / V16) * ROW + 16 * (pc % V16)] = piece(r, k);
    }
  }
  __device__ __forceinline__ void compute(int j, const Chunk& r) {
    const int8_t* xr = bs + (j & 1) * (32 * ROW) + brow * ROW + 16 * h;
#pragma unroll
    for (int u = 0; u < kGS; ++u) {
      const int4 blo = *(const int4*)(xr + u * KSTEP);
      const int4 bhi = SP ? *(const int4*)(xr + u * KSTEP + 32) : make_int4(0, 0, 0, 0);
      const bool live = j * kGS + u < NF;
#pragma unroll
      for (int p = 0; p < kGroupPanelsPerWave; ++p)
        acc[p] = mfma_step<SP>(live ? r.c[p * kGS + u] : 0u, r.m[p * kGS + u], blo, bhi, acc[p]);
    }
  }
  // chunk j: MFMAs from LDS buffer j & 1 (skipped past the end), chunk j + 1's rows to the other
  // buffer, chunk j + kGD's loads into the slot chunk j just freed, then one barrier.
  __device__ __forceinline__ void step(int j, Chunk& cur, const Chunk& nxt) {
    if (j < nch) compute(j, cur);
    put(j + 1, nxt);
    issue(j + kGD, cur);
    block_sync_lds();
  }
};

// At most 128 VGPRs (four waves per SIMD: two blocks per CU).  The fused variant needs a few more
// for its bf16 pieces and spills them outside the main loop only.
template <int LAYOUT, bool FUSED>
__global__ __launch_bounds__(64 * kGroupWaves) __attribute__((amdgpu_waves_per_eu(4)))
void gemv_group_kernel(
    const uint8_t* __restrict__ table) {
  typedef GroupGemv<LAYOUT, FUSED> G;
  __shared__ __attribute__((aligned(16))) int8_t bs[2 * 32 * G::ROW];
  __shared__ float tok_s[32], tok_scale[32];   // fused: 127 / absmax and absmax / 127 per token
  // epilogue staging: per wave one panel's outputs as [token][32 rows], rows padded to 36 floats
  constexpr int kStgRow = 36;
  __shared__ __attribute__((aligned(16))) float stg_all[kGroupWaves][32 * kStgRow];

  const GroupHeader* hdr = (const GroupHeader*)table;
  const int item = blockIdx.x;
  // uniform across the block: a table of another layout or kind, or a grid larger than the
  // table, does nothing
  if (hdr->magic != kGroupMagic || hdr->layout != LAYOUT || hdr->fused != (int)FUSED ||
      item >= hdr->items)
    return;
  const GroupItem it = ((const GroupItem*)(table + sizeof(GroupHeader) +
                                           hdr->count * sizeof(GroupLayer)))[item];
  if (it.layer == kGroupNoItem) return;
  const GroupLayer L = ((const GroupLayer*)(table + sizeof(GroupHeader)))[it.layer];

  G k;
  k.tid = threadIdx.x;
  const int lane = k.tid & 63, wave = k.tid >> 6;
  k.T = L.T;
  k.Keff = L.Keff;
  const int n = L.n;
  const int npanels = (n + kPanel - 1) / kPanel;
  k.NF = k.Keff / G::KSTEP;
  k.nch = (k.NF + kGS - 1) / kGS;
  int P[kGroupPanelsPerWave];
#pragma unroll
  for (int p = 0; p < kGroupPanelsPerWave; ++p) {
    P[p] = (int)it.panel0 + p * kGroupWaves + wave;
    // a panel past the projection re-reads one step of the last real panel at every step (a
    // cache hit: the loads of every chunk stay the same in number) and stores nothing
    const int Pl = min(P[p], npanels - 1);
    k.cp[p] = (g_u32*)L.codes + (size_t)Pl * k.NF * 64 + lane;
    k.mp[p] = G::SP ? (g_u32*)L.meta + (size_t)Pl * k.NF * 64 + lane : nullptr;
    k.cs[p] = P[p] < npanels ? 64 : 0;
  }
  k.xq = (__attribute__((address_space(1))) const int8_t*)L.xq;
  k.bs = bs;
  k.bpieces = k.T * G::V16;
  const int tok = lane & 31;
  k.h = lane >> 5;
  k.brow = min(tok, k.T - 1);                // dead token lanes read a live row
  const float gamma = *(__attribute__((address_space(1))) const float*)L.gamma;
  if constexpr (FUSED) {
    // absmax of each token row over all K (max of the |x| bit patterns: exact, order free), one
    // wave per row, 8 bf16 per lane per load; then the two scales exactly as act_quant_i8 forms
    // them
    for (int t = wave; t < k.T; t += kGroupWaves) {
      g_v4i* rowp = (g_v4i*)(k.xq + (size_t)t * k.Keff * 2);
      uint32_t mx = 0;
#pragma unroll 4
      for (int c = lane; c < k.Keff / 8; c += 64) {
        const v4i u = rowp[c];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t w = (uint32_t)u[q];
          mx = max(mx, max(w & 0x7FFFu, (w >> 16) & 0x7FFFu));
        }
      }
      mx = wave_max_u32(mx);
      if (lane == 0) {
        const float amax = __uint_as_float(mx << 16);
        tok_s[t] = amax > 0.f ? 127.f / amax : 0.f;
        tok_scale[t] = amax / 127.f;
      }
    }
    block_sync_lds();
#pragma unroll
    for (int q = 0; q < G::BPT; ++q) k.qs[q] = tok_s[min((k.tid + q * G::NT) / G::V16, k.T - 1)];
  }
  const float sc = FUSED ? tok_scale[k.brow]
                         : *((__attribute__((address_space(1))) const float*)L.xs + k.brow);

  typename G::Chunk r[kGD];
  // chunk by chunk, in the loop's issue order: the wait for a chunk in the loop is then the same
  // count on the first pass as on every later one (otherwise the compiler takes the smaller one)
#pragma unroll
  for (int q = 0; q < kGD; ++q) {
    k.issue(q, r[q]);
    asm volatile("" ::: "memory");
  }

  k.put(0, r[0]);
  block_sync_lds();
#pragma unroll
  for (int p = 0; p < kGroupPanelsPerWave; ++p) k.acc[p] = v16i{};
  // nch rounded up to the ring depth: the trailing chunks skip their MFMAs, not their loads
  for (int j = 0; j < k.nch; j += kGD) {
#pragma unroll
    for (int q = 0; q < kGD; ++q) k.step(j + q, r[q], r[(q + 1) % kGD]);
  }
  const int h = k.h;
  const bool vec = (n & 3) == 0;
  // A lane holds rows 8g + 4h + i of its token, so storing from the registers writes 32-byte
  // pieces of T token rows per instruction.  A full panel (32 rows inside y, 16-byte aligned rows,
  // no acc output) is first written to the wave's staging region and read back as whole 128-byte
  // token-row lines, eight tokens per store instruction, stored non-temporally (the T = 16 launch
  // 3-4% faster; staged lines stored normally, or the pieces stored non-temporally, were slower).
  float* stg = stg_all[wave];
#pragma unroll
  for (int p = 0; p < kGroupPanelsPerWave; ++p) {
    if (P[p] >= npanels) break;
    if (vec && !L.acc && (P[p] + 1) * kPanel <= n) {
      if (tok < k.T) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          v4f v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = ((float)k.acc[p][4 * g + i] * gamma) * sc;
          *(v4f*)&stg[tok * kStgRow + 8 * g + 4 * h] = v;
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      for (int t0 = 0; t0 < k.T; t0 += 8) {
        const int tt = t0 + (lane >> 3), c4 = 4 * (lane & 7);
        if (tt < k.T) {
          const v4f v = *(const v4f*)&stg[tt * kStgRow + c4];
          float* dst = L.y + (size_t)tt * n + P[p] * kPanel + c4;
          __builtin_nontemporal_store(v, (v4f*)dst);
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      continue;
    }
    if (tok >= k.T) continue;
    const v16i acc = k.acc[p];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int o = P[p] * kPanel + 8 * g + 4 * h;
      const size_t idx = (size_t)tok * n + o;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = ((float)acc[4 * g + i] * gamma) * sc;
      if (vec && o + 3 < n) {
        *(float4*)(L.y + idx) = make_float4(v[0], v[1], v[2], v[3]);
        if (L.acc)
#pragma unroll
          for (int i = 0; i < 4; ++i) L.acc[idx + i] = acc[4 * g + i];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (o + i < n) {
            L.y[idx + i] = v[i];
            if (L.acc) L.acc[idx + i] = acc[4 * g + i];
          }
      }
    }
  }
}

hipError_t launch_fwd_group(const void* table, int64_t items, int layout, int fused,
                            hipStream_t s) {
  const dim3 grid((unsigned)items), block(64 * kGroupWaves);
  const uint8_t* t = (const uint8_t*)table;
  if (layout == kLayoutSparse) {
    if (fused) gemv_group_kernel<kLayoutSparse, true><<<grid, block, 0, s>>>(t);
    else gemv_group_kernel<kLayoutSparse, false><<<grid, block, 0, s>>>(t);
  } else {
    if (fused) gemv_group_kernel<kLayoutDense2, true><<<grid, block, 0, s>>>(t);
    else gemv_group_kernel<kLayoutDense2, false><<<grid, block, 0, s>>>(t);
  }
  return hipGetLastError();
}

}  // namespace bl
