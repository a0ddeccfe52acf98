// Fused decode over a chain of dependent BitLinear layers: layer l + 1 reads layer l's output.
//
// In a decoder each layer's input is the previous layer's output, so a layer's per-token int8
// quantization (BitNet b1.58 page, "The mechanism": absmax per token onto [-127, 127]) can only
// start when the previous layer has finished, and a decode step of separate launches pays one
// quantization launch and one GEMV launch per layer, each a few microseconds of launch and
// memory latency for a few MB of weights.  Here one persistent launch runs the whole chain:
//
//   phase 0      every block takes the max |x| per token over a slice of the first layer's input
//                columns (integer max of the bit patterns: exact and order-free) and stores it
//                in its own slot
//   layer l      a team of S waves shares a 32-row panel (S = 1, 2, 4 or 8: the fewest that keep
//                a wave's share of the K steps within its register budget), so a block of 8
//                waves holds 8 / S panels at a time; the teams load their panels' packed weights
//                first -- they do not depend on the previous layer -- then the block waits at the
//                grid barrier for layer l - 1, takes the per-token absmax as the max of every
//                block's slot, forms the token scales (act_quant_i8's expressions), quantizes the
//                input rows into LDS once (act_quant_i8's expression; for a large input, T x K x 4
//                bytes above kChainSplitBytes, every block quantizes a slice into an int8 copy in
//                the workspace and, after one more grid barrier, copies the int8 rows into LDS
//                instead of reading all of the fp32 rows), and each team runs the
//                sparse MFMAs, sums its waves' int32 partials in LDS in a fixed order, writes
//                y = fl32(fl32(acc * gamma) * scale_t) and keeps the max |y| per token; the block
//                stores its max in its slot for layer l + 1.  With the decode shapes every panel
//                of a layer fits one round of the 64 blocks.
//
// so every layer's y (and int32 accumulators) are bit-identical to act_quant_i8 on the previous
// layer's y followed by bitlinear_fwd.  The grid barrier is a counter every block increments
// once per barrier (after a release fence at agent scope, so its outputs are visible on every XCD)
// and thread 0 of every block polls (then an acquire fence).  The launch is cooperative
// (all blocks resident), and every wait is bounded: after spin_limit polls the block raises the
// workspace's error flag and returns, so a failure ends the kernel instead of hanging it.
#include "chain.hpp"
#include "device_common.hpp"

namespace bl {

namespace {
typedef __attribute__((address_space(1))) const uint32_t g_u32;
typedef __attribute__((address_space(1))) const v4i g_v4i;
typedef __attribute__((address_space(1))) const v4f g_v4f;
}  // namespace

// Bounded wait until `target` arrivals; returns false (after raising the error flag) on timeout.
__device__ __forceinline__ bool chain_wait(uint32_t* ws, uint32_t target, int64_t spin_limit,
                                           int* go_sh) {
  if (threadIdx.x == 0) {
    int go = 1;
    int64_t spins = 0;
    while (__hip_atomic_load(ws, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > spin_limit) {
        __hip_atomic_fetch_or(ws + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        go = 0;
        break;
      }
    }
    *go_sh = go;
    // one acquire for the block: it invalidates this CU's vector cache and the XCD's L2 for every
    // wave, whose later loads the barrier orders after it (a fence in every wave costs as many
    // invalidations)
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  return *go_sh != 0;
}

// This block's outputs of the phase are complete (every wave waited for its stores at the
// barrier); make them visible device-wide, then arrive.
__device__ __forceinline__ void chain_arrive(uint32_t* ws) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");   // this wave's stores are performed
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_fetch_add(ws, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// max |x| bit pattern of 8 bf16 (one 16-byte piece) or 4 fp32 values
__device__ __forceinline__ uint32_t absbits_max_bf16x8(const v4i u) {
  uint32_t m = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t w = (uint32_t)u[q];
    m = max(m, max((w & 0x7FFFu) << 16, w & 0x7FFF0000u));
  }
  return m;
}

template <bool X0_BF16>
__global__ __launch_bounds__(64 * kChainWaves) void chain_kernel(const uint8_t* __restrict__ table,
                                                               const void* __restrict__ x0,
                                                               uint32_t* __restrict__ ws,
                                                               int64_t spin_limit) {
  extern __shared__ __attribute__((aligned(16))) int8_t sm[];
  __shared__ float tok_s[kChainMaxT], tok_scale[kChainMaxT];
  __shared__ uint32_t tok_in[kChainMaxT], tok_out[kChainMaxT];
  __shared__ int go_sh;

  const ChainHeader* hd = (const ChainHeader*)table;
  if (hd->magic != kChainMagic) return;
  const ChainLayer* layers = (const ChainLayer*)(table + sizeof(ChainHeader));
  const int L = hd->L, T = hd->T;
  const int G = gridDim.x, blk = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // per-block partial max |x| of every layer's input: pmax[(l * G + block) * T + t]
  uint32_t* pmax = ws + kChainWsHead;
  // int8 input rows of a split layer
  int8_t* xq = (int8_t*)ws + chain_xq_offset(L, T);
  uint32_t gen = 0;                              // this block's arrivals so far (the same in every block)

  // ---- phase 0: partial per-token absmax of the first layer's input, column slices ----
  {
    const int K0 = layers[0].K;
    constexpr int PE = X0_BF16 ? 8 : 4;          // elements per 16-byte piece
    const int pieces = K0 / PE;
    for (int t = wave; t < T; t += kChainWaves) {
      uint32_t mx = 0;
      for (int p = blk * 64 + lane; p < pieces; p += G * 64) {
        const size_t e = (size_t)t * K0 + (size_t)p * PE;
        if constexpr (X0_BF16) {
          mx = max(mx, absbits_max_bf16x8(*(g_v4i*)((const uint16_t*)x0 + e)));
        } else {
          const v4f v = *(g_v4f*)((const float*)x0 + e);
#pragma unroll
          for (int q = 0; q < 4; ++q) mx = max(mx, __float_as_uint(v[q]) & 0x7FFFFFFFu);
        }
      }
      mx = wave_max_u32(mx);
      if (lane == 0) pmax[(size_t)blk * T + t] = mx;
    }
  }
  chain_arrive(ws);
  gen = 1;

  const int tok = lane & 31, h = lane >> 5;
  // layer records are read-only: each is read one layer ahead, before the wait that invalidates
  // the caches, so the barrier's acquire fence does not put a memory round trip in front of it
  ChainLayer Lnext = layers[0];
  const float* yin = (const float*)x0;           // this layer's fp32 input (layer 0: x0)
  for (int l = 0; l < L; ++l) {
    const ChainLayer Ly = Lnext;
    if (l + 1 < L) Lnext = layers[l + 1];
    const int K = Ly.K, n = Ly.n;
    const int NF = K / 64;
    // a team of S waves shares a panel (S the smallest power of two giving each wave at most
    // kChainMaxSteps K steps); the block's 8 / S teams take panels team0, team0 + teams, ...
    const int S = NF <= kChainMaxSteps ? 1 : NF <= 2 * kChainMaxSteps ? 2
                : NF <= 4 * kChainMaxSteps ? 4 : 8;
    const int tpb = kChainWaves / S;             // teams per block
    const int team = wave / S, wt = wave % S;    // this wave's team and its place in it
    const int per = (NF + S - 1) / S;
    const int s_begin = min(wt * per, NF - 1);
    const int cnt = min(per, NF - wt * per);     // <= 0 for trailing waves of a team
    const int npanels = (n + kPanel - 1) / kPanel;
    const int stride = K + 16;                   // LDS row stride of the staged int8 input
    int* red = (int*)(sm + ((T * stride + 15) & ~15));   // per-wave int32 partials
    g_u32* cbase = (g_u32*)Ly.codes + lane;
    g_u32* mbase = (g_u32*)Ly.meta + lane;
    const int P0 = blk * tpb + team, Pstep = G * tpb;

    uint32_t c0[kChainMaxSteps], m0[kChainMaxSteps];
    // Only the 4-step groups that hold this wave's steps (u < cnt) are read, and multiplied
    // below: the loads a wave has in flight at the barrier stay few (the poll's result returns
    // after them), and no matrix-core time goes to all-zero steps.
    auto load = [&](int P, uint32_t (&c)[kChainMaxSteps], uint32_t (&m)[kChainMaxSteps]) {
#pragma unroll
      for (int g = 0; g < kChainMaxSteps / 4; ++g) {
        if (4 * g >= cnt) break;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int u = 4 * g + v;
          const size_t off = ((size_t)P * NF + min(s_begin + u, NF - 1)) * 64;
          c[u] = __builtin_nontemporal_load(cbase + off);
          m[u] = __builtin_nontemporal_load(mbase + off);
        }
      }
    };
    // the first panel's weights and gamma before the wait: they do not depend on the previous
    // layer
    if (P0 < npanels) load(P0, c0, m0);
    const float gamma = *(__attribute__((address_space(1))) const float*)Ly.gamma;

    // layer l - 1 (or phase 0) complete: every block has made `gen` arrivals
    if (!chain_wait(ws, gen * (uint32_t)G, spin_limit, &go_sh)) return;
    // The per-token absmax (max over every block's slot) and the input rows both come from the
    // previous layer: their loads go out together, then the scales are formed and the rows
    // quantized (act_quant_i8's expression) into LDS (rows t < T, stride K + 16), once for all
    // of the block's panels.  A layer with a large input splits this (kChainSplitBytes): each
    // block quantizes a 1/G slice of the rows into the workspace's int8 rows, and after one more
    // grid barrier every block with panels copies the int8 rows into LDS.
    // 8 positions per piece: 8 fp32 (two 16-byte loads) or 8 bf16 (one).
    const bool has_work = blk * tpb < npanels;   // uniform: the block has at least one panel
    const bool split = (int64_t)T * K * 4 > kChainSplitBytes;   // uniform: the same in every block
    const int ppr = K / 8;                       // pieces per row
    const int per_blk = (T * ppr + G - 1) / G;   // split: pieces per block's slice
    const int pbase = split ? blk * per_blk : 0;
    const int pieces = split ? max(0, min(per_blk, T * ppr - pbase)) : has_work ? T * ppr : 0;
    constexpr int U = 2;                         // pieces in flight per thread
    constexpr int NT = 64 * kChainWaves;
    v4i raw[U][2];
    auto issue = [&](int b0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int pc = pbase + min(b0 + u * NT, pieces - 1);
        const int t = pc / ppr, k = 8 * (pc % ppr);
        const size_t e = (size_t)t * K + k;
        if (l == 0 && X0_BF16) {
          raw[u][0] = *(g_v4i*)((const uint16_t*)x0 + e);
        } else {
          raw[u][0] = *(g_v4i*)(yin + e);
          raw[u][1] = *(g_v4i*)(yin + e + 4);
        }
      }
    };
    if (tid < kChainMaxT) { tok_in[tid] = 0u; tok_out[tid] = 0u; }
    uint32_t pm[(kChainBlocks * kChainMaxT + NT - 1) / NT];
#pragma unroll
    for (int j = 0; j < (kChainBlocks * kChainMaxT + NT - 1) / NT; ++j) {
      const int i = tid + j * NT;
      pm[j] = i < G * T ? pmax[((size_t)l * G) * T + i] : 0u;
    }
    if (pieces > 0) issue(tid);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < (kChainBlocks * kChainMaxT + NT - 1) / NT; ++j)
      if (pm[j]) atomicMax(&tok_in[(tid + j * NT) % T], pm[j]);
    __syncthreads();
    if (tid < T) {
      const float a = __uint_as_float(tok_in[tid]);
      tok_s[tid] = a > 0.f ? 127.f / a : 0.f;
      tok_scale[tid] = a / 127.f;
    }
    __syncthreads();

    for (int b0 = tid; b0 < pieces; b0 += NT * U) {
      if (b0 != tid) issue(b0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int pc = b0 + u * NT;
        if (pc >= pieces) break;
        const int t = (pbase + pc) / ppr, k = 8 * ((pbase + pc) % ppr);
        const float sc = tok_s[t];
        uint32_t out[2];
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          float v[4];
          if (l == 0 && X0_BF16) {
            const uint32_t w0 = (uint32_t)raw[u][0][2 * d];
            const uint32_t w1 = (uint32_t)raw[u][0][2 * d + 1];
            v[0] = __uint_as_float(w0 << 16); v[1] = __uint_as_float(w0 & 0xFFFF0000u);
            v[2] = __uint_as_float(w1 << 16); v[3] = __uint_as_float(w1 & 0xFFFF0000u);
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = __int_as_float(raw[u][d][q]);
          }
          out[d] = q8(v[0], sc) | (q8(v[1], sc) << 8) | (q8(v[2], sc) << 16) | (q8(v[3], sc) << 24);
        }
        if (split) *(uint2*)(xq + (size_t)t * K + k) = make_uint2(out[0], out[1]);
        else *(uint2*)&sm[t * stride + k] = make_uint2(out[0], out[1]);
      }
    }
    if (split) {
      // every slice written: the int8 rows are complete once all blocks arrive
      chain_arrive(ws);
      ++gen;
      if (!chain_wait(ws, gen * (uint32_t)G, spin_limit, &go_sh)) return;
      if (has_work) {
        // row t's K bytes in 1 KB pieces, one direct-to-LDS load per wave each (a short last
        // piece with fewer lanes): no registers hold them, so all of them are in flight at once
        const int cpr = (K + 1023) / 1024;
        for (int c = __builtin_amdgcn_readfirstlane(wave); c < T * cpr; c += kChainWaves) {
          const int t = c / cpr, k0 = (c % cpr) * 1024;
          const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_offset(sm + t * stride + k0));
          if (k0 + 16 * lane < K) lds_dma16(xq + (size_t)t * K + k0 + 16 * lane, m0);
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0));
      }
    }
    __syncthreads();

    if (has_work) {
      // this lane's B fragment of the wave's first step (dead token lanes: row T - 1); the steps
      // follow at immediate offsets of 64 bytes
      const int8_t* xw = sm + min(tok, T - 1) * stride + 16 * h + s_begin * 64;
      // One round: every team multiplies its panel P (P >= npanels: no work, but the team still
      // meets the block at the barriers), the waves' int32 partials are summed in LDS in team
      // order, then y (and acc) and the block's running max |y| per token.
      auto round = [&](int P, const uint32_t (&c)[kChainMaxSteps], const uint32_t (&m)[kChainMaxSteps]) {
        const bool live = P < npanels;
        if (live) {
          v16i acc0 = {}, acc1 = {};
          // B fragments in a ring of three, read two steps ahead of their MFMA.  Reads past the
          // wave's last step (at most five steps: the group's rest and the look-ahead) stay inside
          // the LDS allocation: past the last row they land in the reduction buffer, and they
          // only ever meet a zero code or no MFMA at all.
          // Lanes of tokens past T read nothing: their B columns only feed outputs that are
          // never stored, and the LDS returns data for the live lanes alone.
          const bool rd = tok < T;
          int4 blo[3] = {}, bhi[3] = {};
          if (rd) {
            blo[0] = *(const int4*)xw;
            bhi[0] = *(const int4*)(xw + 32);
            blo[1] = *(const int4*)(xw + 64);
            bhi[1] = *(const int4*)(xw + 96);
          }
#pragma unroll
          for (int g = 0; g < kChainMaxSteps / 4; ++g) {
            if (4 * g >= cnt) break;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int u = 4 * g + v;
              if (u + 2 < kChainMaxSteps && rd) {
                blo[(u + 2) % 3] = *(const int4*)(xw + (u + 2) * 64);
                bhi[(u + 2) % 3] = *(const int4*)(xw + (u + 2) * 64 + 32);
              }
              const uint32_t code = u < cnt ? c[u] : 0u;
              if (u & 1) acc1 = mfma_step<true>(code, m[u], blo[u % 3], bhi[u % 3], acc1);
              else acc0 = mfma_step<true>(code, m[u], blo[u % 3], bhi[u % 3], acc0);
            }
          }
          if (tok < T) {
#pragma unroll
            for (int r = 0; r < 16; ++r) red[(wave * 16 + r) * kChainRedStride + lane] = acc0[r] + acc1[r];
          }
        }
        __syncthreads();
        // The team's 32 x T outputs: item j is token j / 32, panel row j % 32, so a wave's store
        // covers 32 consecutive outputs of a token row.  The accumulator of panel row oo and token
        // t sits in element r = 4 (oo / 8) + oo % 4 of lane 32 ((oo / 4) % 2) + t.
        if (live) {
          for (int j = wt * 64 + lane; j < 32 * T; j += 64 * S) {
            const int t = j >> 5, oo = j & 31;
            const int r = ((oo >> 3) << 2) | (oo & 3);
            const int at = r * kChainRedStride + 32 * ((oo >> 2) & 1) + t;
            int32_t sum = 0;
#pragma unroll
            for (int w = 0; w < kChainWaves; ++w)
              if (w < S) sum += red[(team * S + w) * 16 * kChainRedStride + at];
            const int o = P * kPanel + oo;
            if (o < n) {
              const float v = ((float)sum * gamma) * tok_scale[t];
              Ly.y[(size_t)t * n + o] = v;
              if (Ly.acc) Ly.acc[(size_t)t * n + o] = sum;
              atomicMax(&tok_out[t], __float_as_uint(v) & 0x7FFFFFFFu);
            }
          }
        }
        __syncthreads();   // the reduction buffer is reused by the next round
      };
      // rounds over the block's panels (one round for the decode shapes: the first round's
      // weights were loaded before the wait; a later round loads its own)
      int P = P0;
      for (int base = blk * tpb; base < npanels; base += Pstep, P += Pstep) {
        if (base != blk * tpb && P < npanels) load(P, c0, m0);
        round(P, c0, m0);
      }
    }
    // this block's max |y| per token: a partial of the next layer's input absmax (0 if the
    // block had no panel)
    if (tid < T) pmax[((size_t)(l + 1) * G + blk) * T + tid] = tok_out[tid];
    yin = Ly.y;
    chain_arrive(ws);
    ++gen;
  }
}

__global__ void chain_clear_kernel(uint32_t* __restrict__ ws, int words) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < words) ws[i] = 0u;
}

hipError_t launch_chain(const void* table, int64_t L, int64_t T, int smem, const void* x0,
                        int x_is_bf16, void* ws, int64_t spin_limit, hipStream_t s) {
  // kChainBlocks workgroups (at most one per compute unit; all resident: the launch is
  // cooperative).  Fewer participants make the grid barrier cheaper (its arrivals are atomics on
  // one counter); 64 blocks of 8 waves still stream a layer's weights at a useful rate.
  static int grid = 0;
  if (grid == 0) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    grid = cus < kChainBlocks ? cus : kChainBlocks;
  }
  const int words = (int)(chain_ws_bytes(L, T) / 4);
  chain_clear_kernel<<<(words + 255) / 256, 256, 0, s>>>((uint32_t*)ws, words);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const void* kern = x_is_bf16 ? (const void*)chain_kernel<true> : (const void*)chain_kernel<false>;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 64 * kChainWaves, smem);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorCooperativeLaunchTooLarge;
  const uint8_t* t = (const uint8_t*)table;
  uint32_t* w = (uint32_t*)ws;
  void* args[] = {(void*)&t, (void*)&x0, (void*)&w, (void*)&spin_limit};
  return hipLaunchCooperativeKernel(kern, dim3(grid), dim3(64 * kChainWaves), args, smem, s);
}

}  // namespace bl
