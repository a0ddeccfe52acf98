// C ABI of libbitlinear: host-side validation, then launches on the caller's stream.
// Every check runs before anything is enqueued, so every error path is testable without a GPU.
#include <errno.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <tuple>
#include <vector>

#include "bitlinear.h"
#include "bwd_group.hpp"
#include "chain.hpp"
#include "gemm_group.hpp"
#include "quant_group.hpp"
#include "device_common.hpp"
#include "launch.hpp"
#include "pack_ws.hpp"
#include "pack_group.hpp"

static_assert(BL_PACK_NOALLOC_WS_BYTES == bl::kPackWsBytes, "header states the static workspace size");

namespace {

bool aligned16(const void* p) { return p && ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return p && ((uintptr_t)p & 3u) == 0; }

// Packed K axis: K for 2:4 and DENSE2; (2M - 4) K / M for (M-2):M windows (6:8: 3K/2, 14:16:
// 7K/4).
int64_t keff_of(int64_t K, int M, int layout) {
  return (layout == BL_LAYOUT_SPARSE && M > 4) ? K / M * (2 * M - 4) : K;
}

bool even_m(int M) { return M >= 4 && M <= 16 && M % 2 == 0; }

// K granularity of a layout: whole M-groups and whole MFMA steps on the packed axis (64
// positions for the sparse instruction, 32 for the dense one); lifted layouts also need whole
// lifting chunks of lcm(M, 8) positions.
int64_t k_quantum(int M, int layout) {
  if (layout == BL_LAYOUT_DENSE2) return bl::lcm_i(32, M);
  if (M == 4) return 64;
  for (int64_t k = M;; k += M)
    if (k / M * (2 * M - 4) % 64 == 0 && k % bl::lcm_i(M, 8) == 0) return k;
}

// The N:M mask and layout alone: BL_OK or BL_ENOTSUP.
int check_nm(int N, int M, int layout) {
  if (layout != BL_LAYOUT_SPARSE && layout != BL_LAYOUT_DENSE2) return BL_ENOTSUP;
  if (!even_m(M)) return BL_ENOTSUP;
  if (layout == BL_LAYOUT_SPARSE) {
    // 2:4, or (M-2):M as M/2 - 1 overlapping 2:4 windows
    if (!((N == 2 && M == 4) || (M > 4 && N == M - 2))) return BL_ENOTSUP;
  } else {
    if (N < 1 || N > M) return BL_ENOTSUP;
  }
  return BL_OK;
}

// Shape rules of the packed layout; returns BL_OK and the packed K axis, or a status.
int check_shape(int64_t n, int64_t K, int N, int M, int layout, int64_t* keff) {
  const int nm = check_nm(N, M, layout);
  if (nm != BL_OK) return nm;
  if (n < 1 || K < 1) return BL_EINVAL;
  if (K % k_quantum(M, layout) != 0) return BL_EINVAL;
  if (n > INT32_MAX || K > INT32_MAX) return BL_EINVAL;
  if ((uint64_t)n * (uint64_t)K >= (1ull << 32)) return BL_EINVAL;
  const int64_t ke = keff_of(K, M, layout);
  if (ke * 127 >= (int64_t)INT32_MAX) return BL_EINVAL;
  *keff = ke;
  return BL_OK;
}

// Shape rules of SPARSE6 (a 2:4 matrix re-encoded for decode): those of 2:4 SPARSE.
int check_shape6(int64_t n, int64_t K, int N, int M, int64_t* keff) {
  if (N != 2 || M != 4) return BL_ENOTSUP;
  return check_shape(n, K, 2, 4, BL_LAYOUT_SPARSE, keff);
}

// check_shape for every layout bitlinear_fwd and the decode group accept.
int check_shape_fwd(int64_t n, int64_t K, int N, int M, int layout, int64_t* keff) {
  return layout == BL_LAYOUT_SPARSE6 ? check_shape6(n, K, N, M, keff)
                                     : check_shape(n, K, N, M, layout, keff);
}

int status_of(hipError_t e) { return e == hipSuccess ? BL_OK : BL_EIO; }

// Checks of one act_quant_i8 call (pointers are not looked at when T == 0).
int check_quant(const void* x, int x_dtype, int64_t T, int64_t K, int lift_M, const int8_t* xq,
                const float* x_scale) {
  if (x_dtype != BL_DTYPE_F32 && x_dtype != BL_DTYPE_BF16) return BL_ENOTSUP;
  if (lift_M != 0 && !(even_m(lift_M) && lift_M >= 6)) return BL_EINVAL;
  if (lift_M != 0 && K % bl::lcm_i(lift_M, 8) != 0) return BL_EINVAL;
  if (T < 0 || T > INT32_MAX || K < 8 || K % 8 != 0 || K > (int64_t)1 << 24) return BL_EINVAL;
  if (T == 0) return BL_OK;
  if (!aligned16(x) || !aligned16(xq) || !aligned4(x_scale)) return BL_EINVAL;
  return BL_OK;
}

// Shared checks of one bitlinear_fwd-style projection; returns BL_OK and its packed K axis.
int check_fwd(const int8_t* xq, const float* x_scale, int64_t T, int64_t K, const uint8_t* codes,
              const uint8_t* meta, const float* gamma, int N, int M, int layout, int64_t n,
              const float* y, const int32_t* acc_opt, int64_t* keff) {
  const int st = check_shape_fwd(n, K, N, M, layout, keff);
  if (st != BL_OK) return st;
  if (T < 0 || T > INT32_MAX || (uint64_t)T * (uint64_t)n >= (1ull << 40)) return BL_EINVAL;
  if (layout == BL_LAYOUT_SPARSE6 && T > 32) return BL_ENOTSUP;   // a decode format
  if ((uint64_t)T * (uint64_t)*keff >= (1ull << 31)) return BL_EINVAL;  // 32-bit activation offsets
  if (T == 0) return BL_OK;  // nothing is read or written; pointers may be NULL
  if (!aligned16(xq) || !aligned4(x_scale) || !aligned16(codes) || !aligned16(gamma) ||
      !aligned16(y))
    return BL_EINVAL;
  if (layout == BL_LAYOUT_SPARSE ? !aligned16(meta) : meta != nullptr) return BL_EINVAL;
  if (acc_opt && ((uintptr_t)acc_opt & 3u)) return BL_EINVAL;
  return BL_OK;
}

// Output buffers (y, acc_opt) of a set of projections may not overlap each other or any input
// (xq, x_scale, codes, meta, gamma); inputs may be shared or overlap.  `in_bytes_per_token`: bytes
// of one token row of xq per K_eff position (1 for int8 rows, 2 for the fused group's bf16 rows,
// whose x_scale is not read).  T == 0 projections touch nothing.
int check_fwd_overlaps(const bl_fwd_desc* d, int64_t count, int N, int M, int layout,
                       int in_bytes_per_token) {
  struct Rg { uintptr_t lo, hi; bool out; };
  std::vector<Rg> rs;
  for (int64_t i = 0; i < count; ++i) {
    const bl_fwd_desc& q = d[i];
    if (q.T == 0) continue;
    size_t cb = 0, mb = 0;
    int64_t ke = 0;
    bitlinear_packed_bytes(q.n, q.K, N, M, layout, &cb, &mb, &ke, nullptr);
    rs.push_back({(uintptr_t)q.xq, (uintptr_t)q.xq + (uint64_t)q.T * ke * in_bytes_per_token, false});
    if (in_bytes_per_token == 1)
      rs.push_back({(uintptr_t)q.x_scale, (uintptr_t)q.x_scale + (uint64_t)q.T * 4, false});
    rs.push_back({(uintptr_t)q.codes, (uintptr_t)q.codes + cb, false});
    if (mb) rs.push_back({(uintptr_t)q.meta, (uintptr_t)q.meta + mb, false});
    rs.push_back({(uintptr_t)q.gamma, (uintptr_t)q.gamma + 4, false});
    rs.push_back({(uintptr_t)q.y, (uintptr_t)q.y + (uint64_t)q.T * q.n * 4, true});
    if (q.acc_opt)
      rs.push_back({(uintptr_t)q.acc_opt, (uintptr_t)q.acc_opt + (uint64_t)q.T * q.n * 4, true});
  }
  std::sort(rs.begin(), rs.end(), [](const Rg& a, const Rg& b) { return a.lo < b.lo; });
  uintptr_t out_hi = 0, any_hi = 0;
  for (const Rg& r : rs) {
    if (r.lo < out_hi || (r.out && r.lo < any_hi)) return BL_EINVAL;
    any_hi = std::max(any_hi, r.hi);
    if (r.out) out_hi = std::max(out_hi, r.hi);
  }
  return BL_OK;
}

// Work-item plan of a group.  Items are runs of kGroupPanels panels of one projection; the hardware
// hands workgroup b to XCD b % kXcds, so the plan cuts the projections' items (in projection order)
// into kXcds contiguous runs of about equal weight bytes -- each projection's activation rows then
// land in one or two XCDs' L2 -- and orders each XCD's run largest item first, so the launch ends
// on short items.  Launch position b = p * kXcds + x holds item p of XCD x (padded with empty
// items).
int plan_group(const bl_fwd_desc* d, int64_t count, int N, int M, int layout,
               std::vector<bl::GroupItem>* plan, int in_bytes_per_token) {
  if (!d || count < 1 || count > (1 << 24)) return BL_EINVAL;
  struct It { uint32_t layer, panel0; uint64_t cost; };
  std::vector<It> items;
  uint64_t total = 0;
  for (int64_t i = 0; i < count; ++i) {
    int64_t ke = 0;
    const int st = check_fwd(d[i].xq, d[i].x_scale, d[i].T, d[i].K, d[i].codes, d[i].meta,
                             d[i].gamma, N, M, layout, d[i].n, d[i].y, d[i].acc_opt, &ke);
    if (st != BL_OK) return st;
    if (d[i].T > 32) return BL_EINVAL;
  }
  {
    const int st = check_fwd_overlaps(d, count, N, M, layout, in_bytes_per_token);
    if (st != BL_OK) return st;
  }
  for (int64_t i = 0; i < count; ++i) {
    const int64_t ke = keff_of(d[i].K, M, layout);
    if (d[i].T == 0) continue;
    const int64_t panels = (d[i].n + 31) / 32;
    for (int64_t p0 = 0; p0 < panels; p0 += bl::kGroupPanels) {
      const uint64_t np = (uint64_t)std::min<int64_t>(bl::kGroupPanels, panels - p0);
      items.push_back({(uint32_t)i, (uint32_t)p0, np * (uint64_t)ke});
      total += np * (uint64_t)ke;
      if (items.size() > (size_t)INT32_MAX / (2 * bl::kXcds)) return BL_EINVAL;
    }
  }
  std::vector<std::vector<It>> per(bl::kXcds);
  uint64_t run = 0;
  for (const It& it : items) {
    // XCD of the item's midpoint in the cumulative weight stream
    const uint64_t mid = run + it.cost / 2;
    const int x = (int)std::min<uint64_t>(bl::kXcds - 1, mid * bl::kXcds / std::max<uint64_t>(total, 1));
    per[x].push_back(it);
    run += it.cost;
  }
  size_t depth = 0;
  for (auto& v : per) {
    std::stable_sort(v.begin(), v.end(), [](const It& a, const It& b) { return a.cost > b.cost; });
    depth = std::max(depth, v.size());
  }
  plan->assign(depth * bl::kXcds, bl::GroupItem{bl::kGroupNoItem, 0});
  for (int x = 0; x < bl::kXcds; ++x)
    for (size_t p = 0; p < per[x].size(); ++p)
      (*plan)[p * bl::kXcds + x] = bl::GroupItem{per[x][p].layer, per[x][p].panel0};
  return BL_OK;
}

size_t group_table_bytes(int64_t count, size_t items) {
  const size_t b = sizeof(bl::GroupHeader) + (size_t)count * sizeof(bl::GroupLayer) +
                   items * sizeof(bl::GroupItem);
  return (b + 15) / 16 * 16;
}

// Table size and work items of a group; fused: the descriptors' xq are bf16 rows.
int group_sizes(const bl_fwd_desc* descs, int64_t count, int N, int M, int layout, int fused,
                size_t* table_bytes, int64_t* work_items) {
  std::vector<bl::GroupItem> plan;
  const int st = plan_group(descs, count, N, M, layout, &plan, fused ? 2 : 1);
  if (st != BL_OK) return st;
  if (table_bytes) *table_bytes = group_table_bytes(count, plan.size());
  if (work_items) *work_items = (int64_t)plan.size();
  return BL_OK;
}

// Validates the group and writes its device table; fused: the descriptors' xq are bf16 rows.
int group_build(const bl_fwd_desc* descs, int64_t count, int N, int M, int layout, int fused,
                void* table, size_t table_bytes, void* stream) {
  std::vector<bl::GroupItem> plan;
  const int st = plan_group(descs, count, N, M, layout, &plan, fused ? 2 : 1);
  if (st != BL_OK) return st;
  const size_t bytes = group_table_bytes(count, plan.size());
  if (!aligned16(table)) return BL_EINVAL;
  if (table_bytes < bytes) return BL_ENOSPC;
  std::vector<uint8_t> img(bytes, 0);
  bl::GroupHeader hdr;
  memset(&hdr, 0, sizeof hdr);
  hdr.magic = bl::kGroupMagic;
  hdr.layout = layout;
  hdr.N = N;
  hdr.M = M;
  hdr.count = count;
  hdr.items = (int64_t)plan.size();
  hdr.fused = fused;
  memcpy(img.data(), &hdr, sizeof hdr);
  bl::GroupLayer* rec = (bl::GroupLayer*)(img.data() + sizeof hdr);
  for (int64_t i = 0; i < count; ++i) {
    const bl_fwd_desc& d = descs[i];
    const int64_t ke = keff_of(d.K, M, layout);
    bl::GroupLayer r;
    memset(&r, 0, sizeof r);
    r.xq = d.xq;
    r.xs = fused ? nullptr : d.x_scale;
    r.codes = (const uint32_t*)d.codes;
    r.meta = (const uint32_t*)d.meta;
    r.gamma = d.gamma;
    r.y = d.y;
    r.acc = d.acc_opt;
    r.T = (int32_t)d.T;
    r.Keff = (int32_t)ke;
    r.n = (int32_t)d.n;
    memcpy(&rec[i], &r, sizeof r);
  }
  if (!plan.empty())
    memcpy(img.data() + sizeof hdr + count * sizeof(bl::GroupLayer), plan.data(),
           plan.size() * sizeof(bl::GroupItem));
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(table, img.data(), bytes, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);  // img is released on return
  return status_of(e);
}


// Checks of one bitlinear_bwd call apart from its workspace.
int check_bwd(const uint16_t* dy, int64_t T, int64_t n, const int8_t* xq, const float* x_scale,
              int64_t K, const uint8_t* codes, const uint8_t* meta, const float* gamma, int N,
              int M, int layout, const float* dx, const float* dw, int flags) {
  int64_t ke = 0;
  const int st = check_shape(n, K, N, M, layout, &ke);
  if (st != BL_OK) return st;
  if (T < 0 || T > INT32_MAX) return BL_EINVAL;
  if ((flags & ~(BL_BWD_ACCUM_DX | BL_BWD_ACCUM_DW)) != 0) return BL_EINVAL;
  if (!dx && !dw) return BL_EINVAL;
  const bl::BwdWorkspace w = bl::bwd_workspace(T, n, K);
  const uint64_t lim = 1ull << 30;   // bf16 elements: operands stay below 2^31 bytes
  if ((uint64_t)T * w.n32 >= lim || (uint64_t)K * w.n32 >= lim || (uint64_t)n * w.t32 >= lim ||
      (uint64_t)K * w.t32 >= lim)
    return BL_EINVAL;
  if (dx && T > 0) {
    if (!aligned16(codes) || !aligned4(gamma) || !aligned16(dx)) return BL_EINVAL;
    if (layout == BL_LAYOUT_SPARSE ? !aligned16(meta) : meta != nullptr) return BL_EINVAL;
  }
  if (dw && !aligned16(dw)) return BL_EINVAL;
  if (T > 0) {
    if (!aligned16(dy)) return BL_EINVAL;
    if (dw && (!aligned16(xq) || !aligned4(x_scale))) return BL_EINVAL;
  }
  return BL_OK;
}

// Host plan of a grouped backward: the workspace layout, the prep items, the product jobs and
// their segments.  With ws == NULL the pointers into the workspace are offsets (sizing only).
struct BwdGroupPlan {
  size_t ws_bytes = 0;
  int64_t prep_blocks = 0;
  std::vector<bl::BwdPrep> prep;
  std::vector<bl::BwdJob> jobs;
  std::vector<bl::BwdSeg> segs;
  size_t prep_off = 0, jobs_off = 0, segs_off = 0, table_bytes = 0;
  int64_t t32 = 0;
};

// Per-tile cost of a segment beyond its reduction stages (prologue and epilogue), in stages.
constexpr int64_t kSegCost = 8;

struct Range {
  uintptr_t lo, hi;
};

// Output buffers may not overlap each other or any input, except that projections may name the
// same dx (same pointer, same K): those are summed in descriptor order.
int check_bwd_overlaps(const bl_bwd_desc* d, int64_t count, int64_t T, int N, int M, int layout) {
  std::vector<Range> in;
  struct Out { uintptr_t lo, hi; bool dx; };
  std::vector<Out> out;
  for (int64_t i = 0; i < count; ++i) {
    const bl_bwd_desc& q = d[i];
    size_t cb = 0, mb = 0;
    bitlinear_packed_bytes(q.n, q.K, N, M, layout, &cb, &mb, nullptr, nullptr);
    auto add_in = [&](const void* p, uint64_t bytes) {
      if (p && bytes) in.push_back({(uintptr_t)p, (uintptr_t)p + bytes});
    };
    if (T > 0) {
      add_in(q.dy, (uint64_t)T * q.n * 2);
      if (q.dw) {
        add_in(q.xq, (uint64_t)T * q.K);
        add_in(q.x_scale, (uint64_t)T * 4);
      }
      if (q.dx) {
        add_in(q.codes, cb);
        add_in(q.meta, mb);
        add_in(q.gamma, 4);
      }
    }
    if (q.dx && T > 0)
      out.push_back({(uintptr_t)q.dx, (uintptr_t)q.dx + (uint64_t)T * q.K * 4, true});
    if (q.dw) out.push_back({(uintptr_t)q.dw, (uintptr_t)q.dw + (uint64_t)q.n * q.K * 4, false});
  }
  std::sort(out.begin(), out.end(), [](const Out& a, const Out& b) {
    return a.lo != b.lo ? a.lo < b.lo : a.hi < b.hi;
  });
  // sorted by (start, end), identical ranges are neighbours: a range may start below the running
  // maximum end only as a copy of the dx range just before it
  uintptr_t maxhi = 0;
  for (size_t i = 0; i < out.size(); ++i) {
    const bool same = i > 0 && out[i].dx && out[i - 1].dx && out[i].lo == out[i - 1].lo &&
                      out[i].hi == out[i - 1].hi;
    if (!same && out[i].lo < maxhi) return BL_EINVAL;
    maxhi = std::max(maxhi, out[i].hi);
  }
  std::sort(in.begin(), in.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  std::vector<uintptr_t> pmax(in.size());
  for (size_t i = 0; i < in.size(); ++i) pmax[i] = std::max(in[i].hi, i ? pmax[i - 1] : 0);
  for (const Out& o : out) {
    // inputs starting before o.hi; the largest end among them must stay at or below o.lo
    const size_t k = (size_t)(std::lower_bound(in.begin(), in.end(), o.hi,
                                               [](const Range& r, uintptr_t v) { return r.lo < v; }) -
                              in.begin());
    if (k > 0 && pmax[k - 1] > o.lo) return BL_EINVAL;
  }
  return BL_OK;
}

int plan_bwd_group(const bl_bwd_desc* d, int64_t count, int64_t T, int N, int M, int layout,
                   uint8_t* ws, BwdGroupPlan* P) {
  if (!d || count < 1 || count > (1 << 16)) return BL_EINVAL;
  if (T < 0 || T > INT32_MAX) return BL_EINVAL;
  for (int64_t i = 0; i < count; ++i) {
    const bl_bwd_desc& q = d[i];
    const int st = check_bwd(q.dy, T, q.n, q.xq, q.x_scale, q.K, q.codes, q.meta, q.gamma, N, M,
                             layout, q.dx, q.dw, q.flags);
    if (st != BL_OK) return st;
  }
  {
    const int st = check_bwd_overlaps(d, count, T, N, M, layout);
    if (st != BL_OK) return st;
  }
  auto up = [](size_t v, size_t a) { return (v + a - 1) / a * a; };
  const int64_t t32 = (T + 31) / 32 * 32;
  P->t32 = t32;
  const int tt = (int)((T + 63) / 64);
  size_t off = 0;
  auto carve = [&](size_t bytes) {
    uint8_t* p = ws + off;   // an offset when ws is NULL
    off = up(off + bytes, 256);
    return p;
  };
  // workspace and prep items, in descriptor order
  std::vector<const uint16_t*> dx_a(count), wt(count), dyt(count), xt(count);
  std::map<std::tuple<const int8_t*, const float*, int64_t>, const uint16_t*> xs_seen;
  int64_t blocks = 0;
  auto add_prep = [&](int32_t kind, int64_t nblocks, int a0, int a1, int a2, const void* s0,
                      const void* s1, void* dst) {
    if (nblocks <= 0) return;
    bl::BwdPrep it;
    memset(&it, 0, sizeof it);
    it.kind = kind;
    it.block0 = (int32_t)blocks;
    it.a0 = a0; it.a1 = a1; it.a2 = a2;
    it.src0 = s0; it.src1 = s1; it.dst = dst;
    P->prep.push_back(it);
    blocks += nblocks;
  };
  for (int64_t i = 0; i < count && T > 0; ++i) {
    const bl_bwd_desc& q = d[i];
    const int64_t n32 = (q.n + 31) / 32 * 32;
    if (q.dx) {
      uint16_t* w = (uint16_t*)carve((size_t)q.K * n32 * 2);
      wt[i] = w;
      const int64_t ke = keff_of(q.K, M, layout);
      const int U = (int)(layout == BL_LAYOUT_SPARSE ? ke / 32 : q.K / 16);
      const int64_t groups = q.K / M, pairs = n32 / 2;
      add_prep(bl::kPrepWt, (groups * pairs + 255) / 256, U, (int)groups, (int)pairs, q.codes,
               q.meta, w);
      if (n32 != q.n) {
        uint16_t* p = (uint16_t*)carve((size_t)T * n32 * 2);
        add_prep(bl::kPrepPad, (T * n32 + 255) / 256, (int)q.n, (int)n32, 0, q.dy, nullptr, p);
        dx_a[i] = p;
      } else {
        dx_a[i] = q.dy;
      }
    }
    if (q.dw) {
      uint16_t* p = (uint16_t*)carve((size_t)q.n * t32 * 2);
      const int tn = (int)((q.n + 63) / 64);
      add_prep(bl::kPrepTrDy, (int64_t)tt * tn, (int)q.n, tn, 0, q.dy, nullptr, p);
      dyt[i] = p;
      const auto key = std::make_tuple(q.xq, q.x_scale, q.K);
      const auto hit = xs_seen.find(key);
      if (hit != xs_seen.end()) {
        xt[i] = hit->second;
      } else {
        uint16_t* x = (uint16_t*)carve((size_t)q.K * t32 * 2);
        const int tk = (int)((q.K + 63) / 64);
        add_prep(bl::kPrepTrX, (int64_t)tt * tk, (int)q.K, tk, 0, q.xq, q.x_scale, x);
        xs_seen.emplace(key, x);
        xt[i] = x;
      }
    }
    if (blocks > INT32_MAX) return BL_EINVAL;
  }
  P->ws_bytes = off;
  P->prep_blocks = blocks;

  // products: one per distinct dx (segments = its projections in order), one per dw
  struct Gemm { float* c; int64_t rows_a, rows_b, ldc; int32_t seg0, nseg; int64_t work; };
  std::vector<Gemm> gemms;
  // projections of each distinct dx, in descriptor order; dx buffers in order of first use
  std::map<float*, std::vector<int64_t>> dx_users;
  std::vector<float*> dx_order;
  for (int64_t i = 0; i < count && T > 0; ++i) {
    if (!d[i].dx) continue;
    auto& users = dx_users[d[i].dx];
    if (users.empty()) dx_order.push_back(d[i].dx);
    users.push_back(i);
  }
  for (float* dxp : dx_order) {
    const std::vector<int64_t>& users = dx_users[dxp];
    const int64_t i = users.front();
    Gemm g{dxp, T, d[i].K, d[i].K, (int32_t)P->segs.size(), 0, 0};
    for (const int64_t j : users) {
      const int64_t n32 = (d[j].n + 31) / 32 * 32;
      bl::BwdSeg sg;
      memset(&sg, 0, sizeof sg);
      sg.a = dx_a[j]; sg.b = wt[j]; sg.alpha = d[j].gamma;
      sg.lda = (int32_t)n32; sg.ldb = (int32_t)n32; sg.R = (int32_t)n32;
      sg.accumulate = (d[j].flags & BL_BWD_ACCUM_DX) != 0;
      P->segs.push_back(sg);
      ++g.nseg;
      g.work += n32 / 32 + kSegCost;
    }
    gemms.push_back(g);
  }
  for (int64_t i = 0; i < count; ++i) {
    if (!d[i].dw) continue;
    Gemm g{d[i].dw, d[i].n, d[i].K, d[i].K, (int32_t)P->segs.size(), 1, t32 / 32 + kSegCost};
    bl::BwdSeg sg;
    memset(&sg, 0, sizeof sg);
    sg.a = dyt[i]; sg.b = xt[i]; sg.alpha = nullptr;
    sg.lda = (int32_t)t32; sg.ldb = (int32_t)t32; sg.R = (int32_t)t32;
    sg.accumulate = (d[i].flags & BL_BWD_ACCUM_DW) != 0;
    P->segs.push_back(sg);
    gemms.push_back(g);
  }
  // 8 x 4 tile patches (an XCD's 32 CUs hold one patch at a time, so its operand tiles stay in
  // that XCD's L2), dealt longest first to the least-loaded XCD; each XCD's list runs longest
  // first and block b of the launch takes entry b / 8 of XCD b % 8's list.
  struct Patch { int32_t g, pi, pj; int64_t work, tiles; };
  std::vector<Patch> patches;
  for (size_t g = 0; g < gemms.size(); ++g) {
    const int64_t ti = (gemms[g].rows_a + 255) / 256, tj = (gemms[g].rows_b + 255) / 256;
    for (int64_t pi = 0; pi < ti; pi += 8)
      for (int64_t pj = 0; pj < tj; pj += 4)
        patches.push_back({(int32_t)g, (int32_t)pi, (int32_t)pj, gemms[g].work,
                           std::min<int64_t>(8, ti - pi) * std::min<int64_t>(4, tj - pj)});
  }
  std::stable_sort(patches.begin(), patches.end(),
                   [](const Patch& a, const Patch& b) { return a.work > b.work; });
  std::vector<std::vector<bl::BwdJob>> per(bl::kXcds);
  int64_t load[bl::kXcds] = {};
  for (const Patch& pt : patches) {
    const int x = (int)(std::min_element(load, load + bl::kXcds) - load);
    load[x] += pt.work * pt.tiles;
    const Gemm& g = gemms[pt.g];
    const int64_t ti = (g.rows_a + 255) / 256, tj = (g.rows_b + 255) / 256;
    for (int64_t j = pt.pj; j < std::min<int64_t>(pt.pj + 4, tj); ++j)
      for (int64_t i = pt.pi; i < std::min<int64_t>(pt.pi + 8, ti); ++i) {
        bl::BwdJob jb;
        memset(&jb, 0, sizeof jb);
        jb.c = g.c;
        jb.seg0 = g.seg0; jb.nseg = g.nseg;
        jb.i0 = (int32_t)(i * 256); jb.j0 = (int32_t)(j * 256);
        jb.rows_a = (int32_t)g.rows_a; jb.rows_b = (int32_t)g.rows_b; jb.ldc = (int32_t)g.ldc;
        per[x].push_back(jb);
      }
  }
  size_t depth = 0;
  for (const auto& v : per) depth = std::max(depth, v.size());
  if (depth * bl::kXcds > (size_t)INT32_MAX || P->segs.size() > (size_t)INT32_MAX)
    return BL_EINVAL;
  bl::BwdJob pad;
  memset(&pad, 0, sizeof pad);
  P->jobs.assign(depth * bl::kXcds, pad);
  for (int x = 0; x < bl::kXcds; ++x)
    for (size_t k = 0; k < per[x].size(); ++k) P->jobs[k * bl::kXcds + x] = per[x][k];

  P->prep_off = sizeof(bl::BwdHeader);
  P->jobs_off = up(P->prep_off + P->prep.size() * sizeof(bl::BwdPrep), 16);
  P->segs_off = up(P->jobs_off + P->jobs.size() * sizeof(bl::BwdJob), 16);
  P->table_bytes = up(P->segs_off + P->segs.size() * sizeof(bl::BwdSeg), 16);
  return BL_OK;
}

// Pack tiles of a master (32-row panels x pack_cols column tiles) and its workspace bytes: the
// fixed part and one band region per tile.
int64_t pack_tiles(int64_t n, int64_t K, int layout, int M) {
  const int64_t kb = bl::pack_cols(layout, M);
  return (n + 31) / 32 * ((K + kb - 1) / kb);
}
size_t pack_ws_bytes(int64_t n, int64_t K, int layout, int M) {
  return bl::pack_ws_bytes_for_tiles(pack_tiles(n, K, layout, M));
}
// Grouped pack: per-master workspace slices, each rounded to 256 bytes.
size_t pack_ws_slice(int64_t n, int64_t K, int layout, int M) {
  return (pack_ws_bytes(n, K, layout, M) + 255) / 256 * 256;
}

// Validates a grouped pack: every descriptor as bitlinear_pack; no output (codes, meta, gamma)
// may overlap another output or any master.  Fills the items (ws offsets from `ws`) and returns
// the pack launch's block count.
int plan_pack_group(const bl_pack_desc* d, int64_t count, int N, int M, int layout, uint8_t* ws,
                    std::vector<bl::PackGroupItem>* items, int64_t* pack_blocks,
                    size_t* ws_bytes) {
  if (!d || count < 1 || count > 4096) return BL_EINVAL;
  size_t ws_off = 0;
  struct R { uintptr_t lo, hi; bool out; };
  std::vector<R> rs;
  items->assign((size_t)count, bl::PackGroupItem{});
  for (int64_t i = 0; i < count; ++i) {
    const bl_pack_desc& q = d[i];
    int64_t ke = 0;
    const int st = check_shape(q.n, q.K, N, M, layout, &ke);
    if (st != BL_OK) return st;
    if (!aligned16(q.W) || !aligned16(q.codes) || !aligned16(q.gamma)) return BL_EINVAL;
    if (layout == BL_LAYOUT_SPARSE ? !aligned16(q.meta) : q.meta != nullptr) return BL_EINVAL;
    size_t cb = 0, mb = 0;
    bitlinear_packed_bytes(q.n, q.K, N, M, layout, &cb, &mb, nullptr, nullptr);
    rs.push_back({(uintptr_t)q.W, (uintptr_t)q.W + (uint64_t)q.n * q.K * 4, false});
    rs.push_back({(uintptr_t)q.codes, (uintptr_t)q.codes + cb, true});
    if (mb) rs.push_back({(uintptr_t)q.meta, (uintptr_t)q.meta + mb, true});
    rs.push_back({(uintptr_t)q.gamma, (uintptr_t)q.gamma + 4, true});
    bl::PackGroupItem& it = (*items)[(size_t)i];
    it.W = q.W;
    it.codes = (uint32_t*)q.codes;
    it.meta = (uint32_t*)q.meta;
    it.gamma = q.gamma;
    it.ws = ws + ws_off;
    ws_off += pack_ws_slice(q.n, q.K, layout, M);
    it.n = (int32_t)q.n;
    it.K = (int32_t)q.K;
    it.k_tiles = (int32_t)((q.K + bl::pack_cols(layout, M) - 1) / bl::pack_cols(layout, M));
  }
  // any overlap involving an output is an error (masters may be shared or overlap each other)
  std::sort(rs.begin(), rs.end(), [](const R& a, const R& b) { return a.lo < b.lo; });
  uintptr_t out_hi = 0, any_hi = 0;
  for (const R& r : rs) {
    if (r.lo < out_hi || (r.out && r.lo < any_hi)) return BL_EINVAL;
    any_hi = std::max(any_hi, r.hi);
    if (r.out) out_hi = std::max(out_hi, r.hi);
  }
  // pack blocks in reverse descriptor order
  int64_t blocks = 0;
  for (int64_t i = count - 1; i >= 0; --i) {
    bl::PackGroupItem& it = (*items)[(size_t)i];
    it.block0 = (int32_t)blocks;
    blocks += (int64_t)((it.n + 31) / 32) * it.k_tiles;
    if (blocks > INT32_MAX) return BL_EINVAL;
  }
  *pack_blocks = blocks;
  *ws_bytes = ws_off;
  return BL_OK;
}

// Byte offset of the jobs in a grouped prefill table of `count` projections (16-byte aligned).
size_t gemm_jobs_offset(size_t count) {
  return (sizeof(bl::GemmGroupHeader) + count * sizeof(bl::GemmGroupProj) + 15) / 16 * 16;
}

// Grouped prefill plan: validates the projections (bitlinear_fwd's rules, T > 128 each), checks
// that no output overlaps another output or an input, and lays out the jobs; block b takes entry
// b / 8 of XCD b % 8's list.
//   - When every projection's token tiles split evenly over the XCDs, XCD x takes slab x of the
//     token tiles of every projection, walked as bitlinear_fwd walks it (row tile by row tile,
//     the slab's token tiles fastest), projection after projection with those that read the
//     same activations next to each other: the slab's activation rows stay in that XCD's L2
//     across the projections that share them, and every XCD gets the same work.  On the 3B-alike
//     layer set at 8192 tokens this halves the bytes fetched past L2 of the run order below.
//   - Otherwise each projection's tiles are cut into runs of up to kGemmRun consecutive tile
//     numbers (row tiles fastest, so neighbouring blocks of a run read the same token tile), and
//     runs are dealt longest first to the least-loaded XCD.
constexpr int64_t kGemmRun = 64;   // two block slots on each of an XCD's 32 CUs

int plan_gemm_group(const bl_fwd_desc* d, int64_t count, int N, int M, int layout,
                    std::vector<bl::GemmGroupProj>* projs, std::vector<bl::GemmGroupJob>* jobs) {
  if (!d || count < 1 || count > 4096) return BL_EINVAL;
  struct Rg { uintptr_t lo, hi; bool out; };
  std::vector<Rg> rs;
  projs->assign((size_t)count, bl::GemmGroupProj{});
  for (int64_t i = 0; i < count; ++i) {
    int64_t ke = 0;
    const int st = check_fwd(d[i].xq, d[i].x_scale, d[i].T, d[i].K, d[i].codes, d[i].meta,
                             d[i].gamma, N, M, layout, d[i].n, d[i].y, d[i].acc_opt, &ke);
    if (st != BL_OK) return st;
    if (d[i].T <= 128) return BL_EINVAL;
    const bl_fwd_desc& q = d[i];
    size_t cb = 0, mb = 0;
    bitlinear_packed_bytes(q.n, q.K, N, M, layout, &cb, &mb, nullptr, nullptr);
    rs.push_back({(uintptr_t)q.xq, (uintptr_t)q.xq + (uint64_t)q.T * ke, false});
    rs.push_back({(uintptr_t)q.x_scale, (uintptr_t)q.x_scale + (uint64_t)q.T * 4, false});
    rs.push_back({(uintptr_t)q.codes, (uintptr_t)q.codes + cb, false});
    if (mb) rs.push_back({(uintptr_t)q.meta, (uintptr_t)q.meta + mb, false});
    rs.push_back({(uintptr_t)q.gamma, (uintptr_t)q.gamma + 4, false});
    rs.push_back({(uintptr_t)q.y, (uintptr_t)q.y + (uint64_t)q.T * q.n * 4, true});
    if (q.acc_opt) rs.push_back({(uintptr_t)q.acc_opt, (uintptr_t)q.acc_opt + (uint64_t)q.T * q.n * 4, true});
    bl::GemmGroupProj& r = (*projs)[(size_t)i];
    r.xq = q.xq; r.xs = q.x_scale;
    r.codes = (const uint32_t*)q.codes; r.meta = (const uint32_t*)q.meta;
    r.gamma = q.gamma; r.y = q.y; r.acc = q.acc_opt;
    r.T = (int32_t)q.T; r.Keff = (int32_t)ke; r.n = (int32_t)q.n;
    r.npanels = (int32_t)((q.n + 31) / 32);   // 32-row packed panels
  }
  // inputs may be shared or overlap; an output may overlap nothing
  std::sort(rs.begin(), rs.end(), [](const Rg& a, const Rg& b) { return a.lo < b.lo; });
  uintptr_t out_hi = 0, any_hi = 0;
  for (const Rg& r : rs) {
    if (r.lo < out_hi || (r.out && r.lo < any_hi)) return BL_EINVAL;
    any_hi = std::max(any_hi, r.hi);
    if (r.out) out_hi = std::max(out_hi, r.hi);
  }
  const int64_t BM = bl::gemm_group_tile_rows(), BN = bl::gemm_group_tile_tokens();
  std::vector<std::vector<bl::GemmGroupJob>> per(bl::kXcds);
  bool slabs = true;
  int64_t total = 0;
  for (const bl::GemmGroupProj& r : *projs) {
    const int64_t tn = (r.T + BN - 1) / BN;
    slabs = slabs && tn % bl::kXcds == 0;
    total += tn * ((r.n + BM - 1) / BM);
  }
  if (slabs && total <= (int64_t)1 << 30) {   // the run order below allows as many tiles
    std::vector<int64_t> order;   // projections grouped by activation rows, first-seen order
    std::vector<bool> taken((size_t)count, false);
    for (int64_t i = 0; i < count; ++i) {
      if (taken[(size_t)i]) continue;
      for (int64_t j = i; j < count; ++j)
        if (!taken[(size_t)j] && (*projs)[(size_t)j].xq == (*projs)[(size_t)i].xq) {
          taken[(size_t)j] = true;
          order.push_back(j);
        }
    }
    for (int x = 0; x < bl::kXcds; ++x)
      for (int64_t i : order) {
        const bl::GemmGroupProj& r = (*projs)[(size_t)i];
        const int64_t tm = (r.n + BM - 1) / BM, ntn = (r.T + BN - 1) / BN / bl::kXcds;
        for (int64_t k = 0; k < tm * ntn; ++k)
          per[x].push_back({(int32_t)i, (int32_t)(k / ntn), (int32_t)(x * ntn + k % ntn), 0});
      }
  } else {
    struct Run { int32_t proj; int64_t t0, t1, tiles_m, work; };
    std::vector<Run> runs;
    for (int64_t i = 0; i < count; ++i) {
      const bl::GemmGroupProj& r = (*projs)[(size_t)i];
      const int64_t tm = (r.n + BM - 1) / BM, tiles = tm * ((r.T + BN - 1) / BN);
      for (int64_t t0 = 0; t0 < tiles; t0 += kGemmRun) {
        const int64_t t1 = std::min(tiles, t0 + kGemmRun);
        runs.push_back({(int32_t)i, t0, t1, tm, (t1 - t0) * (int64_t)r.Keff});
      }
      if ((int64_t)runs.size() > (int64_t)1 << 24) return BL_EINVAL;
    }
    std::stable_sort(runs.begin(), runs.end(),
                     [](const Run& a, const Run& b) { return a.work > b.work; });
    int64_t load[bl::kXcds] = {};
    for (const Run& rn : runs) {
      const int x = (int)(std::min_element(load, load + bl::kXcds) - load);
      load[x] += rn.work;
      for (int64_t t = rn.t0; t < rn.t1; ++t)
        per[x].push_back({rn.proj, (int32_t)(t % rn.tiles_m), (int32_t)(t / rn.tiles_m), 0});
    }
  }
  size_t depth = 0;
  for (const auto& v : per) depth = std::max(depth, v.size());
  if (depth * bl::kXcds > (size_t)INT32_MAX) return BL_EINVAL;
  jobs->assign(depth * bl::kXcds, bl::GemmGroupJob{-1, 0, 0, 0});
  for (int x = 0; x < bl::kXcds; ++x)
    for (size_t k = 0; k < per[x].size(); ++k) (*jobs)[k * bl::kXcds + x] = per[x][k];
  return BL_OK;
}

// A fused group's descriptors as plain ones (xq = the bf16 rows; x_scale is not read, the row
// pointer stands in for the NULL check), after the checks that are the fused path's own: no
// lifting (2:4 SPARSE or DENSE2) and bf16 rows addressable with 32-bit offsets.
int fused_as_plain(const bl_fwd_x_desc* d, int64_t count, int M, int layout,
                   std::vector<bl_fwd_desc>* out) {
  if (!d || count < 1 || count > (1 << 24)) return BL_EINVAL;
  if (layout == BL_LAYOUT_SPARSE && M != 4) return BL_ENOTSUP;
  if (layout == BL_LAYOUT_SPARSE6) return BL_ENOTSUP;
  out->resize((size_t)count);
  for (int64_t i = 0; i < count; ++i) {
    if (d[i].T < 0 || d[i].K < 1) return BL_EINVAL;
    if ((uint64_t)d[i].T * (uint64_t)d[i].K * 2u >= (1ull << 31)) return BL_EINVAL;
    bl_fwd_desc& p = (*out)[(size_t)i];
    p.xq = (const int8_t*)d[i].x;
    p.x_scale = (const float*)d[i].x;
    p.T = d[i].T;
    p.K = d[i].K;
    p.codes = d[i].codes;
    p.meta = d[i].meta;
    p.gamma = d[i].gamma;
    p.n = d[i].n;
    p.y = d[i].y;
    p.acc_opt = d[i].acc_opt;
  }
  return BL_OK;
}

// Validation of a chain (see bl_chain_layer in the header); returns BL_OK and the launch's
// dynamic LDS bytes.
constexpr int64_t kChainLdsMax = 163840 - 1024;

int plan_chain(const bl_chain_layer* d, int64_t L, int64_t T, int N, int M, int layout,
               int* smem) {
  if (!d || L < 1 || L > 4096) return BL_EINVAL;
  if (layout != BL_LAYOUT_SPARSE || N != 2 || M != 4) return BL_ENOTSUP;
  if (T < 1 || T > bl::kChainMaxT) return BL_EINVAL;
  int64_t need = 0;
  struct Rg { uintptr_t lo, hi; bool out; };
  std::vector<Rg> rs;
  for (int64_t l = 0; l < L; ++l) {
    const bl_chain_layer& q = d[l];
    int64_t ke = 0;
    const int st = check_shape(q.n, q.K, N, M, layout, &ke);
    if (st != BL_OK) return st;
    if (q.K > bl::kChainMaxK) return BL_EINVAL;
    if (l > 0 && q.K != d[l - 1].n) return BL_EINVAL;
    if ((uint64_t)T * q.K * 4 >= (1ull << 31) || (uint64_t)T * q.n * 4 >= (1ull << 31)) return BL_EINVAL;
    if (!aligned16(q.codes) || !aligned16(q.meta) || !aligned4(q.gamma) || !aligned16(q.y))
      return BL_EINVAL;
    if (q.acc_opt && ((uintptr_t)q.acc_opt & 3u)) return BL_EINVAL;
    need = std::max<int64_t>(need, (T * (q.K + 16) + 15) / 16 * 16 + bl::kChainRedBytes);
    size_t cb = 0, mb = 0;
    bitlinear_packed_bytes(q.n, q.K, N, M, layout, &cb, &mb, nullptr, nullptr);
    rs.push_back({(uintptr_t)q.codes, (uintptr_t)q.codes + cb, false});
    rs.push_back({(uintptr_t)q.meta, (uintptr_t)q.meta + mb, false});
    rs.push_back({(uintptr_t)q.gamma, (uintptr_t)q.gamma + 4, false});
    rs.push_back({(uintptr_t)q.y, (uintptr_t)q.y + (uint64_t)T * q.n * 4, true});
    if (q.acc_opt) rs.push_back({(uintptr_t)q.acc_opt, (uintptr_t)q.acc_opt + (uint64_t)T * q.n * 4, true});
  }
  if (need > kChainLdsMax) return BL_EINVAL;
  std::sort(rs.begin(), rs.end(), [](const Rg& a, const Rg& b) { return a.lo < b.lo; });
  uintptr_t out_hi = 0, any_hi = 0;
  for (const Rg& r : rs) {
    if (r.lo < out_hi || (r.out && r.lo < any_hi)) return BL_EINVAL;
    any_hi = std::max(any_hi, r.hi);
    if (r.out) out_hi = std::max(out_hi, r.hi);
  }
  *smem = (int)need;
  return BL_OK;
}

size_t chain_table_bytes(int64_t L) {
  return (sizeof(bl::ChainHeader) + (size_t)L * sizeof(bl::ChainLayer) + 15) / 16 * 16;
}

}  // namespace

extern "C" {

int bitlinear_layout_version(void) { return BL_LAYOUT_VERSION; }

const char* bitlinear_strerror(int status) {
  switch (status) {
    case BL_OK: return "ok";
    case BL_EINVAL: return "invalid argument, shape, alignment or NULL pointer";
    case BL_ENOTSUP: return "unsupported N:M, layout or dtype";
    case BL_ENOSPC: return "workspace too small";
    case BL_EIO: return "HIP runtime or launch error";
    default: return "unknown status";
  }
}

int bitlinear_packed_bytes(int64_t n, int64_t K, int N, int M, int layout, size_t* codes_bytes,
                           size_t* meta_bytes, int64_t* K_eff, size_t* ws_bytes) {
  int64_t ke = 0;
  const int st = check_shape_fwd(n, K, N, M, layout, &ke);
  if (st != BL_OK) return st;
  const uint64_t n_pad = (uint64_t)((n + 31) / 32) * 32;
  if (layout == BL_LAYOUT_SPARSE6) {
    // three dwords per lane per (32-row panel, 128-column step pair)
    if (codes_bytes) *codes_bytes = (size_t)(n_pad / 32 * (uint64_t)((K + 127) / 128) * 64 * 12);
    if (meta_bytes) *meta_bytes = 0;
    if (K_eff) *K_eff = ke;
    if (ws_bytes) *ws_bytes = 0;
    return BL_OK;
  }
  const uint64_t slots = layout == BL_LAYOUT_SPARSE ? (uint64_t)ke / 2 : (uint64_t)ke;
  if (codes_bytes) *codes_bytes = (size_t)(n_pad * slots / 4);
  if (meta_bytes) *meta_bytes = layout == BL_LAYOUT_SPARSE ? (size_t)(n_pad * slots / 4) : 0;
  if (K_eff) *K_eff = ke;
  if (ws_bytes) *ws_bytes = pack_ws_bytes(n, K, layout, M);
  return BL_OK;
}

int bitlinear_pack(const float* W, int64_t n, int64_t K, int N, int M, int layout, uint8_t* codes,
                   uint8_t* meta, float* gamma, void* ws, size_t ws_bytes, void* stream) {
  int64_t ke = 0;
  const int st = check_shape(n, K, N, M, layout, &ke);
  if (st != BL_OK) return st;
  if (!aligned16(W) || !aligned16(codes) || !aligned16(gamma) || !aligned16(ws)) return BL_EINVAL;
  if (layout == BL_LAYOUT_SPARSE ? !aligned16(meta) : meta != nullptr) return BL_EINVAL;
  if (ws_bytes < pack_ws_bytes(n, K, layout, M)) return BL_ENOSPC;
  return status_of(bl::launch_pack(W, n, K, N, M, layout, (uint32_t*)codes, (uint32_t*)meta, gamma,
                                   ws, pack_tiles(n, K, layout, M), (hipStream_t)stream));
}

int bitlinear_pack_noalloc(const float* W, int64_t n, int64_t K, int N, int M, int layout,
                           uint8_t* codes, uint8_t* meta, float* gamma, void* stream) {
  int64_t ke = 0;
  const int st = check_shape(n, K, N, M, layout, &ke);
  if (st != BL_OK) return st;
  if (!aligned16(W) || !aligned16(codes) || !aligned16(gamma)) return BL_EINVAL;
  if (layout == BL_LAYOUT_SPARSE ? !aligned16(meta) : meta != nullptr) return BL_EINVAL;
  // the static workspace holds the fixed part and band regions for kNoallocTiles tiles; a larger
  // master is packed without the band (two passes), so every shape fits
  if (bl::kPackWsBytes > bl::pack_noalloc_capacity()) return BL_ENOSPC;
  return status_of(bl::launch_pack_noalloc(W, n, K, N, M, layout, (uint32_t*)codes,
                                           (uint32_t*)meta, gamma, (hipStream_t)stream));
}

int bitlinear_pack_group_plan(const bl_pack_desc* descs, int64_t count, int N, int M, int layout,
                              bl_pack_group_plan* plan) {
  if (!plan) return BL_EINVAL;
  std::vector<bl::PackGroupItem> items;
  int64_t blocks = 0;
  size_t wsb = 0;
  const int st = plan_pack_group(descs, count, N, M, layout, nullptr, &items, &blocks, &wsb);
  if (st != BL_OK) return st;
  memset(plan, 0, sizeof *plan);
  plan->table_bytes = sizeof(bl::PackGroupHeader) + (size_t)count * sizeof(bl::PackGroupItem);
  plan->ws_bytes = wsb;
  plan->count = count;
  plan->pack_blocks = blocks;
  plan->N = N;
  plan->M = M;
  plan->layout = layout;
  return BL_OK;
}

int bitlinear_pack_group_build(const bl_pack_desc* descs, int64_t count, int N, int M,
                               int layout, void* ws, size_t ws_bytes, void* table,
                               size_t table_bytes, void* stream) {
  if (!ws || ((uintptr_t)ws & 255u) || !aligned16(table)) return BL_EINVAL;
  std::vector<bl::PackGroupItem> items;
  int64_t blocks = 0;
  size_t wsb = 0;
  const int st = plan_pack_group(descs, count, N, M, layout, (uint8_t*)ws, &items, &blocks, &wsb);
  if (st != BL_OK) return st;
  const size_t bytes = sizeof(bl::PackGroupHeader) + (size_t)count * sizeof(bl::PackGroupItem);
  if (ws_bytes < wsb || table_bytes < bytes) return BL_ENOSPC;
  std::vector<uint8_t> img(bytes, 0);
  bl::PackGroupHeader hdr;
  memset(&hdr, 0, sizeof hdr);
  hdr.magic = bl::kPackGroupMagic;
  hdr.layout = layout;
  hdr.N = N;
  hdr.M = M;
  hdr.count = (int32_t)count;
  hdr.pack_blocks = (int32_t)blocks;
  memcpy(img.data(), &hdr, sizeof hdr);
  memcpy(img.data() + sizeof hdr, items.data(), items.size() * sizeof(bl::PackGroupItem));
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(table, img.data(), bytes, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);  // img is released on return
  return status_of(e);
}

int bitlinear_pack_group(const void* table, const bl_pack_group_plan* plan, void* stream) {
  if (!plan || !aligned16(table)) return BL_EINVAL;
  const int st = check_nm(plan->N, plan->M, plan->layout);
  if (st != BL_OK) return st;
  if (plan->count < 1 || plan->count > 4096 || plan->pack_blocks < 1 ||
      plan->pack_blocks > INT32_MAX)
    return BL_EINVAL;
  return status_of(bl::launch_pack_group(table, plan->count, plan->pack_blocks, plan->layout,
                                         plan->M, (hipStream_t)stream));
}

int bitlinear_gemm_group_plan(const bl_fwd_desc* descs, int64_t count, int N, int M, int layout,
                              bl_gemm_group_plan* plan) {
  if (!plan) return BL_EINVAL;
  std::vector<bl::GemmGroupProj> projs;
  std::vector<bl::GemmGroupJob> jobs;
  const int st = plan_gemm_group(descs, count, N, M, layout, &projs, &jobs);
  if (st != BL_OK) return st;
  memset(plan, 0, sizeof *plan);
  plan->table_bytes = gemm_jobs_offset(projs.size()) + jobs.size() * sizeof(bl::GemmGroupJob);
  plan->jobs = (int64_t)jobs.size();
  plan->N = N;
  plan->M = M;
  plan->layout = layout;
  return BL_OK;
}

int bitlinear_gemm_group_build(const bl_fwd_desc* descs, int64_t count, int N, int M, int layout,
                               void* table, size_t table_bytes, void* stream) {
  if (!aligned16(table)) return BL_EINVAL;
  std::vector<bl::GemmGroupProj> projs;
  std::vector<bl::GemmGroupJob> jobs;
  const int st = plan_gemm_group(descs, count, N, M, layout, &projs, &jobs);
  if (st != BL_OK) return st;
  const size_t pbytes = projs.size() * sizeof(bl::GemmGroupProj);
  const size_t jobs_off = gemm_jobs_offset(projs.size());
  const size_t bytes = jobs_off + jobs.size() * sizeof(bl::GemmGroupJob);
  if (table_bytes < bytes) return BL_ENOSPC;
  std::vector<uint8_t> img(bytes, 0);
  bl::GemmGroupHeader hdr;
  memset(&hdr, 0, sizeof hdr);
  hdr.magic = bl::kGemmGroupMagic;
  hdr.layout = layout;
  hdr.N = N;
  hdr.M = M;
  hdr.count = (int32_t)count;
  hdr.jobs = (int32_t)jobs.size();
  hdr.jobs_off = (int64_t)jobs_off;
  memcpy(img.data(), &hdr, sizeof hdr);
  memcpy(img.data() + sizeof hdr, projs.data(), pbytes);
  memcpy(img.data() + jobs_off, jobs.data(), jobs.size() * sizeof(bl::GemmGroupJob));
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(table, img.data(), bytes, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);  // img is released on return
  return status_of(e);
}

int bitlinear_gemm_group(const void* table, const bl_gemm_group_plan* plan, void* stream) {
  if (!plan || !aligned16(table)) return BL_EINVAL;
  const int st = check_nm(plan->N, plan->M, plan->layout);
  if (st != BL_OK) return st;
  if (plan->jobs < 1 || plan->jobs > INT32_MAX) return BL_EINVAL;
  return status_of(bl::launch_gemm_group(table, plan->jobs, plan->layout, (hipStream_t)stream));
}

int act_quant_i8(const void* x, int x_dtype, int64_t T, int64_t K, int lift_M, int8_t* xq,
                 float* x_scale, void* stream) {
  const int st = check_quant(x, x_dtype, T, K, lift_M, xq, x_scale);
  if (st != BL_OK || T == 0) return st;   // T == 0: nothing is read or written
  return status_of(bl::launch_act_quant(x, x_dtype == BL_DTYPE_BF16, T, K, lift_M, xq, x_scale,
                                        (hipStream_t)stream));
}

int act_quant_i8_group(const bl_quant_desc* descs, int64_t count, int x_dtype, int lift_M,
                       void* stream) {
  if (!descs || count < 1 || count > bl::kQuantGroupMax) return BL_EINVAL;
  struct Rg { uintptr_t lo, hi; bool out; };
  std::vector<Rg> rs;
  bl::QuantGroupArgs a;
  memset(&a, 0, sizeof a);
  int64_t blocks = 0;
  for (int64_t i = 0; i < count; ++i) {
    const bl_quant_desc& d = descs[i];
    const int st = check_quant(d.x, x_dtype, d.T, d.K, lift_M, d.xq, d.x_scale);
    if (st != BL_OK) return st;
    if (d.T == 0) continue;
    const uint64_t ke = lift_M ? (uint64_t)d.K / lift_M * (2 * lift_M - 4) : (uint64_t)d.K;
    const uint64_t xb = x_dtype == BL_DTYPE_BF16 ? 2 : 4;
    rs.push_back({(uintptr_t)d.x, (uintptr_t)d.x + (uint64_t)d.T * d.K * xb, false});
    rs.push_back({(uintptr_t)d.xq, (uintptr_t)d.xq + (uint64_t)d.T * ke, true});
    rs.push_back({(uintptr_t)d.x_scale, (uintptr_t)d.x_scale + (uint64_t)d.T * 4, true});
    const int c = a.count++;
    a.x[c] = d.x;
    a.xq[c] = d.xq;
    a.xs[c] = d.x_scale;
    a.T[c] = (int32_t)d.T;
    a.K[c] = (int32_t)d.K;
    a.block0[c] = (int32_t)blocks;
    blocks += (d.T + 3) / 4;
    if (blocks > INT32_MAX) return BL_EINVAL;
  }
  a.block0[a.count] = (int32_t)blocks;
  // inputs may be shared or overlap; an output may overlap nothing
  std::sort(rs.begin(), rs.end(), [](const Rg& p, const Rg& q) { return p.lo < q.lo; });
  uintptr_t out_hi = 0, any_hi = 0;
  for (const Rg& r : rs) {
    if (r.lo < out_hi || (r.out && r.lo < any_hi)) return BL_EINVAL;
    any_hi = std::max(any_hi, r.hi);
    if (r.out) out_hi = std::max(out_hi, r.hi);
  }
  if (a.count == 0) return BL_OK;
  return status_of(bl::launch_act_quant_group(a, x_dtype == BL_DTYPE_BF16, lift_M,
                                              (hipStream_t)stream));
}

int bitlinear_fwd(const int8_t* xq, const float* x_scale, int64_t T, int64_t K,
                  const uint8_t* codes, const uint8_t* meta, const float* gamma, int N, int M,
                  int layout, int64_t n, float* y, int32_t* acc_opt, void* stream) {
  int64_t ke = 0;
  const int st = check_fwd(xq, x_scale, T, K, codes, meta, gamma, N, M, layout, n, y, acc_opt, &ke);
  if (st != BL_OK || T == 0) return st;
  if (layout == BL_LAYOUT_SPARSE6) {
    if (K > 128 * 128) return BL_ENOTSUP;   // one projection: at most 16 step pairs per wave
    return status_of(bl::launch_fwd6(xq, x_scale, T, K, (const uint32_t*)codes, gamma, n, y,
                                     acc_opt, (hipStream_t)stream));
  }
  return status_of(bl::launch_fwd(xq, x_scale, T, ke, (const uint32_t*)codes, (const uint32_t*)meta,
                                  gamma, layout, n, y, acc_opt, (hipStream_t)stream));
}

int bitlinear_transcode6(const uint8_t* codes, const uint8_t* meta, int64_t n, int64_t K,
                         uint8_t* out, void* stream) {
  int64_t ke = 0;
  const int st = check_shape(n, K, 2, 4, BL_LAYOUT_SPARSE, &ke);
  if (st != BL_OK) return st;
  if (!aligned16(codes) || !aligned16(meta) || !aligned16(out)) return BL_EINVAL;
  size_t cb = 0, mb = 0, ob = 0;
  bitlinear_packed_bytes(n, K, 2, 4, BL_LAYOUT_SPARSE, &cb, &mb, nullptr, nullptr);
  bitlinear_packed_bytes(n, K, 2, 4, BL_LAYOUT_SPARSE6, &ob, nullptr, nullptr, nullptr);
  const uintptr_t o = (uintptr_t)out, c = (uintptr_t)codes, m = (uintptr_t)meta;
  if ((o < c + cb && c < o + ob) || (o < m + mb && m < o + ob)) return BL_EINVAL;
  return status_of(bl::launch_transcode6((const uint32_t*)codes, (const uint32_t*)meta, n, K,
                                         (uint32_t*)out, (hipStream_t)stream));
}

int bitlinear_group_table_bytes(const bl_fwd_desc* descs, int64_t count, int N, int M, int layout,
                                size_t* table_bytes, int64_t* work_items) {
  return group_sizes(descs, count, N, M, layout, 0, table_bytes, work_items);
}

int bitlinear_group_build(const bl_fwd_desc* descs, int64_t count, int N, int M, int layout,
                          void* table, size_t table_bytes, void* stream) {
  return group_build(descs, count, N, M, layout, 0, table, table_bytes, stream);
}

int bitlinear_fwd_group(const void* table, int64_t work_items, int N, int M, int layout,
                        void* stream) {
  const int st = layout == BL_LAYOUT_SPARSE6 ? (N == 2 && M == 4 ? BL_OK : BL_ENOTSUP)
                                             : check_nm(N, M, layout);
  if (st != BL_OK) return st;
  if (work_items < 0 || work_items > INT32_MAX) return BL_EINVAL;
  if (work_items == 0) return BL_OK;
  if (!aligned16(table)) return BL_EINVAL;
  if (layout == BL_LAYOUT_SPARSE6)
    return status_of(bl::launch_fwd6_group(table, work_items, (hipStream_t)stream));
  return status_of(bl::launch_fwd_group(table, work_items, layout, 0, (hipStream_t)stream));
}

int bitlinear_group_fused_table_bytes(const bl_fwd_x_desc* descs, int64_t count, int N, int M,
                                      int layout, size_t* table_bytes, int64_t* work_items) {
  std::vector<bl_fwd_desc> plain;
  const int st = fused_as_plain(descs, count, M, layout, &plain);
  if (st != BL_OK) return st;
  return group_sizes(plain.data(), count, N, M, layout, 1, table_bytes, work_items);
}

int bitlinear_group_fused_build(const bl_fwd_x_desc* descs, int64_t count, int N, int M,
                                int layout, void* table, size_t table_bytes, void* stream) {
  std::vector<bl_fwd_desc> plain;
  const int st = fused_as_plain(descs, count, M, layout, &plain);
  if (st != BL_OK) return st;
  return group_build(plain.data(), count, N, M, layout, 1, table, table_bytes, stream);
}

int bitlinear_fwd_group_fused(const void* table, int64_t work_items, int N, int M, int layout,
                              void* stream) {
  const int st = check_nm(N, M, layout);
  if (st != BL_OK) return st;
  if (layout == BL_LAYOUT_SPARSE && M != 4) return BL_ENOTSUP;
  if (work_items < 0 || work_items > INT32_MAX) return BL_EINVAL;
  if (work_items == 0) return BL_OK;
  if (!aligned16(table)) return BL_EINVAL;
  return status_of(bl::launch_fwd_group(table, work_items, layout, 1, (hipStream_t)stream));
}

int bitlinear_chain_plan(const bl_chain_layer* layers, int64_t L, int64_t T, int N, int M,
                         int layout, bl_chain_plan* plan) {
  if (!plan) return BL_EINVAL;
  int smem = 0;
  const int st = plan_chain(layers, L, T, N, M, layout, &smem);
  if (st != BL_OK) return st;
  memset(plan, 0, sizeof *plan);
  plan->table_bytes = chain_table_bytes(L);
  plan->ws_bytes = bl::chain_ws_bytes(L, T);
  plan->L = L;
  plan->T = T;
  plan->smem = smem;
  return BL_OK;
}

int bitlinear_chain_build(const bl_chain_layer* layers, int64_t L, int64_t T, int N, int M,
                          int layout, void* table, size_t table_bytes, void* stream) {
  int smem = 0;
  const int st = plan_chain(layers, L, T, N, M, layout, &smem);
  if (st != BL_OK) return st;
  if (!aligned16(table)) return BL_EINVAL;
  const size_t bytes = chain_table_bytes(L);
  if (table_bytes < bytes) return BL_ENOSPC;
  std::vector<uint8_t> img(bytes, 0);
  bl::ChainHeader hdr;
  memset(&hdr, 0, sizeof hdr);
  hdr.magic = bl::kChainMagic;
  hdr.L = (int32_t)L;
  hdr.T = (int32_t)T;
  hdr.smem = smem;
  memcpy(img.data(), &hdr, sizeof hdr);
  for (int64_t l = 0; l < L; ++l) {
    bl::ChainLayer r;
    memset(&r, 0, sizeof r);
    r.codes = (const uint32_t*)layers[l].codes;
    r.meta = (const uint32_t*)layers[l].meta;
    r.gamma = layers[l].gamma;
    r.y = layers[l].y;
    r.acc = layers[l].acc_opt;
    r.n = (int32_t)layers[l].n;
    r.K = (int32_t)layers[l].K;
    memcpy(img.data() + sizeof hdr + l * sizeof(bl::ChainLayer), &r, sizeof r);
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(table, img.data(), bytes, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);  // img is released on return
  return status_of(e);
}

int bitlinear_fwd_chain(const void* table, const bl_chain_plan* plan, const void* x0, int x_dtype,
                        void* ws, size_t ws_bytes, int64_t spin_limit, void* stream) {
  if (!plan || !aligned16(table) || !aligned16(x0) || !aligned16(ws)) return BL_EINVAL;
  if (x_dtype != BL_DTYPE_F32 && x_dtype != BL_DTYPE_BF16) return BL_ENOTSUP;
  if (plan->L < 1 || plan->L > 4096 || plan->T < 1 || plan->T > bl::kChainMaxT ||
      plan->smem < 1 || plan->smem > kChainLdsMax)
    return BL_EINVAL;
  if (ws_bytes < bl::chain_ws_bytes(plan->L, plan->T)) return BL_ENOSPC;
  // about a second of polls (each s_sleep 2 is ~128 clocks) unless the caller bounds it
  const int64_t limit = spin_limit > 0 ? spin_limit : (int64_t)1 << 24;
  return status_of(bl::launch_chain(table, plan->L, plan->T, plan->smem, x0,
                                    x_dtype == BL_DTYPE_BF16, ws, limit, (hipStream_t)stream));
}

int bitlinear_bwd_workspace_bytes(int64_t T, int64_t n, int64_t K, size_t* ws_bytes) {
  if (T < 0 || T > INT32_MAX || n < 1 || n > INT32_MAX || K < 1 || K > INT32_MAX || !ws_bytes)
    return BL_EINVAL;
  *ws_bytes = bl::bwd_workspace(T, n, K).total;
  return BL_OK;
}

int bitlinear_bwd(const uint16_t* dy, int64_t T, int64_t n, const int8_t* xq,
                  const float* x_scale, int64_t K, const uint8_t* codes, const uint8_t* meta,
                  const float* gamma, int N, int M, int layout, float* dx, float* dw, int flags,
                  void* ws, size_t ws_bytes, void* stream) {
  const int st = check_bwd(dy, T, n, xq, x_scale, K, codes, meta, gamma, N, M, layout, dx, dw,
                           flags);
  if (st != BL_OK) return st;
  if (!ws || ((uintptr_t)ws & 255u)) return BL_EINVAL;
  if (ws_bytes < bl::bwd_workspace(T, n, K).total) return BL_ENOSPC;
  if (T == 0 && !dw) return BL_OK;   // no rows of dx: nothing to enqueue
  return status_of(bl::launch_bwd(dy, T, n, xq, x_scale, K, (const uint32_t*)codes,
                                  (const uint32_t*)meta, gamma, N, M, layout, dx, dw, flags, ws,
                                  (hipStream_t)stream));
}

int bitlinear_bwd_group_plan(const bl_bwd_desc* descs, int64_t count, int64_t T, int N, int M,
                             int layout, bl_bwd_group_plan* plan) {
  if (!plan) return BL_EINVAL;
  BwdGroupPlan P;
  const int st = plan_bwd_group(descs, count, T, N, M, layout, nullptr, &P);
  if (st != BL_OK) return st;
  memset(plan, 0, sizeof *plan);
  plan->table_bytes = P.table_bytes;
  plan->ws_bytes = P.ws_bytes;
  plan->prep_blocks = P.prep_blocks;
  plan->jobs = (int64_t)P.jobs.size();
  plan->N = N;
  plan->M = M;
  plan->layout = layout;
  return BL_OK;
}

int bitlinear_bwd_group_build(const bl_bwd_desc* descs, int64_t count, int64_t T, int N, int M,
                              int layout, void* ws, size_t ws_bytes, void* table,
                              size_t table_bytes, void* stream) {
  if (!ws || ((uintptr_t)ws & 255u) || !aligned16(table)) return BL_EINVAL;
  BwdGroupPlan P;
  const int st = plan_bwd_group(descs, count, T, N, M, layout, (uint8_t*)ws, &P);
  if (st != BL_OK) return st;
  if (ws_bytes < P.ws_bytes || table_bytes < P.table_bytes) return BL_ENOSPC;
  std::vector<uint8_t> img(P.table_bytes, 0);
  bl::BwdHeader hdr;
  memset(&hdr, 0, sizeof hdr);
  hdr.magic = bl::kBwdMagic;
  hdr.layout = layout;
  hdr.N = N;
  hdr.M = M;
  hdr.T = T;
  hdr.prep_items = (int32_t)P.prep.size();
  hdr.prep_blocks = (int32_t)P.prep_blocks;
  hdr.jobs = (int32_t)P.jobs.size();
  hdr.segs = (int32_t)P.segs.size();
  hdr.prep_off = (int64_t)P.prep_off;
  hdr.jobs_off = (int64_t)P.jobs_off;
  hdr.segs_off = (int64_t)P.segs_off;
  hdr.t32 = P.t32;
  memcpy(img.data(), &hdr, sizeof hdr);
  if (!P.prep.empty())
    memcpy(img.data() + P.prep_off, P.prep.data(), P.prep.size() * sizeof(bl::BwdPrep));
  if (!P.jobs.empty())
    memcpy(img.data() + P.jobs_off, P.jobs.data(), P.jobs.size() * sizeof(bl::BwdJob));
  if (!P.segs.empty())
    memcpy(img.data() + P.segs_off, P.segs.data(), P.segs.size() * sizeof(bl::BwdSeg));
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(table, img.data(), P.table_bytes, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);  // img is released on return
  return status_of(e);
}

int bitlinear_bwd_group(const void* table, const bl_bwd_group_plan* plan, void* stream) {
  if (!plan || !aligned16(table)) return BL_EINVAL;
  const int st = check_nm(plan->N, plan->M, plan->layout);
  if (st != BL_OK) return st;
  if (plan->prep_blocks < 0 || plan->prep_blocks > INT32_MAX || plan->jobs < 0 ||
      plan->jobs > INT32_MAX)
    return BL_EINVAL;
  return status_of(bl::launch_bwd_group(table, plan->prep_blocks, plan->jobs, plan->layout,
                                        plan->M, (hipStream_t)stream));
}

}  // extern "C"
