"""C ABI checks that need no GPU: the library loads, exports every symbol the header declares,
reports packed sizes that match the layout definition, and rejects bad arguments before it
touches the HIP runtime (fake, never dereferenced device addresses are passed)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitlinear.h")


@pytest.fixture(scope="module")
def L():
    from sparsity_amd import bitlinear as B
    if not os.path.exists(B.LIB_PATH):
        from sparsity_amd import build
        build.build()
    return B


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert {"bitlinear_pack", "act_quant_i8", "bitlinear_fwd", "bitlinear_packed_bytes",
            "bitlinear_strerror", "bitlinear_layout_version"} <= set(names)
    lib = ctypes.CDLL(L.LIB_PATH)
    for nm in names:
        assert hasattr(lib, nm), nm


def test_layout_version_and_strerror(L):
    assert L.lib().bitlinear_layout_version() == 2
    for st in (0, -22, -95, -28, -5, 7):
        assert isinstance(L.lib().bitlinear_strerror(st), bytes)


@pytest.mark.parametrize("n,K,N,M,layout", [
    (1, 64, 2, 4, 0), (6912, 2560, 2, 4, 0), (2560, 6912, 2, 4, 0), (11008, 4096, 2, 4, 0),
    (4096, 4096, 6, 8, 0), (45, 384, 6, 8, 0), (33, 288, 2, 4, 1), (33, 288, 6, 8, 1),
    (8640, 3200, 2, 4, 0), (3200, 8640, 2, 4, 0), (100, 96, 4, 4, 1),
    (4096, 4096, 14, 16, 0), (45, 512, 14, 16, 0), (33, 288, 14, 16, 1),
    (45, 240, 4, 6, 0), (33, 480, 8, 10, 0), (33, 384, 10, 12, 0), (33, 224, 12, 14, 0),
    (33, 96, 4, 6, 1), (33, 160, 8, 10, 1), (33, 96, 10, 12, 1), (33, 224, 12, 14, 1)])
def test_packed_bytes_match_layout(L, n, K, N, M, layout):
    st, cb, mb, ke, ws = L.bitlinear_packed_bytes(n, K, N, M, layout)
    assert st == 0
    ncode, nmeta, _ = O.packed_dwords(n, K, N, M, layout)
    assert cb == 4 * ncode and mb == 4 * nmeta and ke == O.k_eff(K, N, M, layout) and ws > 0


@pytest.mark.parametrize("n,K,N,M,layout,want", [
    (64, 100, 2, 4, 0, -22),       # K % 64
    (64, 192, 6, 8, 0, -22),       # 6:8 needs K % 128
    (64, 48, 2, 4, 1, -22),        # DENSE2 needs K % 32
    (0, 256, 2, 4, 0, -22),        # n >= 1
    (64, 256, 3, 4, 0, -95),       # SPARSE supports 2:4 and 6:8 only
    (64, 256, 2, 4, 7, -95),       # unknown layout
    (64, 256, 5, 4, 1, -95),       # N > M
    (64, 256, 2, 32, 1, -95),      # M in {4, 8, 16}
    (64, 128, 14, 16, 0, -22),     # 14:16 needs K % 256
    (64, 256, 12, 16, 0, -95),     # SPARSE windows are (M-2):M
    (64, 256, 6, 16, 0, -95),
    (1 << 20, 1 << 12, 2, 4, 0, -22),  # n*K >= 2^32
    (64, 120, 4, 6, 0, -22),       # 4:6 needs K % 48 (whole lifted MFMA steps)
    (64, 220, 8, 10, 0, -22),      # 8:10 needs K % 40
    (64, 240, 10, 12, 0, -22),     # 10:12 needs K % 192
    (64, 168, 12, 14, 0, -22),     # 12:14 needs K % 112
    (64, 240, 3, 6, 0, -95),       # (M-2):M only
    (64, 224, 2, 7, 1, -95),       # even M only
    (64, 48, 4, 6, 1, -22),        # DENSE2 4:6 needs K % 96
])
def test_packed_bytes_rejects(L, n, K, N, M, layout, want):
    assert L.bitlinear_packed_bytes(n, K, N, M, layout)[0] == want


FAKE = 0x7F0000000000   # 16-byte aligned, never dereferenced (validation fails before use)


def test_pack_rejects_before_launch(L):
    P = FAKE
    ok = dict(W=P, n=64, K=256, N=2, M=4, layout=0, codes=P, meta=P, gamma=P, ws=P, ws_bytes=1 << 24)

    def call(**kw):
        a = dict(ok, **kw)
        return L.bitlinear_pack(a["W"], a["n"], a["K"], a["N"], a["M"], a["layout"], a["codes"],
                                a["meta"], a["gamma"], a["ws"], a["ws_bytes"], None)
    assert call(K=100) == -22
    assert call(N=3) == -95
    assert call(W=None) == -22
    assert call(W=P + 4) == -22
    assert call(codes=P + 8) == -22
    assert call(meta=None) == -22
    assert call(layout=1, meta=P) == -22          # DENSE2 takes no meta buffer
    assert call(gamma=None) == -22
    assert call(ws=None) == -22
    assert call(ws_bytes=16) == -28


def test_act_quant_rejects_before_launch(L):
    P = FAKE
    assert L.act_quant_i8(P, 2, 4, 256, 0, P, P, None) == -95        # dtype
    assert L.act_quant_i8(P, 0, 4, 256, 4, P, P, None) == -22        # lift_M
    assert L.act_quant_i8(P, 0, 4, 264, 16, P, P, None) == -22       # lift 16 needs K % 16
    assert L.act_quant_i8(P, 0, 4, 256, 7, P, P, None) == -22        # odd lift
    assert L.act_quant_i8(P, 0, 4, 256, 18, P, P, None) == -22       # M > 16
    assert L.act_quant_i8(P, 0, 4, 252, 6, P, P, None) == -22        # lift 6 needs K % 24
    assert L.act_quant_i8(P, 0, 4, 308, 14, P, P, None) == -22       # lift 14 needs K % 56
    assert L.act_quant_i8(P, 0, 0, 240, 6, P, P, None) == 0          # valid, nothing enqueued
    assert L.act_quant_i8(P, 0, 0, 280, 10, P, P, None) == 0
    assert L.act_quant_i8(P, 0, 0, 216, 12, P, P, None) == 0
    assert L.act_quant_i8(P, 0, -1, 256, 0, P, P, None) == -22       # T < 0
    assert L.act_quant_i8(P, 0, 4, 100, 0, P, P, None) == -22        # K % 8
    assert L.act_quant_i8(None, 0, 4, 256, 0, P, P, None) == -22
    assert L.act_quant_i8(P, 1, 4, 256, 0, P + 2, P, None) == -22
    assert L.act_quant_i8(P, 0, 0, 256, 0, P, P, None) == 0          # T == 0: nothing enqueued
    assert L.act_quant_i8(None, 0, 0, 256, 0, None, None, None) == 0


def test_fwd_rejects_before_launch(L):
    P = FAKE
    ok = dict(xq=P, xs=P, T=4, K=256, codes=P, meta=P, gamma=P, N=2, M=4, layout=0, n=64, y=P, acc=None)

    def call(**kw):
        a = dict(ok, **kw)
        return L.bitlinear_fwd(a["xq"], a["xs"], a["T"], a["K"], a["codes"], a["meta"], a["gamma"],
                               a["N"], a["M"], a["layout"], a["n"], a["y"], a["acc"], None)
    assert call(K=100) == -22
    assert call(N=6, M=8, K=192) == -22
    assert call(N=1, M=4) == -95
    assert call(T=-1) == -22
    assert call(xq=P + 1) == -22
    assert call(y=None) == -22
    assert call(meta=None) == -22
    assert call(layout=1, meta=P) == -22
    assert call(acc=P + 2) == -22
    assert call(T=0) == 0
    assert call(T=0, xq=None, xs=None, y=None) == 0


@pytest.mark.parametrize("n,K", [(1, 64), (33, 192), (6912, 2560), (2560, 6912), (45, 384)])
def test_sparse6_packed_bytes(L, n, K):
    st, cb, mb, ke, ws = L.bitlinear_packed_bytes(n, K, 2, 4, L.BL_LAYOUT_SPARSE6)
    assert st == 0 and mb == 0 and ke == K and ws == 0
    assert cb == 4 * O.packed6_dwords(n, K)[0]
    # 0.75 of the 2:4 codes + meta once the K axis is whole step pairs
    _, cb2, mb2, _, _ = L.bitlinear_packed_bytes(n, K, 2, 4, 0)
    if K % 128 == 0:
        assert 4 * cb == 3 * (cb2 + mb2)
    assert L.bitlinear_packed_bytes(n, K, 6, 8, L.BL_LAYOUT_SPARSE6)[0] == -95
    assert L.bitlinear_packed_bytes(n, K + 32, 2, 4, L.BL_LAYOUT_SPARSE6)[0] == -22


def test_sparse6_rejects_before_launch(L):
    P, S6 = FAKE, L.BL_LAYOUT_SPARSE6
    ok = dict(xq=P, xs=P, T=4, K=256, codes=P, meta=None, gamma=P, N=2, M=4, layout=S6, n=64, y=P,
              acc=None)

    def call(**kw):
        a = dict(ok, **kw)
        return L.bitlinear_fwd(a["xq"], a["xs"], a["T"], a["K"], a["codes"], a["meta"], a["gamma"],
                               a["N"], a["M"], a["layout"], a["n"], a["y"], a["acc"], None)
    assert call(meta=P) == -22                     # no index dwords
    assert call(T=33) == -95                       # a decode format
    assert call(N=6, M=8, K=256) == -95
    assert call(K=100) == -22
    assert call(K=16384 + 64) == -95               # one projection: K <= 16384
    assert call(codes=P + 4) == -22
    assert call(T=0) == 0
    # re-encoding: the input follows the 2:4 rules, out may not overlap the inputs
    tc = L.bitlinear_transcode6
    assert tc(P, P + (1 << 30), 64, 100, P + (2 << 30), None) == -22
    assert tc(P, P + (1 << 30), 0, 256, P + (2 << 30), None) == -22
    assert tc(P + 8, P + (1 << 30), 64, 256, P + (2 << 30), None) == -22
    assert tc(P, P + (1 << 30), 64, 256, P + 1024, None) == -22     # overlaps codes
    assert tc(P, P + (1 << 30), 64, 256, P + (1 << 30) - 16, None) == -22   # overlaps meta
    # decode group: plain tables only
    arr = (L.BlFwdDesc * 1)(_desc(L, meta=None))
    st, tb, wi = L.bitlinear_group_table_bytes(arr, 2, 4, S6)
    assert st == 0 and wi >= 1
    assert L.bitlinear_group_table_bytes((L.BlFwdDesc * 1)(_desc(L)), 2, 4, S6)[0] == -22
    assert L.bitlinear_group_table_bytes((L.BlFwdDesc * 1)(_desc(L, meta=None, T=33)), 2, 4,
                                         S6)[0] == -95
    assert L.bitlinear_group_table_bytes(arr, 6, 8, S6)[0] == -95
    assert L.bitlinear_fwd_group(FAKE, 3, 6, 8, S6, None) == -95
    xarr = (L.BlFwdXDesc * 1)(L.BlFwdXDesc(x=P, T=4, K=256, codes=P, meta=None, gamma=P, n=64,
                                           y=P + (1 << 34), acc_opt=None))
    assert L.bitlinear_group_fused_table_bytes(xarr, 2, 4, S6)[0] == -95
    # the training-side calls do not take the decode format
    assert L.bitlinear_pack(P, 64, 256, 2, 4, S6, P, None, P, P, 1 << 20, None) == -95


def test_product_path_never_imports_oracle():
    pkg = os.path.join(ROOT, "sparsity_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                txt = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\boracle\b", txt), f


def _desc(L, slot=0, **kw):
    """A group descriptor: inputs share FAKE (allowed), the output sits in its own 16 GiB slot."""
    P = FAKE
    a = dict(xq=P, x_scale=P, T=4, K=256, codes=P, meta=P, gamma=P, n=100,
             y=FAKE + (slot + 1) * (16 << 30), acc_opt=None)
    a.update(kw)
    return L.BlFwdDesc(**a)


def test_group_sizes_and_rejects_before_launch(L):
    arr = (L.BlFwdDesc * 3)(_desc(L), _desc(L, 1, n=6912, K=2560, T=16), _desc(L, 2, T=0, xq=None))
    st, tb, wi = L.bitlinear_group_table_bytes(arr, 2, 4, 0)
    assert st == 0
    # 16 panels of 32 rows per work item (1 + 14 items; the T == 0 projection has none), laid out
    # over the 8 XCDs' launch positions, padded to a whole number of rounds
    assert wi % 8 == 0 and 15 <= wi <= 15 + 8 * 8
    assert tb >= 64 + 3 * 72 + 8 * wi and tb % 16 == 0

    def one(**kw):
        return L.bitlinear_group_table_bytes((L.BlFwdDesc * 1)(_desc(L, **kw)), 2, 4, 0)[0]
    assert one(T=33) == -22                       # a group is decode-sized: T <= 32
    assert one(T=-1) == -22
    assert one(K=100) == -22
    assert one(xq=FAKE + 4) == -22
    assert one(meta=None) == -22
    assert one(acc_opt=FAKE + 2) == -22
    assert L.bitlinear_group_table_bytes((L.BlFwdDesc * 1)(_desc(L)), 3, 4, 0)[0] == -95
    assert L.bitlinear_group_table_bytes((L.BlFwdDesc * 1)(_desc(L, meta=None)), 2, 4, 1)[0] == 0
    lib = L.lib()
    assert lib.bitlinear_group_table_bytes(None, 1, 2, 4, 0, None, None) == -22
    assert lib.bitlinear_group_table_bytes(arr, 0, 2, 4, 0, None, None) == -22
    # build: table too small or misaligned is rejected before anything is copied
    assert L.bitlinear_group_build(arr, 2, 4, 0, FAKE, tb - 16, None) == -28
    assert L.bitlinear_group_build(arr, 2, 4, 0, FAKE + 8, tb, None) == -22
    # launch: argument checks only
    assert L.bitlinear_fwd_group(FAKE, -1, 2, 4, 0, None) == -22
    assert L.bitlinear_fwd_group(FAKE + 4, 3, 2, 4, 0, None) == -22
    assert L.bitlinear_fwd_group(FAKE, 3, 2, 4, 9, None) == -95
    assert L.bitlinear_fwd_group(None, 0, 2, 4, 0, None) == 0   # nothing to launch


def test_group_rejects_overlapping_outputs(L):
    """A decode group's outputs (y, acc_opt) may overlap no other output and no input; inputs may
    be shared.  A T == 0 projection touches nothing."""
    def sizes(*descs, fused=False):
        if fused:
            return L.bitlinear_group_fused_table_bytes((L.BlFwdXDesc * len(descs))(*descs), 2, 4, 0)[0]
        return L.bitlinear_group_table_bytes((L.BlFwdDesc * len(descs))(*descs), 2, 4, 0)[0]
    S = 16 << 30
    assert sizes(_desc(L, 0), _desc(L, 1)) == 0
    assert sizes(_desc(L, 0), _desc(L, 0)) == -22                       # the same y twice
    assert sizes(_desc(L, 0), _desc(L, 1, y=FAKE + S + 4 * 4 * 100 - 16)) == -22   # y ranges overlap
    assert sizes(_desc(L, 0, y=FAKE)) == -22                            # y over the inputs
    assert sizes(_desc(L, 0, acc_opt=FAKE + S + 16)) == -22             # acc over y
    assert sizes(_desc(L, 0, acc_opt=FAKE + 3 * S)) == 0
    assert sizes(_desc(L, 0), _desc(L, 1, acc_opt=FAKE + S)) == -22     # acc over another y
    assert sizes(_desc(L, 0), _desc(L, 1, T=0, y=FAKE + S)) == 0        # T == 0 writes nothing
    assert sizes(_xdesc(L, 0), _xdesc(L, 0), fused=True) == -22
    assert sizes(_xdesc(L, 0, y=FAKE + 2 * 4 * 256 - 16), fused=True) == -22   # y over the bf16 rows
    assert sizes(_xdesc(L, 0, y=FAKE + 2 * 4 * 256 + 16), fused=True) == -22   # y over codes


def _up32(v):
    return (v + 31) // 32 * 32


@pytest.mark.parametrize("T,n,K", [(8192, 3200, 3200), (8192, 8640, 3200), (8192, 3200, 8640),
                                   (1, 45, 64), (0, 100, 256), (33, 96, 128)])
def test_bwd_workspace_bytes(L, T, n, K):
    """Four bf16 operands (W_eff^T, padded dY when n % 32, dY^T, X^^T), 256-byte aligned."""
    st, ws = L.bitlinear_bwd_workspace_bytes(T, n, K)
    assert st == 0
    up = lambda v: (v + 255) // 256 * 256
    n32, t32 = _up32(n), _up32(T)
    want = up(2 * K * n32) + up(2 * T * n32 if n32 != n else 0) + up(2 * n * t32) + up(2 * K * t32)
    assert ws == want
    assert L.bitlinear_bwd_workspace_bytes(-1, n, K)[0] == -22
    assert L.bitlinear_bwd_workspace_bytes(T, 0, K)[0] == -22


def test_bwd_rejects_before_launch(L):
    P = FAKE
    ws_ok = 1 << 30
    ok = dict(dy=P, T=64, n=128, xq=P, xs=P, K=256, codes=P, meta=P, gamma=P, N=2, M=4, layout=0,
              dx=P, dw=P, flags=0, ws=P, wsb=ws_ok)

    def call(**kw):
        a = dict(ok, **kw)
        return L.bitlinear_bwd(a["dy"], a["T"], a["n"], a["xq"], a["xs"], a["K"], a["codes"],
                               a["meta"], a["gamma"], a["N"], a["M"], a["layout"], a["dx"], a["dw"],
                               a["flags"], a["ws"], a["wsb"], None)
    assert call(K=100) == -22                     # packed-layout shape rules
    assert call(N=1, M=4) == -95
    assert call(N=6, M=8, K=192) == -22
    assert call(T=-1) == -22
    assert call(flags=4) == -22
    assert call(dx=None, dw=None) == -22          # nothing asked for
    assert call(dy=P + 2) == -22
    assert call(dy=None) == -22
    assert call(xq=P + 1) == -22
    assert call(xs=P + 2) == -22
    assert call(codes=P + 8) == -22
    assert call(meta=None) == -22
    assert call(layout=1, meta=P) == -22
    assert call(dx=P + 4) == -22
    assert call(dw=P + 4) == -22
    assert call(ws=P + 128) == -22
    assert call(wsb=L.bitlinear_bwd_workspace_bytes(64, 128, 256)[1] - 1) == -28
    # operands of 2^31 bytes or more (32-bit offsets inside the kernels)
    assert call(T=1 << 20, n=1024, K=256) == -22
    # dX only with no tokens: nothing to do, nothing enqueued, token buffers may be NULL
    assert call(T=0, dw=None, dy=None, xq=None, xs=None) == 0


GB = 1 << 30


def _bdesc(L, slot, **kw):
    """A grouped-backward descriptor whose buffers sit in their own 1 GiB slot of fake space."""
    base = FAKE + slot * 16 * GB
    a = dict(dy=base, xq=base + GB, x_scale=base + 2 * GB, K=256, codes=base + 3 * GB,
             meta=base + 4 * GB, gamma=base + 5 * GB, n=128, dx=base + 6 * GB, dw=base + 7 * GB,
             flags=0, reserved=0)
    a.update(kw)
    return L.BlBwdDesc(**a)


def _bplan(L, descs, T=64, N=2, M=4, layout=0):
    return L.bitlinear_bwd_group_plan((L.BlBwdDesc * len(descs))(*descs), T, N, M, layout)


def test_bwd_group_plan_sizes(L):
    """One projection needs the workspace of bitlinear_bwd; projections sharing an activation
    share its transposed copy; jobs fill whole rounds of the 8 XCDs."""
    T, n, K = 300, 300, 640
    st, plan = _bplan(L, [_bdesc(L, 0, n=n, K=K)], T=T)
    assert st == 0
    assert plan.ws_bytes == L.bitlinear_bwd_workspace_bytes(T, n, K)[1]
    assert (plan.N, plan.M, plan.layout) == (2, 4, 0)
    tiles_dx = 2 * 3                         # ceil(300 / 256) x ceil(640 / 256)
    tiles_dw = 2 * 3
    assert plan.jobs % 8 == 0 and tiles_dx + tiles_dw <= plan.jobs < tiles_dx + tiles_dw + 8 * 8
    # prep blocks: W_eff^T (K/M groups x n32/2 row pairs, 256 per block), dY pad (T x n32),
    # dY^T and X^^T (64 x 64 tiles)
    n32, tt = _up32(n), (T + 63) // 64
    want = (-(-(K // 4 * n32 // 2) // 256) + -(-(T * n32) // 256) + tt * ((n + 63) // 64)
            + tt * ((K + 63) // 64))
    assert plan.prep_blocks == want
    up = lambda v: (v + 255) // 256 * 256
    t32 = _up32(T)
    # two projections reading one activation (same xq, x_scale, K) and summing into one dx
    a = _bdesc(L, 0, n=n, K=K)
    b = _bdesc(L, 1, n=n, K=K, xq=a.xq, x_scale=a.x_scale, dx=a.dx, flags=1)
    st, p2 = _bplan(L, [a, b], T=T)
    assert st == 0
    assert p2.ws_bytes == 2 * plan.ws_bytes - up(2 * K * t32)
    assert p2.prep_blocks == 2 * plan.prep_blocks - tt * ((K + 63) // 64)
    # T == 0: dx untouched, dw zeroed by the product launch; nothing to prepare
    st, p0 = _bplan(L, [_bdesc(L, 0, dy=None, xq=None, x_scale=None)], T=0)
    assert st == 0 and p0.prep_blocks == 0 and p0.ws_bytes == 0 and p0.jobs == 8
    st, p0 = _bplan(L, [_bdesc(L, 0, dw=None)], T=0)
    assert st == 0 and p0.jobs == 0


def test_bwd_group_rejects_before_launch(L):
    ok = _bdesc(L, 0)
    assert _bplan(L, [ok])[0] == 0
    assert _bplan(L, [_bdesc(L, 0, K=100)])[0] == -22
    assert _bplan(L, [ok], N=1)[0] == -95
    assert _bplan(L, [ok], T=-1)[0] == -22
    assert _bplan(L, [_bdesc(L, 0, flags=4)])[0] == -22
    assert _bplan(L, [_bdesc(L, 0, dx=None, dw=None)])[0] == -22
    assert _bplan(L, [_bdesc(L, 0, dy=FAKE + 2)])[0] == -22
    assert _bplan(L, [_bdesc(L, 0, meta=None)])[0] == -22
    lib = L.lib()
    assert lib.bitlinear_bwd_group_plan(None, 1, 64, 2, 4, 0, ctypes.byref(L.BlBwdGroupPlan())) == -22
    assert lib.bitlinear_bwd_group_plan((L.BlBwdDesc * 1)(ok), 0, 64, 2, 4, 0,
                                        ctypes.byref(L.BlBwdGroupPlan())) == -22
    assert lib.bitlinear_bwd_group_plan((L.BlBwdDesc * 1)(ok), 1, 64, 2, 4, 0, None) == -22
    # outputs: a shared dx must be the same buffer with the same K; nothing else may overlap
    b = _bdesc(L, 1)
    assert _bplan(L, [ok, _bdesc(L, 1, dx=ok.dx)])[0] == 0
    assert _bplan(L, [ok, _bdesc(L, 1, dx=ok.dx + 64)])[0] == -22       # partial overlap
    assert _bplan(L, [ok, _bdesc(L, 1, dx=ok.dx, K=512)])[0] == -22      # same start, other K
    assert _bplan(L, [ok, _bdesc(L, 1, dw=ok.dw)])[0] == -22             # dw shared
    assert _bplan(L, [ok, _bdesc(L, 1, dw=ok.dx + 1024)])[0] == -22      # dw inside a dx
    assert _bplan(L, [ok, _bdesc(L, 1, dx=ok.dw)])[0] == -22             # dx on a dw
    assert _bplan(L, [_bdesc(L, 0, dw=ok.dx + 64 * 256 * 4)])[0] == 0    # adjacent: fine
    # an output over any input of the group
    assert _bplan(L, [ok, _bdesc(L, 1, dx=ok.dy)])[0] == -22
    assert _bplan(L, [ok, _bdesc(L, 1, dw=ok.xq)])[0] == -22
    assert _bplan(L, [ok, _bdesc(L, 1, dw=ok.gamma - 8)])[0] == -22
    assert _bplan(L, [ok, _bdesc(L, 1, dx=ok.codes + 2048)])[0] == -22   # codes: 4096 bytes
    assert _bplan(L, [ok, _bdesc(L, 1, dx=ok.codes + 4096)])[0] == 0
    assert _bplan(L, [ok, b])[0] == 0
    # build: workspace / table checks come before anything is copied
    st, plan = _bplan(L, [ok, b])
    arr = (L.BlBwdDesc * 2)(ok, b)
    W, TB = FAKE + 64 * 16 * GB, FAKE + 80 * 16 * GB
    assert L.bitlinear_bwd_group_build(arr, 64, 2, 4, 0, W, plan.ws_bytes - 1, TB,
                                       plan.table_bytes, None) == -28
    assert L.bitlinear_bwd_group_build(arr, 64, 2, 4, 0, W, plan.ws_bytes, TB,
                                       plan.table_bytes - 16, None) == -28
    assert L.bitlinear_bwd_group_build(arr, 64, 2, 4, 0, W + 128, plan.ws_bytes, TB,
                                       plan.table_bytes, None) == -22
    assert L.bitlinear_bwd_group_build(arr, 64, 2, 4, 0, W, plan.ws_bytes, TB + 8,
                                       plan.table_bytes, None) == -22
    # launch: argument checks only
    assert L.bitlinear_bwd_group(TB, None, None) == -22
    assert L.bitlinear_bwd_group(TB + 4, plan, None) == -22
    bad = L.BlBwdGroupPlan.from_buffer_copy(plan)
    bad.layout = 7
    assert L.bitlinear_bwd_group(TB, bad, None) == -95
    bad = L.BlBwdGroupPlan.from_buffer_copy(plan)
    bad.jobs = -1
    assert L.bitlinear_bwd_group(TB, bad, None) == -22


def _pdesc(L, slot, **kw):
    base = FAKE + slot * 16 * GB
    a = dict(W=base, n=128, K=256, codes=base + GB, meta=base + 2 * GB, gamma=base + 3 * GB)
    a.update(kw)
    return L.BlPackDesc(**a)


def _pplan(L, descs, N=2, M=4, layout=0):
    return L.bitlinear_pack_group_plan((L.BlPackDesc * len(descs))(*descs), N, M, layout)


def test_pack_group_plan_and_rejects_before_launch(L):
    """Tiles of 32 rows x 256 columns per master, dealt in reverse master order; one workspace
    slice per master; the single call's shape and alignment rules; no output overlaps."""
    a, b = _pdesc(L, 0, n=300, K=640), _pdesc(L, 1, n=64, K=256)
    st, plan = _pplan(L, [a, b])
    assert st == 0
    assert plan.count == 2 and plan.pack_blocks == 10 * 3 + 2 * 1
    assert plan.table_bytes == 64 + 2 * 64
    up = lambda b: (b + 255) // 256 * 256
    wa = L.bitlinear_packed_bytes(300, 640, 2, 4, 0)[4]
    wb = L.bitlinear_packed_bytes(64, 256, 2, 4, 0)[4]
    assert plan.ws_bytes == up(wa) + up(wb)     # each master's bitlinear_pack workspace
    assert _pplan(L, [_pdesc(L, 0, K=100)])[0] == -22
    assert _pplan(L, [a], N=3)[0] == -95
    assert _pplan(L, [_pdesc(L, 0, W=FAKE + 4)])[0] == -22
    assert _pplan(L, [_pdesc(L, 0, gamma=FAKE + 3 * GB + 4)])[0] == -22
    assert _pplan(L, [_pdesc(L, 0, meta=None)])[0] == -22
    assert _pplan(L, [_pdesc(L, 0, meta=FAKE + 2 * GB)], layout=1)[0] == -22
    assert _pplan(L, [_pdesc(L, 0, meta=None)], layout=1)[0] == 0
    lib = L.lib()
    assert lib.bitlinear_pack_group_plan(None, 1, 2, 4, 0, ctypes.byref(L.BlPackGroupPlan())) == -22
    assert lib.bitlinear_pack_group_plan((L.BlPackDesc * 1)(a), 0, 2, 4, 0,
                                         ctypes.byref(L.BlPackGroupPlan())) == -22
    # masters may be shared; outputs may not overlap each other or a master
    assert _pplan(L, [a, _pdesc(L, 1, W=a.W)])[0] == 0
    assert _pplan(L, [a, _pdesc(L, 1, codes=a.codes)])[0] == -22
    assert _pplan(L, [a, _pdesc(L, 1, gamma=a.codes + 16)])[0] == -22
    assert _pplan(L, [a, _pdesc(L, 1, meta=a.W + 4096)])[0] == -22
    assert _pplan(L, [_pdesc(L, 0, codes=FAKE + 1024)])[0] == -22   # own output inside own W
    # build and launch argument checks (nothing is copied or launched)
    arr = (L.BlPackDesc * 2)(a, b)
    W, TB = FAKE + 64 * 16 * GB, FAKE + 80 * 16 * GB
    assert L.bitlinear_pack_group_build(arr, 2, 4, 0, W, plan.ws_bytes - 1, TB, plan.table_bytes,
                                        None) == -28
    assert L.bitlinear_pack_group_build(arr, 2, 4, 0, W, plan.ws_bytes, TB, plan.table_bytes - 16,
                                        None) == -28
    assert L.bitlinear_pack_group_build(arr, 2, 4, 0, W + 16, plan.ws_bytes, TB, plan.table_bytes,
                                        None) == -22
    assert L.bitlinear_pack_group(TB, None, None) == -22
    bad = L.BlPackGroupPlan.from_buffer_copy(plan)
    bad.N = 3
    assert L.bitlinear_pack_group(TB, bad, None) == -95
    bad = L.BlPackGroupPlan.from_buffer_copy(plan)
    bad.pack_blocks = 0
    assert L.bitlinear_pack_group(TB, bad, None) == -22


def _gdesc(L, slot, **kw):
    """A grouped-prefill descriptor whose buffers sit in their own 1 GiB slots of fake space."""
    base = FAKE + slot * 16 * GB
    a = dict(xq=base, x_scale=base + GB, T=300, K=640, codes=base + 2 * GB, meta=base + 3 * GB,
             gamma=base + 4 * GB, n=300, y=base + 5 * GB, acc_opt=None)
    a.update(kw)
    return L.BlFwdDesc(**a)


def _gplan(L, descs, N=2, M=4, layout=0):
    return L.bitlinear_gemm_group_plan((L.BlFwdDesc * len(descs))(*descs), N, M, layout)


def test_gemm_group_plan_xcd_slabs(L):
    """Token tiles that divide by 8 in every projection: each XCD takes the same eighth of every
    projection's tiles, so the launch holds exactly the tiles (no padding jobs); one projection
    whose token tiles do not divide by 8 sends the group back to the run plan."""
    a = _gdesc(L, 0, T=1024, n=300, K=640)     # 2 row tiles x 8 token tiles
    b = _gdesc(L, 1, T=2048, n=1000, K=256)    # 4 x 16
    c = _gdesc(L, 2, T=1024, n=45, K=640, xq=a.xq, x_scale=a.x_scale)   # 1 x 8, shares a's rows
    st, plan = _gplan(L, [a, b, c])
    assert st == 0
    assert plan.jobs == 16 + 64 + 8
    assert plan.table_bytes == (64 + 3 * 72 + 15) // 16 * 16 + 16 * plan.jobs
    # T = 129 (2 token tiles) does not divide: the run plan pads every XCD to the depth of the
    # deepest one (a's 16 tiles in one run)
    st, plan2 = _gplan(L, [a, _gdesc(L, 1, T=129, n=64)])
    assert st == 0 and plan2.jobs == 8 * 16


def test_gemm_group_plan_and_rejects_before_launch(L):
    """256 x 128 output tiles per projection, runs of up to 64 tiles dealt to the least-loaded XCD
    (heaviest tiles first), launch position p * 8 + x; bitlinear_fwd's rules with T > 128; no
    output overlaps an input or another output."""
    a = _gdesc(L, 0)                                     # 2 x 3 tiles, K_eff 320
    b = _gdesc(L, 1, T=1000, n=1000, K=256)              # 4 x 8 tiles, K_eff 128
    st, plan = _gplan(L, [a, b])
    assert st == 0
    assert plan.jobs == 8 * 32                            # b's 32 tiles on one XCD set the depth
    assert plan.table_bytes == 64 + 144 + 16 * plan.jobs  # header, 2 x 72 (16-aligned), jobs
    assert (plan.N, plan.M, plan.layout) == (2, 4, 0)
    # 2048 tiles in 32 runs of 64: four runs per XCD, no padding
    st, plan2 = _gplan(L, [_gdesc(L, 0, T=8192, n=8192, K=256)])
    assert st == 0 and plan2.jobs == 2048
    # the big projection's runs first, four per XCD; the small one's two tiles go to one XCD
    st, plan3 = _gplan(L, [_gdesc(L, 0, T=129, n=64), _gdesc(L, 1, T=8192, n=8192, K=256)])
    assert st == 0 and plan3.jobs == 8 * 258
    assert _gplan(L, [_gdesc(L, 0, T=128)])[0] == -22   # prefill-sized only
    assert _gplan(L, [_gdesc(L, 0, T=0)])[0] == -22
    assert _gplan(L, [_gdesc(L, 0, K=100)])[0] == -22
    assert _gplan(L, [_gdesc(L, 0, xq=FAKE + 4)])[0] == -22
    assert _gplan(L, [_gdesc(L, 0, y=FAKE + 5 * GB + 8)])[0] == -22
    assert _gplan(L, [_gdesc(L, 0, meta=None)])[0] == -22
    assert _gplan(L, [_gdesc(L, 0, T=1 << 22, K=1024)])[0] == -22   # 32-bit activation offsets
    assert _gplan(L, [a], N=3)[0] == -95
    assert _gplan(L, [_gdesc(L, 0, meta=None)], layout=1)[0] == 0
    lib = L.lib()
    assert lib.bitlinear_gemm_group_plan(None, 1, 2, 4, 0, ctypes.byref(L.BlGemmGroupPlan())) == -22
    assert lib.bitlinear_gemm_group_plan((L.BlFwdDesc * 1)(a), 0, 2, 4, 0,
                                         ctypes.byref(L.BlGemmGroupPlan())) == -22
    assert lib.bitlinear_gemm_group_plan((L.BlFwdDesc * 1)(a), 1, 2, 4, 0, None) == -22
    # inputs may be shared; an output may overlap nothing
    assert _gplan(L, [a, _gdesc(L, 1, xq=a.xq, x_scale=a.x_scale, codes=a.codes,
                                meta=a.meta, gamma=a.gamma)])[0] == 0
    assert _gplan(L, [a, _gdesc(L, 1, y=a.y)])[0] == -22
    assert _gplan(L, [a, _gdesc(L, 1, y=a.y + 300 * 300 * 4 - 16)])[0] == -22
    assert _gplan(L, [a, _gdesc(L, 1, y=a.y + 300 * 300 * 4)])[0] == 0      # adjacent
    assert _gplan(L, [a, _gdesc(L, 1, y=a.codes + 1024)])[0] == -22
    assert _gplan(L, [a, _gdesc(L, 1, xq=a.y + 64)])[0] == -22
    assert _gplan(L, [_gdesc(L, 0, acc_opt=FAKE + 5 * GB + 4096)])[0] == -22   # acc inside y
    assert _gplan(L, [_gdesc(L, 0, acc_opt=FAKE + 6 * GB)])[0] == 0
    # build and launch argument checks (nothing is copied or launched)
    arr = (L.BlFwdDesc * 2)(a, b)
    TB = FAKE + 80 * 16 * GB
    assert L.bitlinear_gemm_group_build(arr, 2, 4, 0, TB, plan.table_bytes - 16, None) == -28
    assert L.bitlinear_gemm_group_build(arr, 2, 4, 0, TB + 8, plan.table_bytes, None) == -22
    assert L.bitlinear_gemm_group(TB, None, None) == -22
    assert L.bitlinear_gemm_group(TB + 4, plan, None) == -22
    bad = L.BlGemmGroupPlan.from_buffer_copy(plan)
    bad.N = 3
    assert L.bitlinear_gemm_group(TB, bad, None) == -95
    bad = L.BlGemmGroupPlan.from_buffer_copy(plan)
    bad.jobs = 0
    assert L.bitlinear_gemm_group(TB, bad, None) == -22


def _qdesc(L, slot, **kw):
    """A grouped-quantization descriptor whose buffers sit in their own 1 GiB slots."""
    base = FAKE + slot * 16 * GB
    a = dict(x=base, T=5, K=512, xq=base + GB, x_scale=base + 2 * GB)
    a.update(kw)
    return L.BlQuantDesc(**a)


def _qgroup(L, descs, dtype=1, lift=0):
    return L.act_quant_i8_group((L.BlQuantDesc * len(descs))(*descs), dtype, lift, None)


def test_act_quant_group_rejects_before_launch(L):
    """act_quant_i8's rules per matrix, 1..16 matrices, outputs overlapping nothing; groups with
    nothing to do return OK without touching the runtime."""
    assert _qgroup(L, [_qdesc(L, 0, T=0, x=None, xq=None, x_scale=None)]) == 0
    assert _qgroup(L, [_qdesc(L, i, T=0) for i in range(16)]) == 0
    assert _qgroup(L, [_qdesc(L, i, T=0) for i in range(17)]) == -22
    lib = L.lib()
    assert lib.act_quant_i8_group(None, 1, 1, 0, None) == -22
    assert lib.act_quant_i8_group((L.BlQuantDesc * 1)(_qdesc(L, 0)), 0, 1, 0, None) == -22
    assert _qgroup(L, [_qdesc(L, 0)], dtype=7) == -95
    assert _qgroup(L, [_qdesc(L, 0)], lift=4) == -22
    assert _qgroup(L, [_qdesc(L, 0, K=520)], lift=16) == -22
    assert _qgroup(L, [_qdesc(L, 0, K=12)]) == -22
    assert _qgroup(L, [_qdesc(L, 0, T=-1)]) == -22
    assert _qgroup(L, [_qdesc(L, 0), _qdesc(L, 1, x=FAKE + 16 * GB + 8)]) == -22
    assert _qgroup(L, [_qdesc(L, 0, xq=FAKE + GB + 4)]) == -22
    assert _qgroup(L, [_qdesc(L, 0, x_scale=FAKE + 2 * GB + 2)]) == -22
    # outputs may not overlap an input or another output (checked before anything is launched)
    a = _qdesc(L, 0)
    assert _qgroup(L, [a, _qdesc(L, 1, xq=a.xq)]) == -22
    assert _qgroup(L, [a, _qdesc(L, 1, xq=a.xq + 5 * 512 - 16)]) == -22
    assert _qgroup(L, [a, _qdesc(L, 1, x_scale=a.x + 64)]) == -22
    assert _qgroup(L, [_qdesc(L, 0, xq=FAKE + 1024)]) == -22         # own xq inside own x
    assert _qgroup(L, [a, _qdesc(L, 1, x_scale=a.x_scale + 16)]) == -22


def _xdesc(L, slot=0, **kw):
    P = FAKE
    a = dict(x=P, T=4, K=256, codes=P, meta=P, gamma=P, n=100,
             y=FAKE + (slot + 1) * (16 << 30), acc_opt=None)
    a.update(kw)
    return L.BlFwdXDesc(**a)


def test_fused_group_sizes_and_rejects_before_launch(L):
    """The fused group plans exactly like the plain one; it refuses lifted layouts."""
    xs = (L.BlFwdXDesc * 3)(_xdesc(L), _xdesc(L, 1, n=6912, K=2560, T=16), _xdesc(L, 2, T=0, x=None))
    ps = (L.BlFwdDesc * 3)(_desc(L), _desc(L, 1, n=6912, K=2560, T=16), _desc(L, 2, T=0, xq=None))
    assert L.bitlinear_group_fused_table_bytes(xs, 2, 4, 0) == L.bitlinear_group_table_bytes(ps, 2, 4, 0)

    def one(N=2, M=4, layout=0, **kw):
        return L.bitlinear_group_fused_table_bytes((L.BlFwdXDesc * 1)(_xdesc(L, **kw)), N, M, layout)[0]
    assert one() == 0
    assert one(N=6, M=8, K=512) == -95             # lifted layouts are not fused
    assert one(N=14, M=16, K=512) == -95
    assert one(N=6, M=8, layout=1, meta=None) == 0  # dense 2-bit 6:8 has no lifting
    assert one(T=33) == -22
    assert one(x=FAKE + 8) == -22
    assert one(x=None) == -22
    assert L.bitlinear_group_fused_build(xs, 2, 4, 0, FAKE, 16, None) == -28
    assert L.bitlinear_fwd_group_fused(FAKE, 3, 6, 8, 0, None) == -95
    assert L.bitlinear_fwd_group_fused(FAKE + 4, 3, 2, 4, 0, None) == -22
    assert L.bitlinear_fwd_group_fused(None, 0, 2, 4, 0, None) == 0


def _cdesc(L, slot, n, K, **kw):
    """A chain layer whose buffers sit in their own 16 GiB slot of fake space."""
    base = FAKE + slot * 16 * GB
    a = dict(codes=base, meta=base + GB, gamma=base + 2 * GB, n=n, K=K, y=base + 3 * GB,
             acc_opt=None)
    a.update(kw)
    return L.BlChainLayer(**a)


def _cplan(L, layers, T=4, N=2, M=4, layout=0):
    return L.bitlinear_chain_plan((L.BlChainLayer * len(layers))(*layers), T, N, M, layout)


def test_chain_plan_sizes_and_rejects(L):
    """A chain's table, workspace and LDS size; its layers must chain (K == previous n), be 2:4
    and fit the per-wave step budget; outputs may not overlap anything."""
    dims = [(6912, 2560), (2560, 6912), (6912, 2560)]
    st, plan = _cplan(L, [_cdesc(L, i, n, K) for i, (n, K) in enumerate(dims)], T=16)
    assert st == 0
    assert plan.L == 3 and plan.T == 16
    assert plan.table_bytes == (64 + 3 * 56 + 15) // 16 * 16
    # per-workgroup absmax slots (64 workgroups), then from a 256-byte boundary the int8 rows of
    # the largest accepted K
    assert plan.ws_bytes == (4 * (64 + 4 * 64 * 16) + 255) // 256 * 256 + 16 * 8192
    # the widest layer's int8 input rows, then the eight waves' int32 partials
    assert plan.smem == 16 * (6912 + 16) + 8 * 16 * 65 * 4
    ok = [_cdesc(L, 0, 128, 256), _cdesc(L, 1, 64, 128)]
    assert _cplan(L, ok)[0] == 0
    assert _cplan(L, [_cdesc(L, 0, 128, 256), _cdesc(L, 1, 64, 192)])[0] == -22   # K != prev n
    assert _cplan(L, ok, N=6, M=8)[0] == -95                                         # 2:4 only
    assert _cplan(L, ok, layout=1)[0] == -95
    assert _cplan(L, ok, T=0)[0] == -22
    assert _cplan(L, ok, T=33)[0] == -22
    assert _cplan(L, [_cdesc(L, 0, 64, 8256)])[0] == -22                            # K > 8192
    assert _cplan(L, [_cdesc(L, 0, 64, 8192)], T=32)[0] == -22                      # LDS
    assert _cplan(L, [_cdesc(L, 0, 64, 4096)], T=32)[0] == -22
    assert _cplan(L, [_cdesc(L, 0, 64, 4032)], T=32)[0] == 0
    assert _cplan(L, [_cdesc(L, 0, 64, 100)])[0] == -22
    assert _cplan(L, [_cdesc(L, 0, 64, 128, codes=FAKE + 8)])[0] == -22
    assert _cplan(L, [_cdesc(L, 0, 64, 128, y=FAKE + 4)])[0] == -22
    # outputs: a y over another layer's y, over weights, or an acc over a y
    assert _cplan(L, [_cdesc(L, 0, 128, 256), _cdesc(L, 1, 64, 128, y=FAKE + 3 * GB + 64)])[0] == -22
    assert _cplan(L, [_cdesc(L, 0, 128, 256, y=FAKE + 16)])[0] == -22
    assert _cplan(L, [_cdesc(L, 0, 128, 256, acc_opt=FAKE + 3 * GB + 16)])[0] == -22
    assert _cplan(L, [_cdesc(L, 0, 128, 256, acc_opt=FAKE + 5 * GB)])[0] == 0
    lib = L.lib()
    assert lib.bitlinear_chain_plan(None, 1, 4, 2, 4, 0, None) == -22
    # launch: argument checks only
    assert L.bitlinear_fwd_chain(FAKE, plan, FAKE + 4, 1, FAKE, plan.ws_bytes, 0, None) == -22
    assert L.bitlinear_fwd_chain(FAKE, plan, FAKE, 7, FAKE, plan.ws_bytes, 0, None) == -95
    assert L.bitlinear_fwd_chain(FAKE, plan, FAKE, 1, FAKE, plan.ws_bytes - 4, 0, None) == -28
    assert L.bitlinear_fwd_chain(FAKE, None, FAKE, 1, FAKE, plan.ws_bytes, 0, None) == -22
    assert L.bitlinear_chain_build((L.BlChainLayer * 1)(_cdesc(L, 0, 64, 128)), 4, 2, 4, 0,
                                   FAKE, 16, None) == -28
