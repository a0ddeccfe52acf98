"""Grouped decode forward (bitlinear_fwd_group) vs the CPU oracle, through the C ABI.

Every projection of a group must give the oracle's int32 accumulators bit for bit and its fp32
outputs within 1e-5 relative, and the very bits of a separate bitlinear_fwd call.  Groups mix
shapes: ragged rows (n not a multiple of 32, nor of 4), K with a partial last chunk and K of many
chunks, T from 0 to 32, several work items per projection, shared activation buffers.
"""
import numpy as np
import pytest

import oracle as O
from parity_util import assert_y_close, dev, f32_bits, host
from synth import act_normal, master_weights, rng

pytestmark = pytest.mark.gpu

S = pytest.importorskip("sparsity_amd")

CASES_NM = [(2, 4, O.LAYOUT_SPARSE), (6, 8, O.LAYOUT_SPARSE), (14, 16, O.LAYOUT_SPARSE),
            (2, 4, O.LAYOUT_DENSE2), (4, 4, O.LAYOUT_DENSE2)]


def _kq(N, M, layout):
    return 32 if layout == O.LAYOUT_DENSE2 else {4: 64, 8: 128, 16: 256}[M]


def _make(n, K, T, N, M, layout, seed, x=None):
    """One projection: oracle results plus the device buffers of a group entry."""
    import torch
    g = rng(seed)
    W = master_weights(g, n, K)
    if x is None:
        x = act_normal(g, max(T, 1), K)[:T]
    ref = O.pack(W, N, M, layout)
    lift = M if (layout == O.LAYOUT_SPARSE and M in O.WINDOW_M) else 0
    codes, meta, gamma = S.pack(dev(W), N, M, layout)
    if T:
        xq, sc = S.act_quant(dev(x), lift)
        q, s = O.act_quant(x, 0)
        acc_ref = O.acc_dense(ref["W_eff"], q)
        y_ref = O.rescale(acc_ref, ref["gamma"], s)
    else:
        ke = K // lift * (2 * lift - 4) if lift else K
        xq = torch.zeros((0, ke), dtype=torch.int8, device="cuda")
        sc = torch.zeros(4, dtype=torch.float32, device="cuda")[:0]
        acc_ref = np.zeros((0, n), np.int64)
        y_ref = np.zeros((0, n))
    y = torch.full((T, n), float("nan"), dtype=torch.float32, device="cuda")
    acc = torch.full((T, n), -7, dtype=torch.int32, device="cuda")
    return dict(xq=xq, scale=sc, K=K, codes=codes, meta=meta, gamma=gamma, n=n, y=y, acc=acc,
                acc_ref=acc_ref, y_ref=y_ref, T=T)


def _check(p, what):
    acc = host(p["acc"])
    nbad = int((acc != p["acc_ref"]).sum())
    assert nbad == 0, f"{what}: {nbad} accumulators differ"
    assert_y_close(host(p["y"]), p["y_ref"], what=what)
    if p["T"]:
        # same bits as one bitlinear_fwd call on the same buffers
        y1 = S.fwd(p["xq"], p["scale"], p["K"], p["codes"], p["meta"], p["gamma"], p["n"],
                   *p["nm"])
        assert np.array_equal(f32_bits(host(y1)), f32_bits(host(p["y"]))), what


@pytest.mark.parametrize("N,M,layout", CASES_NM)
def test_group_mixed_shapes(N, M, layout):
    kq = _kq(N, M, layout)
    shapes = [  # (n, K, T)
        (200, 5 * kq, 1),        # ragged rows, K of 5 steps' worth (partial chunk)
        (45, 2 * kq, 3),         # n not a multiple of 4: element stores
        (600, 26 * kq, 16),      # several work items, K over 3 chunks with a partial one
        (96, kq, 32),            # one K quantum, full token tile
        (64, 3 * kq, 0),         # no tokens: skipped
        (257, 9 * kq, 7),        # 9 panels = two work items, the second with surplus waves
    ]
    projs = []
    for i, (n, K, T) in enumerate(shapes):
        p = _make(n, K, T, N, M, layout, seed=100 * i + M + 7 * layout)
        p["nm"] = (N, M, layout)
        projs.append(p)
    grp = S.FwdGroup(projs, N, M, layout)
    grp()
    for i, p in enumerate(projs):
        _check(p, f"projection {i} {shapes[i]}")


def test_group_shared_activations_and_relaunch():
    """Q/K/V-style: three projections read one xq; new activations written into the same buffers
    are picked up by the next launch without rebuilding the table."""
    import torch
    K, T = 512, 5
    g = rng(77)
    x1 = act_normal(g, T, K)
    x2 = act_normal(g, T, K)
    xq, sc = S.act_quant(dev(x1))
    projs = []
    for i, n in enumerate((512, 128, 128)):
        W = master_weights(rng(500 + i), n, K)
        ref = O.pack(W, 2, 4, O.LAYOUT_SPARSE)
        codes, meta, gamma = S.pack(dev(W), 2, 4)
        projs.append(dict(xq=xq, scale=sc, K=K, codes=codes, meta=meta, gamma=gamma, n=n,
                          y=torch.empty((T, n), device="cuda"),
                          acc=torch.empty((T, n), dtype=torch.int32, device="cuda"), ref=ref))
    grp = S.FwdGroup(projs)
    for x in (x1, x2):
        S.act_quant(dev(x), out=(xq, sc))
        grp()
        q, s = O.act_quant(x, 0)
        for p in projs:
            acc_ref = O.acc_dense(p["ref"]["W_eff"], q)
            assert np.array_equal(host(p["acc"]), acc_ref)
            assert_y_close(host(p["y"]), O.rescale(acc_ref, p["ref"]["gamma"], s))


FUSED_NM = [(2, 4, O.LAYOUT_SPARSE), (2, 4, O.LAYOUT_DENSE2), (6, 8, O.LAYOUT_DENSE2),
            (4, 4, O.LAYOUT_DENSE2)]


def _bf16(x):
    """bf16 device tensor from the synth generator's rounding, and its fp32 values."""
    import torch
    from synth import to_bf16
    vals, bits = to_bf16(x)
    return vals, torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


@pytest.mark.parametrize("N,M,layout", FUSED_NM)
def test_fused_group_matches_oracle_and_plain(N, M, layout):
    """Fused quantization inside the grouped GEMV: accumulators bit-exact and outputs within 1e-5
    of the oracle, and every output bit-identical to act_quant_i8 + the plain group on the same
    bf16 rows.  Ragged n, T from 0 to 32, K over several chunks, shared activation rows."""
    import torch
    kq = _kq(N, M, layout)
    shapes = [(200, 5 * kq, 1), (45, 2 * kq, 3), (600, 26 * kq, 16), (96, kq, 32), (64, 3 * kq, 0),
              (257, 9 * kq, 7)]
    fused, plain = [], []
    for i, (n, K, T) in enumerate(shapes):
        g = rng(900 + 10 * i + M + layout)
        W = master_weights(g, n, K)
        # a heavy-tailed row and an all-zero row exercise absmax and the zero-scale case
        x = act_normal(g, T, K) if T else np.zeros((0, K), np.float32)
        if T >= 3:
            x[1] *= 40.0
            x[2] = 0.0
        xv, xd = _bf16(x)
        ref = O.pack(W, N, M, layout)
        codes, meta, gamma = S.pack(dev(W), N, M, layout)
        q, s = O.act_quant(xv, 0)
        acc_ref = O.acc_dense(ref["W_eff"], q)
        yf = torch.full((T, n), float("nan"), device="cuda")
        af = torch.full((T, n), -7, dtype=torch.int32, device="cuda")
        fused.append(dict(x=xd, K=K, codes=codes, meta=meta, gamma=gamma, n=n, y=yf, acc=af,
                          acc_ref=acc_ref, y_ref=O.rescale(acc_ref, ref["gamma"], s), T=T))
        if T:
            xq, sc = S.act_quant(xd)
        else:
            xq = torch.zeros((0, K), dtype=torch.int8, device="cuda")
            sc = torch.zeros(4, dtype=torch.float32, device="cuda")[:0]
        plain.append(dict(xq=xq, scale=sc, K=K, codes=codes, meta=meta, gamma=gamma, n=n,
                          y=torch.full((T, n), float("nan"), device="cuda"),
                          acc=torch.full((T, n), -7, dtype=torch.int32, device="cuda")))
    S.FusedGroup(fused, N, M, layout)()
    S.FwdGroup(plain, N, M, layout)()
    for i, (f, p) in enumerate(zip(fused, plain)):
        what = f"fused projection {i} {shapes[i]}"
        assert np.array_equal(host(f["acc"]), f["acc_ref"]), f"{what}: accumulators"
        assert_y_close(host(f["y"]), f["y_ref"], what=what)
        assert np.array_equal(f32_bits(host(f["y"])), f32_bits(host(p["y"]))), f"{what}: != plain"
        assert np.array_equal(host(f["acc"]), host(p["acc"])), f"{what}: acc != plain"


def test_fused_group_shared_rows_and_new_contents():
    """Q/K/V-style: three projections read one bf16 activation buffer; new contents written into
    it are quantized by the next launch without a rebuild."""
    import torch
    K, T = 512, 5
    g = rng(78)
    x1, x2 = act_normal(g, T, K), act_normal(g, T, K) * 3.0
    v1, xd = _bf16(x1)
    v2, xd2 = _bf16(x2)
    projs = []
    for i, n in enumerate((512, 128, 160)):
        W = master_weights(rng(600 + i), n, K)
        ref = O.pack(W, 2, 4, O.LAYOUT_SPARSE)
        codes, meta, gamma = S.pack(dev(W), 2, 4)
        projs.append(dict(x=xd, K=K, codes=codes, meta=meta, gamma=gamma, n=n,
                          y=torch.empty((T, n), device="cuda"),
                          acc=torch.empty((T, n), dtype=torch.int32, device="cuda"), ref=ref))
    grp = S.FusedGroup(projs)
    for vals, src in ((v1, None), (v2, xd2)):
        if src is not None:
            xd.copy_(src)
        grp()
        q, s = O.act_quant(vals, 0)
        for p in projs:
            acc_ref = O.acc_dense(p["ref"]["W_eff"], q)
            assert np.array_equal(host(p["acc"]), acc_ref)
            assert_y_close(host(p["y"]), O.rescale(acc_ref, p["ref"]["gamma"], s))
