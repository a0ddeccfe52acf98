"""Grouped prefill forward (bitlinear_gemm_group) through the C ABI.

The group's contract is bitlinear_fwd per descriptor, bit for bit, so every case compares y and
the int32 accumulators with separate bitlinear_fwd calls on the same buffers; the small cases
also check the CPU oracle directly (accumulators bit for bit, y within 1e-5 relative).  Groups
mix shapes: ragged rows and tokens (n and T not multiples of the 256 x 128 output tile), one K
quantum and many, a projection of more than one 64-tile run, per-projection T, shared
activations, and the packings the single call accepts.
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


def _lift(M, layout):
    return M if (layout == O.LAYOUT_SPARSE and M in O.WINDOW_M) else 0


def _make(n, K, T, N, M, layout, seed, with_acc=True):
    """One projection: oracle results plus the device buffers of a group entry."""
    import torch
    g = rng(seed)
    W = master_weights(g, n, K)
    x = act_normal(g, T, K)
    ref = O.pack(W, N, M, layout)
    codes, meta, gamma = S.pack(dev(W), N, M, layout)
    xq, sc = S.act_quant(dev(x), _lift(M, layout))
    q, s = O.act_quant(x, 0)
    acc_ref = O.acc_dense(ref["W_eff"], q)
    y = torch.full((T, n), float("nan"), dtype=torch.float32, device="cuda")
    acc = torch.full((T, n), -7, dtype=torch.int32, device="cuda") if with_acc else None
    return dict(xq=xq, scale=sc, K=K, codes=codes, meta=meta, gamma=gamma, n=n, y=y, acc=acc,
                acc_ref=acc_ref, y_ref=O.rescale(acc_ref, ref["gamma"], s), T=T, q=q, s=s)


def _single(p, N, M, layout):
    y, acc = S.fwd(p["xq"], p["scale"], p["K"], p["codes"], p["meta"], p["gamma"], p["n"], N, M,
                   layout, want_acc=True)
    return host(y), host(acc)


@pytest.mark.parametrize("N,M,layout", CASES_NM)
def test_gemm_group_mixed_shapes(N, M, layout):
    kq = _kq(N, M, layout)
    shapes = [  # (n, K, T)
        (300, 5 * kq, 200),      # ragged rows and tokens: 2 x 2 tiles, both partial at the edge
        (45, 2 * kq, 129),       # one partial row tile; a token tile holding one token
        (520, 6 * kq, 260),
        (256, kq, 256),          # whole tiles, one K quantum
        (257, 9 * kq, 131),      # a row tile of one row
        (2304, kq, 1100),        # 9 x 9 tiles: two runs, dealt to different XCDs
    ]
    projs = [_make(n, K, T, N, M, layout, seed=100 * i + M + 7 * layout, with_acc=i % 2 == 0)
             for i, (n, K, T) in enumerate(shapes)]
    grp = S.GemmGroup(projs, N, M, layout)
    grp()
    for i, p in enumerate(projs):
        what = f"projection {i} {shapes[i]}"
        if p["acc"] is not None:
            nbad = int((host(p["acc"]) != p["acc_ref"]).sum())
            assert nbad == 0, f"{what}: {nbad} accumulators differ from the oracle"
        assert_y_close(host(p["y"]), p["y_ref"], what=what)
        y1, acc1 = _single(p, N, M, layout)
        assert np.array_equal(f32_bits(y1), f32_bits(host(p["y"]))), f"{what}: y != bitlinear_fwd"
        if p["acc"] is not None:
            assert np.array_equal(acc1, host(p["acc"])), f"{what}: acc != bitlinear_fwd"


@pytest.mark.parametrize("N,M,layout", CASES_NM)
def test_gemm_group_xcd_slabs(N, M, layout):
    """Token tiles that split evenly over the 8 XCDs (T a multiple of 8 x 128) take the slab plan:
    each XCD walks its slab of every projection, projections reading the same activations next
    to each other (here the first and the third share one xq and are launched apart).  Every
    output against the oracle and against bitlinear_fwd, bit for bit."""
    import torch
    kq = _kq(N, M, layout)
    a = _make(300, 2 * kq, 1024, N, M, layout, seed=900 + M + 7 * layout)          # ragged rows
    b = _make(45, kq, 2048, N, M, layout, seed=901 + M + 7 * layout, with_acc=False)
    W = master_weights(rng(902 + M + 7 * layout), 257, 2 * kq)                      # a 1-row tile
    ref = O.pack(W, N, M, layout)
    codes, meta, gamma = S.pack(dev(W), N, M, layout)
    acc_ref = O.acc_dense(ref["W_eff"], a["q"])
    c = dict(xq=a["xq"], scale=a["scale"], K=a["K"], codes=codes, meta=meta, gamma=gamma, n=257,
             y=torch.full((1024, 257), float("nan"), dtype=torch.float32, device="cuda"),
             acc=torch.full((1024, 257), -7, dtype=torch.int32, device="cuda"), acc_ref=acc_ref,
             y_ref=O.rescale(acc_ref, ref["gamma"], a["s"]), T=1024)
    projs = [a, b, c]
    S.GemmGroup(projs, N, M, layout)()
    for i, p in enumerate(projs):
        what = f"projection {i}"
        if p["acc"] is not None:
            nbad = int((host(p["acc"]) != p["acc_ref"]).sum())
            assert nbad == 0, f"{what}: {nbad} accumulators differ from the oracle"
        assert_y_close(host(p["y"]), p["y_ref"], what=what)
        y1, acc1 = _single(p, N, M, layout)
        assert np.array_equal(f32_bits(y1), f32_bits(host(p["y"]))), f"{what}: y != bitlinear_fwd"


def test_gemm_group_shared_activations_new_contents_and_graph():
    """Q/K/V-style projections read one xq; new activations written into the same buffers are
    picked up by the next launch without a rebuild; a captured launch replays to the same bits
    (several replays, eager work in between)."""
    import torch
    K, T = 768, 333
    g = rng(78)
    x1, x2 = act_normal(g, T, K), act_normal(g, T, K)
    xq, sc = S.act_quant(dev(x1))
    projs = []
    for i, n in enumerate((768, 256, 256)):
        W = master_weights(rng(600 + i), n, K)
        ref = O.pack(W, 2, 4, O.LAYOUT_SPARSE)
        codes, meta, gamma = S.pack(dev(W), 2, 4)
        projs.append(dict(xq=xq, scale=sc, K=K, codes=codes, meta=meta, gamma=gamma, n=n,
                          y=torch.empty((T, n), device="cuda"),
                          acc=torch.empty((T, n), dtype=torch.int32, device="cuda"), ref=ref))
    grp = S.GemmGroup(projs)
    for x in (x1, x2):
        S.act_quant(dev(x), out=(xq, sc))
        grp()
        q, s = O.act_quant(x, 0)
        for p in projs:
            acc_ref = O.acc_dense(p["ref"]["W_eff"], q)
            assert np.array_equal(host(p["acc"]), acc_ref)
            assert_y_close(host(p["y"]), O.rescale(acc_ref, p["ref"]["gamma"], s))
    want = [(host(p["y"]), host(p["acc"])) for p in projs]
    cap = torch.cuda.Stream()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=cap):
        grp()
    for _ in range(3):
        for p in projs:
            p["y"].fill_(float("nan"))
            p["acc"].fill_(-7)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        for p, (y0, a0) in zip(projs, want):
            assert np.array_equal(f32_bits(host(p["y"])), f32_bits(y0)), "graph replay differs"
            assert np.array_equal(host(p["acc"]), a0)


def test_gemm_group_layer_set_full_size():
    """The training-step layer set (QKV 3 x 3200^2 and gate/up 8640 x 3200 on one activation, O
    3200^2 and down 3200 x 8640 on their own) at 8192 tokens, 2:4: the whole outputs against
    bitlinear_fwd on the same device, bit for bit."""
    import torch
    T = 8192
    g = rng(79)
    acts = {}
    for key, K in (("x", 3200), ("o", 3200), ("d", 8640)):
        xq, sc = S.act_quant(dev(act_normal(g, T, K)))
        acts[key] = (xq, sc, K)
    specs = [("x", 3200)] * 3 + [("o", 3200)] + [("x", 8640)] * 2 + [("d", 3200)]
    projs = []
    for i, (key, n) in enumerate(specs):
        xq, sc, K = acts[key]
        codes, meta, gamma = S.pack(dev(master_weights(rng(800 + i), n, K)), 2, 4)
        projs.append(dict(xq=xq, scale=sc, K=K, codes=codes, meta=meta, gamma=gamma, n=n,
                          y=torch.empty((T, n), device="cuda")))
    S.GemmGroup(projs)()
    for i, p in enumerate(projs):
        y1 = S.fwd(p["xq"], p["scale"], p["K"], p["codes"], p["meta"], p["gamma"], p["n"])
        assert torch.equal(y1.view(torch.int32), p["y"].view(torch.int32)), f"projection {i}"
        del y1
    torch.cuda.empty_cache()
