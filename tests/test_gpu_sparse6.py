"""SPARSE6 (2:4 re-encoded at 6 bits per group) through the C ABI against the CPU oracle.

Bit-exact: the re-encoded stream (against oracle.pack6 of the oracle's own slots) and the int32
accumulators of the 6-bit decode (single projection and group).  Within 1e-5 relative: y.  At the
decode projections' full sizes the stream is compared on sampled 32-row panels (the oracle's
pure-Python encoder is slow), every output against the oracle, and the 6-bit decode must equal
the 2:4 decode of the same packed masters bit for bit (y and acc).
"""
import numpy as np
import pytest

import oracle as O
from parity_util import as_u32, assert_y_close, dev, host
from synth import act_normal, master_weights, rng

pytestmark = pytest.mark.gpu

S = pytest.importorskip("sparsity_amd")
S6 = O.LAYOUT_SPARSE6


def _stream_ref(W):
    n, K = W.shape
    ref = O.pack(W, 2, 4, O.LAYOUT_SPARSE)
    vals, idx = O.weight_slots(ref["W_eff"], ref["keep"], 2, 4, O.LAYOUT_SPARSE)
    return ref, O.pack6(vals, idx, n, K)


@pytest.mark.parametrize("n,K", [(1, 64), (33, 192), (70, 320), (45, 384), (257, 640)])
def test_transcode_matches_oracle(n, K):
    W = master_weights(rng(n * 7 + K), n, K)
    W[:, :16] = 0.0                                  # all-zero groups: state 0
    W[3 % n, 16:24] = [0.5, 0.5, 0.5, 0.5, -1, 1, -1, 1]   # ties: the lower positions are kept
    ref, want = _stream_ref(W)
    codes, meta, gamma = S.pack(dev(W), 2, 4)
    got = as_u32(S.transcode6(codes, meta, n, K))
    assert got.shape == want.shape
    nbad = int((got != want).sum())
    assert nbad == 0, f"{nbad} stream dwords differ (n={n}, K={K})"


def _fwd6_case(n, K, T, seed):
    g = rng(seed)
    W = master_weights(g, n, K)
    x = act_normal(g, T, K)
    ref = O.pack(W, 2, 4)
    xq_ref, sc_ref = O.act_quant(x)
    acc_ref = O.acc_dense(ref["W_eff"], xq_ref)
    y_ref = O.rescale(acc_ref, ref["gamma"], sc_ref)
    codes, meta, gamma = S.pack(dev(W), 2, 4)
    st = S.transcode6(codes, meta, n, K)
    xq, sc = S.act_quant(dev(x))
    y, acc = S.fwd(xq, sc, K, st, None, gamma, n, 2, 4, S6, want_acc=True)
    nbad = int((host(acc) != acc_ref).sum())
    assert nbad == 0, f"{nbad} accumulators differ (T={T}, n={n}, K={K})"
    assert_y_close(host(y), y_ref)
    return (xq, sc, codes, meta, gamma, st), (y, acc)


@pytest.mark.parametrize("T", [1, 3, 16, 17, 32])
@pytest.mark.parametrize("n,K", [(33, 192), (200, 320), (257, 640), (64, 2560)])
def test_fwd6_matches_oracle(n, K, T):
    _fwd6_case(n, K, T, seed=T * 31 + K + n)


def test_fwd6_long_rows_without_lds_staging():
    # T * (K + 16) past the LDS budget: B operands come straight from L2
    _fwd6_case(40, 6912, 32, seed=6912)
    _fwd6_case(40, 16384, 9, seed=16384)


def test_fwd6_edge_tokens_and_zero_rows():
    import torch
    g = rng(5)
    n, K, T = 70, 256, 16
    W = master_weights(g, n, K)
    W[7] = 0.0
    x = act_normal(g, T, K)
    x[0] = 0.0
    x[5, :4] = [127.0, 2.5, -3.5, 0.5]
    x[5, 4:] = 0.0
    ref = O.forward(W, x, 2, 4)
    codes, meta, gamma = S.pack(dev(W), 2, 4)
    st = S.transcode6(codes, meta, n, K)
    xq, sc = S.act_quant(dev(x))
    y, acc = S.fwd(xq, sc, K, st, None, gamma, n, 2, 4, S6, want_acc=True)
    assert np.array_equal(host(acc), ref["acc"])
    assert_y_close(host(y), ref["y"])
    xq0 = torch.zeros((0, K), dtype=torch.int8, device="cuda")
    sc0 = torch.zeros(4, dtype=torch.float32, device="cuda")[:0]
    assert S.fwd(xq0, sc0, K, st, None, gamma, n, 2, 4, S6).shape == (0, n)


def test_group6_mixed_shapes_matches_single_and_oracle():
    import torch
    shapes = [(200, 320, 16), (33, 192, 1), (257, 640, 32), (64, 2560, 4), (100, 448, 0),
              (520, 256, 17)]
    projs, refs = [], []
    for i, (n, K, T) in enumerate(shapes):
        g = rng(100 + i)
        W = master_weights(g, n, K)
        x = act_normal(g, max(T, 1), K)[:T]
        codes, meta, gamma = S.pack(dev(W), 2, 4)
        st = S.transcode6(codes, meta, n, K)
        xq, sc = S.act_quant(dev(x)) if T else (torch.zeros((0, K), dtype=torch.int8, device="cuda"),
                                                torch.zeros(4, dtype=torch.float32, device="cuda")[:0])
        y = torch.full((max(T, 1), n), float("nan"), device="cuda")[:T]
        acc = torch.zeros((max(T, 1), n), dtype=torch.int32, device="cuda")[:T]
        projs.append(dict(xq=xq, scale=sc, K=K, codes=st, meta=None, gamma=gamma, n=n, y=y,
                          acc=acc if T else None))
        refs.append(O.forward(W, x, 2, 4) if T else None)
    grp = S.FwdGroup(projs, 2, 4, S6)
    for _ in range(2):                             # relaunch: same results
        grp()
        for p, r in zip(projs, refs):
            if r is None:
                continue
            assert np.array_equal(host(p["acc"]), r["acc"])
            assert_y_close(host(p["y"]), r["y"])
            ys, accs = S.fwd(p["xq"], p["scale"], p["K"], p["codes"], None, p["gamma"], p["n"], 2,
                             4, S6, want_acc=True)
            assert torch.equal(ys, p["y"]) and torch.equal(accs, p["acc"])


def test_group6_full_decode_shapes():
    """FFN up 6912x2560 and down 2560x6912 at T = 1, 4, 16 in one SPARSE6 group, as the decode
    benchmark runs them: sampled panels of each stream bit-exact against the oracle's, every
    output against the oracle, and bitwise equal to the 2:4 group of the same packed masters."""
    import torch
    from synth import workload_inputs
    d = workload_inputs("decode", 0)
    p4, p6 = [], []
    for name, K in (("up", 2560), ("down", 6912)):
        W = d[f"W:{name}"]
        n = W.shape[0]
        ref = O.pack(W, 2, 4)
        codes, meta, gamma = S.pack(dev(W), 2, 4)
        st = S.transcode6(codes, meta, n, K)
        st_h = as_u32(st)
        vals, idx = O.weight_slots(ref["W_eff"], ref["keep"], 2, 4, O.LAYOUT_SPARSE)
        nc = -(-K // 128)
        for P in (0, 1, n // 64, n // 32 - 1):
            rows = slice(32 * P, 32 * P + 32)
            want = O.pack6(vals[rows], idx[rows], 32, K)
            assert np.array_equal(st_h[P * nc * 192:(P + 1) * nc * 192], want), f"{name} panel {P}"
        print(f"decode {name}: sampled stream panels bit-exact", flush=True)
        for T in (1, 4, 16):
            x = d[f"X:{K}"][:T]
            xq, sc = S.act_quant(dev(x))
            for lst, c, m in ((p4, codes, meta), (p6, st, None)):
                lst.append(dict(xq=xq, scale=sc, K=K, codes=c, meta=m, gamma=gamma, n=n,
                                y=torch.empty((T, n), device="cuda"),
                                acc=torch.empty((T, n), dtype=torch.int32, device="cuda"),
                                ref=ref, x=x, name=f"{name} T={T}"))
    S.FwdGroup(p4)()
    S.FwdGroup(p6, 2, 4, S6)()
    for a, b in zip(p4, p6):
        assert torch.equal(b["acc"], a["acc"]), b["name"]
        assert torch.equal(b["y"], a["y"]), b["name"]
        q, s = O.act_quant(b["x"], 0)
        acc_ref = O.acc_dense(b["ref"]["W_eff"], q)
        assert np.array_equal(host(b["acc"]), acc_ref), f"decode {b['name']}: accumulators"
        assert_y_close(host(b["y"]), O.rescale(acc_ref, b["ref"]["gamma"], s), what=b["name"])
        y1, a1 = S.fwd(b["xq"], b["scale"], b["K"], b["codes"], None, b["gamma"], b["n"], 2, 4,
                       S6, want_acc=True)
        assert torch.equal(a1, b["acc"]) and torch.equal(y1, b["y"]), b["name"]
        print(f"decode {b['name']}: SPARSE6 ok", flush=True)
