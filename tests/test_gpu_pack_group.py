"""Grouped pack (bitlinear_pack_group) through the C ABI.

Its contract is bitlinear_pack per master, bit for bit, so every case compares each master's
gamma, codes and meta with a single bitlinear_pack call (itself checked against the CPU oracle in
test_gpu_parity.py), and one case compares a whole group with the oracle directly.
"""
import numpy as np
import pytest

import oracle as O
from parity_util import dev, f32_bits, host
from synth import master_weights, rng

pytestmark = pytest.mark.gpu

S = pytest.importorskip("sparsity_amd")

CASES_NM = [(2, 4, O.LAYOUT_SPARSE), (6, 8, O.LAYOUT_SPARSE), (14, 16, O.LAYOUT_SPARSE),
            (2, 4, O.LAYOUT_DENSE2), (5, 8, O.LAYOUT_DENSE2)]


def _kq(M, layout):
    return 32 if layout == O.LAYOUT_DENSE2 else {4: 64, 8: 128, 16: 256}[M]


def _same(out, ref, what):
    c, m, g = out
    rc, rm, rg = ref
    assert np.array_equal(f32_bits(host(g)), f32_bits(host(rg))), f"{what}: gamma"
    assert np.array_equal(host(c), host(rc)), f"{what}: codes"
    if rm is not None:
        assert np.array_equal(host(m), host(rm)), f"{what}: meta"


def _masters(N, M, layout, seed):
    g = rng(seed)
    kq = _kq(M, layout)
    shapes = [(45, 2 * kq * 2), (300, 3 * 256), (32, kq * 4), (97, 1024)]
    out = []
    for n, K in shapes:
        K = max(kq, K // kq * kq)
        out.append(master_weights(g, n, K))
    return out


@pytest.mark.parametrize("N,M,layout", CASES_NM)
def test_pack_group_matches_single_calls(N, M, layout):
    Ws = [dev(W) for W in _masters(N, M, layout, seed=11 + M + 3 * layout)]
    grp = S.PackGroup([dict(W=W) for W in Ws], N, M, layout)
    grp()
    for i, W in enumerate(Ws):
        _same(grp.outputs[i], S.pack(W, N, M, layout), f"master {i}")


def test_pack_group_against_oracle_and_exact_gamma():
    """A group holding a master whose mean |w| sits exactly between two fp32 values (the exact
    fallback decides gamma), a zero master and a random one, against the oracle."""
    n, K = 32, 64
    W0 = np.ones((n, K), np.float32)
    W0[7, 9] = np.float32(1.0 + 3 * (n * K) * 2.0 ** -24)
    W0[::2] *= -1
    W1 = np.zeros((64, 128), np.float32)
    W2 = master_weights(rng(5), 200, 512)
    grp = S.PackGroup([dict(W=dev(W)) for W in (W0, W1, W2)], 2, 4, O.LAYOUT_SPARSE)
    grp()
    for (c, m, gm), W in zip(grp.outputs, (W0, W1, W2)):
        ref = O.pack(W, 2, 4, O.LAYOUT_SPARSE)
        assert f32_bits(host(gm)[0]) == f32_bits(ref["gamma"])
        assert np.array_equal(host(c).view(np.uint32), ref["codes"])
        assert np.array_equal(host(m).view(np.uint32), ref["meta"])
    assert int(f32_bits(host(grp.outputs[0][2])[0])) == 0x3F800002


def test_pack_group_rereads_masters_and_replays_in_a_graph():
    """Built once: updated masters (same buffers) are packed at the next launch; a captured
    launch replays bit-identically (several replays with eager work in between)."""
    import torch
    Ws = [dev(W) for W in _masters(2, 4, O.LAYOUT_SPARSE, seed=77)]
    grp = S.PackGroup([dict(W=W) for W in Ws])
    grp()
    g = rng(78)
    for W in Ws:
        W.copy_(dev(master_weights(g, *W.shape)))
    grp()
    want = [S.pack(W) for W in Ws]
    for i in range(len(Ws)):
        _same(grp.outputs[i], want[i], f"updated master {i}")
    cap = torch.cuda.Stream()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=cap):
        grp()
    for _ in range(3):
        for c, m, gm in grp.outputs:
            c.zero_()
            m.zero_()
            gm.zero_()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        for i in range(len(Ws)):
            _same(grp.outputs[i], want[i], f"graph replay, master {i}")


def test_pack_group_training_layer_set_full_size():
    """The training-step layer set's seven masters (3200 x 3200 x 4, 8640 x 3200 x 2,
    3200 x 8640) in one group, as the training-step benchmark packs them."""
    from synth import workload_inputs
    d = workload_inputs("train_step", 0)
    names = ("q", "k", "v", "o", "gate", "up", "down")
    Ws = [dev(d[f"W:{L}"]) for L in names]
    grp = S.PackGroup([dict(W=W) for W in Ws])
    grp()
    for i, (L, W) in enumerate(zip(names, Ws)):
        _same(grp.outputs[i], S.pack(W), L)
    ref = O.pack(d["W:o"], 2, 4, O.LAYOUT_SPARSE)
    c, m, gm = grp.outputs[3]
    assert f32_bits(host(gm)[0]) == f32_bits(ref["gamma"])
    assert np.array_equal(host(c).view(np.uint32), ref["codes"])
    assert np.array_equal(host(m).view(np.uint32), ref["meta"])
