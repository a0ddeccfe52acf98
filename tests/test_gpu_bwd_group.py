"""Grouped backward (bitlinear_bwd_group) through the C ABI.

The group's contract is the sequence of bitlinear_bwd calls in descriptor order, bit for bit, so
every case compares against those calls made one after another (bitlinear_bwd itself is checked
against the CPU oracle in test_gpu_bwd.py).  One case also checks a whole group against the
oracle directly, on integer output gradients and power-of-two token scales, where every partial
sum is exact in fp32.
"""
import numpy as np
import pytest

import oracle as O
from parity_util import dev, f32_bits, host
from synth import act_normal, grad_bf16, grad_int_bf16, master_weights, rng

pytestmark = pytest.mark.gpu

S = pytest.importorskip("sparsity_amd")


def _bf16_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _layer_set(T, specs, N, M, layout, seed, integer=False):
    """specs: (n, K, x_id, dx_id, want_dw, accum_dx, accum_dw) per projection.  Projections with the
    same x_id read one activation; the same dx_id means one dx buffer.  Returns the projections
    and the shared tensors."""
    import torch
    g = rng(seed)
    xs, dxs, projs = {}, {}, []
    for (n, K, x_id, dx_id, want_dw, acc_dx, acc_dw) in specs:
        if x_id not in xs:
            if integer:
                q = g.integers(-127, 128, size=(T, K)).astype(np.int8)
                xs[x_id] = (dev(q), dev(np.full(T, 2.0 ** -7, np.float32)), q,
                            np.full(T, 2.0 ** -7, np.float32))
            else:
                x = act_normal(g, T, K)
                xq, sc = S.act_quant(dev(x), 0)
                xs[x_id] = (xq, sc, None, None)
        W = master_weights(g, n, K)
        codes, meta, gamma = S.pack(dev(W), N, M, layout)
        dy, bits = (grad_int_bf16(g, T, n) if integer else grad_bf16(g, T, n, 1.0))
        if dx_id is not None and dx_id not in dxs:
            dxs[dx_id] = torch.from_numpy(g.integers(-9, 9, size=(T, K)).astype(np.float32)).cuda()
        dw = (torch.from_numpy(g.integers(-9, 9, size=(n, K)).astype(np.float32)).cuda()
              if want_dw else None)
        xq, sc = xs[x_id][0], xs[x_id][1]
        projs.append(dict(dy=_bf16_dev(bits), dy_f=dy, xq=xq, scale=sc, K=K, codes=codes,
                          meta=meta, gamma=gamma, n=n,
                          dx=dxs[dx_id] if dx_id is not None else None, dw=dw,
                          accumulate=(acc_dx, acc_dw), W=W, x_id=x_id))
    return projs, xs, dxs


def _outputs(projs, dxs):
    return [host(t) for t in dxs.values()] + [host(p["dw"]) for p in projs if p["dw"] is not None]


def _sequential(projs, T, N, M, layout):
    for p in projs:
        S.bwd(p["dy"], p["xq"], p["scale"], p["K"], p["codes"], p["meta"], p["gamma"], p["n"], N,
              M, layout, want_dx=p["dx"] is not None, want_dw=p["dw"] is not None,
              out=(p["dx"], p["dw"]), accumulate=p["accumulate"])


def _snapshot(projs, dxs):
    return [t.clone() for t in dxs.values()] + [p["dw"].clone() for p in projs
                                                if p["dw"] is not None]


def _restore(projs, dxs, snap):
    outs = list(dxs.values()) + [p["dw"] for p in projs if p["dw"] is not None]
    for t, s in zip(outs, snap):
        t.copy_(s)


def _group_vs_sequential(projs, dxs, T, N, M, layout):
    import torch
    snap = _snapshot(projs, dxs)
    _sequential(projs, T, N, M, layout)
    torch.cuda.synchronize()
    want = _outputs(projs, dxs)
    _restore(projs, dxs, snap)
    grp = S.BwdGroup(projs, T, N, M, layout)
    grp()
    torch.cuda.synchronize()
    got = _outputs(projs, dxs)
    for i, (a, b) in enumerate(zip(got, want)):
        assert np.array_equal(f32_bits(a), f32_bits(b)), f"output {i} differs from the sequential calls"
    return grp, snap, want


# (n, K, x_id, dx_id, want_dw, accum_dx, accum_dw)
QKV_SET = [(320, 512, "a", "a", True, False, False),      # Q: overwrites dx_a
           (96, 512, "a", "a", True, True, False),        # K: narrow, adds
           (300, 512, "a", "a", True, True, True),        # V: ragged n (padded dY), adds; dw adds
           (512, 640, "o", "o", True, False, False)]      # O: own activation and dx


@pytest.mark.parametrize("N,M,layout", [(2, 4, O.LAYOUT_SPARSE), (6, 8, O.LAYOUT_SPARSE),
                                        (2, 4, O.LAYOUT_DENSE2)])
@pytest.mark.parametrize("T", [300, 64, 1])
def test_group_matches_sequential_calls(N, M, layout, T):
    projs, xs, dxs = _layer_set(T, QKV_SET, N, M, layout, seed=T + 7 * M + layout)
    _group_vs_sequential(projs, dxs, T, N, M, layout)


def test_group_flag_mixes_and_partial_outputs():
    """A later projection without BL_BWD_ACCUM_DX overwrites what the earlier ones summed; dx-only
    and dw-only projections; the first term accumulating onto an existing dx."""
    specs = [(256, 768, "a", "a", False, True, False),    # adds onto the existing dx, no dw
             (160, 768, "a", "a", True, True, False),
             (224, 768, "a", "a", True, False, True),     # overwrites: the two above are lost
             (128, 768, "a", "a", False, True, False),
             (192, 768, "b", None, True, False, True)]    # dw only, accumulating
    projs, xs, dxs = _layer_set(130, specs, 2, 4, O.LAYOUT_SPARSE, seed=44)
    _group_vs_sequential(projs, dxs, 130, 2, 4, O.LAYOUT_SPARSE)


def test_group_against_oracle_exact():
    """Integer dY in [-8, 8] and token scale 2^-7: dX = fl(fl(g1 S1) + fl(g2 S2)) and dW exact."""
    import torch
    T = 200
    specs = [(288, 512, "a", "a", True, False, False),
             (96, 512, "a", "a", True, True, False),
             (256, 1024, "b", "b", True, False, False)]
    projs, xs, dxs = _layer_set(T, specs, 2, 4, O.LAYOUT_SPARSE, seed=91, integer=True)
    S.BwdGroup(projs, T)()
    torch.cuda.synchronize()
    want_dx = {}
    for p in projs:
        ref = O.pack(p["W"], 2, 4, O.LAYOUT_SPARSE)
        q, sc = xs[p["x_id"]][2], xs[p["x_id"]][3]
        dx_ref, dw_ref = O.backward(p["dy_f"], ref["W_eff"], ref["gamma"], q, sc)
        term = dx_ref.astype(np.float32)
        want_dx[p["x_id"]] = term if not p["accumulate"][0] else want_dx[p["x_id"]] + term
        assert np.array_equal(f32_bits(host(p["dw"])), f32_bits(dw_ref.astype(np.float32)))
    for k, t in dxs.items():
        assert np.array_equal(f32_bits(host(t)), f32_bits(want_dx[k])), f"dx {k}"


def test_group_reads_new_contents_and_replays_in_a_graph():
    """Built once: new dY contents are picked up at the next launch; a captured launch replays
    bit-identically to the eager one (several replays with eager work in between)."""
    import torch
    T = 256
    specs = [(256, 512, "a", "a", True, False, False), (512, 512, "a", "a", True, True, False)]
    projs, xs, dxs = _layer_set(T, specs, 2, 4, O.LAYOUT_SPARSE, seed=12)
    grp, snap, _ = _group_vs_sequential(projs, dxs, T, 2, 4, O.LAYOUT_SPARSE)
    # new output gradients in the same buffers
    g = rng(13)
    for p in projs:
        _, bits = grad_bf16(g, T, p["n"], 1.0)
        p["dy"].copy_(_bf16_dev(bits))
    _restore(projs, dxs, snap)
    _sequential(projs, T, 2, 4, O.LAYOUT_SPARSE)
    torch.cuda.synchronize()
    want = _outputs(projs, dxs)
    _restore(projs, dxs, snap)
    grp()
    torch.cuda.synchronize()
    for a, b in zip(_outputs(projs, dxs), want):
        assert np.array_equal(f32_bits(a), f32_bits(b))
    cap = torch.cuda.Stream()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=cap):
        grp()
    for _ in range(3):
        _restore(projs, dxs, snap)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        for a, b in zip(_outputs(projs, dxs), want):
            assert np.array_equal(f32_bits(a), f32_bits(b)), "graph replay differs"


def test_group_no_tokens():
    """T == 0: dx is left alone, dw is zeroed (or left unchanged when accumulating)."""
    import torch
    g = rng(3)
    W = master_weights(g, 64, 256)
    codes, meta, gamma = S.pack(dev(W), 2, 4)
    dw0 = torch.full((64, 256), 3.0, device="cuda")
    dw1 = torch.full((64, 256), 5.0, device="cuda")
    empty_dy = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    empty_x = torch.empty((0, 256), dtype=torch.int8, device="cuda")
    empty_s = torch.empty((0,), dtype=torch.float32, device="cuda")
    base = dict(dy=empty_dy, xq=empty_x, scale=empty_s, K=256, codes=codes, meta=meta,
                gamma=gamma, n=64, dx=None)
    S.BwdGroup([dict(base, dw=dw0), dict(base, dw=dw1, accumulate=(False, True))], 0)()
    torch.cuda.synchronize()
    assert np.all(host(dw0) == 0.0) and np.all(host(dw1) == 5.0)


def test_group_layer_set_shapes_sampled():
    """The training-step layer set (QKV 3 x 3200^2 and gate/up 8640 x 3200 on one activation, O
    3200^2 and down 3200 x 8640 on their own) at 8192 tokens, against the sequential calls on the
    same device (whole outputs compared bitwise)."""
    import torch
    T = 8192
    specs = [(3200, 3200, "x", "x", True, False, False)] + \
            [(3200, 3200, "x", "x", True, True, False)] * 2 + \
            [(3200, 3200, "x", "x", True, True, False)] + \
            [(8640, 3200, "x", "x", True, True, False)] * 2 + \
            [(3200, 8640, "d", "d", True, False, False)]
    projs, xs, dxs = _layer_set(T, specs, 2, 4, O.LAYOUT_SPARSE, seed=77)
    _group_vs_sequential(projs, dxs, T, 2, 4, O.LAYOUT_SPARSE)
    torch.cuda.empty_cache()
