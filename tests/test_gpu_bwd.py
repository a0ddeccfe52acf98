"""Straight-through backward (bitlinear_bwd) vs the CPU oracle, through the C ABI.

Exact cases use integer output gradients and the token scale 2^-7: every partial sum of both
products is then exactly representable in fp32, so dX = fl32(gamma * S) and dW must match the
oracle bit for bit whatever the summation order.  General cases (bf16 N(0,1) gradients, scales from
act_quant) are checked against the bound of fp32 summation in any order, derived from the
arithmetic: with exact products (bf16 x bf16, or bf16 x +-1) and R terms, each partial sum is
rounded at most R - 1 times, so |S' - S| <= 2 R u sum|terms| (u = 2^-24; the factor 2 also covers
an accumulator that truncates), plus one rounding u |result| for the gamma product and the store.
"""
import numpy as np
import pytest

import oracle as O
from parity_util import dev, f32_bits, host
from synth import act_normal, grad_bf16, grad_int_bf16, master_weights, rng

pytestmark = pytest.mark.gpu

S = pytest.importorskip("sparsity_amd")

U = 2.0 ** -24
CASES_NM = [(2, 4, O.LAYOUT_SPARSE), (6, 8, O.LAYOUT_SPARSE), (14, 16, O.LAYOUT_SPARSE),
            (2, 4, O.LAYOUT_DENSE2), (4, 4, O.LAYOUT_DENSE2)]


def _kq(M, layout):
    return 32 if layout == O.LAYOUT_DENSE2 else {4: 64, 8: 128, 16: 256}[M]


def _bf16_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _assert_within(got, ref, mag, R, what):
    """|got - ref| <= 2 R u mag + u |ref| elementwise (mag = sum of |terms|)."""
    got = np.asarray(got, np.float64)
    bound = 2.0 * R * U * mag + U * np.abs(ref) + 1e-45
    err = np.abs(got - ref)
    bad = err > bound
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} elements outside the fp32 summation bound; "
                             f"first at {i}: gpu {got[i]!r} ref {ref[i]!r} bound {bound[i]!r}")


def _setup(T, n, K, N, M, layout, seed, integer):
    g = rng(seed)
    W = master_weights(g, n, K)
    ref = O.pack(W, N, M, layout)
    codes, meta, gamma = S.pack(dev(W), N, M, layout)
    if integer:
        dy, dy_bits = grad_int_bf16(g, T, n)
        q = g.integers(-127, 128, size=(T, K)).astype(np.int8)
        scale = np.full(T, 2.0 ** -7, np.float32)
        xq, sc = dev(q), dev(scale)
    else:
        dy, dy_bits = grad_bf16(g, T, n, 1.0)
        x = act_normal(g, T, K)
        xq, sc = S.act_quant(dev(x), 0)
        q, scale = O.act_quant(x, 0)
        assert np.array_equal(host(xq), q)
    return dict(W=W, ref=ref, codes=codes, meta=meta, gamma=gamma, dy=dy, dyd=_bf16_dev(dy_bits),
                q=q, scale=scale, xq=xq, sc=sc, T=T, n=n, K=K, nm=(N, M, layout))


def _run(c, **kw):
    return S.bwd(c["dyd"], c["xq"], c["sc"], c["K"], c["codes"], c["meta"], c["gamma"], c["n"],
                 *c["nm"], **kw)


@pytest.mark.parametrize("N,M,layout", CASES_NM)
def test_bwd_exact_integer(N, M, layout):
    """Ragged everything: T = 300 (two 256-token tiles, a partial 32-token pad), n = 300 (padded
    dY copy for dX, two row tiles for dW), K past two 256-wide column tiles."""
    kq = _kq(M, layout)
    K = -(-600 // kq) * kq
    c = _setup(300, 300, K, N, M, layout, seed=31 + M + 5 * layout, integer=True)
    dx, dw = _run(c)
    dx_ref, dw_ref = O.backward(c["dy"], c["ref"]["W_eff"], c["ref"]["gamma"], c["q"], c["scale"])
    assert np.array_equal(f32_bits(host(dx)), f32_bits(dx_ref.astype(np.float32))), "dX bits"
    assert np.array_equal(f32_bits(host(dw)), f32_bits(dw_ref.astype(np.float32))), "dW bits"


@pytest.mark.parametrize("N,M,layout", CASES_NM)
@pytest.mark.parametrize("T,n", [(256, 256), (77, 512), (513, 96), (1, 32)])
def test_bwd_random_within_bound(N, M, layout, T, n):
    kq = _kq(M, layout)
    K = max(kq, -(-384 // kq) * kq)
    c = _setup(T, n, K, N, M, layout, seed=T + n + M, integer=False)
    dx, dw = _run(c)
    W_eff, gamma = c["ref"]["W_eff"], c["ref"]["gamma"]
    dx_ref, dw_ref = O.backward(c["dy"], W_eff, gamma, c["q"], c["scale"])
    ady = np.abs(c["dy"].astype(np.float64))
    mag_dx = np.float64(gamma) * (ady @ np.abs(W_eff.astype(np.float64)))
    xh = np.abs(O.dequant_act(c["q"], c["scale"]).astype(np.float64))
    mag_dw = ady.T @ xh
    _assert_within(host(dx), dx_ref, mag_dx, n, "dX")
    _assert_within(host(dw), dw_ref, mag_dw, T, "dW")


def test_bwd_accumulate_and_partial_outputs():
    """BL_BWD_ACCUM_* add into the outputs (one more fp32 rounding); a NULL output is skipped."""
    import torch
    c = _setup(96, 128, 256, 2, 4, O.LAYOUT_SPARSE, seed=5, integer=True)
    dx_ref, dw_ref = O.backward(c["dy"], c["ref"]["W_eff"], c["ref"]["gamma"], c["q"], c["scale"])
    g = rng(6)
    prev_dx = g.integers(-50, 50, size=dx_ref.shape).astype(np.float32)
    prev_dw = g.integers(-50, 50, size=dw_ref.shape).astype(np.float32)
    dx, dw = dev(prev_dx), dev(prev_dw)
    _run(c, out=(dx, dw), accumulate=(True, True))
    assert np.array_equal(f32_bits(host(dx)), f32_bits((prev_dx + dx_ref.astype(np.float32))))
    assert np.array_equal(f32_bits(host(dw)), f32_bits((prev_dw + dw_ref.astype(np.float32))))
    # dW only, overwrite: dx stays as it is
    dw2 = torch.full((128, 256), float("nan"), device="cuda")
    _run(c, out=(None, dw2), want_dx=False)
    assert np.array_equal(f32_bits(host(dw2)), f32_bits(dw_ref.astype(np.float32)))
    # dX only
    dx2 = torch.full((96, 256), float("nan"), device="cuda")
    _run(c, out=(dx2, None), want_dw=False)
    assert np.array_equal(f32_bits(host(dx2)), f32_bits(dx_ref.astype(np.float32)))


def test_bwd_no_tokens():
    """T == 0: dW is written as zeros, or left unchanged when accumulating."""
    import torch
    c = _setup(0, 64, 128, 2, 4, O.LAYOUT_SPARSE, seed=8, integer=True)
    dw = torch.full((64, 128), 3.0, device="cuda")
    _run(c, out=(None, dw), accumulate=(False, True), want_dx=False)
    assert np.all(host(dw) == 3.0)
    _run(c, out=(None, dw), want_dx=False)
    assert np.all(host(dw) == 0.0)


def test_bwd_windows_and_dense_storage_agree():
    """The same master packed as 6:8 windows and as dense 2-bit codes has one W_eff: dX is the same
    bits from both (and dW never depends on the packing)."""
    g = rng(68)
    T, n, K = 200, 320, 512
    W = master_weights(g, n, K)
    dy, bits = grad_bf16(g, T, n, 1.0)
    x = act_normal(g, T, K)
    xq, sc = S.act_quant(dev(x), 0)
    dyd = _bf16_dev(bits)
    outs = []
    for layout in (O.LAYOUT_SPARSE, O.LAYOUT_DENSE2):
        codes, meta, gamma = S.pack(dev(W), 6, 8, layout)
        outs.append([host(t) for t in S.bwd(dyd, xq, sc, K, codes, meta, gamma, n, 6, 8, layout)])
    assert np.array_equal(f32_bits(outs[0][0]), f32_bits(outs[1][0]))
    assert np.array_equal(f32_bits(outs[0][1]), f32_bits(outs[1][1]))
