"""Pins of the oracle's straight-through backward against hand-derived values, exact arithmetic,
brute-force loops, a library cast and the adjoint identities of the pinned forward.

Sparse-BitNet technical summary, Training Strategie (Dual STE): the quantizers and the Top-N
selection are passed straight through and the gradient reaches every master weight, so
dX = gamma * dY W_eff and dW = dY^T X^ with X^ = bf16(fp32(q * scale_t)).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from golden_io import hexu32, read_kv


def _floats(vals):
    return np.array([float(v) for v in vals])


def _u32_to_f32(vals):
    return np.array(vals, dtype=np.uint32).view(np.float32)


def _bf16_values(g, shape, scale=1.0):
    """Random values on the bfloat16 grid (kept 8 significant bits), as fp32."""
    v = (g.standard_normal(shape) * scale).astype(np.float32)
    return O.bf16_round(v)


# ------------------------------------------------------------------------------------------
# hand-derived tiny case
# ------------------------------------------------------------------------------------------

def test_backward_golden_tiny():
    kv = read_kv("bwd_tiny.txt")
    W = np.stack([_floats(kv["W_row0"]), _floats(kv["W_row1"])]).astype(np.float32)
    W_eff, gamma, keep = O.effective_weights(W, 2, 4)
    assert float(gamma) == 1.0
    want_eff = np.stack([_floats(kv["W_eff_row0"]), _floats(kv["W_eff_row1"])])
    assert np.array_equal(W_eff, want_eff)
    q = np.stack([_floats(kv["q_row0"]), _floats(kv["q_row1"])]).astype(np.int8)
    scale = _floats(kv["scale"]).astype(np.float32)
    xhat = O.dequant_act(q, scale)
    assert np.array_equal(xhat, np.stack([_floats(kv["Xhat_row0"]), _floats(kv["Xhat_row1"])]))
    dy = np.stack([_floats(kv["dY_row0"]), _floats(kv["dY_row1"])])
    dx, dw = O.backward(dy, W_eff, gamma, q, scale)
    assert np.array_equal(dx, np.stack([_floats(kv["dX_row0"]), _floats(kv["dX_row1"])]))
    assert np.array_equal(dw, np.stack([_floats(kv["dW_row0"]), _floats(kv["dW_row1"])]))
    # masked weights get gradient (Dual STE): row 0 masks k = 1, 3; row 1 masks k = 0, 3
    assert not keep[0, 3] and dw[0, 3] != 0
    assert not keep[1, 0] and dw[1, 0] != 0 and dw[1, 3] != 0


def test_dequant_golden_roundings():
    kv = read_kv("bwd_tiny.txt")
    q = np.array([int(v) for v in kv["deq_q"]], dtype=np.int8)
    s = _u32_to_f32(hexu32(kv["deq_scale"]))
    want = hexu32(kv["deq_xhat"])
    got = O.dequant_act(q[:, None], s)[:, 0]
    assert [int(b) for b in got.view(np.uint32)] == want


# ------------------------------------------------------------------------------------------
# bfloat16 rounding
# ------------------------------------------------------------------------------------------

def _bf16_nearest_exact(v: np.float32) -> float:
    """Nearest bfloat16 to v by exact comparison of the two bracketing grid points."""
    u = int(np.float32(v).view(np.uint32))
    lo = np.uint32(u & 0xFFFF0000).view(np.float32)        # truncation toward zero
    hi_bits = (u & 0xFFFF0000) + 0x10000
    hi = np.uint32(hi_bits).view(np.float32)               # next grid point away from zero
    fv, flo, fhi = Fraction(float(v)), Fraction(float(lo)), Fraction(float(hi))
    dlo, dhi = abs(fv - flo), abs(fhi - fv)
    if dlo < dhi:
        return float(lo)
    if dhi < dlo:
        return float(hi)
    return float(lo) if ((u >> 16) & 1) == 0 else float(hi)


@pytest.mark.parametrize("seed", range(3))
def test_bf16_round_exact_nearest(seed):
    g = np.random.default_rng(seed)
    v = (g.standard_normal(3000) * np.exp2(g.integers(-140, 120, size=3000))).astype(np.float32)
    # exact ties and values one fp32 ulp either side of a tie
    ties = np.uint32(g.integers(0x00800000, 0x7F000000, size=300) & 0xFFFF0000 | 0x8000)
    v = np.concatenate([v, ties.view(np.float32), (ties + 1).view(np.float32),
                        (ties - 1).view(np.float32), -ties.view(np.float32)])
    got = O.bf16_round(v)
    want = np.array([_bf16_nearest_exact(x) for x in v])
    assert np.array_equal(got.astype(np.float64), want)


def test_bf16_round_matches_torch_cast():
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(9)
    v = (g.standard_normal(20000) * np.exp2(g.integers(-130, 100, size=20000))).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(O.bf16_round(v), ref)


# ------------------------------------------------------------------------------------------
# brute force, identities, mask independence
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("N,M,layout", [(2, 4, O.LAYOUT_SPARSE), (6, 8, O.LAYOUT_SPARSE),
                                        (2, 4, O.LAYOUT_DENSE2)])
def test_backward_bruteforce_loops(N, M, layout):
    """Python loops over exact rationals on a 3 x 5 x 16 case."""
    g = np.random.default_rng(40 + M)
    T, n, K = 3, 5, 16
    W = g.normal(0, 0.02, size=(n, K)).astype(np.float32)
    x = g.standard_normal((T, K)).astype(np.float32)
    dy = _bf16_values(g, (T, n))
    W_eff, gamma, _ = O.effective_weights(W, N, M)
    q, s = O.act_quant(x, 0)
    dx, dw = O.backward(dy, W_eff, gamma, q, s)
    for t in range(T):
        for k in range(K):
            acc = Fraction(0)
            for o in range(n):
                acc += Fraction(float(dy[t, o])) * int(W_eff[o, k])
            want = Fraction(float(gamma)) * acc
            assert abs(Fraction(float(dx[t, k])) - want) <= Fraction(1, 2**50) * (abs(want) + 1), (t, k)
    for o in range(n):
        for k in range(K):
            acc = Fraction(0)
            for t in range(T):
                p32 = np.float32(np.float32(q[t, k]) * np.float32(s[t]))
                xh = Fraction(_bf16_nearest_exact(p32))
                acc += Fraction(float(dy[t, o])) * xh
            assert abs(Fraction(float(dw[o, k])) - acc) <= Fraction(1, 2**50) * (abs(acc) + 1), (o, k)


@pytest.mark.parametrize("N,M,layout", [(2, 4, O.LAYOUT_SPARSE), (6, 8, O.LAYOUT_SPARSE),
                                        (14, 16, O.LAYOUT_SPARSE), (2, 4, O.LAYOUT_DENSE2),
                                        (4, 4, O.LAYOUT_DENSE2)])
def test_backward_adjoint_identities(N, M, layout):
    """<dX, X^> = <dY, Y> = <dW, gamma W_eff>, Y from the pinned forward (int64 accumulators).

    Power-of-two token scales make X^ = q * scale exact, so the forward's Y = X^ (gamma W_eff)^T
    holds exactly and both identities must agree to fp64 rounding.  A dropped term, a wrong sign,
    a missing gamma or a transposed gradient breaks them."""
    g = np.random.default_rng(7 * M + N)
    T, n, K = 24, 40, 256
    W = g.normal(0, 0.02, size=(n, K)).astype(np.float32)
    p = O.pack(W, N, M, layout)
    q = g.integers(-127, 128, size=(T, K)).astype(np.int8)
    scale = np.exp2(g.integers(-9, -3, size=T)).astype(np.float32)
    dy = _bf16_values(g, (T, n))
    dx, dw = O.backward(dy, p["W_eff"], p["gamma"], q, scale)
    acc = O.acc_dense(p["W_eff"], q)
    y64 = acc.astype(np.float64) * np.float64(p["gamma"]) * scale.astype(np.float64)[:, None]
    xhat = q.astype(np.float64) * scale.astype(np.float64)[:, None]
    lhs = float(np.sum(dy.astype(np.float64) * y64))
    mag = float(np.sum(np.abs(dy.astype(np.float64) * y64))) + 1e-30
    assert abs(float(np.sum(dx * xhat)) - lhs) <= 1e-12 * mag
    wq = np.float64(p["gamma"]) * p["W_eff"].astype(np.float64)
    assert abs(float(np.sum(dw * wq)) - lhs) <= 1e-12 * mag
    # a transposed weight gradient would fail the identity (the shapes are not square)
    assert dw.shape == (n, K) and dx.shape == (T, K)


def test_weight_gradient_ignores_mask():
    """Dual STE: dW is the same for every N:M (the mask passes gradient to masked weights);
    dX sees only the kept ternary weights, so it changes with the mask."""
    g = np.random.default_rng(5)
    T, n, K = 16, 24, 64
    W = g.normal(0, 0.02, size=(n, K)).astype(np.float32)
    x = g.standard_normal((T, K)).astype(np.float32)
    q, s = O.act_quant(x, 0)
    dy = _bf16_values(g, (T, n))
    outs = {}
    for N, M in ((2, 4), (6, 8), (4, 4)):
        W_eff, gamma, keep = O.effective_weights(W, N, M)
        outs[(N, M)] = O.backward(dy, W_eff, gamma, q, s) + (keep,)
    dw24 = outs[(2, 4)][1]
    assert np.array_equal(dw24, outs[(6, 8)][1]) and np.array_equal(dw24, outs[(4, 4)][1])
    keep24 = outs[(2, 4)][2]
    assert np.all(dw24[~keep24] != 0)            # masked positions get (nonzero) gradient
    assert not np.array_equal(outs[(2, 4)][0], outs[(4, 4)][0])


def test_integer_inputs_are_exact():
    """Integer dY with the token scale 2^-7: every partial sum of the two products is exactly
    representable, so dX / gamma and 128 dW equal int64 products."""
    g = np.random.default_rng(12)
    T, n, K = 64, 96, 128
    W = g.normal(0, 0.02, size=(n, K)).astype(np.float32)
    W_eff, gamma, _ = O.effective_weights(W, 2, 4)
    q = g.integers(-127, 128, size=(T, K)).astype(np.int8)
    scale = np.full(T, 2.0 ** -7, np.float32)
    dyi = g.integers(-8, 9, size=(T, n))
    dx, dw = O.backward(dyi.astype(np.float32), W_eff, gamma, q, scale)
    assert np.array_equal(dx, np.float64(gamma) * (dyi @ W_eff.astype(np.int64)))
    assert np.array_equal(dw * 128, (dyi.T @ q.astype(np.int64)).astype(np.float64))
