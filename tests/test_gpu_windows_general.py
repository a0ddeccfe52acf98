"""(2N-2):2N beyond 6:8 and 14:16 -- 4:6, 8:10, 10:12, 12:14 -- through the C ABI.

Every (M-2):M group is decomposed into M/2 - 1 overlapping 2:4 windows (SlideSparse abstract,
Sliding Window Decomposition) with the activations lifted to match.  Against the oracle: gamma,
codes and meta bit for bit, lifted int8 activations and scales bit for bit, int32 accumulators bit
for bit (GEMV and GEMM paths, ragged rows and tokens, several pack tiles), y within 1e-5; the
window product equals the dense-stored product of the same masked weights; the backward's dX and
dW are bit-exact on integer output gradients; a grouped pack equals the single calls.
"""
import numpy as np
import pytest

import oracle as O
from parity_util import as_u32, assert_y_close, bf16_dev, dev, f32_bits, host
from synth import act_normal, grad_int_bf16, master_weights, rng, to_bf16

pytestmark = pytest.mark.gpu

S = pytest.importorskip("sparsity_amd")

NEW_M = [6, 10, 12, 14]
# K of each case: several pack tiles with a partial last one, whole lifted MFMA steps, and a
# multiple of the dense-storage quantum lcm(32, M) where the dense comparison runs
K_SP = {6: 1200, 10: 1040, 12: 1152, 14: 1120}
K_BOTH = {6: 960, 10: 1120, 12: 1152, 14: 1120}    # valid for SPARSE windows and DENSE2


@pytest.mark.parametrize("M", NEW_M)
@pytest.mark.parametrize("layout", [O.LAYOUT_SPARSE, O.LAYOUT_DENSE2])
def test_pack(M, layout):
    K = K_SP[M] if layout == O.LAYOUT_SPARSE else K_BOTH[M]
    for n, seed in ((45, 1), (200, 2)):
        W = master_weights(rng(100 * M + seed), n, K)
        ref = O.pack(W, M - 2, M, layout)
        codes, meta, gamma = S.pack(dev(W), M - 2, M, layout)
        assert f32_bits(host(gamma)[0]) == f32_bits(ref["gamma"])
        assert np.array_equal(as_u32(codes), ref["codes"])
        if layout == O.LAYOUT_SPARSE:
            assert np.array_equal(as_u32(meta), ref["meta"])
    # ties: discrete magnitudes with signed zeros
    g = rng(7 * M)
    W = g.choice(np.array([0.0, -0.0, 0.01, -0.01, 0.02, -0.02], np.float32), size=(70, K))
    ref = O.pack(W, M - 2, M, layout)
    codes, meta, _ = S.pack(dev(W), M - 2, M, layout)
    assert np.array_equal(as_u32(codes), ref["codes"])
    if layout == O.LAYOUT_SPARSE:
        assert np.array_equal(as_u32(meta), ref["meta"])


@pytest.mark.parametrize("M", NEW_M)
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("T", [1, 5, 130])
def test_act_quant_lifted(M, dtype, T):
    K = K_SP[M]
    g = rng(T + M)
    x = act_normal(g, T, K)
    if T > 3:
        x[2] = 0.0
    if dtype == "bf16":
        x, bits = to_bf16(x)
        xd = bf16_dev(bits)
    else:
        xd = dev(x)
    xq_ref, sc_ref = O.act_quant(x, M)
    xq, sc = S.act_quant(xd, M)
    assert np.array_equal(host(xq), xq_ref)
    assert np.array_equal(f32_bits(host(sc)), f32_bits(sc_ref))


@pytest.mark.parametrize("M", NEW_M)
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_act_quant_lifted_long_rows(M, dtype):
    """Rows past the register budget of the one-wave-per-token kernel (the two-pass kernel)."""
    q = {6: 48, 10: 40, 12: 192, 14: 112}[M]
    K = (20000 // q) * q
    g = rng(M + 1)
    x = act_normal(g, 3, K)
    x[1, K - 1] = 400.0
    if dtype == "bf16":
        x, bits = to_bf16(x)
        xd = bf16_dev(bits)
    else:
        xd = dev(x)
    xq_ref, sc_ref = O.act_quant(x, M)
    xq, sc = S.act_quant(xd, M)
    assert np.array_equal(host(xq), xq_ref)
    assert np.array_equal(f32_bits(host(sc)), f32_bits(sc_ref))


@pytest.mark.parametrize("M", NEW_M)
@pytest.mark.parametrize("T", [1, 16, 77, 300])
def test_fwd_windows_against_oracle_and_dense_storage(M, T):
    """GEMV (T <= 32) and GEMM paths: accumulators equal the oracle's dense int64 product of the
    masked ternary weights, and the dense-stored (DENSE2) path of the same weights, bit for bit."""
    n, K = 200, K_BOTH[M]
    g = rng(1000 * M + T)
    W = master_weights(g, n, K)
    x = act_normal(g, T, K)
    ref = O.pack(W, M - 2, M, O.LAYOUT_SPARSE)
    acc_ref = O.acc_dense(ref["W_eff"], O.act_quant(x, 0)[0])
    xl_ref, sl_ref = O.act_quant(x, M)
    c1, m1, g1 = S.pack(dev(W), M - 2, M, O.LAYOUT_SPARSE)
    c2, _, g2 = S.pack(dev(W), M - 2, M, O.LAYOUT_DENSE2)
    xl, sl = S.act_quant(dev(x), M)
    xd, sd = S.act_quant(dev(x), 0)
    y1, a1 = S.fwd(xl, sl, K, c1, m1, g1, n, M - 2, M, O.LAYOUT_SPARSE, want_acc=True)
    _, a2 = S.fwd(xd, sd, K, c2, None, g2, n, M - 2, M, O.LAYOUT_DENSE2, want_acc=True)
    assert np.array_equal(host(a1), acc_ref)
    assert np.array_equal(host(a2), acc_ref)
    assert_y_close(host(y1), O.rescale(acc_ref, ref["gamma"], sl_ref))


@pytest.mark.parametrize("M", NEW_M)
def test_bwd_exact_integer(M):
    """Integer output gradients and token scale 2^-7: dX and dW bit-exact (every partial sum is
    exact in fp32), windows and dense storage alike."""
    T, n, K = 300, 200, K_BOTH[M]
    g = rng(77 + M)
    W = master_weights(g, n, K)
    ref = O.pack(W, M - 2, M, O.LAYOUT_SPARSE)
    dy, dy_bits = grad_int_bf16(g, T, n)
    q = g.integers(-127, 128, size=(T, K)).astype(np.int8)
    scale = np.full(T, 2.0 ** -7, np.float32)
    dx_ref, dw_ref = O.backward(dy, ref["W_eff"], ref["gamma"], q, scale)
    for layout in (O.LAYOUT_SPARSE, O.LAYOUT_DENSE2):
        codes, meta, gamma = S.pack(dev(W), M - 2, M, layout)
        dx, dw = S.bwd(bf16_dev(dy_bits), dev(q), dev(scale), K, codes, meta, gamma, n, M - 2, M,
                       layout)
        assert np.array_equal(f32_bits(host(dx)), f32_bits(dx_ref.astype(np.float32)))
        assert np.array_equal(f32_bits(host(dw)), f32_bits(dw_ref.astype(np.float32)))


def test_grouped_pack_equals_single_calls():
    """One grouped pack of 10:12 masters of different shapes equals bitlinear_pack per master."""
    g = rng(1012)
    masters = [dev(master_weights(g, n, 1152)) for n in (64, 100, 33)]
    grp = S.PackGroup([dict(W=W) for W in masters], 10, 12)
    grp()
    for W, (c, m, ga) in zip(masters, grp.outputs):
        c1, m1, g1 = S.pack(W, 10, 12)
        assert np.array_equal(host(c), host(c1)) and np.array_equal(host(m), host(m1))
        assert f32_bits(host(ga)[0]) == f32_bits(host(g1)[0])
