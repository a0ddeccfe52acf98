"""HIP path vs the CPU oracle through the C ABI, at sizes the oracle finishes in seconds.

Bit-exact: gamma, packed codes and meta, int8 activations, activation scales, int32 accumulators.
Within 1e-5 relative: the rescaled fp32 outputs.  Shapes span several tiles with ragged tails in
rows (n not a multiple of 32), K (partial 256-wide pack tiles) and tokens (T not a multiple of 32
or of the GEMM tile), plus the degenerate cases of the method.
"""
import numpy as np
import pytest

import oracle as O
from parity_util import as_u32, assert_y_close, bf16_dev, dev, f32_bits, host
from synth import act_normal, act_student_t, master_weights, rng, to_bf16

pytestmark = pytest.mark.gpu

S = pytest.importorskip("sparsity_amd")

CASES_NM = [(2, 4, O.LAYOUT_SPARSE), (6, 8, O.LAYOUT_SPARSE), (2, 4, O.LAYOUT_DENSE2),
            (6, 8, O.LAYOUT_DENSE2), (4, 4, O.LAYOUT_DENSE2), (14, 16, O.LAYOUT_SPARSE),
            (14, 16, O.LAYOUT_DENSE2)]


def _lift(N, M, layout):
    return M if (layout == O.LAYOUT_SPARSE and M in O.WINDOW_M) else 0


def _kq(N, M, layout):
    """K granularity of a layout: whole sparse-MFMA steps on the packed axis."""
    if layout == O.LAYOUT_DENSE2:
        return 32
    return {4: 64, 8: 128, 16: 256}[M]


def _pack_gpu(W, N, M, layout):
    codes, meta, gamma = S.pack(dev(W), N, M, layout)
    return (as_u32(codes), None if meta is None else as_u32(meta), host(gamma)[0])


def _check_pack(W, N, M, layout):
    ref = O.pack(W, N, M, layout)
    codes, meta, gamma = _pack_gpu(W, N, M, layout)
    assert f32_bits(gamma) == f32_bits(ref["gamma"]), (gamma, ref["gamma"])
    assert codes.shape == ref["codes"].shape
    nbad = int((codes != ref["codes"]).sum())
    assert nbad == 0, f"{nbad} code dwords differ"
    if layout == O.LAYOUT_SPARSE:
        assert np.array_equal(meta, ref["meta"])
    return ref


# ---------------------------------------------------------------------------------------------
# pack
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("N,M,layout", CASES_NM)
@pytest.mark.parametrize("n,K", [(45, 256), (96, 384), (200, 1024), (33, 640)])
def test_pack_random(N, M, layout, n, K):
    if K % _kq(N, M, layout):
        pytest.skip(f"{N}:{M} windows need K % {_kq(N, M, layout)} == 0")
    W = master_weights(rng(n * 7 + K + M), n, K)
    _check_pack(W, N, M, layout)


@pytest.mark.parametrize("N,M,layout", CASES_NM[:3])
def test_pack_ties_and_exact_halves(N, M, layout):
    # half the magnitudes 0.5 and half 1.5 -> gamma = 1 exactly: w = +-0.5 sits exactly on the
    # rounding boundary (rint(0.5) = 0), w = +-1.5 rounds to 2 and clips; groups are full of ties
    g = rng(1)
    n, K = 64, 256
    mag = np.where(np.arange(n * K).reshape(n, K) % 2 == 0, 0.5, 1.5).astype(np.float32)
    mag = mag.ravel()[g.permutation(n * K)].reshape(n, K)
    W = (mag * g.choice([-1.0, 1.0], size=(n, K))).astype(np.float32)
    ref = _check_pack(W, N, M, layout)
    assert float(ref["gamma"]) == 1.0
    assert np.any(np.abs(W) == 0.5 * float(ref["gamma"]))
    # signed zeros on top of the same magnitudes (gamma moves off 1; parity must still hold)
    W[3, :16] = -0.0
    W[4, :32] = 0.0
    _check_pack(W, N, M, layout)


def test_pack_discrete_ties():
    g = rng(2)
    W = g.choice(np.array([0.0, -0.0, 0.01, -0.01, 0.02, -0.02], np.float32), size=(70, 512))
    for N, M, layout in CASES_NM:
        _check_pack(W.astype(np.float32), N, M, layout)


@pytest.mark.parametrize("layout", [O.LAYOUT_SPARSE, O.LAYOUT_DENSE2])
def test_pack_zero_matrix(layout):
    W = np.zeros((40, 128), np.float32)
    W[1, 5] = -0.0
    ref = _check_pack(W, 2, 4, layout)
    assert float(ref["gamma"]) == 0.0


def test_pack_subnormal_and_wide_range():
    g = rng(3)
    tiny = (g.integers(-5, 6, size=(32, 64)) * np.float32(2.0 ** -149)).astype(np.float32)
    _check_pack(tiny, 2, 4, O.LAYOUT_SPARSE)
    wide = (g.standard_normal((64, 256)) * np.exp2(g.integers(-140, 100, size=(64, 256)))).astype(np.float32)
    _check_pack(wide, 2, 4, O.LAYOUT_SPARSE)
    _check_pack(wide, 6, 8, O.LAYOUT_SPARSE)


@pytest.mark.parametrize("bump,want", [(1, 0x3F800000), (3, 0x3F800002)])
def test_pack_gamma_at_fp32_midpoint(bump, want):
    # all |w| = 1 except one: the exact mean is 1 + bump * 2^-24, exactly halfway between two fp32
    # values, so no fp64 error bound can decide the rounding and the exact path must (ties to even)
    n, K = 32, 64
    W = np.ones((n, K), np.float32)
    W[7, 9] = np.float32(1.0 + bump * (n * K) * 2.0 ** -24)
    W[::2] *= -1
    ref = _check_pack(W, 2, 4, O.LAYOUT_SPARSE)
    assert int(f32_bits(ref["gamma"])) == want


# ---------------------------------------------------------------------------------------------
# act_quant
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("lift", [0, 8, 16])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("T,K", [(1, 256), (7, 4096), (64, 8640), (300, 512)])
def test_act_quant(lift, dtype, T, K):
    g = rng(T + K + lift)
    x = act_student_t(g, T, K) if K == 4096 else act_normal(g, T, K)
    x[0, :8] = [127.0, 2.5, -3.5, 0.5, 0.0, -0.0, 1.0, -127.0]
    if T > 3:
        x[2] = 0.0                      # all-zero token
        x[3] = x[3] * np.float32(2.0 ** -100)
    if dtype == "bf16":
        x, bits = to_bf16(x)
        xd = bf16_dev(bits)
    else:
        xd = dev(x)
    xq_ref, sc_ref = O.act_quant(x, lift)
    xq, sc = S.act_quant(xd, lift)
    assert np.array_equal(host(xq), xq_ref)
    assert np.array_equal(f32_bits(host(sc)), f32_bits(sc_ref))


@pytest.mark.parametrize("lift", [0, 8, 16])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("K", [2560, 6144, 8192, 12288, 16384, 16400])
def test_act_quant_row_widths(lift, dtype, K):
    """Every register budget of the one-wave-per-token kernel (4 to 32 chunks per lane) and the
    fallback to the two-pass kernel for longer rows (fp32 past 8192, bf16 past 16384), with a
    token count that leaves the last block of four tokens partly empty."""
    g = rng(K + lift + (dtype == "bf16"))
    T = 5
    x = act_normal(g, T, K)
    x[1, K - 1] = -300.0                # absmax in the last element of a row
    x[4, :] = 0.0
    if dtype == "bf16":
        x, bits = to_bf16(x)
        xd = bf16_dev(bits)
    else:
        xd = dev(x)
    xq_ref, sc_ref = O.act_quant(x, lift)
    xq, sc = S.act_quant(xd, lift)
    assert np.array_equal(host(xq), xq_ref)
    assert np.array_equal(f32_bits(host(sc)), f32_bits(sc_ref))


def test_act_quant_empty():
    import torch
    x = torch.zeros((0, 256), dtype=torch.float32, device="cuda")
    xq, sc = S.act_quant(x)
    assert xq.shape == (0, 256)


# ---------------------------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------------------------

def _fwd_case(n, K, T, N, M, layout, seed, x=None):
    g = rng(seed)
    W = master_weights(g, n, K)
    if x is None:
        x = act_normal(g, T, K)
    ref = O.pack(W, N, M, layout)
    lift = _lift(N, M, layout)
    xq_ref, sc_ref = O.act_quant(x, lift)
    acc_ref = O.acc_dense(ref["W_eff"], O.act_quant(x, 0)[0])
    y_ref = O.rescale(acc_ref, ref["gamma"], sc_ref)

    codes, meta, gamma = S.pack(dev(W), N, M, layout)
    xq, sc = S.act_quant(dev(x), lift)
    y, acc = S.fwd(xq, sc, K, codes, meta, gamma, n, N, M, layout, want_acc=True)
    acc_h = host(acc)
    nbad = int((acc_h != acc_ref).sum())
    assert nbad == 0, f"{nbad} accumulators differ (T={T}, n={n}, K={K}, {N}:{M}, layout {layout})"
    assert_y_close(host(y), y_ref)
    return y, acc


@pytest.mark.parametrize("N,M,layout", CASES_NM)
@pytest.mark.parametrize("T", [1, 3, 16, 32])
def test_fwd_gemv(N, M, layout, T):
    K = {64: 320, 128: 384, 256: 512, 32: 320}[_kq(N, M, layout)]
    _fwd_case(200, K, T, N, M, layout, seed=T * 13 + M)


@pytest.mark.parametrize("N,M,layout", CASES_NM)
@pytest.mark.parametrize("T", [33, 130, 257])
def test_fwd_gemm(N, M, layout, T):
    K = 384 if M == 8 and layout == O.LAYOUT_SPARSE else 512
    _fwd_case(300, K, T, N, M, layout, seed=T * 17 + M)


@pytest.mark.parametrize("N,M,layout,K", [(2, 4, O.LAYOUT_SPARSE, 320), (2, 4, O.LAYOUT_SPARSE, 704),
                                          (6, 8, O.LAYOUT_SPARSE, 640), (2, 4, O.LAYOUT_DENSE2, 352)])
def test_fwd_gemm_partial_stage(N, M, layout, K):
    # K steps that do not fill the last 128-byte stage of the large-tile GEMM
    _fwd_case(520, K, 300, N, M, layout, seed=K)


@pytest.mark.parametrize("N,M,layout,K", [(2, 4, O.LAYOUT_SPARSE, 1600), (2, 4, O.LAYOUT_SPARSE, 1536),
                                          (2, 4, O.LAYOUT_SPARSE, 832), (6, 8, O.LAYOUT_SPARSE, 1024),
                                          (2, 4, O.LAYOUT_DENSE2, 800), (14, 16, O.LAYOUT_SPARSE, 768)])
def test_fwd_gemm_stage_counts(N, M, layout, K):
    # the large-tile GEMM over odd and even counts of 128-byte K stages, with and without a
    # partial last stage, ragged rows and tokens
    _fwd_case(300, K, 257, N, M, layout, seed=K + M)


def test_fwd_edge_tokens():
    g = rng(9)
    T, K = 70, 256
    x = act_normal(g, T, K)
    x[0] = 0.0
    x[5, :4] = [127.0, 2.5, -3.5, 0.5]
    x[5, 4:] = 0.0
    _fwd_case(64, K, T, 2, 4, O.LAYOUT_SPARSE, seed=9, x=x)
    _fwd_case(64, K, 16, 2, 4, O.LAYOUT_SPARSE, seed=9, x=x[:16])


def test_fwd_tiny_workload_and_determinism():
    from synth import workload_inputs
    d = workload_inputs("tiny", 0)
    W, x = d["W:w"], d["X:256"]
    ref = O.forward(W, x, 2, 4)
    codes, meta, gamma = S.pack(dev(W), 2, 4)
    xq, sc = S.act_quant(dev(x))
    outs = [S.fwd(xq, sc, 256, codes, meta, gamma, 256, want_acc=True) for _ in range(2)]
    for y, acc in outs:
        assert np.array_equal(host(acc), ref["acc"])
        assert_y_close(host(y), ref["y"])
    assert np.array_equal(f32_bits(host(outs[0][0])), f32_bits(host(outs[1][0])))


def test_fwd_zero_tokens_is_noop():
    import torch
    W = master_weights(rng(4), 64, 256)
    codes, meta, gamma = S.pack(dev(W), 2, 4)
    xq = torch.zeros((0, 256), dtype=torch.int8, device="cuda")
    sc = torch.zeros(4, dtype=torch.float32, device="cuda")[:0]
    y = S.fwd(xq, sc, 256, codes, meta, gamma, 64)
    assert y.shape == (0, 64)


def test_six_eight_lifted_equals_dense_path():
    """The lifted 2:4-window product equals the dense-stored product of the same masked weights."""
    g = rng(21)
    n, K, T = 256, 512, 100
    W = master_weights(g, n, K)
    x = act_normal(g, T, K)
    c1, m1, g1 = S.pack(dev(W), 6, 8, O.LAYOUT_SPARSE)
    c2, _, g2 = S.pack(dev(W), 6, 8, O.LAYOUT_DENSE2)
    xl, sl = S.act_quant(dev(x), 8)
    xd, sd = S.act_quant(dev(x), 0)
    _, a1 = S.fwd(xl, sl, K, c1, m1, g1, n, 6, 8, O.LAYOUT_SPARSE, want_acc=True)
    _, a2 = S.fwd(xd, sd, K, c2, None, g2, n, 6, 8, O.LAYOUT_DENSE2, want_acc=True)
    assert np.array_equal(host(a1), host(a2))


def test_fourteen_sixteen_lifted_equals_dense_path():
    """14:16 through seven 2:4 windows equals the dense-stored product of the same weights."""
    g = rng(1416)
    n, K, T = 200, 768, 70
    W = master_weights(g, n, K)
    x = act_normal(g, T, K)
    c1, m1, g1 = S.pack(dev(W), 14, 16, O.LAYOUT_SPARSE)
    c2, _, g2 = S.pack(dev(W), 14, 16, O.LAYOUT_DENSE2)
    xl, sl = S.act_quant(dev(x), 16)
    xd, sd = S.act_quant(dev(x), 0)
    for TT in (T, 16):   # the GEMM and the GEMV paths
        _, a1 = S.fwd(xl[:TT], sl[:TT], K, c1, m1, g1, n, 14, 16, O.LAYOUT_SPARSE, want_acc=True)
        _, a2 = S.fwd(xd[:TT], sd[:TT], K, c2, None, g2, n, 14, 16, O.LAYOUT_DENSE2, want_acc=True)
        assert np.array_equal(host(a1), host(a2))
        q, _ = O.act_quant(x[:TT], 0)
        assert np.array_equal(host(a1), O.acc_dense(O.pack(W, 14, 16)["W_eff"], q))
