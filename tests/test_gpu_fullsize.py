"""Parity at the benchmark workloads' full sizes, in the launch configurations bench.py times.

Packed codes, metadata, gamma and int8 activations are compared in full, bit for bit.  Outputs are
compared in full where the oracle's int64 product is cheap (decode), else on sampled tokens (all
output rows) and sampled rows (all tokens).  Inputs come from the seeded generators in synth/.
"""
import numpy as np
import pytest

import oracle as O
from parity_util import assert_y_close, dev, f32_bits, host
from synth import workload_grads, workload_inputs

pytestmark = pytest.mark.gpu

S = pytest.importorskip("sparsity_amd")


def _bf16_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _check_pack(W, N, M, layout, what):
    ref = O.pack(W, N, M, layout)
    codes, meta, gamma = S.pack(dev(W), N, M, layout)
    assert f32_bits(host(gamma)[0]) == f32_bits(ref["gamma"]), f"{what}: gamma"
    assert np.array_equal(host(codes).view(np.uint32), ref["codes"]), f"{what}: codes"
    if meta is not None:
        assert np.array_equal(host(meta).view(np.uint32), ref["meta"]), f"{what}: meta"
    return ref, (codes, meta, gamma)


def _check_quant(x, bits, lift, what):
    xq, sc = S.act_quant(_bf16_dev(bits), lift)
    q_ref, s_ref = O.act_quant(x, lift)
    assert np.array_equal(host(xq), q_ref), f"{what}: int8 activations"
    assert np.array_equal(f32_bits(host(sc)), f32_bits(s_ref)), f"{what}: token scales"
    return xq, sc


def _check_sampled(ref, x, y, acc, toks, rows, what):
    """Accumulators and outputs of sampled tokens (all rows) and sampled rows (all tokens)."""
    q, s = O.act_quant(x, 0)
    acc_t = O.acc_dense(ref["W_eff"], q[toks])
    assert np.array_equal(acc[toks], acc_t), f"{what}: accumulators of sampled tokens"
    assert_y_close(y[toks], O.rescale(acc_t, ref["gamma"], s[toks]), what=f"{what} sampled tokens")
    acc_r = O.acc_dense(ref["W_eff"][rows], q)
    assert np.array_equal(acc[:, rows], acc_r), f"{what}: accumulators of sampled rows"
    assert_y_close(y[:, rows], O.rescale(acc_r, ref["gamma"], s), what=f"{what} sampled rows")


def test_decode_full_size_grouped():
    """FFN up 6912x2560 and down 2560x6912 (2:4) at T = 1, 4, 16 in one grouped launch, as the
    decode benchmark runs them; every output compared; single-projection calls and the fused
    (in-kernel quantization) group agree bitwise."""
    import torch
    d = workload_inputs("decode", 0)
    projs = []
    for name, K in (("up", 2560), ("down", 6912)):
        W = d[f"W:{name}"]
        ref, (codes, meta, gamma) = _check_pack(W, 2, 4, O.LAYOUT_SPARSE, f"decode {name}")
        print(f"decode {name}: pack bit-exact", flush=True)
        for T in (1, 4, 16):
            x, bits = d[f"X:{K}"][:T], d[f"Xbits:{K}"][:T]
            xq, sc = _check_quant(x, bits, 0, f"decode {name} T={T}")
            n = W.shape[0]
            projs.append(dict(xq=xq, scale=sc, K=K, codes=codes, meta=meta, gamma=gamma, n=n,
                              y=torch.empty((T, n), device="cuda"),
                              acc=torch.empty((T, n), dtype=torch.int32, device="cuda"),
                              ref=ref, x=x, name=f"{name} T={T}"))
    S.FwdGroup(projs)()
    # the same projections with quantization fused into the grouped GEMV: bitwise the same
    fused = []
    for name, K in (("up", 2560), ("down", 6912)):
        for T in (1, 4, 16):
            p = next(q for q in projs if q["name"] == f"{name} T={T}")
            fused.append(dict(x=_bf16_dev(d[f"Xbits:{K}"][:T]), K=K, codes=p["codes"],
                              meta=p["meta"], gamma=p["gamma"], n=p["n"],
                              y=torch.empty_like(p["y"]), acc=torch.empty_like(p["acc"]), ref=p))
    S.FusedGroup(fused)()
    for f in fused:
        assert np.array_equal(f32_bits(host(f["y"])), f32_bits(host(f["ref"]["y"]))), f["ref"]["name"]
        assert np.array_equal(host(f["acc"]), host(f["ref"]["acc"])), f["ref"]["name"]
    print("decode fused group: bitwise equal to act_quant + group", flush=True)
    for p in projs:
        q, s = O.act_quant(p["x"], 0)
        acc_ref = O.acc_dense(p["ref"]["W_eff"], q)
        assert np.array_equal(host(p["acc"]), acc_ref), f"decode {p['name']}: accumulators"
        assert_y_close(host(p["y"]), O.rescale(acc_ref, p["ref"]["gamma"], s), what=p["name"])
        y1 = S.fwd(p["xq"], p["scale"], p["K"], p["codes"], p["meta"], p["gamma"], p["n"])
        assert np.array_equal(f32_bits(host(y1)), f32_bits(host(p["y"]))), p["name"]
        print(f"decode {p['name']}: ok", flush=True)


def test_prefill_full_size():
    """4096 Student-t tokens x 4096 -> 11008 (2:4), the large-tile GEMM."""
    d = workload_inputs("prefill", 0)
    W, x, bits = d["W:gate_up"], d["X:4096"], d["Xbits:4096"]
    ref, (codes, meta, gamma) = _check_pack(W, 2, 4, O.LAYOUT_SPARSE, "prefill")
    print("prefill: pack bit-exact", flush=True)
    xq, sc = _check_quant(x, bits, 0, "prefill")
    y, acc = S.fwd(xq, sc, 4096, codes, meta, gamma, 11008, want_acc=True)
    g = np.random.default_rng(11)
    toks = np.unique(np.concatenate([[0, 4095], g.choice(4096, 30, replace=False)]))
    rows = np.unique(np.concatenate([[0, 11007], g.choice(11008, 30, replace=False)]))
    _check_sampled(ref, x, host(y), host(acc), toks, rows, "prefill")
    print("prefill: sampled outputs ok", flush=True)


def test_six_eight_full_size():
    """6:8 through three 2:4 windows, 2048 x 4096 -> 4096: pack and lifted activations bit-exact,
    sampled outputs against the oracle, and the dense-stored path bitwise equal at full size."""
    d = workload_inputs("six_eight", 0)
    W, x, bits = d["W:w"], d["X:4096"], d["Xbits:4096"]
    ref, (cs, ms, gs) = _check_pack(W, 6, 8, O.LAYOUT_SPARSE, "6:8 windows")
    _, (cd, _, gd) = _check_pack(W, 6, 8, O.LAYOUT_DENSE2, "6:8 dense")
    print("6:8: both packs bit-exact", flush=True)
    xl, sl = _check_quant(x, bits, 8, "6:8 lifted")
    xd, sd = _check_quant(x, bits, 0, "6:8 plain")
    ys, accs = S.fwd(xl, sl, 4096, cs, ms, gs, 4096, 6, 8, O.LAYOUT_SPARSE, want_acc=True)
    yd = S.fwd(xd, sd, 4096, cd, None, gd, 4096, 6, 8, O.LAYOUT_DENSE2)
    assert np.array_equal(f32_bits(host(ys)), f32_bits(host(yd))), "windows path != dense path"
    g = np.random.default_rng(68)
    toks = np.unique(np.concatenate([[0, 2047], g.choice(2048, 30, replace=False)]))
    rows = np.unique(np.concatenate([[0, 4095], g.choice(4096, 30, replace=False)]))
    _check_sampled(ref, x, host(ys), host(accs), toks, rows, "6:8")
    print("6:8: sampled outputs ok", flush=True)


def test_train_step_full_size():
    """3B-alike layer set at 8192 tokens: all seven masters packed bit-exactly, both activation
    matrices quantized bit-exactly, each forward checked on sampled tokens and rows."""
    d = workload_inputs("train_step", 0)
    Q = {K: _check_quant(d[f"X:{K}"], d[f"Xbits:{K}"], 0, f"train X:{K}") for K in (3200, 8640)}
    g = np.random.default_rng(35)
    for L in ("q", "k", "v", "o", "gate", "up", "down"):
        W = d[f"W:{L}"]
        n, K = W.shape
        ref, (codes, meta, gamma) = _check_pack(W, 2, 4, O.LAYOUT_SPARSE, f"train {L}")
        xq, sc = Q[K]
        y, acc = S.fwd(xq, sc, K, codes, meta, gamma, n, want_acc=True)
        toks = np.unique(np.concatenate([[0, 8191], g.choice(8192, 6, replace=False)]))
        rows = np.unique(np.concatenate([[0, n - 1], g.choice(n, 6, replace=False)]))
        _check_sampled(ref, d[f"X:{K}"], host(y), host(acc), toks, rows, f"train {L}")
        print(f"train {L} {n}x{K}: pack bit-exact, sampled outputs ok", flush=True)


def test_fourteen_sixteen_full_size():
    """14:16 through seven 2:4 windows at the 6:8 workload's shapes (2048 x 4096 -> 4096, same
    seeded master and activations): packs and lifted activations bit-exact, sampled outputs
    against the oracle, the dense-stored path bitwise equal at full size."""
    d = workload_inputs("six_eight", 0)
    W, x, bits = d["W:w"], d["X:4096"], d["Xbits:4096"]
    ref, (cs, ms, gs) = _check_pack(W, 14, 16, O.LAYOUT_SPARSE, "14:16 windows")
    _, (cd, _, gd) = _check_pack(W, 14, 16, O.LAYOUT_DENSE2, "14:16 dense")
    print("14:16: both packs bit-exact", flush=True)
    xl, sl = _check_quant(x, bits, 16, "14:16 lifted")
    xd, sd = _check_quant(x, bits, 0, "14:16 plain")
    ys, accs = S.fwd(xl, sl, 4096, cs, ms, gs, 4096, 14, 16, O.LAYOUT_SPARSE, want_acc=True)
    yd = S.fwd(xd, sd, 4096, cd, None, gd, 4096, 14, 16, O.LAYOUT_DENSE2)
    assert np.array_equal(f32_bits(host(ys)), f32_bits(host(yd))), "windows path != dense path"
    g = np.random.default_rng(1416)
    toks = np.unique(np.concatenate([[0, 2047], g.choice(2048, 30, replace=False)]))
    rows = np.unique(np.concatenate([[0, 4095], g.choice(4096, 30, replace=False)]))
    _check_sampled(ref, x, host(ys), host(accs), toks, rows, "14:16")
    print("14:16: sampled outputs ok", flush=True)


U = 2.0 ** -24


def _within(got, ref, bound, what):
    got = np.asarray(got, np.float64)
    bad = np.abs(got - ref) > bound + 1e-45
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} outside the fp32 summation bound; first at "
                             f"{i}: gpu {got[i]!r} ref {ref[i]!r} bound {bound[i]!r}")


def test_train_step_backward_full_size_grouped():
    """The layer set's grouped backward at 8192 tokens, launched as the training-step benchmark
    launches it (the six K = 3200 projections summing into one dX in layer order, down into its
    own): sampled dW rows and columns of every projection, sampled dX tokens and columns, against
    the oracle's backward on the same slices, within the bound of fp32 summation in any order
    (2 R u sum|terms| + u |ref| per product, plus u |partial sum| per dX accumulation)."""
    import torch
    T = 8192
    d = workload_inputs("train_step", 0)
    gr = workload_grads("train_step", 0)
    Q = {K: _check_quant(d[f"X:{K}"], d[f"Xbits:{K}"], 0, f"bwd X:{K}") for K in (3200, 8640)}
    q_ref = {K: O.act_quant(d[f"X:{K}"], 0) for K in Q}
    dX = {K: torch.empty((T, K), dtype=torch.float32, device="cuda") for K in Q}
    projs, refs, seen = [], [], set()
    for L in ("q", "k", "v", "o", "gate", "up", "down"):
        W = d[f"W:{L}"]
        n, K = W.shape
        ref, (codes, meta, gamma) = _check_pack(W, 2, 4, O.LAYOUT_SPARSE, f"bwd {L}")
        projs.append(dict(dy=_bf16_dev(gr[f"dYbits:{L}"]), xq=Q[K][0], scale=Q[K][1], K=K,
                          codes=codes, meta=meta, gamma=gamma, n=n, dx=dX[K],
                          dw=torch.empty((n, K), dtype=torch.float32, device="cuda"),
                          accumulate=(K in seen, False)))
        refs.append((L, ref, n, K))
        seen.add(K)
    S.BwdGroup(projs, T)()
    torch.cuda.synchronize()
    print("grouped backward done", flush=True)
    g = np.random.default_rng(808)
    toks = np.unique(np.concatenate([[0, T - 1], g.choice(T, 2, replace=False)]))
    sums = {K: (np.zeros((len(toks), K)), np.zeros((len(toks), K)))
            for K in Q}   # running reference sum and its bound, sampled dX rows
    for (L, ref, n, K), p in zip(refs, projs):
        dy = gr[f"dY:{L}"].astype(np.float64)
        q, sc = q_ref[K]
        W_eff, gamma = ref["W_eff"], ref["gamma"]
        dw = host(p["dw"])
        rows = np.unique(np.concatenate([[0, n - 1], g.choice(n, 2, replace=False)]))
        cols = np.unique(np.concatenate([[0, K - 1], g.choice(K, 2, replace=False)]))
        # dW rows: dW[o] = dY[:, o]^T X^, over all K
        _, dw_r = O.backward(dy[:, rows], W_eff[rows], gamma, q, sc)
        xh = np.abs(O.dequant_act(q, sc).astype(np.float64))
        mag = np.abs(dy[:, rows]).T @ xh
        _within(dw[rows], dw_r, 2 * T * U * mag + U * np.abs(dw_r), f"{L} dW rows")
        # dW columns: dW[:, k] = dY^T X^[:, k], over all out-features
        _, dw_c = O.backward(dy, W_eff[:, cols], gamma, q[:, cols], sc)
        mag = np.abs(dy).T @ xh[:, cols]
        _within(dw[:, cols], dw_c, 2 * T * U * mag + U * np.abs(dw_c), f"{L} dW columns")
        del xh
        # dX tokens: this projection's term of the running sum in layer order
        dx_t, _ = O.backward(dy[toks], W_eff, gamma, q[toks], sc[toks])
        mag = np.float64(gamma) * (np.abs(dy[toks]) @ np.abs(W_eff.astype(np.float64)))
        r, b = sums[K]
        r += dx_t
        b += 2 * n * U * mag + U * np.abs(dx_t)
        if p["accumulate"][0]:
            b += U * np.abs(r)
        print(f"{L} {n}x{K}: sampled dW rows and columns ok", flush=True)
    for K in Q:
        r, b = sums[K]
        _within(host(dX[K])[toks], r, b, f"dX:{K} sampled tokens")
        print(f"dX:{K}: sampled tokens ok", flush=True)


def test_backward_full_size_exact_dw():
    """dW at the gate projection's full size (8192 tokens, 8640 x 3200) on inputs for which every
    partial sum is exact in fp32, so dW must equal the oracle bit for bit whatever the summation
    order: |x| in [0.5, 1] with absmax 1 per token gives q in [64, 127] and X^ = bf16(q / 127)
    multiples of 2^-8 in [0.5, 1]; dY in {-1, 0, +1}; |dW| * 2^8 <= 8192 * 256 < 2^24.  X^
    without its bf16 rounding (or rounded otherwise) has 24-bit mantissas and moves the sums off
    the 2^-8 grid, which the bit-exact comparison catches (checked below on the oracle itself)."""
    import torch
    T, n, K = 8192, 8640, 3200
    g = np.random.default_rng(8192)
    x = (g.uniform(0.5, 1.0, (T, K)) * g.choice([-1.0, 1.0], (T, K))).astype(np.float32)
    x[np.arange(T), g.integers(0, K, T)] = 1.0                 # absmax 1 in every token
    dy_bits = g.choice(np.array([0x3F80, 0xBF80, 0x0000], np.uint16), (T, n), p=[0.3, 0.3, 0.4])
    dy = np.where(dy_bits == 0x3F80, 1.0, np.where(dy_bits == 0xBF80, -1.0, 0.0))
    q, sc = O.act_quant(x, 0)
    assert np.abs(q).min() >= 64
    xq, s = S.act_quant(dev(x))
    assert np.array_equal(host(xq), q) and np.array_equal(f32_bits(host(s)), f32_bits(sc))
    W = (torch.randn((n, K), generator=torch.Generator(device="cuda").manual_seed(5),
                     device="cuda") * 0.02).contiguous()
    codes, meta, gamma = S.pack(W, 2, 4)
    _, dw = S.bwd(_bf16_dev(dy_bits), xq, s, K, codes, meta, gamma, n, want_dx=False)
    dw = host(dw)
    xh = O.dequant_act(q, sc).astype(np.float64)
    rows = np.unique(np.concatenate([[0, n - 1], g.choice(n, 62, replace=False)]))
    cols = np.unique(np.concatenate([[0, K - 1], g.choice(K, 62, replace=False)]))
    ref_r = dy[:, rows].T @ xh                                 # exact: integers / 256 below 2^24
    ref_c = dy.T @ xh[:, cols]
    assert np.array_equal(ref_r * 256, np.round(ref_r * 256))
    nbad = int((dw[rows].astype(np.float64) != ref_r).sum())
    assert nbad == 0, f"{nbad} of the sampled dW rows' entries differ"
    nbad = int((dw[:, cols].astype(np.float64) != ref_c).sum())
    assert nbad == 0, f"{nbad} of the sampled dW columns' entries differ"
    # sensitivity: the same sums over X^ without its bf16 rounding leave the 2^-8 grid
    x_unrounded = (np.asarray(q, np.float32) * sc[:, None]).astype(np.float64)
    slip = dy[:, rows[:4]].T @ x_unrounded
    assert (slip != ref_r[:4]).mean() > 0.99
    print("full-size dW: sampled rows and columns bit-exact", flush=True)
