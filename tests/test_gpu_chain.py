"""Fused decode over a chain of dependent layers (bitlinear_fwd_chain) through the C ABI.

Each layer's input is the previous layer's fp32 output.  Per layer, the GPU's int32 accumulators
must equal the oracle's (act_quant of that layer's input, int64 product of the packed ternary
weights) bit for bit and y must be within 1e-5 of the oracle's rescale, the input being the
GPU's own previous y (the oracle rounds y once from fp64, the GPU's rescale rounds twice in
fp32, so feeding the oracle's y forward would compare different inputs).  The chain must also
equal act_quant_i8 + bitlinear_fwd called layer by layer, bit for bit, and a wait forced to give
up from the host (a spin limit of one poll) must end the launch with the error word set.
"""
import numpy as np
import pytest

import oracle as O
from parity_util import assert_y_close, dev, host
from synth import act_normal, master_weights, rng, to_bf16

pytestmark = pytest.mark.gpu

S = pytest.importorskip("sparsity_amd")


def _layers(g, dims):
    import torch
    out = []
    for (n, K) in dims:
        W = master_weights(g, n, K)
        ref = O.pack(W, 2, 4)
        c, m, ga = S.pack(dev(W), 2, 4)
        out.append(dict(codes=c, meta=m, gamma=ga, n=n, K=K, ref=ref))
    return out


def _run_chain(layers, T, x0):
    import torch
    for ly in layers:
        ly["acc"] = torch.empty((T, ly["n"]), dtype=torch.int32, device="cuda")
    ch = S.Chain([{k: v for k, v in ly.items() if k != "ref"} for ly in layers], T)
    ch(x0)
    assert ch.error() == 0
    return ch


def _check_against_oracle(layers, ch, x0_host):
    inp = x0_host
    for l, ly in enumerate(layers):
        q, s = O.act_quant(inp)
        acc_ref = O.acc_dense(ly["ref"]["W_eff"], q)
        acc = host(ch.accs[l])
        assert np.array_equal(acc, acc_ref), f"layer {l}: accumulators differ"
        y = host(ch.ys[l])
        assert_y_close(y, O.rescale(acc_ref, ly["ref"]["gamma"], s), what=f"layer {l} y")
        inp = y


def _check_against_calls(layers, ch, x0, T):
    """act_quant_i8 + bitlinear_fwd layer by layer, on the same inputs: bitwise equal."""
    import torch
    inp = x0
    for l, ly in enumerate(layers):
        xq, sc = S.act_quant(inp)
        y, acc = S.fwd(xq, sc, ly["K"], ly["codes"], ly["meta"], ly["gamma"], ly["n"], want_acc=True)
        torch.cuda.synchronize()
        assert torch.equal(acc, ch.accs[l]), f"layer {l}: accumulators differ from the calls"
        assert torch.equal(y, ch.ys[l]), f"layer {l}: y differs from the calls"
        inp = y


DIMS = [(320, 256), (192, 320), (448, 192), (128, 448), (100, 128)]


@pytest.mark.parametrize("T", [1, 5, 16, 32])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_chain_matches_oracle_layer_by_layer(T, dtype):
    import torch
    g = rng(60 + T)
    layers = _layers(g, DIMS)
    x = act_normal(g, T, DIMS[0][1])
    if dtype == "bf16":
        xh, bits = to_bf16(x)
        x0 = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        xh = x
        x0 = dev(x)
    ch = _run_chain(layers, T, x0)
    _check_against_oracle(layers, ch, xh)
    _check_against_calls(layers, ch, x0, T)


@pytest.mark.parametrize("T,dims", [
    (32, [(2304, 2112), (128, 2304), (2112, 128), (64, 2112)]),
    (17, [(256, 3904), (3904, 256), (128, 3904)]),
])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_chain_split_input_layers(T, dims, dtype):
    """Layers whose fp32 input exceeds 256 KB (T x K x 4) take the two-stage input: every block
    quantizes a slice of the rows into the workspace's int8 rows, then every block copies them
    into LDS (K not a multiple of 1 KB: a short last piece per row).  Split layers at the start
    (bf16 or fp32 first input) and after an unsplit one."""
    import torch
    g = rng(80 + T)
    layers = _layers(g, dims)
    x = act_normal(g, T, dims[0][1])
    if dtype == "bf16":
        xh, bits = to_bf16(x)
        x0 = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        xh = x
        x0 = dev(x)
    ch = _run_chain(layers, T, x0)
    _check_against_oracle(layers, ch, xh)
    _check_against_calls(layers, ch, x0, T)


def test_chain_degenerate_rows():
    """A zero input row (absmax 0: q = 0, scale 0, y = 0 all along the chain) and a heavy-tailed
    row next to ordinary ones."""
    import torch
    g = rng(70)
    layers = _layers(g, DIMS[:3])
    x = act_normal(g, 6, DIMS[0][1])
    x[2] = 0.0
    x[4] *= 1e4
    ch = _run_chain(layers, 6, dev(x))
    _check_against_oracle(layers, ch, x)
    for l in range(3):
        assert not host(ch.ys[l])[2].any()


@pytest.mark.parametrize("T", [1, 16])
def test_chain_full_size_decode_layers(T):
    """Four decode layers (FFN up 6912 x 2560, down 2560 x 6912, up, down) chained, bf16 input."""
    import torch
    g = rng(71)
    dims = [(6912, 2560), (2560, 6912), (6912, 2560), (2560, 6912)]
    layers = _layers(g, dims)
    xh, bits = to_bf16(act_normal(g, T, 2560))
    x0 = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    ch = _run_chain(layers, T, x0)
    _check_against_calls(layers, ch, x0, T)
    _check_against_oracle(layers, ch, xh)


def test_chain_bounded_wait_gives_up_and_recovers():
    """A spin limit of one poll makes the first waits give up: the launch ends with the error
    word set (outputs invalid).  The next launch with the default limit is correct."""
    import torch
    g = rng(72)
    layers = _layers(g, DIMS)
    T = 4
    x = act_normal(g, T, DIMS[0][1])
    x0 = dev(x)
    for ly in layers:
        ly["acc"] = torch.empty((T, ly["n"]), dtype=torch.int32, device="cuda")
    ch = S.Chain([{k: v for k, v in ly.items() if k != "ref"} for ly in layers], T)
    ch(x0, spin_limit=1)
    assert ch.error() != 0
    ch(x0)
    assert ch.error() == 0
    _check_against_oracle(layers, ch, x)
