"""Grouped activation quantization (act_quant_i8_group) through the C ABI.

Each matrix of a group must give the CPU oracle's int8 rows and token scales bit for bit (the
same bar as act_quant_i8), and so the very bits of separate act_quant_i8 calls.  Groups mix row
lengths across every register budget of the one-wave-per-token kernel (a short-row matrix in a
group sized for long rows loads only its own chunks), token counts from 0 to a few hundred, and
both activation dtypes and the lifted layouts; a row past the register budget sends the group to
one launch per matrix.
"""
import numpy as np
import pytest

import oracle as O
from parity_util import bf16_dev, dev, f32_bits, host
from synth import act_normal, rng, to_bf16

pytestmark = pytest.mark.gpu

S = pytest.importorskip("sparsity_amd")


def _matrices(shapes, dtype, seed):
    g = rng(seed)
    hs, ds = [], []
    for (T, K) in shapes:
        x = act_normal(g, T, K)
        if T > 2:
            x[1, K - 1] = -300.0            # absmax in a row's last element
            x[2] = 0.0                      # an all-zero token
        if dtype == "bf16":
            x, bits = to_bf16(x)
            d = bf16_dev(bits)
        else:
            d = dev(x)
        hs.append(x)
        ds.append(d)
    return hs, ds


@pytest.mark.parametrize("lift", [0, 8, 16])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_quant_group_matches_oracle_and_single_calls(lift, dtype):
    kmax = 16384 if dtype == "bf16" else 8192
    shapes = [(7, 2560), (0, 512), (64, 512), (257, 6912 if dtype == "bf16" else 4096),
              (1, kmax), (3, 16), (130, 1024)]
    hs, ds = _matrices(shapes, dtype, seed=31 + lift + (dtype == "bf16"))
    outs = S.act_quant_group(ds, lift)
    for i, ((T, K), x, d, (xq, sc)) in enumerate(zip(shapes, hs, ds, outs)):
        q_ref, s_ref = O.act_quant(x, lift)
        assert np.array_equal(host(xq), q_ref), f"matrix {i} {T}x{K}: int8 rows"
        assert np.array_equal(f32_bits(host(sc)), f32_bits(s_ref)), f"matrix {i}: scales"
        if T:
            xq1, sc1 = S.act_quant(d, lift)
            assert np.array_equal(host(xq1), host(xq)) and \
                np.array_equal(f32_bits(host(sc1)), f32_bits(host(sc)))


def test_quant_group_long_rows_fall_back():
    """A bf16 row of 16400 elements is past the register budget: every matrix then gets its own
    launch, with the same results."""
    shapes = [(5, 16400), (9, 2560), (4, 6912)]
    hs, ds = _matrices(shapes, "bf16", seed=5)
    for (xq, sc), x in zip(S.act_quant_group(ds), hs):
        q_ref, s_ref = O.act_quant(x, 0)
        assert np.array_equal(host(xq), q_ref)
        assert np.array_equal(f32_bits(host(sc)), f32_bits(s_ref))


def test_quant_group_shared_input_and_graph_replay():
    """Two quantizations of one shared input in one group; a captured launch replays to the same
    bits (several replays with eager work in between)."""
    import torch
    hs, ds = _matrices([(33, 4096)], "bf16", seed=8)
    x, d = hs[0], ds[0]
    outs = [S.act_quant(d, 0)]          # buffers reused by the group below
    want = [O.act_quant(x, 0)]
    res = S.act_quant_group([d, d], 0, outs=[outs[0], (torch.empty_like(outs[0][0]),
                                                       torch.empty_like(outs[0][1]))])
    for xq, sc in res:
        assert np.array_equal(host(xq), want[0][0])
        assert np.array_equal(f32_bits(host(sc)), f32_bits(want[0][1]))
    cap = torch.cuda.Stream()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=cap):
        S.act_quant_group([d, d], 0, outs=res)
    for _ in range(3):
        for xq, sc in res:
            xq.fill_(77)
            sc.fill_(-1.0)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        for xq, sc in res:
            assert np.array_equal(host(xq), want[0][0]), "graph replay differs"
            assert np.array_equal(f32_bits(host(sc)), f32_bits(want[0][1]))


def test_quant_group_training_step_sizes_sampled():
    """The training step's two activation matrices (8192 x 3200 and 8192 x 8640, bf16) in one
    group; 48 sampled rows of each against the oracle (every row is quantized on its own, so a
    sampled row is an exact check), plus the first and last rows."""
    T = 8192
    hs, ds = _matrices([(T, 3200), (T, 8640)], "bf16", seed=17)
    outs = S.act_quant_group(ds)
    g = rng(18)
    for x, (xq, sc) in zip(hs, outs):
        rows = np.unique(np.concatenate([[0, T - 1], g.integers(0, T, 48)]))
        q_ref, s_ref = O.act_quant(x[rows], 0)
        assert np.array_equal(host(xq)[rows], q_ref)
        assert np.array_equal(f32_bits(host(sc))[rows], f32_bits(s_ref))
