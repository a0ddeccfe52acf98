"""The exact gamma fallback at full size: once per master, not once per pack block.

A training-step gate master (8640 x 3200) whose exact mean |w| lies exactly halfway between two
fp32 values: no fp64 error bound can decide the rounding, so the exact exponent-binned pass must
(ties to even).  gamma, codes and meta are compared with the oracle, and the pack is timed against
the same call on an ordinary master of that size: the fallback adds one pass over W.
"""
import numpy as np
import pytest

import oracle as O
from parity_util import as_u32, dev, f32_bits, host
from synth import master_weights, rng

pytestmark = pytest.mark.gpu

S = pytest.importorskip("sparsity_amd")

# diagnostic flag in bitlinear_pack's workspace: after the fp64 partials (1024 x 8 bytes), the
# exact pass's per-block word slots (256 x 128), its nine counter lines (9 x 128), gamma and tau
EXACT_USED_OFFSET = 1024 * 8 + 256 * 128 + 9 * 128 + 8


def _midpoint(n, K):
    W = np.ones((n, K), np.float32)
    W[7, 9] = np.float32(1.0 + (n * K) * 2.0 ** -24)   # exact mean 1 + 2^-24: a tie -> 1.0
    W[1::2] *= -1
    return W


def _time_pack(torch, Wd, ws, out, reps=7):
    for _ in range(2):
        S.pack(Wd, out=out, ws=ws)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record()
        S.pack(Wd, out=out, ws=ws)
        b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev]))


def test_gamma_midpoint_full_size_gate_master():
    import torch
    n, K = 8640, 3200
    W = _midpoint(n, K)
    Wd = dev(W)
    cb, mb, _, wsb = S.packed_bytes(n, K)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    out = (torch.empty(cb, dtype=torch.uint8, device="cuda"),
           torch.empty(mb, dtype=torch.uint8, device="cuda"),
           torch.empty(4, dtype=torch.float32, device="cuda")[:1])
    codes, meta, gamma = S.pack(Wd, out=out, ws=ws)
    ref = O.pack(W, 2, 4)
    assert int(f32_bits(host(gamma)[0])) == 0x3F800000 == int(f32_bits(ref["gamma"]))
    assert host(ws)[EXACT_USED_OFFSET] == 1, "the exact fallback did not decide gamma"
    assert np.array_equal(as_u32(codes), ref["codes"])
    assert np.array_equal(as_u32(meta), ref["meta"])

    t_exact = _time_pack(torch, Wd, ws, out)
    Wn = dev(master_weights(rng(53), n, K))
    t_plain = _time_pack(torch, Wn, ws, out)
    assert host(ws)[EXACT_USED_OFFSET] == 0
    print(f"pack 8640x3200: exact fallback {t_exact:.3f} ms, certified {t_plain:.3f} ms, "
          f"ratio {t_exact / t_plain:.2f}")
    assert t_exact <= 2.0 * t_plain, (t_exact, t_plain)
