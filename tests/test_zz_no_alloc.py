"""bitlinear_pack_noalloc (the pack for callers that cannot allocate) against bitlinear_pack.

Through the C ABI: the allocation-free entry point keeps its workspace in a static per-device
array that every call shares, so it is checked on calls in a row -- each compared bit for bit with
bitlinear_pack (caller workspace) on the same master, and with the oracle -- the second smaller
than the first, including a master whose gamma needs the exact fallback right after one that did
not (the shared state of the previous call must not leak into the next).
"""
import ctypes

import numpy as np
import pytest

import oracle as O
from parity_util import dev, f32_bits, host
from synth import master_weights, rng

pytestmark = pytest.mark.gpu

S = pytest.importorskip("sparsity_amd")


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _outs(n, K, N, M, layout):
    import torch
    cb, mb, _, wsb = S.packed_bytes(n, K, N, M, layout)
    mk = lambda b: torch.full((max(b, 16),), 0xAB, dtype=torch.uint8, device="cuda")
    return mk(cb), (mk(mb) if mb else None), torch.full((4,), float("nan"), device="cuda"), wsb


def _both(W, N, M, layout):
    """(noalloc outputs, bitlinear_pack outputs), each (codes u8, meta u8 or None, gamma f32)."""
    import torch
    n, K = W.shape
    Wd = dev(W)
    c1, m1, g1, _ = _outs(n, K, N, M, layout)
    st = S.lib().bitlinear_pack_noalloc(Wd.data_ptr(), n, K, N, M, layout, c1.data_ptr(),
                                        None if m1 is None else m1.data_ptr(), g1.data_ptr(),
                                        _stream())
    assert st == 0, st
    c2, m2, g2, wsb = _outs(n, K, N, M, layout)
    ws = torch.full((wsb,), 0x5A, dtype=torch.uint8, device="cuda")
    st = S.lib().bitlinear_pack(Wd.data_ptr(), n, K, N, M, layout, c2.data_ptr(),
                                None if m2 is None else m2.data_ptr(), g2.data_ptr(),
                                ws.data_ptr(), wsb, _stream())
    assert st == 0, st
    fetch = lambda c, m, g: (host(c), None if m is None else host(m), host(g)[0])
    return fetch(c1, m1, g1), fetch(c2, m2, g2)


def _check(W, N, M, layout):
    (c1, m1, g1), (c2, m2, g2) = _both(W, N, M, layout)
    assert f32_bits(g1) == f32_bits(g2)
    assert np.array_equal(c1, c2)
    if m1 is not None:
        assert np.array_equal(m1, m2)
    ref = O.pack(W, N, M, layout)
    assert f32_bits(g1) == f32_bits(ref["gamma"])
    assert np.array_equal(c1[:ref["codes"].size * 4].view(np.uint32), ref["codes"])
    if m1 is not None:
        assert np.array_equal(m1[:ref["meta"].size * 4].view(np.uint32), ref["meta"])
    return g1


def _midpoint(n, K, bump=1):
    """All |w| = 1 except one, so the exact mean is 1 + bump * 2^-24, halfway between two fp32
    values: no fp64 bound can decide the rounding and the exact fallback must (ties to even)."""
    W = np.ones((n, K), np.float32)
    W[3, 5] = np.float32(1.0 + bump * (n * K) * 2.0 ** -24)
    W[1::2] *= -1
    return W


@pytest.mark.parametrize("N,M,layout", [(2, 4, O.LAYOUT_SPARSE), (6, 8, O.LAYOUT_SPARSE),
                                        (4, 4, O.LAYOUT_DENSE2)])
def test_noalloc_pack_calls_in_a_row(N, M, layout):
    g = rng(51)
    big = master_weights(g, 300, 1024)      # ragged rows, four 256-wide tiles
    small = master_weights(g, 40, 256)
    _check(big, N, M, layout)
    _check(small, N, M, layout)


def test_noalloc_pack_exact_fallback_after_certified_call():
    g = rng(52)
    _check(master_weights(g, 256, 512), 2, 4, O.LAYOUT_SPARSE)        # certified gamma
    assert int(f32_bits(_check(_midpoint(64, 256), 2, 4, O.LAYOUT_SPARSE))) == 0x3F800000
    assert int(f32_bits(_check(_midpoint(32, 128, 3), 2, 4, O.LAYOUT_SPARSE))) == 0x3F800002
    _check(master_weights(g, 33, 256), 2, 4, O.LAYOUT_SPARSE)         # certified again


def test_noalloc_pack_rejects_like_pack():
    lib = S.lib()
    assert lib.bitlinear_pack_noalloc(None, 32, 256, 2, 4, 0, None, None, None, None) == -22
    assert lib.bitlinear_pack_noalloc(None, 32, 100, 2, 4, 0, None, None, None, None) == -22
    assert lib.bitlinear_pack_noalloc(None, 32, 256, 3, 4, 0, None, None, None, None) == -95
