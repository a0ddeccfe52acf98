"""The torch wrappers refuse wrong output buffers before anything reaches the C ABI (CPU only).

The C ABI receives bare device pointers and cannot see buffer sizes, so the wrappers check dtype,
device, contiguity and element count of every buffer they pass.  Stand-in tensor objects that
report a CUDA device let the checks run without a GPU; a wrong buffer must raise ValueError
before any library call that could enqueue work.
"""
import pytest
import torch

import sparsity_amd as S

DEV = torch.device("cuda:0")


class FakeT:
    """A stand-in for a CUDA tensor: shape, dtype, device and contiguity only."""

    def __init__(self, shape, dtype, device=DEV, contiguous=True):
        self.shape = tuple(shape) if isinstance(shape, (tuple, list)) else (shape,)
        self.dtype = dtype
        self.device = device
        self.is_cuda = device.type == "cuda"
        self._contig = contiguous

    def numel(self):
        n = 1
        for d in self.shape:
            n *= d
        return n

    def dim(self):
        return len(self.shape)

    def is_contiguous(self):
        return self._contig

    def data_ptr(self):
        raise AssertionError("a checked buffer reached the C ABI")


def _pack_out(n, K, N=2, M=4, layout=S.BL_LAYOUT_SPARSE):
    cb, mb, _, wsb = S.packed_bytes(n, K, N, M, layout)
    return (FakeT(cb, torch.uint8), FakeT(mb, torch.uint8) if mb else None,
            FakeT(1, torch.float32)), FakeT(wsb, torch.uint8)


def test_pack_checks_outputs():
    n, K = 64, 256
    W = FakeT((n, K), torch.float32)
    (c, m, g), ws = _pack_out(n, K)
    cases = {
        "codes": ((FakeT(c.numel() - 1, torch.uint8), m, g), ws),
        "meta": ((c, FakeT(m.numel(), torch.int8), g), ws),
        "gamma": ((c, m, FakeT(1, torch.float64)), ws),
        "ws": ((c, m, g), FakeT(ws.numel() - 16, torch.uint8)),
        "device": ((c, m, FakeT(1, torch.float32, device=torch.device("cuda:1"))), ws),
        "contiguous": ((FakeT(c.numel(), torch.uint8, contiguous=False), m, g), ws),
    }
    for name, (out, w) in cases.items():
        with pytest.raises(ValueError):
            S.pack(W, out=out, ws=w)
    (c2, _, g2), ws2 = _pack_out(n, K, 4, 4, S.BL_LAYOUT_DENSE2)
    with pytest.raises(ValueError):   # dense 2-bit codes carry no meta
        S.pack(W, 4, 4, S.BL_LAYOUT_DENSE2, out=(c2, FakeT(16, torch.uint8), g2), ws=ws2)


def test_act_quant_checks_outputs():
    T, K = 5, 256
    x = FakeT((T, K), torch.bfloat16)
    with pytest.raises(ValueError):
        S.act_quant(x, out=(FakeT((T, K - 1), torch.int8), FakeT(T, torch.float32)))
    with pytest.raises(ValueError):
        S.act_quant(x, out=(FakeT((T, K), torch.uint8), FakeT(T, torch.float32)))
    with pytest.raises(ValueError):
        S.act_quant(x, out=(FakeT((T, K), torch.int8), FakeT(T - 1, torch.float32)))
    with pytest.raises(ValueError):   # lifted 6:8 rows are 1.5 K long
        S.act_quant(x, 8, out=(FakeT((T, K), torch.int8), FakeT(T, torch.float32)))
    with pytest.raises(ValueError):
        S.act_quant_group([x], outs=[(FakeT((T, K), torch.int8), FakeT(T, torch.int32))])


def test_fwd_checks_shapes_and_buffers():
    T, K, n = 4, 256, 96
    cb, mb, ke, _ = S.packed_bytes(n, K)
    xq, sc = FakeT((T, K), torch.int8), FakeT(T, torch.float32)
    codes, meta, gamma = FakeT(cb, torch.uint8), FakeT(mb, torch.uint8), FakeT(1, torch.float32)
    y = FakeT((T, n), torch.float32)
    ok = dict(xq=xq, scale=sc, K=K, codes=codes, meta=meta, gamma=gamma, n=n)

    def call(**kw):
        a = dict(ok)
        out = kw.pop("out", (y, None))
        a.update(kw)
        return S.fwd(a["xq"], a["scale"], a["K"], a["codes"], a["meta"], a["gamma"], a["n"],
                     out=out)
    bad = [
        dict(xq=FakeT((T, K + 64), torch.int8)),          # row length is not K_eff
        dict(scale=FakeT(T - 1, torch.float32)),
        dict(codes=FakeT(cb - 4, torch.uint8)),
        dict(meta=FakeT(mb - 4, torch.uint8)),
        dict(meta=None),
        dict(gamma=FakeT(1, torch.float16)),
        dict(n=n + 64),                                    # codes too short for more rows
        dict(out=(FakeT((T, n - 1), torch.float32), None)),
        dict(out=(y, FakeT((T, n), torch.float32))),       # acc must be int32
        dict(out=(y, FakeT((T, n - 1), torch.int32))),
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            call(**kw)
    with pytest.raises(ValueError):   # windows need the lifted rows: 1.5 K for 6:8
        cb8, mb8, _, _ = S.packed_bytes(n, K, 6, 8)
        S.fwd(xq, sc, K, FakeT(cb8, torch.uint8), FakeT(mb8, torch.uint8), gamma, n, 6, 8,
              out=(y, None))
