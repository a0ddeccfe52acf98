"""The one-pass pack's coding band and its two fix-up paths, through the C ABI.

bitlinear_pack codes each kept weight in its one pass over W against a band around the
threshold estimated from a sample of W, lists the kept weights inside the band, and once the exact
gamma is known either sets the listed codes (tau inside the band, list complete) or packs every
tile again.  Whichever path runs, gamma, codes and meta must equal the oracle's bit for bit.  The
workspace's diagnostic words say which path ran: ordinary masters must take the listed-codes path
(otherwise the pack would read W twice), and the masters built here to defeat the band -- weights
crowded at the threshold, a sample that misses the one large piece, a master smaller than one
sampling chunk -- must take the repack path and still be exact.
"""
import numpy as np
import pytest

import oracle as O
from parity_util import dev, f32_bits, host
from synth import master_weights, rng

pytestmark = pytest.mark.gpu

S = pytest.importorskip("sparsity_amd")

# bitlinear_pack's workspace: fp64 sum slots (1024 x 8), the exact pass's word slots (256 x 128)
# and nine counter lines (9 x 128); then gamma, tau, exact_used, fix_mode, tau_lo, tau_hi,
# band_ok, overflow (4 bytes each)
_BASE = 1024 * 8 + 256 * 128 + 9 * 128
FIX_MODE = _BASE + 12
BAND_OK = _BASE + 24
OVERFLOW = _BASE + 28


def _word(ws, off):
    return int(host(ws)[off:off + 4].view(np.uint32)[0])


def _pack_checked(W, N=2, M=4, layout=O.LAYOUT_SPARSE):
    import torch
    n, K = W.shape
    wsb = S.packed_bytes(n, K, N, M, layout)[3]
    ws = torch.full((wsb,), 0xAB, dtype=torch.uint8, device="cuda")   # stale contents
    codes, meta, gamma = S.pack(dev(W), N, M, layout, ws=ws)
    ref = O.pack(W, N, M, layout)
    assert int(f32_bits(host(gamma)[0])) == int(f32_bits(ref["gamma"])), "gamma"
    assert np.array_equal(host(codes).view(np.uint32), ref["codes"]), "codes"
    if meta is not None:
        assert np.array_equal(host(meta).view(np.uint32), ref["meta"]), "meta"
    return ws


@pytest.mark.parametrize("n,K,N,M,layout", [
    (1024, 1024, 2, 4, O.LAYOUT_SPARSE),
    (640, 2048, 6, 8, O.LAYOUT_SPARSE),
    (512, 3072, 14, 16, O.LAYOUT_SPARSE),
    (1000, 1536, 2, 4, O.LAYOUT_DENSE2),
])
def test_ordinary_masters_take_the_listed_codes_path(n, K, N, M, layout):
    W = master_weights(rng(n + K + M), n, K)
    ws = _pack_checked(W, N, M, layout)
    assert _word(ws, BAND_OK) == 1
    assert _word(ws, OVERFLOW) == 0
    assert _word(ws, FIX_MODE) == 0, "an ordinary master fell back to a second pass over W"


def test_weights_crowded_at_the_threshold_overflow_and_repack():
    # every other 4-group holds four weights of magnitude 1; the others keep two weights of
    # magnitude x (1 +- 1e-3) and two of about 0.01.  mean |w| is about (4 + 2x) / 8, so with
    # x = 2/7 the kept x-weights sit on tau = gamma / 2: far more band entries than a tile holds
    g = rng(91)
    n, K = 512, 1024
    W = np.empty((n, K), np.float32)
    grp = W.reshape(n, K // 4, 4)
    big = (np.arange(K // 4) % 2 == 0)
    sgn = np.where(g.random((n, K // 4, 4)) < 0.5, -1.0, 1.0)
    x = (2.0 / 7.0) * (1.0 + 1e-3 * g.standard_normal((n, K // 4, 2)))
    small = 0.01 * g.random((n, K // 4, 2))
    vals = np.concatenate([x, small], axis=2)
    perm = np.argsort(g.random((n, K // 4, 4)), axis=2)
    vals = np.take_along_axis(vals, perm, axis=2)
    grp[:] = np.where(big[None, :, None], 1.0, vals) * sgn
    ws = _pack_checked(W)
    assert _word(ws, OVERFLOW) == 1
    assert _word(ws, FIX_MODE) == 1


def test_sample_that_misses_the_mass_repacks():
    # tiny weights everywhere but one 256-byte piece of huge ones: the sample either misses it
    # (estimate far below gamma) or holds it (estimate far above, standard error huge)
    g = rng(92)
    n, K = 1024, 1024
    W = (1e-3 * g.standard_normal((n, K))).astype(np.float32)
    W[517, 320:384] = 1.0e4 * np.where(g.random(64) < 0.5, -1.0, 1.0)
    ws = _pack_checked(W)
    assert _word(ws, FIX_MODE) == 1


@pytest.mark.parametrize("n,K,layout", [(1, 32, O.LAYOUT_DENSE2), (1, 512, O.LAYOUT_SPARSE),
                                        (7, 128, O.LAYOUT_SPARSE)])
def test_master_without_a_whole_sampling_chunk_repacks(n, K, layout):
    # fewer than 1024 weights: not one 4 KB sampling chunk, so no band (a small master is
    # otherwise sampled whole)
    W = master_weights(rng(93 + K), n, K)
    ws = _pack_checked(W, 2, 4, layout)
    assert _word(ws, BAND_OK) == 0
    assert _word(ws, FIX_MODE) == 1


@pytest.mark.parametrize("n,K", [(3, 384), (8, 512), (33, 640)])
def test_small_masters_sampled_whole(n, K):
    # the band follows the sample's standard error: usable from a few thousand weights on; below
    # that (3 x 384) it may be too wide and the fix-up repacks -- exact either way
    W = master_weights(rng(93 + n), n, K)
    ws = _pack_checked(W)
    if n * K >= 4096:
        assert _word(ws, BAND_OK) == 1


def test_group_mixes_both_paths():
    """One grouped pack holding an ordinary master (listed codes) and a crowded one (repack):
    each master's slice of the workspace records its own path, and every output equals the
    single call's."""
    import torch
    g = rng(94)
    A = master_weights(g, 768, 1024)
    n, K = 256, 512
    # groups of four ones alternate with groups of four weights near 1/3: mean |w| about 2/3, so
    # tau sits on the kept third-weights
    B = np.where(np.arange(K) % 8 < 4, 1.0, 1.0 / 3.0 * (1.0 + 1e-3 * g.standard_normal((n, K))))
    B = (B * np.where(g.random((n, K)) < 0.5, -1.0, 1.0)).astype(np.float32)
    Ws = [dev(A), dev(B)]
    grp = S.PackGroup([dict(W=W) for W in Ws])
    grp()
    torch.cuda.synchronize()
    for i, W in enumerate(Ws):
        c, m, gm = grp.outputs[i]
        rc, rm, rg = S.pack(W)
        assert torch.equal(gm, rg) and torch.equal(c, rc) and torch.equal(m, rm), f"master {i}"
    slice_bytes = (S.packed_bytes(768, 1024)[3] + 255) // 256 * 256
    ws = grp.ws
    assert _word(ws, FIX_MODE) == 0
    assert _word(ws, slice_bytes + FIX_MODE) == 1
    ref = O.pack(np.asarray(B), 2, 4, O.LAYOUT_SPARSE)
    assert np.array_equal(host(grp.outputs[1][0]).view(np.uint32), ref["codes"])


def test_noalloc_beyond_its_band_regions_matches_pack():
    """bitlinear_pack_noalloc's static workspace holds band regions for 8192 tiles (67 M weights);
    a larger master is packed there without the band (two passes over W) and must equal
    bitlinear_pack, which has a region for every tile and takes the one-pass path."""
    import ctypes
    import torch
    n, K = 8224, 8192                     # 257 panels x 32 tiles = 8224 tiles
    g = torch.Generator(device="cuda")
    g.manual_seed(95)
    Wd = (torch.randn((n, K), generator=g, device="cuda") * 0.02).contiguous()
    cb, mb, _, wsb = S.packed_bytes(n, K)
    outs = [(torch.full((cb,), 0xAB, dtype=torch.uint8, device="cuda"),
             torch.full((mb,), 0xAB, dtype=torch.uint8, device="cuda"),
             torch.full((4,), float("nan"), device="cuda")) for _ in range(2)]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    c, m, gm = outs[0]
    assert S.lib().bitlinear_pack_noalloc(Wd.data_ptr(), n, K, 2, 4, O.LAYOUT_SPARSE,
                                          c.data_ptr(), m.data_ptr(), gm.data_ptr(), stream) == 0
    ws = torch.full((wsb,), 0x5A, dtype=torch.uint8, device="cuda")
    c2, m2, g2 = S.pack(Wd, out=outs[1], ws=ws)
    torch.cuda.synchronize()
    assert _word(ws, FIX_MODE) == 0 and _word(ws, BAND_OK) == 1
    assert torch.equal(gm[:1], g2[:1]) and torch.equal(c, c2) and torch.equal(m, m2)
