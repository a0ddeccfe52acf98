"""Pins of the CPU oracle against the pages' definitions, closed forms and brute force.

None of these tests needs a GPU.  Each test checks the oracle against something other
than itself: hand-derived golden values (tests/golden), exact rational arithmetic,
exhaustive search, closed-form thresholds or statistics, or a library routine.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from golden_io import hexu32, read_kv, read_lines


def f32_from_bits(vals):
    return np.array(vals, dtype=np.uint32).view(np.float32)


def bits(x):
    return int(np.float32(x).view(np.uint32))


# ------------------------------------------------------------------------------------------
# gamma
# ------------------------------------------------------------------------------------------

def test_gamma_closed_forms():
    kv = read_kv("gamma_closed_forms.txt")
    for c in range(1, 7):
        W = f32_from_bits(hexu32(kv[f"case{c}_W"])).reshape(1, -1)
        want = hexu32(kv[f"case{c}_gamma"])[0]
        assert bits(O.absmean_gamma(W)) == want, c


def _fraction_to_f32_bruteforce(r: Fraction) -> np.float32:
    """Nearest fp32 to r (ties to even) by checking the neighbours of a candidate exactly."""
    c = np.float32(float(r))
    cands = {c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(0))}
    best = None
    for v in sorted(cands, key=float):
        d = abs(Fraction(float(v)) - r)
        even = bits(v) % 2 == 0
        key = (d, not even)
        if best is None or key < best[0]:
            best = (key, v)
    return np.float32(best[1])


@pytest.mark.parametrize("seed", range(6))
def test_gamma_rational_bruteforce(seed):
    g = np.random.default_rng(seed)
    kind = seed % 3
    if kind == 0:
        W = g.normal(0, 0.02, size=(7, 13)).astype(np.float32)
    elif kind == 1:   # very wide exponent range, including subnormals
        W = (g.standard_normal((5, 11)) * np.exp2(g.integers(-149, 100, size=(5, 11)))).astype(np.float32)
    else:             # tiny values only: the mean may be subnormal
        W = (g.integers(-9, 10, size=(3, 8)) * np.float32(2.0 ** -149)).astype(np.float32)
    exact = sum(Fraction(float(abs(w))) for w in W.ravel()) / W.size
    assert bits(O.absmean_gamma(W)) == bits(_fraction_to_f32_bruteforce(exact))


def test_round_ratio_matches_numpy_cast():
    g = np.random.default_rng(3)
    xs = list(np.abs(g.standard_normal(200)) * np.exp2(g.integers(-160, 120, 200)))
    # exact fp32 midpoints and values one fp64 ulp either side of them
    for k in range(1, 40):
        m = (2 * k + 1) * 2.0 ** -25
        xs += [1.0 + m, np.nextafter(1.0 + m, 2.0), np.nextafter(1.0 + m, 0.0)]
    xs += [2.0 ** -150, 3 * 2.0 ** -150, 2.0 ** -149 * 1.5, 5e-324, 1.0]
    for x in xs:
        fr = Fraction(float(x))
        got = O.round_ratio_to_f32(fr.numerator, fr.denominator)
        want = np.float32(np.float64(x))   # numpy's fp64 -> fp32 cast rounds to nearest even
        assert bits(got) == bits(want), x


def test_gamma_invariances():
    g = np.random.default_rng(11)
    W = g.normal(0, 0.02, size=(64, 96)).astype(np.float32)
    gam = O.absmean_gamma(W)
    perm = g.permutation(W.size)
    assert bits(O.absmean_gamma(W.ravel()[perm].reshape(96, 64))) == bits(gam)
    assert bits(O.absmean_gamma(-W)) == bits(gam)
    for k in (-3, 5, 17):
        assert bits(O.absmean_gamma(W * np.float32(2.0 ** k))) == bits(np.float32(gam * 2.0 ** k))
    c = np.float32(0.0173)
    Wc = np.where(g.random(W.shape) < 0.5, c, -c).astype(np.float32)
    assert bits(O.absmean_gamma(Wc)) == bits(c)


def test_gamma_gaussian_statistic():
    g = np.random.default_rng(5)
    sigma = 0.02
    W = g.normal(0, sigma, size=(1024, 1024)).astype(np.float32)
    want = sigma * math.sqrt(2 / math.pi)      # E|w| for N(0, sigma^2)
    assert abs(float(O.absmean_gamma(W)) / want - 1) < 3e-3


# ------------------------------------------------------------------------------------------
# mask
# ------------------------------------------------------------------------------------------

def test_mask_golden():
    for line in read_lines("mask_ties.txt"):
        nm, w, kept = [s.strip() for s in line.split("|")]
        N, M = map(int, nm.split())
        W = np.array([float(v) for v in w.split()], dtype=np.float32).reshape(1, M)
        got = np.nonzero(O.nm_mask(W, N, M)[0])[0].tolist()
        assert got == [int(v) for v in kept.split()], line


def _topn_bruteforce(a, N):
    """The unique N-subset whose kept entries all precede every dropped entry in the order
    (|w| descending, index ascending)."""
    M = len(a)
    found = []
    for S in itertools.combinations(range(M), N):
        ok = all((abs(a[i]) > abs(a[j])) or (abs(a[i]) == abs(a[j]) and i < j)
                 for i in S for j in range(M) if j not in S)
        if ok:
            found.append(S)
    assert len(found) == 1
    return list(found[0])


@pytest.mark.parametrize("N,M", [(2, 4), (6, 8), (1, 4), (4, 4)])
def test_mask_bruteforce(N, M):
    g = np.random.default_rng(N * 10 + M)
    pool = np.array([0.0, -0.0, 0.25, -0.25, 0.5, -0.5, 1.0], dtype=np.float32)
    W = g.choice(pool, size=(40, M * 6)).astype(np.float32)
    W[:20] = g.normal(0, 0.02, size=(20, M * 6)).astype(np.float32)
    keep = O.nm_mask(W, N, M)
    for r in range(W.shape[0]):
        for gi in range(W.shape[1] // M):
            grp = [float(v) for v in W[r, gi * M:(gi + 1) * M]]
            want = _topn_bruteforce(grp, N)
            assert np.nonzero(keep[r, gi * M:(gi + 1) * M])[0].tolist() == want
    assert np.all(keep.reshape(W.shape[0], -1, M).sum(-1) == N)


# ------------------------------------------------------------------------------------------
# ternarize
# ------------------------------------------------------------------------------------------

def test_ternarize_golden():
    kv = read_kv("ternarize_worked.txt")
    W = np.array([float(v) for v in kv["W"]], dtype=np.float32).reshape(1, -1)
    gam = O.absmean_gamma(W)
    assert float(gam) == float(kv["gamma"][0])
    assert O.ternarize(W, gam).ravel().tolist() == [int(v) for v in kv["t"]]
    Wn = np.array([float(v) for v in kv["Wneg"]], dtype=np.float32).reshape(1, -1)
    assert O.ternarize(Wn, O.absmean_gamma(Wn)).ravel().tolist() == [int(v) for v in kv["tneg"]]


def test_ternarize_threshold_closed_form():
    """fl32(|w|/gamma) > 0.5  <=>  |w| * 2^25 > gamma * (2^24 + 1)  (RNE; spacing above 0.5 is 2^-24).

    Both sides of the right-hand comparison are exact in fp64 (a power-of-two scaling, and a
    24-bit by 25-bit product)."""
    g = np.random.default_rng(7)
    gammas = np.abs(g.normal(0, 0.02, 64)).astype(np.float32)
    for gam in gammas:
        base = float(gam) * 0.5
        near = [np.float32(base * (1 + k * 2.0 ** -26)) for k in range(-6, 7)]
        near += [np.nextafter(np.float32(base), np.float32(1)), np.nextafter(np.float32(base), np.float32(0))]
        far = list((g.normal(0, 0.05, 200)).astype(np.float32))
        w = np.array(near + [-v for v in near] + far, dtype=np.float32).reshape(1, -1)
        t = O.ternarize(w, gam).ravel()
        a = np.abs(w.ravel()).astype(np.float64)
        want = np.where(a * 2.0 ** 25 > np.float64(gam) * (2.0 ** 24 + 1), np.sign(w.ravel()), 0)
        assert np.array_equal(t, want.astype(np.int8))


def test_ternarize_zero_gamma_and_symmetry():
    W = np.zeros((4, 8), np.float32)
    assert O.absmean_gamma(W) == 0 and not O.ternarize(W, O.absmean_gamma(W)).any()
    g = np.random.default_rng(2)
    W = g.normal(0, 0.02, (32, 64)).astype(np.float32)
    gam = O.absmean_gamma(W)
    assert np.array_equal(O.ternarize(-W, gam), -O.ternarize(W, gam))


def test_ternary_gaussian_zero_fraction():
    """P(|w| <= gamma/2) for Gaussian w with gamma = E|w| is 2*Phi(sqrt(2/pi)/2) - 1 ~= 0.3101."""
    g = np.random.default_rng(9)
    W = g.normal(0, 0.02, (1024, 1024)).astype(np.float32)
    t = O.ternarize(W, O.absmean_gamma(W))
    want = math.erf(math.sqrt(2 / math.pi) / 2 / math.sqrt(2))
    assert abs((t == 0).mean() - want) < 2e-3


# ------------------------------------------------------------------------------------------
# 6:8 windows
# ------------------------------------------------------------------------------------------

def test_windows_golden():
    kv = read_kv("windows_68.txt")
    table = O.window_table_68()
    for sfx in ("", "_b", "_c"):
        kept = [int(v) for v in kv["kept" + sfx]]
        wins = table[sum(1 << p for p in kept)]
        for w in range(3):
            assert wins[w] == [int(v) for v in kv[f"w{w}{sfx}"]]


def test_windows_1416_golden():
    kv = read_kv("windows_1416.txt")
    table = O.window_table(16)
    for sfx in ("", "_b", "_c"):
        kept = [int(v) for v in kv["kept" + sfx]]
        wins = table[sum(1 << p for p in kept)]
        for w in range(7):
            assert wins[w] == [int(v) for v in kv[f"w{w}{sfx}"]]


@pytest.mark.parametrize("prefix,M", [("m6", 6), ("m6b", 6), ("m10", 10), ("m10b", 10),
                                      ("m12", 12), ("m14", 14)])
def test_windows_general_golden(prefix, M):
    """Hand-derived decompositions of 4:6, 8:10, 10:12 and 12:14 groups (windows_general.txt)."""
    kv = read_kv("windows_general.txt")
    kept = [int(v) for v in kv[prefix + "_kept"]]
    wins = O.window_table(M)[sum(1 << p for p in kept)]
    assert len(wins) == M // 2 - 1
    for w in range(M // 2 - 1):
        assert wins[w] == [int(v) for v in kv[f"{prefix}_w{w}"]]


@pytest.mark.parametrize("M,count", [(6, 15), (8, 28), (10, 45), (12, 66), (14, 91), (16, 120)])
def test_windows_cover_every_mask(M, count):
    """Every (M-2):M mask splits into M/2 - 1 windows of two kept positions each, each position
    inside its window's span (the decomposition is lossless for every mask)."""
    table = O.window_table(M)
    assert len(table) == count
    for mask, wins in table.items():
        assert len(wins) == M // 2 - 1
        flat = sorted(p for w in wins for p in w)
        assert flat == [p for p in range(M) if mask >> p & 1]
        for w, ps in enumerate(wins):
            assert len(ps) == 2 and all(2 * w <= p <= 2 * w + 3 for p in ps)


# ------------------------------------------------------------------------------------------
# pack layout
# ------------------------------------------------------------------------------------------

# K per group size M: whole groups and whole 64-position sparse MFMA steps on the lifted axis
GENERAL_K = {4: 256, 6: 240, 8: 256, 10: 240, 12: 384, 14: 224, 16: 256}


def test_pack_golden_unit():
    kv = read_kv("pack_2of4_unit.txt")
    half = np.array([float(v) for v in kv["W"]], dtype=np.float32)
    W = np.concatenate([half, -half]).reshape(1, 64)
    p = O.pack(W, 2, 4, O.LAYOUT_SPARSE)
    assert float(p["gamma"]) == 1.0
    vals, idx = O.weight_slots(p["W_eff"], p["keep"], 2, 4, O.LAYOUT_SPARSE)
    assert vals[0, :16].tolist() == [int(v) for v in kv["slot_codes_unit0"]]
    assert idx[0, :16].tolist() == [int(v) for v in kv["slot_idx_unit0"]]
    codes, meta = p["codes"], p["meta"]
    assert codes.size == 64 and meta.size == 64
    assert codes[0] == hexu32(kv["code_dword_0"])[0]
    assert codes[32] == hexu32(kv["code_dword_32"])[0]
    assert meta[0] == hexu32(kv["meta_dword_0"])[0]
    assert meta[32] == hexu32(kv["meta_dword_32"])[0]
    pad = hexu32(kv["pad_meta"])[0]
    others = [i for i in range(64) if i not in (0, 32)]
    assert not codes[others].any()
    assert np.all(meta[others] == pad)


def test_pack_golden_tiling():
    # two panels, several fragments, SPARSE and DENSE2 (tests/golden/pack_tiling.txt)
    kv = read_kv("pack_tiling.txt")
    W = np.zeros((33, 128), dtype=np.float32)
    for key, v in kv.items():
        if key.startswith("w "):
            r, k0 = (int(t) for t in key.split()[1:])
            W[r, k0:k0 + 4] = [float(t) for t in v]
    for layout, pre in ((O.LAYOUT_SPARSE, "sparse"), (O.LAYOUT_DENSE2, "dense")):
        p = O.pack(W, 2, 4, layout)
        assert float(p["gamma"]) == float(np.float32(9 / (33 * 128)))
        codes = p["codes"]
        assert codes.size == int(kv[f"{pre}_dwords"][0])
        exp_c = {int(k.split()[1]): hexu32(v)[0] for k, v in kv.items()
                 if k.startswith(f"{pre}_code ")}
        for d, v in exp_c.items():
            assert int(codes[d]) == v, (pre, d, hex(int(codes[d])), hex(v))
        others = np.array([d for d in range(codes.size) if d not in exp_c])
        assert not codes[others].any()
        if layout == O.LAYOUT_SPARSE:
            meta = p["meta"]
            exp_m = {int(k.split()[1]): hexu32(v)[0] for k, v in kv.items()
                     if k.startswith("sparse_meta ")}
            for d, v in exp_m.items():
                assert int(meta[d]) == v, (d, hex(int(meta[d])), hex(v))
            others = np.array([d for d in range(meta.size) if d not in exp_m])
            assert np.all(meta[others] == O.PAD_META)


@pytest.mark.parametrize("N,M,layout", [(2, 4, O.LAYOUT_SPARSE), (6, 8, O.LAYOUT_SPARSE),
                                        (14, 16, O.LAYOUT_SPARSE), (2, 4, O.LAYOUT_DENSE2),
                                        (6, 8, O.LAYOUT_DENSE2), (14, 16, O.LAYOUT_DENSE2),
                                        (4, 6, O.LAYOUT_SPARSE), (8, 10, O.LAYOUT_SPARSE),
                                        (10, 12, O.LAYOUT_SPARSE), (12, 14, O.LAYOUT_SPARSE)])
def test_pack_roundtrip(N, M, layout):
    g = np.random.default_rng(N + M + layout)
    n, K = 45, GENERAL_K[M]
    W = g.normal(0, 0.02, (n, K)).astype(np.float32)
    p = O.pack(W, N, M, layout)
    vals, idx = O.unpack_slots(p["codes"], p["meta"], n, K, N, M, layout)
    dense = O.slots_to_dense(vals, idx, K, N, M, layout)
    assert np.array_equal(dense, p["W_eff"])
    nnz = (p["W_eff"] != 0).reshape(n, K // M, M).sum(-1)
    assert nnz.max() <= N


# ------------------------------------------------------------------------------------------
# 6-bit 2:4 decode encoding (SPARSE6)
# ------------------------------------------------------------------------------------------

def test_state6_golden_table():
    table = read_kv("state6.txt")
    assert sorted(int(k) for k in table) == list(range(54))
    for k, v in table.items():
        s = int(k)
        i, j, *w = (int(t) for t in v)
        assert O.state6_decode(s)[:2] == (i, j)
        assert O.state6_dense(s) == tuple(w)
        assert O.state6(i, j, w[i], w[j]) == s
    for s in range(54, 64):
        with pytest.raises(ValueError):
            O.state6_decode(s)


def test_state6_bijection():
    # every 2:4 mask (a pair of kept positions) with every pair of ternary values: 54 distinct
    # states below 54, each decoding back to its mask and values
    seen = set()
    for i in range(4):
        for j in range(i + 1, 4):
            for a in (-1, 0, 1):
                for b in (-1, 0, 1):
                    s = O.state6(i, j, a, b)
                    assert 0 <= s < 54 and s not in seen
                    seen.add(s)
                    assert O.state6_decode(s) == (i, j, a, b)
                    w = [0] * 4
                    w[i], w[j] = a, b
                    assert O.state6_dense(s) == tuple(w)
    assert len(seen) == O.STATE6_COUNT == 54 <= 64


def _golden_pack6():
    kv = read_kv("pack6_unit.txt")
    n, K = int(kv["n"][0]), int(kv["K"][0])
    W = np.zeros((n, K), dtype=np.int8)
    keep = np.zeros((n, K), dtype=bool)
    keep[:, 0::4] = keep[:, 1::4] = True          # all-zero groups keep (0, 1)
    for key, v in kv.items():
        if key.startswith("g "):
            r, g = (int(t) for t in key.split()[1:])
            w0, w1, w2, w3, i, j = (int(t) for t in v)
            W[r, 4 * g:4 * g + 4] = (w0, w1, w2, w3)
            keep[r, 4 * g:4 * g + 4] = False
            keep[r, 4 * g + i] = keep[r, 4 * g + j] = True
    exp = {int(key.split()[1]): hexu32(v)[0] for key, v in kv.items() if key.startswith("d ")}
    return n, K, W, keep, int(kv["dwords"][0]), exp


def test_pack6_golden_unit():
    n, K, W, keep, nd, exp = _golden_pack6()
    assert O.packed6_dwords(n, K) == (nd, 64, 2)
    vals, idx = O.weight_slots(W, keep, 2, 4, O.LAYOUT_SPARSE)
    out = O.pack6(vals, idx, n, K)
    assert out.size == nd
    for d, v in exp.items():
        assert int(out[d]) == v, (d, hex(int(out[d])), hex(v))
    others = np.array([d for d in range(nd) if d not in exp])
    assert not out[others].any()
    Wd, kd = O.unpack6(out, n, K)
    assert np.array_equal(Wd, W) and np.array_equal(kd, keep)


@pytest.mark.parametrize("n,K", [(1, 64), (45, 384), (70, 320), (64, 256)])
def test_pack6_roundtrip_from_pack(n, K):
    # the 2:4 packed buffers of a master, through their slots, re-encode to a stream whose
    # decoded weights and mask are the master's effective weights and mask
    g = np.random.default_rng(n + K)
    Wm = g.normal(0, 0.02, (n, K)).astype(np.float32)
    Wm[:, :8] = 0.0                                # all-zero groups
    p = O.pack(Wm, 2, 4, O.LAYOUT_SPARSE)
    vals, idx = O.unpack_slots(p["codes"], p["meta"], n, K, 2, 4, O.LAYOUT_SPARSE)
    s = O.pack6(vals, idx, n, K)
    assert s.size == O.packed6_dwords(n, K)[0]
    Wd, kd = O.unpack6(s, n, K)
    assert np.array_equal(Wd, p["W_eff"]) and np.array_equal(kd, p["keep"])
    # 0.1875 bytes per weight once rows and step pairs are whole
    if n % 32 == 0 and K % 128 == 0:
        assert s.size * 4 == n * K * 6 // 32


# ------------------------------------------------------------------------------------------
# activation quantization
# ------------------------------------------------------------------------------------------

def test_act_quant_golden():
    kv = read_kv("act_quant_worked.txt")
    x = np.array([[float(v) for v in kv[f"x{i}"]] for i in range(3)], dtype=np.float32)
    q, scale = O.act_quant(x)
    for i in range(3):
        assert q[i].tolist() == [int(v) for v in kv[f"q{i}"]]
    assert scale[0] == np.float32(1.0)
    assert scale[1] == np.float32(np.float32(0.5) / np.float32(127))
    assert scale[2] == 0


def test_act_quant_invariants():
    g = np.random.default_rng(4)
    x = g.standard_normal((33, 200)).astype(np.float32)
    x[5] = 0
    q, scale = O.act_quant(x)
    nz = np.abs(x).max(1) > 0
    assert np.all(np.abs(q[nz]).max(1) == 127) and not q[~nz].any()
    for k in (-7, 3, 20):
        q2, s2 = O.act_quant(x * np.float32(2.0 ** k))
        assert np.array_equal(q2, q)
        assert np.array_equal(s2, (scale * np.float32(2.0 ** k)).astype(np.float32))


def test_act_quant_close_to_real_rounding():
    """Against rint(x * 127 / absmax) in fp64: any difference sits at a near-half-integer."""
    g = np.random.default_rng(8)
    x = (0.5 * g.standard_t(4, (64, 512))).astype(np.float32)
    q, _ = O.act_quant(x)
    am = np.abs(x).max(1, keepdims=True).astype(np.float64)
    real = x.astype(np.float64) * 127 / am
    ref = np.rint(real)
    diff = q != ref
    assert np.all(np.abs(q - ref)[diff] == 1)
    assert np.all(np.abs(np.abs(real[diff] - np.floor(real[diff])) - 0.5) < 1e-4)


def test_lift_1416():
    kv = read_kv("windows_1416.txt")
    q = np.arange(2 * 32, dtype=np.int64).reshape(2, 32).astype(np.int8)
    L = O.lift(q, 16)
    assert L.shape == (2, 56)
    want = [int(v) for v in kv["lift16"]]
    assert L[0, :28].tolist() == want
    assert L[0, 28:].tolist() == [16 + v for v in want]
    assert O.k_eff(256, 14, 16, O.LAYOUT_SPARSE) == 448


def test_lift_68():
    q = np.arange(2 * 16, dtype=np.int64).reshape(2, 16).astype(np.int8)
    L = O.lift_68(q)
    assert L.shape == (2, 24)
    assert L[0].tolist() == [0, 1, 2, 3, 2, 3, 4, 5, 4, 5, 6, 7, 8, 9, 10, 11, 10, 11, 12, 13, 12, 13, 14, 15]


def test_lift_general():
    """Written out by hand from the lifting rule (window w of a group = its positions 2w..2w+3):
    4:6 makes 8 of every 6 values, 8:10 16 of every 10, 10:12 20 of 12, 12:14 24 of 14."""
    q = np.arange(12, dtype=np.int64).reshape(1, 12).astype(np.int8)
    assert O.lift(q, 6)[0].tolist() == [0, 1, 2, 3, 2, 3, 4, 5, 6, 7, 8, 9, 8, 9, 10, 11]
    q = np.arange(10, dtype=np.int64).reshape(1, 10).astype(np.int8)
    assert O.lift(q, 10)[0].tolist() == [0, 1, 2, 3, 2, 3, 4, 5, 4, 5, 6, 7, 6, 7, 8, 9]
    q = np.arange(12, dtype=np.int64).reshape(1, 12).astype(np.int8)
    assert O.lift(q, 12)[0].tolist() == [0, 1, 2, 3, 2, 3, 4, 5, 4, 5, 6, 7, 6, 7, 8, 9,
                                         8, 9, 10, 11]
    q = np.arange(14, dtype=np.int64).reshape(1, 14).astype(np.int8)
    assert O.lift(q, 14)[0].tolist() == [0, 1, 2, 3, 2, 3, 4, 5, 4, 5, 6, 7, 6, 7, 8, 9,
                                         8, 9, 10, 11, 10, 11, 12, 13]
    assert [O.k_eff(k, m - 2, m, O.LAYOUT_SPARSE) for k, m in ((240, 6), (240, 10), (384, 12),
                                                              (224, 14))] == [320, 384, 640, 384]


# ------------------------------------------------------------------------------------------
# accumulation and rescale
# ------------------------------------------------------------------------------------------

def test_acc_bruteforce_tiny():
    g = np.random.default_rng(12)
    W = g.integers(-1, 2, (3, 8)).astype(np.int8)
    q = g.integers(-127, 128, (2, 8)).astype(np.int8)
    acc = O.acc_dense(W, q)
    for t in range(2):
        for o in range(3):
            s = 0
            for k in range(8):
                s += int(W[o][k]) * int(q[t][k])
            assert acc[t][o] == s


@pytest.mark.parametrize("N,M,layout", [(2, 4, O.LAYOUT_SPARSE), (6, 8, O.LAYOUT_SPARSE),
                                        (14, 16, O.LAYOUT_SPARSE), (2, 4, O.LAYOUT_DENSE2),
                                        (14, 16, O.LAYOUT_DENSE2), (4, 6, O.LAYOUT_SPARSE),
                                        (8, 10, O.LAYOUT_SPARSE), (10, 12, O.LAYOUT_SPARSE),
                                        (12, 14, O.LAYOUT_SPARSE)])
def test_acc_forms_agree(N, M, layout):
    """Form i (dense int64 matmul of W_eff) equals form ii (add/sub over packed slots); for the
    (M-2):M windows the lifted 2:4 windows against lifted activations equal the dense product
    (lossless)."""
    g = np.random.default_rng(20 + N)
    n, K, T = 40, GENERAL_K[M], 9
    W = g.normal(0, 0.02, (n, K)).astype(np.float32)
    x = g.standard_normal((T, K)).astype(np.float32)
    p = O.pack(W, N, M, layout)
    lift = M if (layout == O.LAYOUT_SPARSE and M in O.WINDOW_M) else 0
    xq, _ = O.act_quant(x, lift)
    q, _ = O.act_quant(x, 0)
    vals, idx = O.unpack_slots(p["codes"], p["meta"], n, K, N, M, layout)
    assert np.array_equal(O.acc_addsub(vals, idx, xq, layout), O.acc_dense(p["W_eff"], q))


def test_tokens_independent():
    g = np.random.default_rng(13)
    W = g.normal(0, 0.02, (64, 128)).astype(np.float32)
    x = g.standard_normal((16, 128)).astype(np.float32)
    big = O.forward(W, x, 2, 4)
    small = O.forward(W, x[:1], 2, 4)
    assert np.array_equal(big["acc"][:1], small["acc"]) and np.array_equal(big["y"][:1], small["y"])


def test_rescale_exact_cases():
    acc = np.array([[0, 3, -5]], dtype=np.int64)
    y = O.rescale(acc, np.float32(0.5), np.array([0.25], np.float32))
    assert y.tolist() == [[0.0, 0.375, -0.625]]
    y0 = O.rescale(acc, np.float32(0.5), np.array([0.0], np.float32))
    assert not y0.any()


def test_tiny_workload_invariants():
    from synth import workload_inputs
    d = workload_inputs("tiny", 0)
    W, x = d["W:w"], d["X:256"]
    out = O.forward(W, x, 2, 4)
    assert out["y"].shape == (16, 256) and np.all(np.isfinite(out["y"]))
    nnz = (out["W_eff"] != 0).reshape(256, 64, 4).sum(-1)
    assert nnz.max() <= 2
    assert np.all(np.abs(out["acc"]) < 2 ** 31)
