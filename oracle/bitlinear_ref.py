"""Plain numpy oracle of the sparse ternary BitLinear forward (test infrastructure only).

Sources (pages; cited by title and section):
  [SB]  "Sparse-BitNet: 1.58-bit LLMs are Naturally Friendly to Semi-Structured
        Sparsity" -- abstract (newx.sg page) and the technical summary
        (gist.science page, section 2 "Methodologie", Kerncomponenten:
        Sparse-BitLinear, Maskering, Forward Pass; Training Strategie:
        Dynamisch Masker).
  [B158] "BitNet b1.58: Ternary Weights for 1.58-bit LLMs" (fanout blog page) --
        section "The mechanism" (absmean weight quantization, Eqs. 1-3 of the
        paper; activations scaled per token to [-Qb, Qb]) and "Algorithm /
        figure walkthrough" steps 3-5.
  [SS]  SlideSparse abstract on the page "Is 2:4 Sparsity Still Worth It?
        Semi-Structured Sparsity versus Quantization in LLM Inference" --
        Sliding Window Decomposition of (2N-2):2N blocks into N-1 overlapping
        2:4 windows, and Activation Lifting.

Readings taken where the pages are silent or garbled (the page [B158] lost the
formulas of Eqs. 1-3 in extraction):
  * gamma = mean |W| over the whole dense master matrix (per tensor), computed
    exactly and rounded once to fp32 (round half to even).  No epsilon.
    gamma == 0 gives an all-zero ternary matrix.
  * W~ = clip(rint(fl32(W / gamma)), -1, 1) with rint = round half to even.
  * N:M mask: per row, per contiguous group of M along K starting at k = 0,
    keep the N largest |w| of the continuous master; ties go to the lower
    index; exactly N positions are kept even when their ternary code is 0.
    The mask multiplies the ternary matrix (quantize first, then mask; gamma
    comes from the dense master).
  * Activations: absmax_t = max_k |x_tk|; s_t = fl32(127 / absmax_t);
    q = clamp(rint(fl32(x * s_t)), -127, 127); scale_t = fl32(absmax_t / 127);
    absmax_t == 0 gives q = 0 and scale_t = 0.
  * (2N-2):2N windows (6:8 and 14:16): with M = 2N, window w in 0..N-2 covers
    positions 2w..2w+3 of an M-group; kept positions are assigned in ascending
    order, each to the lowest window that covers it and holds fewer than 2
    (for 6:8: w0 takes kept positions in 0..3, at most 2; w1 takes the
    remaining ones in 2..5, at most 2; w2 takes the rest).  Lifted activations:
    x'[(2M-4)g + 4w + j] = x[Mg + 2w + j] (6:8: 12 per 8, 14:16: 28 per 16).
  * Output: y = acc * gamma * scale_t evaluated in fp64, rounded to fp32.
  * Backward ([SB] Training Strategie, Dual STE): the rounding, the clip and the Top-N
    selection are passed straight through, so with W_q = gamma * W_eff the layer is
    y = X^ W_q^T and its gradients are dX = dY W_q = gamma * (dY W_eff) and
    dW = dY^T X^.  dW reaches every master weight, masked ones included: it does not
    depend on the mask.  dY is bfloat16 (the Sparse-BitNet summary trains in BF16);
    X^ is the dequantized activation held in bfloat16:
    X^ = bf16(fp32(q * scale_t)), both roundings to nearest even.  The gradient
    w.r.t. gamma and the token scales is not propagated (straight through).

Packed layout (layout id 2), the format of the library's packed buffers:
  A *slot* is one kept weight.  SPARSE layout (2:4, or 6:8 / 14:16 lifted into
  2:4 windows): each 4-wide window j of a row's (lifted) K axis holds slots 2j and
  2j+1 -- the kept positions in ascending order -- with a 2-bit ternary code
  (00 = 0, 01 = +1, 10 = -1; 11 is never written) and a 2-bit position index 0..3
  within the window.
  DENSE2 layout: every position is a slot with a 2-bit code and no index.
  A *unit* is 16 consecutive slots of one row (row r, unit c) and is stored as
  one little-endian code dword -- slot i at bits 8*(i%4) + 2*(i//4) -- and,
  for SPARSE, one meta dword -- slot i's index at bits 2*i.  Units are tiled
  for 64-lane fragments: rows are padded to a multiple of 32 (padded rows:
  codes 0, every window's indices (0, 1)), and unit (r, c) lives at dword
  ((r // 32) * (U // 2) + c // 2) * 64 + (c % 2) * 32 + r % 32, where U is the
  number of units per row (K_eff / 32 for SPARSE, K / 16 for DENSE2).
  SPARSE6 (a 2:4 matrix re-encoded for decode, 6 bits per 4-wide group): the pages
  fix no sub-2-bit format, so this one is the plainest: the 54 states of a group
  (6 kept-position pairs x 3 x 3 ternary values) numbered 9 * pair + 3 * digit(lower)
  + digit(upper), and laid out for 16-row MFMA tiles (pack6 states the tiling).

Pinned functions (tests/test_oracle_*.py) and what pins them:
  absmean_gamma      rational brute force, closed forms, permutation and 2^k
                     scaling invariance, ties at fp32 midpoints, subnormals
  round_ratio_to_f32 numpy's correctly rounded fp64 -> fp32 cast
  nm_mask            exhaustive subset search on tie-heavy groups
  ternarize          worked example with an exact half, the closed-form
                     threshold |w| * 2^25 > gamma * (2^24 + 1), sign symmetry
  window_table       worked examples (6:8, 14:16); every valid 6:8 and 14:16
                     mask is decomposed and reconstructs
  pack / unpack      hand-encoded dwords (tests/golden), round trip
  act_quant          worked example with exact halves, invariants
  acc_dense          brute-force Python loops on tiny inputs; agrees with the
                     add/sub form acc_addsub; 6:8 and 14:16 lifted == dense
  rescale            zero case and exact small products
  bf16_round         hand-derived ties and neighbours, exact rational nearest search,
                     torch's CPU float32 -> bfloat16 cast
  dequant_act        hand-derived values (tests/golden/bwd_tiny.txt), exact products
  state6 / pack6     the 54 states written out by hand (tests/golden/state6.txt),
                     bijection over every 2:4 mask and ternary pair, hand-encoded
                     stream dwords over two panels and two step pairs
                     (tests/golden/pack6_unit.txt), round trip through unpack6
  backward           hand-derived tiny case (tests/golden/bwd_tiny.txt), brute-force Python
                     loops, the adjoint identities <dX, X^> = <dY, Y> = <dW, W_q> against
                     the pinned forward, mask independence of dW
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import Dict, List, Tuple

import numpy as np

LAYOUT_SPARSE = 0
LAYOUT_DENSE2 = 1
QB = 127                  # activation range [-Qb, Qb]
PANEL = 32                # rows per tile panel
PAD_META = 0x44444444     # meta dword of a padded row: every window (0, 1)

__all__ = [
    "LAYOUT_SPARSE", "LAYOUT_DENSE2", "QB", "PAD_META",
    "round_ratio_to_f32", "absmean_gamma", "nm_mask", "ternarize", "effective_weights",
    "WINDOW_M", "window_table", "window_table_68", "k_eff", "packed_dwords", "weight_slots",
    "pack", "unpack_slots", "slots_to_dense", "act_quant", "lift", "lift_68", "acc_dense",
    "acc_addsub", "rescale", "forward", "bf16_round", "dequant_act", "backward",
    "LAYOUT_SPARSE6", "STATE6_PAIRS", "STATE6_COUNT", "state6", "state6_decode", "state6_dense",
    "packed6_dwords", "pack6", "unpack6",
]


# ----------------------------------------------------------------------------------------------
# gamma: absmean scale ([B158] "The mechanism", absmean weight quantization; [SB] 2, the scale
# is taken from the dense master before the mask is applied)
# ----------------------------------------------------------------------------------------------

def round_ratio_to_f32(num: int, den: int) -> np.float32:
    """Round the nonnegative rational num/den to the nearest fp32, ties to even (exact)."""
    assert num >= 0 and den > 0
    if num == 0:
        return np.float32(0.0)
    # binary exponent E with 2^E <= num/den < 2^(E+1)
    E = num.bit_length() - den.bit_length()
    if E >= 0:
        if num < (den << E):
            E -= 1
    else:
        if (num << -E) < den:
            E -= 1
    # quantum of the fp32 grid at that exponent (subnormals share 2^-149)
    qe = max(E, -126) - 23
    if qe >= 0:
        q, r = divmod(num, den << qe)
        d = den << qe
    else:
        q, r = divmod(num << -qe, den)
        d = den
    if 2 * r > d or (2 * r == d and (q & 1)):
        q += 1
    val = math.ldexp(float(q), qe)
    out = np.float32(val)
    assert float(out) == val, "value out of fp32 range"
    return out


def absmean_gamma(W: np.ndarray) -> np.float32:
    """gamma = mean |W| over every entry of the dense fp32 master, exact then rounded once.

    Every finite fp32 magnitude is m * 2^(max(e,1) - 150) with integer significand m < 2^24
    and biased exponent e, i.e. an integer multiple of 2^-149.  The sum of all magnitudes is
    therefore an exact integer S in units of 2^-149 and gamma = RNE_fp32(S / (count * 2^149)).
    """
    a = np.abs(np.asarray(W, dtype=np.float32)).ravel()
    count = a.size
    assert count > 0
    bits = a.view(np.uint32)
    e = (bits >> 23).astype(np.int64)
    assert np.all(e < 255), "non-finite weights are outside the contract"
    m = (bits & 0x7FFFFF).astype(np.int64)
    m = np.where(e > 0, m | (1 << 23), m)
    shift = np.maximum(e, 1) - 1
    S = 0
    for s in np.unique(shift):
        S += int(m[shift == s].sum(dtype=np.int64)) << int(s)
    return round_ratio_to_f32(S, count << 149)


# ----------------------------------------------------------------------------------------------
# N:M mask on the continuous master ([SB] 2, Maskering; Dynamisch Masker)
# ----------------------------------------------------------------------------------------------

def nm_mask(W: np.ndarray, N: int, M: int) -> np.ndarray:
    """Boolean keep-mask: per row, per contiguous M-group along K, the N largest |w|.

    Ties are broken toward the lower index (a stable sort of -|w|).  |-0.0| == |+0.0|.
    """
    W = np.asarray(W, dtype=np.float32)
    n, K = W.shape
    assert K % M == 0 and 0 < N <= M
    g = np.abs(W).reshape(n, K // M, M)
    order = np.argsort(-g, axis=-1, kind="stable")
    keep = np.zeros(g.shape, dtype=bool)
    np.put_along_axis(keep, order[..., :N], True, axis=-1)
    return keep.reshape(n, K)


# ----------------------------------------------------------------------------------------------
# ternarization ([B158] "The mechanism": divide by gamma, round, clip to [-1, 1])
# ----------------------------------------------------------------------------------------------

def ternarize(W: np.ndarray, gamma: np.float32) -> np.ndarray:
    """W~ = clip(rint(fl32(W / gamma)), -1, 1), rint = round half to even; all zero if gamma == 0."""
    W = np.asarray(W, dtype=np.float32)
    if float(gamma) == 0.0:
        return np.zeros(W.shape, dtype=np.int8)
    q = W / np.float32(gamma)            # IEEE fp32 division
    assert q.dtype == np.float32
    return np.clip(np.rint(q), -1, 1).astype(np.int8)


def effective_weights(W: np.ndarray, N: int, M: int) -> Tuple[np.ndarray, np.float32, np.ndarray]:
    """W_eff = mask * ternary(W) ([SB] 2, Forward Pass: quantize, then apply the mask).

    Returns (W_eff int8 [n][K], gamma, keep mask).
    """
    gamma = absmean_gamma(W)
    t = ternarize(W, gamma)
    keep = nm_mask(W, N, M)
    return np.where(keep, t, 0).astype(np.int8), gamma, keep


# ----------------------------------------------------------------------------------------------
# (2N-2):2N sliding windows ([SS] Sliding Window Decomposition): 4:6, 6:8, ..., 14:16
# ----------------------------------------------------------------------------------------------

WINDOW_M = (6, 8, 10, 12, 14, 16)   # group sizes M = 2N decomposed into N - 1 overlapping 2:4 windows


def _assign_windows(kept: List[int], M: int) -> List[List[int]]:
    """Kept positions of an M-group (M - 2 of them) -> positions per window.

    Window w (0 <= w < M/2 - 1) covers positions 2w..2w+3.  Positions are taken in ascending
    order, each by the lowest window that covers it and still holds fewer than two.
    """
    nw = M // 2 - 1
    assert len(kept) == M - 2
    wins: List[List[int]] = [[] for _ in range(nw)]
    for p in sorted(kept):
        for w in range(nw):
            if 2 * w <= p <= 2 * w + 3 and len(wins[w]) < 2:
                wins[w].append(p)
                break
        else:
            raise AssertionError(f"no window for position {p} of {sorted(kept)}")
    assert all(len(w) == 2 for w in wins), kept
    return wins


def _assign_windows_68(kept: List[int]) -> List[List[int]]:
    """6:8 case of _assign_windows (windows 0..3, 2..5, 4..7)."""
    return _assign_windows(kept, 8)


def window_table(M: int) -> Dict[int, List[List[int]]]:
    """keep-bitmask of an M-group (bit p = position p kept) -> positions per window."""
    table = {}
    for drop in range(M):
        for drop2 in range(drop + 1, M):
            kept = [p for p in range(M) if p not in (drop, drop2)]
            mask = sum(1 << p for p in kept)
            table[mask] = _assign_windows(kept, M)
    return table


def window_table_68() -> Dict[int, List[List[int]]]:
    return window_table(8)


# ----------------------------------------------------------------------------------------------
# slots and the packed layout
# ----------------------------------------------------------------------------------------------

def k_eff(K: int, N: int, M: int, layout: int) -> int:
    """Length of the packed K axis: K for 2:4 and DENSE2, (2M - 4) K / M for (M-2):M windows
    (3K/2 for 6:8, 7K/4 for 14:16)."""
    if layout == LAYOUT_DENSE2:
        return K
    if (N, M) == (2, 4):
        return K
    if M in WINDOW_M and N == M - 2:
        return K * (2 * M - 4) // M
    raise ValueError("SPARSE layout supports 2:4 and (M-2):M for even M = 6..16")


def packed_dwords(n: int, K: int, N: int, M: int, layout: int) -> Tuple[int, int, int]:
    """(code dwords, meta dwords, n_pad) of a packed matrix."""
    n_pad = -(-n // PANEL) * PANEL
    ke = k_eff(K, N, M, layout)
    if layout == LAYOUT_DENSE2:
        assert K % 32 == 0
        return n_pad * K // 16, 0, n_pad
    assert ke % 64 == 0
    return n_pad * ke // 32, n_pad * ke // 32, n_pad


def weight_slots(W_eff: np.ndarray, keep: np.ndarray, N: int, M: int, layout: int):
    """Per-row slot codes (int8 in {-1,0,1}) and window indices (uint8 0..3, SPARSE only)."""
    n, K = W_eff.shape
    if layout == LAYOUT_DENSE2:
        return W_eff.astype(np.int8).copy(), None
    if (N, M) == (2, 4):
        kg = keep.reshape(n, K // 4, 4)
        pos = np.argsort(~kg, axis=-1, kind="stable")[..., :2]          # kept positions, ascending
        vals = np.take_along_axis(W_eff.reshape(n, K // 4, 4), pos, axis=-1)
        return vals.reshape(n, K // 2).astype(np.int8), pos.reshape(n, K // 2).astype(np.uint8)
    if M in WINDOW_M and N == M - 2:
        table = window_table(M)
        G = K // M
        kg = keep.reshape(n, G, M)
        bitmask = (kg.astype(np.int64) << np.arange(M)).sum(axis=-1)
        # dense position (0..M-1) of each of the M-2 slots per group, for every valid bitmask
        lut = np.zeros((1 << M, N), dtype=np.int64)
        for msk, wins in table.items():
            lut[msk] = [p for w in wins for p in w]
        assert np.all(np.isin(bitmask, list(table.keys())))
        pos = lut[bitmask]                                                # [n][G][M-2]
        vals = np.take_along_axis(W_eff.reshape(n, G, M), pos, axis=-1)
        window_start = 2 * (np.arange(N) // 2)                            # 0,0,2,2,4,4,...
        local = pos - window_start
        return vals.reshape(n, G * N).astype(np.int8), local.reshape(n, G * N).astype(np.uint8)
    raise ValueError("unsupported N:M")


_CODE_SHIFT = np.array([8 * (i % 4) + 2 * (i // 4) for i in range(16)], dtype=np.uint32)
_META_SHIFT = np.array([2 * i for i in range(16)], dtype=np.uint32)


def _tile(units: np.ndarray) -> np.ndarray:
    """[n_pad][U] unit dwords -> flat tiled order (panel, fragment, lane)."""
    n_pad, U = units.shape
    t = units.reshape(n_pad // PANEL, PANEL, U // 2, 2)      # [P][r][F][h]
    return np.ascontiguousarray(t.transpose(0, 2, 3, 1)).reshape(-1)


def _untile(flat: np.ndarray, n_pad: int, U: int) -> np.ndarray:
    t = flat.reshape(n_pad // PANEL, U // 2, 2, PANEL)       # [P][F][h][r]
    return np.ascontiguousarray(t.transpose(0, 3, 1, 2)).reshape(n_pad, U)


def pack(W: np.ndarray, N: int, M: int, layout: int = LAYOUT_SPARSE):
    """Mask + ternarize + pack a fp32 master (the library's pack call, layout id 2).

    Returns dict(codes=uint32[...], meta=uint32[...] or None, gamma=fp32, K_eff, n_pad,
    W_eff, keep).
    """
    W = np.asarray(W, dtype=np.float32)
    n, K = W.shape
    W_eff, gamma, keep = effective_weights(W, N, M)
    vals, idx = weight_slots(W_eff, keep, N, M, layout)
    ncode, nmeta, n_pad = packed_dwords(n, K, N, M, layout)
    S = vals.shape[1]
    U = S // 16
    v = np.zeros((n_pad, S), dtype=np.int8)
    v[:n] = vals
    code2 = np.where(v < 0, 2, v).astype(np.uint32)                  # 0 -> 00, +1 -> 01, -1 -> 10
    code_units = (code2.reshape(n_pad, U, 16) << _CODE_SHIFT).sum(
        axis=-1, dtype=np.uint64).astype(np.uint32)
    codes = _tile(code_units)
    meta = None
    if layout == LAYOUT_SPARSE:
        ix = np.zeros((n_pad, S), dtype=np.uint8)
        ix[:, 1::2] = 1                                      # padded rows: windows (0, 1)
        ix[:n] = idx
        meta_units = (ix.reshape(n_pad, U, 16).astype(np.uint32) << _META_SHIFT).sum(
            axis=-1, dtype=np.uint64).astype(np.uint32)
        meta = _tile(meta_units)
        assert meta.size == nmeta
    assert codes.size == ncode
    return dict(codes=codes, meta=meta, gamma=gamma, K_eff=S * 2 if layout == LAYOUT_SPARSE else S,
                n_pad=n_pad, W_eff=W_eff, keep=keep)


def unpack_slots(codes: np.ndarray, meta, n: int, K: int, N: int, M: int, layout: int):
    """Inverse of the tiling and bit packing: (slot codes int8 [n][S], indices uint8 or None)."""
    ncode, nmeta, n_pad = packed_dwords(n, K, N, M, layout)
    codes = np.asarray(codes).view(np.uint32).reshape(-1)
    assert codes.size == ncode
    ke = k_eff(K, N, M, layout)
    S = ke // 2 if layout == LAYOUT_SPARSE else ke
    U = S // 16
    cu = _untile(codes, n_pad, U)[:n]                                    # [n][U]
    raw = (cu[..., None] >> _CODE_SHIFT) & 3                              # [n][U][16]
    assert not np.any(raw == 3), "code 11 is never written"
    vals = np.where(raw == 2, -1, raw).astype(np.int8).reshape(n, S)
    if layout == LAYOUT_DENSE2:
        return vals, None
    mu = _untile(np.asarray(meta).view(np.uint32).reshape(-1), n_pad, U)[:n]
    idx = ((mu[..., None] >> _META_SHIFT) & 3).astype(np.uint8).reshape(n, S)
    return vals, idx


def slots_to_dense(vals: np.ndarray, idx, K: int, N: int, M: int, layout: int) -> np.ndarray:
    """Scatter slots back to the dense [n][K] ternary matrix (6:8 windows summed back)."""
    n = vals.shape[0]
    if layout == LAYOUT_DENSE2:
        return vals.astype(np.int8)
    S = vals.shape[1]
    window = np.arange(S) // 2
    lifted_pos = 4 * window[None, :] + idx.astype(np.int64)               # position on K_eff axis
    if (N, M) == (2, 4):
        dense_pos = lifted_pos
    else:
        L = 2 * M - 4                                                     # lifted per M dense
        g, rem = lifted_pos // L, lifted_pos % L
        dense_pos = M * g + 2 * (rem // 4) + (rem % 4)
    out = np.zeros((n, K), dtype=np.int64)
    rows = np.repeat(np.arange(n)[:, None], S, axis=1)
    np.add.at(out, (rows, dense_pos), vals.astype(np.int64))
    return out.astype(np.int8)


# ----------------------------------------------------------------------------------------------
# 6-bit 2:4 decode encoding (layout id 2 SPARSE6).  The Bitnet.cpp abstract (aitopics "bitnet"
# tag page) motivates ternary formats below 2 bits per weight; the pages fix no format.  A 2:4
# group has C(4,2) = 6 kept-position pairs and 3 x 3 ternary values on them: 54 states, which
# fit in 6 bits (0.1875 bytes per weight against the 0.25 of 2-bit codes plus 2-bit indices).
# ----------------------------------------------------------------------------------------------

LAYOUT_SPARSE6 = 2
STATE6_PAIRS = ((0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3))   # kept positions, state // 9
STATE6_COUNT = 54
_TERN_DIGIT = {0: 0, 1: 1, -1: 2}           # ternary value -> digit
_DIGIT_TERN = (0, 1, -1)


def state6(i: int, j: int, a: int, b: int) -> int:
    """State of a 2:4 group keeping positions i < j, with ternary value a at i and b at j:
    9 * (index of (i, j) in STATE6_PAIRS) + 3 * digit(a) + digit(b), digit(0, +1, -1) = 0, 1, 2."""
    return 9 * STATE6_PAIRS.index((i, j)) + 3 * _TERN_DIGIT[int(a)] + _TERN_DIGIT[int(b)]


def state6_decode(s: int) -> Tuple[int, int, int, int]:
    """(i, j, a, b) of a state 0..53; states 54..63 are never written."""
    if not 0 <= s < STATE6_COUNT:
        raise ValueError(f"6-bit state {s} is not one of the 54 states")
    p, r = divmod(s, 9)
    i, j = STATE6_PAIRS[p]
    return i, j, _DIGIT_TERN[r // 3], _DIGIT_TERN[r % 3]


def state6_dense(s: int) -> Tuple[int, int, int, int]:
    """The group's four effective ternary weights (zero where not kept)."""
    i, j, a, b = state6_decode(s)
    w = [0, 0, 0, 0]
    w[i], w[j] = a, b
    return tuple(w)


def packed6_dwords(n: int, K: int) -> Tuple[int, int, int]:
    """(stream dwords, n_pad, step pairs) of a SPARSE6 matrix: rows padded to 32, the K axis
    to whole 128-column step pairs; three dwords per lane per (panel, step pair)."""
    if K % 64 != 0:
        raise ValueError("SPARSE6 needs K % 64 == 0 (the 2:4 packed K axis)")
    n_pad = -(-n // PANEL) * PANEL
    NC = -(-K // 128)
    return (n_pad // PANEL) * NC * 64 * 3, n_pad, NC


def _state6_matrix(vals: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """[n][S] 2:4 slot values / indices (two slots per 4-wide group) -> [n][K/4] states."""
    n, S = vals.shape
    st = np.zeros((n, S // 2), dtype=np.int64)
    for r in range(n):
        for g in range(S // 2):
            i, j = int(idx[r, 2 * g]), int(idx[r, 2 * g + 1])
            st[r, g] = state6(i, j, int(vals[r, 2 * g]), int(vals[r, 2 * g + 1]))
    return st


def pack6(vals: np.ndarray, idx: np.ndarray, n: int, K: int) -> np.ndarray:
    """2:4 slots (weight_slots / unpack_slots of a 2:4 SPARSE matrix) -> SPARSE6 stream dwords.

    Unit: one 32-row panel P and one step pair c (128 columns: 32 groups).  Lane l (0..63) holds
    96 bits, little-endian over its three dwords, field f at bits 6f..6f+5; field
    f = 8 * s2 + 4 * rt + g' (s2, rt in {0, 1}, g' in 0..3) is the state of row 32P + 16rt + l % 16,
    group 32c + 16s2 + 4(l // 16) + g'.  Lane l's dwords sit at dword ((P * NC + c) * 64 + l) * 3.
    Padded rows and groups past K hold state 0 (positions (0, 1), both values 0: zero weights).
    """
    nd, n_pad, NC = packed6_dwords(n, K)
    st = np.zeros((n_pad, NC * 32), dtype=np.int64)
    st[:n, :K // 4] = _state6_matrix(vals, idx)
    out = np.zeros(nd, dtype=np.uint32)
    for P in range(n_pad // PANEL):
        for c in range(NC):
            for l in range(64):
                bits = 0
                for s2 in range(2):
                    for rt in range(2):
                        for gq in range(4):
                            f = 8 * s2 + 4 * rt + gq
                            row = PANEL * P + 16 * rt + l % 16
                            grp = 32 * c + 16 * s2 + 4 * (l // 16) + gq
                            bits |= int(st[row, grp]) << (6 * f)
                base = ((P * NC + c) * 64 + l) * 3
                for d in range(3):
                    out[base + d] = (bits >> (32 * d)) & 0xFFFFFFFF
    return out


def unpack6(stream: np.ndarray, n: int, K: int) -> Tuple[np.ndarray, np.ndarray]:
    """Inverse of pack6: (effective ternary weights int8 [n][K], kept mask bool [n][K])."""
    nd, n_pad, NC = packed6_dwords(n, K)
    stream = np.asarray(stream).view(np.uint32).reshape(-1)
    assert stream.size == nd
    W = np.zeros((n_pad, NC * 128), dtype=np.int8)
    keep = np.zeros((n_pad, NC * 128), dtype=bool)
    for P in range(n_pad // PANEL):
        for c in range(NC):
            for l in range(64):
                base = ((P * NC + c) * 64 + l) * 3
                bits = sum(int(stream[base + d]) << (32 * d) for d in range(3))
                for f in range(16):
                    s2, rt, gq = f // 8, (f // 4) % 2, f % 4
                    row = PANEL * P + 16 * rt + l % 16
                    grp = 32 * c + 16 * s2 + 4 * (l // 16) + gq
                    i, j, a, b = state6_decode((bits >> (6 * f)) & 63)
                    W[row, 4 * grp + i], W[row, 4 * grp + j] = a, b
                    keep[row, 4 * grp + i] = keep[row, 4 * grp + j] = True
    return W[:n, :K], keep[:n, :K]


# ----------------------------------------------------------------------------------------------
# activations ([B158] "The mechanism", Activations: per-token symmetric 8-bit, [-Qb, Qb];
# [SS] Activation Lifting for 6:8)
# ----------------------------------------------------------------------------------------------

def lift(q: np.ndarray, M: int) -> np.ndarray:
    """x'[t][(2M-4)g + 4w + j] = x[t][Mg + 2w + j], w = 0..M/2-2, j = 0..3."""
    T, K = q.shape
    G = K // M
    src = np.array([2 * w + j for w in range(M // 2 - 1) for j in range(4)])   # 2M-4 per group
    cols = (M * np.arange(G)[:, None] + src[None, :]).reshape(-1)
    return q[:, cols]


def lift_68(q: np.ndarray) -> np.ndarray:
    """x'[t][12g + 4w + j] = x[t][8g + 2w + j], w = 0..2, j = 0..3."""
    return lift(q, 8)


def act_quant(x: np.ndarray, lift_M: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Per-token absmax int8 quantization (Qb = 127).  Returns (xq int8 [T][K_eff], scale fp32 [T])."""
    x = np.asarray(x, dtype=np.float32)
    absmax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    nz = absmax > 0
    s = np.zeros_like(absmax)
    s[nz] = np.float32(QB) / absmax[nz]                          # fp32 division
    prod = x * s[:, None]                                        # fp32 multiply
    q = np.clip(np.rint(prod), -QB, QB).astype(np.int8)
    scale = (absmax / np.float32(QB)).astype(np.float32)
    scale[~nz] = 0.0
    if lift_M in WINDOW_M:
        q = lift(q, lift_M)
    else:
        assert lift_M == 0
    return q, scale


# ----------------------------------------------------------------------------------------------
# accumulation and rescale ([B158] "The mechanism": a ternary MAC is add, subtract or skip;
# integer accumulation of int8 activations, then rescale by gamma and the token scale)
# ----------------------------------------------------------------------------------------------

def acc_dense(W_eff: np.ndarray, q: np.ndarray) -> np.ndarray:
    """acc[t][o] = sum_k W_eff[o][k] * q[t][k] in int64 (form i: dense matmul)."""
    return np.asarray(q, np.int64) @ np.asarray(W_eff, np.int64).T


def acc_addsub(vals: np.ndarray, idx, xq: np.ndarray, layout: int) -> np.ndarray:
    """Form ii: per slot, add the activation under a +1 code, subtract it under a -1 code.

    ``xq`` is on the packed K axis (lifted for 6:8 and 14:16).
    """
    T = xq.shape[0]
    n, S = vals.shape
    if layout == LAYOUT_DENSE2:
        pos = np.broadcast_to(np.arange(S), (n, S))
    else:
        pos = 4 * (np.arange(S) // 2)[None, :] + idx.astype(np.int64)
    xq64 = xq.astype(np.int64)
    acc = np.zeros((T, n), dtype=np.int64)
    for o in range(n):
        plus = pos[o][vals[o] == 1]
        minus = pos[o][vals[o] == -1]
        acc[:, o] = xq64[:, plus].sum(axis=1) - xq64[:, minus].sum(axis=1)
    return acc


def rescale(acc: np.ndarray, gamma: np.float32, scale: np.ndarray) -> np.ndarray:
    """y = acc * gamma * scale_t, evaluated in fp64 and rounded to fp32."""
    y = np.asarray(acc, np.float64) * np.float64(gamma) * np.asarray(scale, np.float64)[:, None]
    return y.astype(np.float32)


def forward(W: np.ndarray, x: np.ndarray, N: int, M: int, layout: int = LAYOUT_SPARSE) -> Dict:
    """Whole path: pack the master, quantize (and lift) x, accumulate, rescale."""
    p = pack(W, N, M, layout)
    lift = M if (layout == LAYOUT_SPARSE and M in WINDOW_M) else 0
    xq, scale = act_quant(x, lift)
    acc = acc_dense(p["W_eff"], act_quant(x, 0)[0])
    y = rescale(acc, p["gamma"], scale)
    p.update(xq=xq, scale=scale, acc=acc, y=y)
    return p


# ----------------------------------------------------------------------------------------------
# backward ([SB] technical summary, Training Strategie: Dual STE -- the quantizer and the Top-N
# selection are bypassed by straight-through estimators and the gradient reaches every master
# weight, the masked ones too; the plain-language section says the same of removed weights)
# ----------------------------------------------------------------------------------------------

def bf16_round(v: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to the nearest bfloat16 (8 significant bits), ties to even.

    Returned as fp32 values.  v = m * 2^e with 0.5 <= |m| < 1 (frexp); the bfloat16 grid near v
    has spacing 2^(e - 8), or 2^-133 below the normal range (e < -125).
    """
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    _, e = np.frexp(v)
    step = np.exp2(np.maximum(e, -125) - 8).astype(np.float64)
    return (np.rint(v / step) * step).astype(np.float32)


def dequant_act(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """X^[t][k] = bf16(fp32(q[t][k] * scale_t)): the dequantized activation in bfloat16."""
    prod = np.asarray(q, np.float32) * np.asarray(scale, np.float32)[:, None]   # fp32 multiply
    return bf16_round(prod)


def backward(dy: np.ndarray, W_eff: np.ndarray, gamma: np.float32, q: np.ndarray,
             scale: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Straight-through gradients of y = X^ (gamma W_eff)^T, in fp64.

    dy: [T][n] bfloat16 values (as floats); W_eff: [n][K] ternary (mask applied); q: [T][K] int8
    (not lifted) with scale [T].  Returns dX [T][K] = gamma * (dY @ W_eff) and
    dW [n][K] = dY^T @ X^ (the gradient of every master weight, masked or kept).
    """
    dy64 = np.asarray(dy, np.float64)
    dx = np.float64(gamma) * (dy64 @ np.asarray(W_eff, np.float64))
    dw = dy64.T @ dequant_act(q, scale).astype(np.float64)
    return dx, dw
