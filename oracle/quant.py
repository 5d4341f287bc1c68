"""Load-time quantisers, plain and slow -- TEST INFRASTRUCTURE ONLY.

Same rules as the rest of oracle/: only tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg may import it; it shares no code with the GPU
library.

What is computed (mdjawad.com DGX Spark feed, section "Fewer bytes per weight:
NVFP4"): each block of 16 consecutive weights gets a scale chosen so that its
largest magnitude maps to 6, the largest E2M1 value; the block scales are E4M3,
and one FP32 number per tensor brings them into E4M3's range.  Readings where
the pages stop:

  * NVFP4 tensor scale: s_T = the FP32 value nearest to amax(W) / (6 * 448), so
    the largest block scale lands at 448, the largest E4M3 value (1 for an
    all-zero tensor).  It is the stored FP32 number, and every later decision
    is taken against that stored value, because it is what dequantisation
    multiplies by.
  * block scale code = nearest E4M3 value to amax_b / (6 s_T); element code =
    nearest E2M1 value to w / (s_b s_T) with s_b the decoded block scale
    (element code 0 where s_b == 0).
  * MXFP4 (block of 32, E8M0 scale; the Ling-3.0 article leaves the recipe
    open): the smallest power of two 2^e with amax_b / 2^e <= 6, code e + 127
    clamped to 0..254 (127 for an all-zero block); elements nearest E2M1 of
    w / 2^e.
  * FP8 rows: s_row = the FP32 value nearest to amax_row / 448 (1 for an
    all-zero row); codes = nearest E4M3 of w / s_row.
  * "Nearest": the grid value closest to the exact quotient; a quotient exactly
    halfway between two grid values takes the even code; magnitudes above the
    largest value saturate to it; a value that rounds to zero gets the
    positive-zero code.

Every decision here is exact.  The quotients are never formed: q >= mid is
decided as |w| >= mid * den, and that product is exact in float64 (a midpoint
of E2M1 has at most 3 significant bits and one of E4M3 at most 5; 6 has 2; an
E4M3 scale 4; an FP32 scale 24: at most 31 of float64's 53 bits).  The two FP32
scales are rounded from exact rationals (fractions.Fraction).

A kernel that forms the quotient in FP32 (one or two roundings, each at most
2^-24 relative) can only land on the other side of a midpoint when the exact
quotient lies within about 2^-23 of it, relatively.  `quantize_detail` marks
every decision whose exact quotient lies within AMBIGUOUS_REL = 2^-22 of a
midpoint (or on it) and names the code on the other side; nothing else may
differ.  For an NVFP4 block whose scale decision is so marked, it also gives
the elements as decided under the other scale.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

NVFP4, MXFP4, FP8_ROW = 1, 2, 3

# E2M1 magnitudes of codes 0..7 (the pages' value set)
_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _e4m3_magnitudes() -> np.ndarray:
    """Magnitudes of E4M3FN codes 0..126 (bias 7, subnormals, 0x7F is NaN)."""
    out = []
    for c in range(127):
        e, m = c >> 3, c & 7
        out.append((m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(out)


_E4M3 = _e4m3_magnitudes()
_MID_E2M1 = (_E2M1[:-1] + _E2M1[1:]) / 2      # exact in float64
_MID_E4M3 = (_E4M3[:-1] + _E4M3[1:]) / 2

AMBIGUOUS_REL = 2.0 ** -22


def _nearest_even(a: float, grid: np.ndarray) -> int:
    """Index of the grid value nearest to a >= 0, ties to the even index,
    saturating at the last value (brute force over the whole grid)."""
    if a >= grid[-1]:
        return len(grid) - 1
    d = np.abs(grid - a)
    best = np.flatnonzero(d == d.min())
    even = [int(i) for i in best if i % 2 == 0]
    return even[0] if even else int(best[0])


def e2m1_rne(q: float) -> int:
    """E2M1 code (sign in bit 3) of q, rounded to nearest even, saturating."""
    i = _nearest_even(abs(float(q)), _E2M1)
    return (8 | i) if (q < 0 and i != 0) else i


def e4m3_rne(t: float) -> int:
    """E4M3FN code of t >= 0, rounded to nearest even, saturating at 448."""
    return _nearest_even(float(t), _E4M3)


def f32_nearest(x: Fraction) -> np.float32:
    """The FP32 value nearest to the rational x (ties to the even significand),
    chosen by exact comparison among the float32 neighbours of a first guess."""
    guess = np.float32(float(x))
    cands = [np.nextafter(guess, np.float32(-np.inf)), guess, np.nextafter(guess, np.float32(np.inf))]
    best = None
    for c in cands:
        if not np.isfinite(c):
            continue
        d = abs(Fraction(float(c)) - x)
        key = (d, int(np.array(c, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def _decide(a: np.ndarray, den, mids: np.ndarray):
    """Nearest grid index of the exact quotient a / den (a >= 0, den > 0; every
    mids[i] * den exact in float64), ties to the even index, saturating.
    Returns (index, ambiguous, other) with `other` the index on the other side of
    the midpoint that marks the decision ambiguous (= index where not)."""
    a = np.asarray(a, np.float64)
    den = np.broadcast_to(np.asarray(den, np.float64), a.shape)
    P = den[..., None] * mids                      # exact products
    A = a[..., None]
    above = A > P
    tie = A == P
    n = np.arange(1, mids.size + 1)                # index just above midpoint i
    idx = above.sum(-1) + (tie & (n % 2 == 0)).sum(-1)
    near = np.abs(A - P) <= AMBIGUOUS_REL * A
    near |= tie
    amb = near.any(-1)
    i = np.argmax(near, -1)                        # the (first) close midpoint
    # chosen side of that midpoint: above -> i + 1, else i; the other side
    chosen_above = idx > i
    other = np.where(amb, np.where(chosen_above, i, i + 1), idx)
    return idx.astype(np.int64), amb, other.astype(np.int64)


def _signed(idx: np.ndarray, neg: np.ndarray, sign_bit: int) -> np.ndarray:
    """Code with the sign bit set for negative inputs, except for zero."""
    return np.where(neg & (idx != 0), idx | sign_bit, idx).astype(np.uint8)


def _bf16_values(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def tensor_scale_nvfp4(w: np.ndarray) -> np.float32:
    amax = float(np.max(np.abs(w))) if w.size else 0.0
    return f32_nearest(Fraction(amax) / 2688) if amax > 0 else np.float32(1.0)


def quantize_detail(fmt: int, w_bf16_bits: np.ndarray) -> dict:
    """Quantise a [d_out][d_in] matrix given as bf16 bit patterns.

    Returns a dict:
      codes, scales, tensor_scale -- the logical layout fp4g_pack takes (NVFP4 /
        MXFP4 codes u8[d_out][d_in/2] with column 2j in bits 0-3; scales
        u8[d_out][d_in/16] E4M3 or u8[d_out][d_in/32] E8M0; FP8 codes
        u8[d_out][d_in], scales f32[d_out]);
      el, el_amb, el_alt -- element codes u8[d_out][d_in] (sign in bit 3, or 7
        for FP8), whether each decision is near a midpoint, and the code on the
        other side;
      scale_amb, scale_alt -- the same for NVFP4 block scales (all False for
        MXFP4, whose decisions are exact powers of two);
      el_if_alt, el_if_alt_amb, el_if_alt_alt -- NVFP4 only: the elements under
        the block's other scale code (equal to el where the scale is not
        ambiguous)."""
    w = _bf16_values(w_bf16_bits)
    d_out, d_in = w.shape
    a, neg = np.abs(w), w < 0
    out: dict = {}
    if fmt == FP8_ROW:
        scales = np.zeros(d_out, np.float32)
        for r in range(d_out):
            amax = float(np.max(a[r]))
            scales[r] = f32_nearest(Fraction(amax) / 448) if amax > 0 else np.float32(1.0)
        idx, amb, alt = _decide(a, scales.astype(np.float64)[:, None], _MID_E4M3)
        out.update(codes=_signed(idx, neg, 0x80), scales=scales, tensor_scale=1.0,
                   el=_signed(idx, neg, 0x80), el_amb=amb, el_alt=_signed(alt, neg, 0x80))
        return out
    blk = 16 if fmt == NVFP4 else 32
    nb = d_in // blk
    ab = a.reshape(d_out, nb, blk)
    amax_b = ab.max(-1)
    if fmt == NVFP4:
        s_t = tensor_scale_nvfp4(w)
        st = float(s_t)
        sidx, samb, salt = _decide(amax_b, 6.0 * st, _MID_E4M3)

        def elements(sc_idx):
            den = _E4M3[sc_idx] * st                  # exact: 4 x 24 bits
            safe = np.where(den > 0, den, 1.0)
            i, m, o = _decide(ab, safe[..., None], _MID_E2M1)
            z = (den == 0)[..., None]
            i, m, o = np.where(z, 0, i), np.where(z, False, m), np.where(z, 0, o)
            return i.reshape(d_out, d_in), m.reshape(d_out, d_in), o.reshape(d_out, d_in)

        el, el_amb, el_alt = elements(sidx)
        el2, el2_amb, el2_alt = elements(np.where(samb, salt, sidx))
        scales = sidx.astype(np.uint8)
        out.update(scale_amb=samb, scale_alt=salt.astype(np.uint8), tensor_scale=float(s_t),
                   el_if_alt=_signed(el2, neg, 8), el_if_alt_amb=el2_amb, el_if_alt_alt=_signed(el2_alt, neg, 8))
    else:
        e = np.zeros((d_out, nb), np.int64)
        for r in range(d_out):
            for b in range(nb):
                m = float(amax_b[r, b])
                if m == 0.0:
                    continue
                k = int(np.floor(np.log2(m))) - 3      # 2^k * 6 < m for a start
                while m > 6.0 * 2.0 ** k:               # exact comparisons
                    k += 1
                while m <= 6.0 * 2.0 ** (k - 1):
                    k -= 1
                e[r, b] = k
        code = np.clip(e + 127, 0, 254)
        code = np.where(amax_b == 0, 127, code)
        scale = np.exp2((code - 127).astype(np.float64))
        i, m_, o = _decide(ab, scale[..., None], _MID_E2M1)
        el, el_amb, el_alt = i.reshape(d_out, d_in), m_.reshape(d_out, d_in), o.reshape(d_out, d_in)
        scales = code.astype(np.uint8)
        out.update(scale_amb=np.zeros((d_out, nb), bool), scale_alt=scales.copy(), tensor_scale=1.0)
    el_s = _signed(el, neg, 8)
    codes = (el_s[:, 0::2] | (el_s[:, 1::2] << 4)).astype(np.uint8)
    out.update(codes=codes, scales=scales, el=el_s, el_amb=el_amb, el_alt=_signed(el_alt, neg, 8))
    if fmt == MXFP4:
        out.update(el_if_alt=out["el"], el_if_alt_amb=out["el_amb"], el_if_alt_alt=out["el_alt"])
    return out


def quantize(fmt: int, w_bf16_bits: np.ndarray):
    """(codes, scales, tensor_scale) of quantize_detail."""
    d = quantize_detail(fmt, w_bf16_bits)
    return d["codes"], d["scales"], d["tensor_scale"]


def elements_of(fmt: int, codes: np.ndarray) -> np.ndarray:
    """Element codes u8[d_out][d_in] of logical codes (NVFP4/MXFP4 nibbles
    unpacked, low nibble first; FP8 as is)."""
    c = np.asarray(codes, np.uint8)
    if fmt == FP8_ROW:
        return c
    return np.stack([c & 15, c >> 4], axis=-1).reshape(c.shape[0], -1)
