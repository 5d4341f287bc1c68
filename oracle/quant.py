"""Load-time quantisers, plain and slow -- TEST INFRASTRUCTURE ONLY.

Same rules as the rest of oracle/: only tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg may import it; it shares no code with the GPU
library.

What is computed (mdjawad.com DGX Spark feed, section "Fewer bytes per weight:
NVFP4"): each block of 16 consecutive weights gets a scale chosen so that its
largest magnitude maps to 6 (the largest E2M1 value), stored as E4M3; one FP32
scale per tensor brings the block scales into the range E4M3 can represent.
Readings where the pages stop:

  * NVFP4 tensor scale s_T = amax(W) / (6 * 448), so the largest block scale is
    at most 448, the largest E4M3 value; s_T = 1 for an all-zero tensor.
  * block scale code = E4M3_RNE(amax_b / (6 * s_T)); element code =
    E2M1_RNE(w / (s_b * s_T)) with s_b the decoded block scale (codes 0 where
    s_b == 0).
  * MXFP4 (block of 32, E8M0 scale; the article leaves the recipe open): the
    smallest power of two 2^e with amax_b / 2^e <= 6, code e + 127 clamped to
    0..254 (127 for an all-zero block); elements E2M1_RNE(w / 2^e).
  * FP8 rows: s_row = amax_row / 448 (1 for an all-zero row); codes =
    E4M3_RNE(w / s_row).
  * Rounding: to the nearest representable value, ties to the even code;
    magnitudes above the largest value saturate to it; a value that rounds to
    zero gets the positive-zero code.
  * The scale arithmetic (the divisions and products above) is done in FP32,
    one rounding per operation in the order written, because its results decide
    integer codes; the GPU kernels take the same decisions in the same precision.

The roundings are brute force: the nearest of the format's enumerated values.
"""
from __future__ import annotations

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


def _nearest_even(a: float, grid: np.ndarray) -> int:
    """Index of the grid value nearest to a >= 0, ties to the even index,
    saturating at the last value."""
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


def _f32(x) -> np.float32:
    return np.float32(x)


def quantize(fmt: int, w_bf16_bits: np.ndarray):
    """Quantise a [d_out][d_in] matrix given as bf16 bit patterns.  Returns
    (codes, scales, tensor_scale) in the logical layout fp4g_pack takes:
    NVFP4/MXFP4 codes u8[d_out][d_in/2] (column 2j in bits 0-3), scales
    u8[d_out][d_in/16] E4M3 or u8[d_out][d_in/32] E8M0; FP8 codes u8[d_out][d_in],
    scales f32[d_out]."""
    bits = np.asarray(w_bf16_bits, dtype=np.uint16)
    d_out, d_in = bits.shape
    w = (bits.astype(np.uint32) << 16).view(np.float32)  # exact bf16 -> f32
    if fmt == FP8_ROW:
        codes = np.zeros((d_out, d_in), np.uint8)
        scales = np.zeros(d_out, np.float32)
        for r in range(d_out):
            amax = _f32(np.max(np.abs(w[r])))
            s = _f32(amax / _f32(448.0)) if amax > 0 else _f32(1.0)
            scales[r] = s
            for k in range(d_in):
                q = _f32(w[r, k] / s)
                c = e4m3_rne(abs(float(q)))
                codes[r, k] = (0x80 | c) if (q < 0 and c != 0) else c
        return codes, scales, 1.0
    blk = 16 if fmt == NVFP4 else 32
    el = np.zeros((d_out, d_in), np.uint8)
    scales = np.zeros((d_out, d_in // blk), np.uint8)
    if fmt == NVFP4:
        amax_t = _f32(np.max(np.abs(w)))
        s_t = _f32(amax_t / _f32(2688.0)) if amax_t > 0 else _f32(1.0)
        six_st = _f32(_f32(6.0) * s_t)
    else:
        s_t = _f32(1.0)
    for r in range(d_out):
        for b in range(d_in // blk):
            seg = w[r, b * blk:(b + 1) * blk]
            amax = _f32(np.max(np.abs(seg)))
            if fmt == NVFP4:
                sc = e4m3_rne(float(_f32(amax / six_st)))
                scales[r, b] = sc
                den = _f32(_f32(_E4M3[sc]) * s_t)
                for k in range(blk):
                    el[r, b * blk + k] = e2m1_rne(float(_f32(seg[k] / den))) if _E4M3[sc] > 0 else 0
            else:
                if amax > 0:
                    e = int(np.ceil(np.log2(float(_f32(amax / _f32(6.0))))))
                    # the smallest power of two with amax / 2^e <= 6, checked exactly
                    while float(amax) / 2.0 ** e > 6.0:
                        e += 1
                    while e > -127 and float(amax) / 2.0 ** (e - 1) <= 6.0:
                        e -= 1
                    code = min(max(e + 127, 0), 254)
                else:
                    code = 127
                scales[r, b] = code
                for k in range(blk):
                    el[r, b * blk + k] = e2m1_rne(float(seg[k]) / 2.0 ** (code - 127))
    codes = (el[:, 0::2] | (el[:, 1::2] << 4)).astype(np.uint8)
    return codes, scales, float(s_t)
