"""W4A8: 4-bit weights times 8-bit activations, plain and slow -- TEST INFRASTRUCTURE ONLY.

Same rules as the rest of oracle/: only tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg may import it; it shares no code with the GPU
library.

What is computed (magicnetworld.com Ling-3.0 MoE article, sec. 5 and sec. 6:
the measured configuration is W4A8, MXFP4 expert weights with 8-bit
activations; the feed's "Fewer bytes per weight: NVFP4" gives the block-scale
idea).  The pages do not say how the activations are quantised; readings:

  * activations quantise per vector in blocks of 32 consecutive columns
    (aligned at column 0) to MXFP8: one E8M0 scale 2^e per block, e the
    smallest integer with amax_block / 2^e <= 448 (the largest E4M3 value, so
    no element saturates), code e + 127 clamped to 0..254, 127 for an all-zero
    block -- the same recipe as the MXFP4 weight quantiser;
  * elements: E4M3FN of x / 2^e, round to nearest, ties to the even code; a
    value that rounds to zero gets the +0 code;
  * the product is exact: y[m][r] = sum_k w[r][k] * e4m3(code[m][k]) * 2^e, in
    FP64 (weights dequantised as the GEMV oracle does).

The element rounding is oracle.quant's brute-force E4M3 rounding.
"""
from __future__ import annotations

import numpy as np

from . import dequant
from .quant import _E4M3, e4m3_rne

E4M3_MAX = 448.0


def block_exponent(amax: float) -> int:
    """The smallest e with amax / 2^e <= 448 (checked exactly), clamped so the
    E8M0 code e + 127 stays in 0..254; 0 for an all-zero block."""
    if amax == 0.0:
        return 0
    e = int(np.floor(np.log2(amax / E4M3_MAX)))
    while amax / 2.0 ** e > E4M3_MAX:
        e += 1
    while amax / 2.0 ** (e - 1) <= E4M3_MAX:
        e -= 1
    return min(max(e, -127), 127)


def quantize_mxfp8(x_bf16_bits: np.ndarray):
    """Quantise bf16 activations [M][d_in] (d_in % 32 == 0), given as bit
    patterns, to (codes u8 [M][d_in] E4M3FN, scales u8 [M][d_in / 32] E8M0)."""
    bits = np.asarray(x_bf16_bits, dtype=np.uint16)
    if bits.ndim == 1:
        bits = bits[None, :]
    M, d_in = bits.shape
    x = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    codes = np.zeros((M, d_in), np.uint8)
    scales = np.zeros((M, d_in // 32), np.uint8)
    for m in range(M):
        for b in range(d_in // 32):
            seg = x[m, 32 * b:32 * (b + 1)]
            e = block_exponent(float(np.max(np.abs(seg))))
            scales[m, b] = e + 127
            for k in range(32):
                q = seg[k] / 2.0 ** e  # exact: a power-of-two division of a bf16 value
                c = e4m3_rne(abs(q))
                codes[m, 32 * b + k] = (0x80 | c) if (q < 0 and c != 0) else c
    return codes, scales


def dequant_mxfp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """FP64 values of MXFP8 activations."""
    codes = np.asarray(codes, dtype=np.uint8)
    mag = _E4M3[(codes & 0x7F).astype(np.int64)]
    val = np.where(codes & 0x80, -mag, mag)
    e = np.repeat(np.asarray(scales, dtype=np.int64) - 127, 32, axis=1)
    return val * np.exp2(e.astype(np.float64))


def gemv(fmt, w_codes, w_scales, tensor_scale, x_bf16_bits):
    """Y[m][r] = sum_k w[r][k] * xq[m][k] in FP64 with xq the MXFP8 activations;
    also returns A[m][r] = sum_k |w[r][k] * xq[m][k]| (the tolerance scale)."""
    W = dequant(fmt, w_codes, w_scales, tensor_scale)
    codes, scales = quantize_mxfp8(x_bf16_bits)
    Xq = dequant_mxfp8(codes, scales)
    return Xq @ W.T, np.abs(Xq) @ np.abs(W).T
