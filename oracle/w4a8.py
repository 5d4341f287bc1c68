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


def _bf16_bits_of(v: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of FP64 values: FP32 round to nearest even, then bf16
    round to nearest even (the intermediate h between the two halves of a
    layer is bf16 on every path)."""
    f = np.asarray(v, np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    r = (f + 0x7FFF + ((f >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def moe(get_expert, shared, X_bits, logits, k: int):
    """W4A8 mixture-of-experts layer in FP64 (the Ling-3.0 article's measured
    configuration: MXFP4 experts, 8-bit activations): the routing of oracle.moe
    (top-k by logit, ties to the lower index, softmax over the k picks), each
    expert's gate and up on x quantised to MXFP8, h = bf16(SiLU(g) u), down on h
    quantised to MXFP8, y = sum_j g_j d_j + d_shared.  Returns dict(ids, w, y,
    tol) with tol the sum of the gate-weighted magnitude sums of the downs."""
    from . import silu_mul, topk_softmax

    X_bits = np.asarray(X_bits, np.uint16)
    ids, w = topk_softmax(logits, k)
    M = X_bits.shape[0]
    ys, tols = [], []
    for m in range(M):
        picks = [(int(ids[m, j]), w[m, j]) for j in range(k)] + ([(None, 1.0)] if shared is not None else [])
        y = 0.0
        tol = 0.0
        for e, c in picks:
            ex = shared if e is None else get_expert(e)
            g, _ = gemv(ex["gate"]["format"], ex["gate"]["codes"], ex["gate"]["scales"], ex["gate"]["tensor_scale"],
                        X_bits[m][None, :])
            u, _ = gemv(ex["up"]["format"], ex["up"]["codes"], ex["up"]["scales"], ex["up"]["tensor_scale"],
                        X_bits[m][None, :])
            h = _bf16_bits_of(silu_mul(g, u))
            dn = ex["down"]
            d, Ad = gemv(dn["format"], dn["codes"], dn["scales"], dn["tensor_scale"], h)
            y = y + c * d[0]
            tol = tol + c * Ad[0]
        ys.append(y)
        tols.append(tol)
    return {"ids": ids, "w": w, "y": np.stack(ys), "tol": np.stack(tols)}
