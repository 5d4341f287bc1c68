"""Reference packer for the tiled weight layout -- TEST INFRASTRUCTURE ONLY.

The packed layout is this library's own format (it is not from the pages); its
definition is the prose of fp4g_packed_bytes in include/fp4gemv.h.  This module
writes that prose out with numpy reshapes so that the GPU packer can be checked
byte for byte against it.  It shares no code with the GPU packer.
"""
from __future__ import annotations

import numpy as np

NVFP4, MXFP4, FP8_ROW = 1, 2, 3


def packed_bytes(fmt: int, d_out: int, d_in: int) -> int:
    if d_out < 1 or d_in < 32 or d_in % 32:
        return 0
    R, C = -(-d_out // 64), -(-d_in // 256)
    tile = {NVFP4: 9216, MXFP4: 8704, FP8_ROW: 16384}[fmt]
    return R * C * tile + (R * 64 * 4 if fmt == FP8_ROW else 0)


def pack(fmt: int, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Logical (codes, scales) -> packed bytes (uint8 vector)."""
    d_out = codes.shape[0]
    d_in = codes.shape[1] * (1 if fmt == FP8_ROW else 2)
    R, C = -(-d_out // 64), -(-d_in // 256)
    if fmt == FP8_ROW:
        cp = np.zeros((R * 64, C * 256), np.uint8)
        cp[:d_out, :d_in] = codes
        # [g][l][c][j][16] -> [g][c][j][l][16]
        t = cp.reshape(R, 64, C, 16, 16).transpose(0, 2, 3, 1, 4).reshape(R * C * 16384)
        rs = np.zeros(R * 64, np.float32)
        rs[:d_out] = scales
        return np.concatenate([t, rs.view(np.uint8)])
    per = 16 if fmt == NVFP4 else 8
    cp = np.zeros((R * 64, C * 128), np.uint8)
    cp[:d_out, : d_in // 2] = codes
    sp = np.zeros((R * 64, C * per), np.uint8)
    sp[:d_out, : scales.shape[1]] = scales
    ct = cp.reshape(R, 64, C, 8, 16).transpose(0, 2, 3, 1, 4).reshape(R, C, 8192)
    st = sp.reshape(R, 64, C, per).transpose(0, 2, 1, 3).reshape(R, C, 64 * per)
    return np.concatenate([ct, st], axis=2).reshape(-1)
