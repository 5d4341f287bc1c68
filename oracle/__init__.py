"""CPU oracle (FP64) for the decode GEMV library -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may
import this package.  It shares no code with the GPU library and never calls it;
the GPU library never imports it.  Everything here is plain: decoders from closed
forms, sequential FP64 sums (oracle.c), and numpy glue that composes them in the
order the pages describe.

Sources for what is computed (the pages carry no code):
  * mdjawad.com DGX Spark feed, "Decode speed is bytes divided by bandwidth":
    y = W x with one multiply and one add per weight; "Fewer bytes per weight:
    NVFP4": E2M1 elements, E4M3 scale per 16 consecutive weights, FP32 tensor
    scale (formula lost in extraction; read as a product); "More tokens per
    weight read": the verify pass multiplies each matrix by K+1 vectors.
  * magicnetworld.com Ling-3.0 MoE decode article, sec. 3 and the sec. 4
    flowchart: 8 of 512 routed experts plus 1 shared expert per token; MXFP4
    expert weights (block of 32 with an E8M0 scale is the reading taken); sec. 7:
    FP8 output layer; sec. 8: M tokens touch the union of their experts, about
    512 * (1 - (1 - 8/512)^M) of them.

Parity pins: see tests/test_oracle_pins.py (the MoE layer end to end through its
invariants: identical experts ignore the routing, top-1 is the argmax expert's
output, the output is the gate-weighted sum).  Parity unpinned: the bf16 rounding
of the MLP intermediate h, which this oracle keeps in FP64 (the GPU's h is held
to it within the tolerance bound plus half a bf16 step).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

NVFP4, MXFP4, FP8_ROW = 1, 2, 3

_HERE = Path(__file__).resolve().parent
_LIB_PATH = _HERE / "liboracle.so"
_lib = None


def build(verbose: bool = False) -> Path:
    """Compile oracle.c into liboracle.so with gcc (plain C, -O2, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-shared", "-fPIC", "-o", str(_LIB_PATH),
           str(_HERE / "oracle.c"), "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not _LIB_PATH.exists() or _LIB_PATH.stat().st_mtime < (_HERE / "oracle.c").stat().st_mtime:
            build()
        L = ctypes.CDLL(str(_LIB_PATH))
        d, u, i32, i64, vp = ctypes.c_double, ctypes.c_uint, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
        for name in ("or_e2m1", "or_e4m3", "or_e8m0"):
            getattr(L, name).restype = d
            getattr(L, name).argtypes = [u]
        L.or_bf16.restype = d
        L.or_bf16.argtypes = [ctypes.c_uint16]
        L.or_silu.restype = d
        L.or_silu.argtypes = [d]
        for name in ("or_gemv", "or_gemv_dx"):
            f = getattr(L, name)
            f.restype = i32
            f.argtypes = [i32, i64, i64, vp, vp, d, i32, vp, vp, i64, vp, vp, i32]
        L.or_dequant.restype = i32
        L.or_dequant.argtypes = [i32, i64, i64, vp, vp, d, vp]
        L.or_silu_mul.restype = None
        L.or_silu_mul.argtypes = [i64, vp, vp, vp]
        L.or_topk_softmax.restype = i32
        L.or_topk_softmax.argtypes = [i32, i32, i32, vp, vp, vp]
        _lib = L
    return _lib


def _nthreads() -> int:
    return max(1, min(64, os.cpu_count() or 1))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _np(t):
    """numpy view of a CPU torch tensor or array (bf16 viewed as uint16)."""
    try:
        import torch
        if isinstance(t, torch.Tensor):
            t = t.detach().cpu()
            if t.dtype == torch.bfloat16:
                t = t.view(torch.uint16) if hasattr(torch, "uint16") else t.view(torch.int16)
            return np.ascontiguousarray(t.numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(t)


# ---- scalar decoders -------------------------------------------------------------
def e2m1(code: int) -> float:
    return lib().or_e2m1(code)


def e4m3(b: int) -> float:
    return lib().or_e4m3(b)


def e8m0(b: int) -> float:
    return lib().or_e8m0(b)


def bf16(h: int) -> float:
    return lib().or_bf16(h)


def silu(z: float) -> float:
    return lib().or_silu(z)


# ---- products ---------------------------------------------------------------------
def gemv(fmt, codes, scales, tensor_scale, X, rows=None, nthreads=None):
    """(Y, A) in float64, both [M][nrows]: Y = W[rows] x_m, A = sum |w x|.

    X: bf16 bit patterns (uint16 [M][d_in]) or float64 [M][d_in] (exact inputs)."""
    codes = _np(codes).astype(np.uint8, copy=False)
    scales = _np(scales)
    scales = scales.astype(np.float32 if fmt == FP8_ROW else np.uint8, copy=False)
    X = _np(X)
    if X.ndim == 1:
        X = X[None, :]
    d_out = codes.shape[0]
    d_in = codes.shape[1] * (1 if fmt == FP8_ROW else 2)
    M = X.shape[0]
    if rows is None:
        r = None
        nrows = d_out
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = r.shape[0]
    Y = np.zeros((M, nrows), np.float64)
    A = np.zeros((M, nrows), np.float64)
    nt = nthreads or _nthreads()
    if X.dtype == np.float64:
        f = lib().or_gemv_dx
    else:
        X = X.view(np.uint16)
        f = lib().or_gemv
    X = np.ascontiguousarray(X)
    rc = f(fmt, d_out, d_in, _ptr(codes), _ptr(scales), float(tensor_scale), M, _ptr(X),
           None if r is None else _ptr(r), nrows, _ptr(Y), _ptr(A), nt)
    if rc != 0:
        raise ValueError("oracle gemv: bad arguments")
    return Y, A


def dequant(fmt, codes, scales, tensor_scale=1.0) -> np.ndarray:
    codes = _np(codes).astype(np.uint8, copy=False)
    scales = _np(scales).astype(np.float32 if fmt == FP8_ROW else np.uint8, copy=False)
    d_out = codes.shape[0]
    d_in = codes.shape[1] * (1 if fmt == FP8_ROW else 2)
    W = np.zeros((d_out, d_in), np.float64)
    if lib().or_dequant(fmt, d_out, d_in, _ptr(codes), _ptr(scales), float(tensor_scale), _ptr(W)) != 0:
        raise ValueError("oracle dequant: bad arguments")
    return W


def silu_mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g = np.ascontiguousarray(g, dtype=np.float64)
    u = np.ascontiguousarray(u, dtype=np.float64)
    h = np.zeros_like(g)
    lib().or_silu_mul(g.size, _ptr(g), _ptr(u), _ptr(h))
    return h


def gate_up_silu(gate: dict, up: dict, X, rows=None, nthreads=None):
    """Fused MLP front half in FP64: returns dict(h, g, u, Ag, Au), each [M][nrows]."""
    g, Ag = gemv(gate["format"], gate["codes"], gate["scales"], gate["tensor_scale"], X, rows, nthreads)
    u, Au = gemv(up["format"], up["codes"], up["scales"], up["tensor_scale"], X, rows, nthreads)
    return {"h": silu_mul(g, u), "g": g, "u": u, "Ag": Ag, "Au": Au}


def topk_softmax(logits, k: int):
    """(ids int32 [M][k], w float64 [M][k]); descending logit, ties to lower index."""
    L = np.ascontiguousarray(_np(logits), dtype=np.float32)
    if L.ndim == 1:
        L = L[None, :]
    M, E = L.shape
    ids = np.zeros((M, k), np.int32)
    w = np.zeros((M, k), np.float64)
    if lib().or_topk_softmax(M, E, k, _ptr(L), _ptr(ids), _ptr(w)) != 0:
        raise ValueError("oracle topk: bad arguments")
    return ids, w


def moe_expert(expert: dict, x_row, h_in=None, nthreads=None):
    """One expert on one token: d = down(SiLU(gate x) * (up x)).

    expert: {"gate","up","down"} logical matrices.  x_row: bf16 bits [hidden].
    h_in: optional given intermediate (bf16 bits or float64 [d_ff]) to feed the
    down projection instead of the FP64 one (stage-wise checking).
    Returns dict(h, d, Ad, hg) with hg the gate/up result dict."""
    hg = gate_up_silu(expert["gate"], expert["up"], x_row, nthreads=nthreads)
    h = hg["h"][0] if h_in is None else h_in
    dn = expert["down"]
    d, Ad = gemv(dn["format"], dn["codes"], dn["scales"], dn["tensor_scale"], np.asarray(h)[None, :],
                 nthreads=nthreads)
    return {"h": hg["h"][0], "d": d[0], "Ad": Ad[0], "hg": hg}


def moe(get_expert, shared, X, logits, k: int, h_given=None, nthreads=None):
    """MoE layer in FP64 (article sec. 3 / sec. 4 flowchart).

    get_expert(e) -> {"gate","up","down"}; shared: same or None.
    X bf16 bits [M][hidden]; logits f32 [M][E].
    h_given: optional callable (m, slot) -> intermediate to feed down (slot k is
    the shared expert).  nthreads: host threads per product (default: all).  Returns dict(ids, w, y, tol) with tol[m] the per-output
    tolerance scale sum_j w_j A_down,j + A_down,shared."""
    X = _np(X)
    ids, w = topk_softmax(logits, k)
    M = X.shape[0]
    ys, tols = [], []
    for m in range(M):
        y = None
        tol = None
        for j in range(k):
            ex = get_expert(int(ids[m, j]))
            hin = None if h_given is None else h_given(m, j)
            r = moe_expert(ex, X[m], hin, nthreads)
            contrib = w[m, j] * r["d"]
            t = w[m, j] * r["Ad"]
            y = contrib if y is None else y + contrib
            tol = t if tol is None else tol + t
        if shared is not None:
            hin = None if h_given is None else h_given(m, k)
            r = moe_expert(shared, X[m], hin, nthreads)
            y = y + r["d"]
            tol = tol + r["Ad"]
        ys.append(y)
        tols.append(tol)
    return {"ids": ids, "w": w, "y": np.stack(ys), "tol": np.stack(tols)}
