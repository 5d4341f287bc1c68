"""Python binding of libfp4gemv.so: decode GEMV over NVFP4 / MXFP4 / FP8 weights on
MI355X (gfx950).

Argument marshalling only: every step of every product runs in the HIP kernels
of the shared library (include/fp4gemv.h).  PyTorch provides device memory and
the current stream.  The names follow the C ABI.  Importing this package fails
loudly when the library has not been built; there is no fallback path.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass, field
from pathlib import Path

import torch

__all__ = [
    "NVFP4", "MXFP4", "FP8_ROW", "PATH_AUTO", "PATH_VALU", "PATH_MFMA", "PATH_A8",
    "ACT_BF16", "ACT_MXFP8", "OP_GEMV", "OP_GATE_UP", "OP_MOE", "OP_LMHEAD", "OP_GROUPED", "OP_LMHEAD_ARGMAX", "MAX_GROUP", "MAX_M", "MAX_M_WIDE", "Fp4gError", "PackedWeight", "MoeLayer",
    "lib", "abi_version", "status_string", "packed_bytes", "workspace_bytes", "pack", "unpack",
    "validate", "quantize", "fp4_gemv", "fp4_skinny_gemm", "fp4_skinny_gemm_noalloc", "NOALLOC_SCRATCH_BYTES", "fp4_gemv_grouped", "Group", "fp4_gate_up_silu", "moe_route_gemv",
    "fp8_lmhead_gemv", "fp8_lmhead_argmax", "LIB_PATH"
]

NVFP4, MXFP4, FP8_ROW = 1, 2, 3
PATH_AUTO, PATH_VALU, PATH_MFMA, PATH_A8 = 0, 1, 2, 3
OP_GEMV, OP_GATE_UP, OP_MOE, OP_LMHEAD, OP_GROUPED, OP_LMHEAD_ARGMAX = 1, 2, 3, 4, 5, 6
MAX_GROUP = 4
MAX_M, MAX_M_WIDE = 8, 16  # vectors per call; the wider range on the matrix-core path only
LAYOUT_TILE64x256 = 0x46344731

LIB_PATH = Path(__file__).resolve().parent / "libfp4gemv.so"


class WeightDesc(ctypes.Structure):
    _fields_ = [
        ("format", ctypes.c_uint32),
        ("layout_tag", ctypes.c_uint32),
        ("d_out", ctypes.c_int32),
        ("d_in", ctypes.c_int32),
        ("packed", ctypes.c_void_p),
        ("packed_bytes", ctypes.c_uint64),
        ("tensor_scale", ctypes.c_float),
        ("reserved", ctypes.c_uint32),
    ]


class GroupDesc(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("reserved", ctypes.c_int32), ("w", WeightDesc * MAX_GROUP)]


class MoeDesc(ctypes.Structure):
    _fields_ = [
        ("num_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("d_ff", ctypes.c_int32),
        ("gate", WeightDesc),
        ("up", WeightDesc),
        ("down", WeightDesc),
        ("stride_gate", ctypes.c_uint64),
        ("stride_up", ctypes.c_uint64),
        ("stride_down", ctypes.c_uint64),
        ("has_shared", ctypes.c_int32),
        ("act", ctypes.c_int32),
        ("sh_gate", WeightDesc),
        ("sh_up", WeightDesc),
        ("sh_down", WeightDesc),
    ]


_VP, _I32, _U32, _U64, _F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_float
_SIGNATURES = {
    "fp4g_abi_version": (_U32, []),
    "fp4g_status_string": (ctypes.c_char_p, [_I32]),
    "fp4g_packed_bytes": (_U64, [_U32, _I32, _I32]),
    "fp4g_pack": (_I32, [_U32, _I32, _I32, _VP, _VP, _F, _VP, _U64, ctypes.POINTER(WeightDesc), _VP]),
    "fp4g_unpack": (_I32, [ctypes.POINTER(WeightDesc), _VP, _VP, _VP]),
    "fp4g_quantize": (_I32, [_U32, _I32, _I32, _VP, _VP, _VP, _VP, _VP, _U64, _VP]),
    "fp4g_validate": (_I32, [ctypes.POINTER(WeightDesc), _VP, _VP]),
    "fp4g_workspace_bytes": (_U64, [_I32, _VP, _I32]),
    "fp4g_workspace_check": (_I32, [_I32, _VP, _I32, _VP, _U64, ctypes.POINTER(_U64), _VP]),
    "fp4_gemv": (_I32, [ctypes.POINTER(WeightDesc), _VP, _VP, _VP, _U64, _VP]),
    "fp4_skinny_gemm": (_I32, [ctypes.POINTER(WeightDesc), _VP, _I32, _VP, _I32, _VP, _U64, _VP]),
    "fp4_skinny_gemm_noalloc": (_I32, [ctypes.POINTER(WeightDesc), _VP, _I32, _VP, _I32, _VP]),
    "fp4_gemv_grouped": (_I32, [ctypes.POINTER(GroupDesc), _VP, _I32, ctypes.POINTER(_VP), _I32, _VP, _U64, _VP]),
    "fp4_gate_up_silu": (_I32, [ctypes.POINTER(WeightDesc), ctypes.POINTER(WeightDesc), _VP, _I32, _VP, _I32,
                                _VP, _U64, _VP]),
    "moe_route_gemv": (_I32, [ctypes.POINTER(MoeDesc), _VP, _VP, _I32, _VP, _VP, _VP, _VP, _VP, _U64, _VP]),
    "fp8_lmhead_gemv": (_I32, [ctypes.POINTER(WeightDesc), _VP, _I32, _VP, _VP, _U64, _VP]),
    "fp8_lmhead_argmax": (_I32, [ctypes.POINTER(WeightDesc), _VP, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _U64, _VP]),
}

_lib = None


def lib():
    """The loaded shared library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise ImportError(f"{LIB_PATH} is missing: build it with bit_weight_gemv_fp4_amd.build.build()")
        L = ctypes.CDLL(str(LIB_PATH))
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class Fp4gError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def _check(status: int, where: str):
    if status != 0:
        raise Fp4gError(status, where)


def abi_version() -> int:
    return lib().fp4g_abi_version()


def status_string(status: int) -> str:
    return lib().fp4g_status_string(status).decode()


def packed_bytes(fmt: int, d_out: int, d_in: int) -> int:
    return lib().fp4g_packed_bytes(fmt, d_out, d_in)


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


@dataclass
class PackedWeight:
    """A packed matrix: the C descriptor plus the device buffer it points into."""
    desc: WeightDesc
    buf: torch.Tensor
    keep: list = field(default_factory=list)

    @property
    def format(self) -> int:
        return self.desc.format

    @property
    def d_out(self) -> int:
        return self.desc.d_out

    @property
    def d_in(self) -> int:
        return self.desc.d_in

    @property
    def nbytes(self) -> int:
        return packed_bytes(self.format, self.d_out, self.d_in)

    def view(self, offset: int, d_out: int | None = None, d_in: int | None = None) -> "PackedWeight":
        """Descriptor of a matrix stored at byte `offset` inside the same buffer."""
        d = WeightDesc()
        ctypes.pointer(d)[0] = self.desc
        d.packed = self.desc.packed + offset
        d.packed_bytes = self.desc.packed_bytes - offset
        if d_out is not None:
            d.d_out = d_out
        if d_in is not None:
            d.d_in = d_in
        return PackedWeight(d, self.buf, self.keep)


def pack(fmt: int, codes: torch.Tensor, scales: torch.Tensor, tensor_scale: float = 1.0,
         out: torch.Tensor | None = None, offset: int = 0, stream=None) -> PackedWeight:
    """Pack logical (codes, scales) device tensors into the tiled layout.

    codes: uint8 [d_out, d_in/2] (FP4) or [d_out, d_in] (FP8); scales: uint8
    [d_out, d_in/16] (NVFP4), [d_out, d_in/32] (MXFP4) or float32 [d_out] (FP8).
    out/offset: pack into an existing uint8 device buffer at a byte offset."""
    assert codes.is_contiguous() and scales.is_contiguous()
    d_out = codes.shape[0]
    d_in = codes.shape[1] * (1 if fmt == FP8_ROW else 2)
    nb = packed_bytes(fmt, d_out, d_in)
    if nb == 0:
        raise Fp4gError(2, "pack")
    if out is None:
        out = torch.empty(nb, dtype=torch.uint8, device=codes.device)
        offset = 0
    desc = WeightDesc()
    _check(lib().fp4g_pack(fmt, d_out, d_in, _ptr(codes), _ptr(scales), float(tensor_scale),
                           out.data_ptr() + offset, out.numel() - offset, ctypes.byref(desc), _stream(stream)),
           "fp4g_pack")
    return PackedWeight(desc, out)


def quantize(fmt: int, w: torch.Tensor, stream=None):
    """Quantise a bf16 matrix [d_out, d_in] on the device: returns (codes, scales,
    tensor_scale) in the logical layout `pack` takes."""
    assert w.dtype == torch.bfloat16 and w.dim() == 2 and w.is_contiguous()
    d_out, d_in = w.shape
    dev = w.device
    if fmt == FP8_ROW:
        codes = torch.empty((d_out, d_in), dtype=torch.uint8, device=dev)
        scales = torch.empty(d_out, dtype=torch.float32, device=dev)
    else:
        codes = torch.empty((d_out, d_in // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((d_out, d_in // (16 if fmt == NVFP4 else 32)), dtype=torch.uint8, device=dev)
    ts = torch.empty(1, dtype=torch.float32, device=dev)
    scratch = torch.empty(256, dtype=torch.uint8, device=dev)
    _check(lib().fp4g_quantize(fmt, d_out, d_in, w.data_ptr(), codes.data_ptr(), scales.data_ptr(), ts.data_ptr(),
                               scratch.data_ptr(), 256, _stream(stream)), "fp4g_quantize")
    return codes, scales, float(ts.item())


def unpack(W: PackedWeight, stream=None):
    fmt = W.format
    dev = W.buf.device
    if fmt == FP8_ROW:
        codes = torch.empty((W.d_out, W.d_in), dtype=torch.uint8, device=dev)
        scales = torch.empty((W.d_out,), dtype=torch.float32, device=dev)
    else:
        codes = torch.empty((W.d_out, W.d_in // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((W.d_out, W.d_in // (16 if fmt == NVFP4 else 32)), dtype=torch.uint8, device=dev)
    _check(lib().fp4g_unpack(ctypes.byref(W.desc), codes.data_ptr(), scales.data_ptr(), _stream(stream)),
           "fp4g_unpack")
    return codes, scales


def validate(W: PackedWeight, stream=None) -> int:
    """Number of NaN scale codes (FP8: NaN element codes + non-finite row scales).
    Synchronises the stream."""
    bad = torch.empty(1, dtype=torch.int64, device=W.buf.device)
    _check(lib().fp4g_validate(ctypes.byref(W.desc), bad.data_ptr(), _stream(stream)), "fp4g_validate")
    return int(bad.item())


def workspace_bytes(op: int, desc, M: int) -> int:
    d = desc.desc if isinstance(desc, (PackedWeight, MoeLayer, Group)) else desc
    return lib().fp4g_workspace_bytes(op, ctypes.addressof(d), M)


def workspace_check(op: int, desc, M: int, ws: torch.Tensor, stream=None) -> int:
    """Non-zero 8-byte words in the part of `ws` the call (op, desc, M) needs
    zero-filled (0: the workspace may be used).  Synchronises the stream."""
    d = desc.desc if isinstance(desc, (PackedWeight, MoeLayer, Group)) else desc
    n = ctypes.c_uint64(0)
    _check(lib().fp4g_workspace_check(op, ctypes.addressof(d), M, ws.data_ptr(), ws.numel() * ws.element_size(),
                                      ctypes.byref(n), _stream(stream)), "fp4g_workspace_check")
    return int(n.value)


_ws_cache: dict = {}


def _workspace(op, desc, M, device, ws):
    """A zero-filled workspace of the size the call needs.  The library leaves its
    exchange slots at zero after every call, so a per-device buffer is reused by
    all products; MoE layers get one per layer shape (they keep tables there too).
    Calls that share a workspace must be ordered on one stream (pass `ws`
    otherwise)."""
    need = workspace_bytes(op, desc, M)
    if ws is not None:
        return ws, need
    if need == 0:
        return None, 0
    dev = torch.device(device)
    if dev.type == "cuda" and dev.index is None:  # "cuda" and "cuda:0" name one buffer
        dev = torch.device("cuda", torch.cuda.current_device())
    key = dev
    if op == OP_MOE:
        # MoE keeps tables after its slots: one workspace per layer shape
        d = desc.desc
        key = (dev, "moe", d.num_experts, d.top_k, d.hidden, d.d_ff, d.has_shared, d.gate.format)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < need:
        buf = torch.zeros(max(need, 1 << 20), dtype=torch.uint8, device=dev)
        _ws_cache[key] = buf
    return buf, need


def _bits(t: torch.Tensor) -> int:
    assert t.dtype == torch.bfloat16 and t.is_contiguous()
    return t.data_ptr()


def fp4_gemv(W: PackedWeight, x: torch.Tensor, y: torch.Tensor | None = None, ws=None, stream=None) -> torch.Tensor:
    """y = W x for one bf16 vector x [d_in]; returns float32 [d_out]."""
    if y is None:
        y = torch.empty(W.d_out, dtype=torch.float32, device=x.device)
    wsb, need = _workspace(OP_GEMV, W, 1, x.device, ws)
    _check(lib().fp4_gemv(ctypes.byref(W.desc), _bits(x), y.data_ptr(), _ptr(wsb),
                          wsb.numel() if wsb is not None else 0, _stream(stream)), "fp4_gemv")
    return y


def fp4_skinny_gemm(W: PackedWeight, X: torch.Tensor, Y: torch.Tensor | None = None, path: int = PATH_AUTO,
                    ws=None, stream=None) -> torch.Tensor:
    """Y[m] = W X[m] for X bf16 [M, d_in], M in 1..16 (above 8 on the matrix-core path);
    returns float32 [M, d_out]."""
    M = X.shape[0]
    if Y is None:
        Y = torch.empty((M, W.d_out), dtype=torch.float32, device=X.device)
    wsb, need = _workspace(OP_GEMV, W, M, X.device, ws)
    _check(lib().fp4_skinny_gemm(ctypes.byref(W.desc), _bits(X), M, Y.data_ptr(), path, _ptr(wsb),
                                 wsb.numel() if wsb is not None else 0, _stream(stream)), "fp4_skinny_gemm")
    return Y


NOALLOC_SCRATCH_BYTES = 16 << 20


def fp4_skinny_gemm_noalloc(W: PackedWeight, X: torch.Tensor, Y: torch.Tensor, path: int = PATH_AUTO,
                            stream=None) -> torch.Tensor:
    """fp4_skinny_gemm with the library's fixed scratch array as its workspace: no
    device memory is allocated (Y must be given).  Calls on one GPU must be
    ordered with each other."""
    _check(lib().fp4_skinny_gemm_noalloc(ctypes.byref(W.desc), _bits(X), X.shape[0], Y.data_ptr(), path,
                                         _stream(stream)), "fp4_skinny_gemm_noalloc")
    return Y


class Group:
    """Matrices of one format and d_in that multiply the same input."""

    def __init__(self, members):
        members = list(members)
        if not 1 <= len(members) <= MAX_GROUP:
            raise ValueError(f"a group holds 1..{MAX_GROUP} matrices")
        self.members = members  # keeps the buffers alive
        self.desc = GroupDesc()
        self.desc.n = len(members)
        for i, W in enumerate(members):
            self.desc.w[i] = W.desc


def fp4_gemv_grouped(G: Group, X: torch.Tensor, Ys=None, path: int = PATH_AUTO, ws=None, stream=None):
    """Ys[i][m] = W_i X[m] for every member W_i of G (NVFP4/MXFP4, or FP8 rows),
    X bf16 [M, d_in] (or [d_in]); returns the list of float32 [M, d_out_i] outputs."""
    X2 = X if X.dim() == 2 else X.view(1, -1)
    M = X2.shape[0]
    if Ys is None:
        Ys = [torch.empty((M, W.d_out), dtype=torch.float32, device=X.device) for W in G.members]
    ptrs = (_VP * len(Ys))(*[y.data_ptr() for y in Ys])
    wsb, need = _workspace(OP_GROUPED, G, M, X.device, ws)
    _check(lib().fp4_gemv_grouped(ctypes.byref(G.desc), _bits(X2), M, ptrs, path, _ptr(wsb),
                                  wsb.numel() if wsb is not None else 0, _stream(stream)), "fp4_gemv_grouped")
    return Ys


def fp4_gate_up_silu(Wg: PackedWeight, Wu: PackedWeight, X: torch.Tensor, H: torch.Tensor | None = None,
                     path: int = PATH_AUTO, ws=None, stream=None) -> torch.Tensor:
    """H = bf16(SiLU(Wg X) * (Wu X)) for X bf16 [M, d_in] (an NVFP4/MXFP4 pair, or
    an FP8 row-scaled pair); returns bf16 [M, d_out].  PATH_A8 (MXFP4 pairs):
    both products take X quantised to MXFP8."""
    X2 = X if X.dim() == 2 else X.view(1, -1)
    M = X2.shape[0]
    if H is None:
        H = torch.empty((M, Wg.d_out), dtype=torch.bfloat16, device=X.device)
    wsb, need = _workspace(OP_GATE_UP, Wg, M, X.device, ws)
    _check(lib().fp4_gate_up_silu(ctypes.byref(Wg.desc), ctypes.byref(Wu.desc), _bits(X2), M, H.data_ptr(), path,
                                  _ptr(wsb), wsb.numel() if wsb is not None else 0, _stream(stream)),
           "fp4_gate_up_silu")
    return H if X.dim() == 2 else H.view(-1)


def fp8_lmhead_gemv(W: PackedWeight, X: torch.Tensor, logits: torch.Tensor | None = None, ws=None,
                    stream=None) -> torch.Tensor:
    """logits[m] = s_row * (E4M3 W) X[m] for X bf16 [M, d_in] (or [d_in])."""
    X2 = X if X.dim() == 2 else X.view(1, -1)
    M = X2.shape[0]
    if logits is None:
        logits = torch.empty((M, W.d_out), dtype=torch.float32, device=X.device)
    wsb, need = _workspace(OP_LMHEAD, W, M, X.device, ws)
    _check(lib().fp8_lmhead_gemv(ctypes.byref(W.desc), _bits(X2), M, logits.data_ptr(), _ptr(wsb),
                                 wsb.numel() if wsb is not None else 0, _stream(stream)), "fp8_lmhead_gemv")
    return logits if X.dim() == 2 else logits.view(-1)


def fp8_lmhead_argmax(W: PackedWeight, X: torch.Tensor, row_begin: int = 0, n_rows: int | None = None,
                      logits: bool = False, ws=None, stream=None):
    """Greedy pick over rows [row_begin, row_begin + n_rows) of an FP8 head for X
    bf16 [M, d_in] (or [d_in]): returns (row int32 [M], logit float32 [M],
    logits float32 [M, n_rows] or None)."""
    X2 = X if X.dim() == 2 else X.view(1, -1)
    M = X2.shape[0]
    n = W.d_out - row_begin if n_rows is None else n_rows
    L = torch.empty((M, n), dtype=torch.float32, device=X.device) if logits else None
    idx = torch.empty(M, dtype=torch.int32, device=X.device)
    val = torch.empty(M, dtype=torch.float32, device=X.device)
    wsb, need = _workspace(OP_LMHEAD_ARGMAX, W, M, X.device, ws)
    _check(lib().fp8_lmhead_argmax(ctypes.byref(W.desc), _bits(X2), M, row_begin, n, _ptr(L), idx.data_ptr(),
                                   val.data_ptr(), _ptr(wsb), wsb.numel() if wsb is not None else 0,
                                   _stream(stream)), "fp8_lmhead_argmax")
    return idx, val, L


@dataclass
class MoeLayer:
    """One MoE layer: routed experts stored back to back in three buffers."""
    desc: MoeDesc
    keep: list = field(default_factory=list)


ACT_BF16, ACT_MXFP8 = 0, 1


def moe_layer(gate: PackedWeight, up: PackedWeight, down: PackedWeight, num_experts: int, top_k: int,
              stride_gate: int, stride_up: int, stride_down: int, shared: tuple | None = None,
              act: int = ACT_BF16) -> MoeLayer:
    """Describe a layer whose expert e is at gate/up/down + e * stride (bytes);
    `gate`, `up`, `down` describe expert 0 and span all experts' bytes.  act:
    ACT_BF16, or ACT_MXFP8 (W4A8: MXFP8 activations, MXFP4 experts)."""
    d = MoeDesc()
    d.act = act
    d.num_experts, d.top_k = num_experts, top_k
    d.hidden, d.d_ff = gate.d_in, gate.d_out
    d.gate, d.up, d.down = gate.desc, up.desc, down.desc
    d.stride_gate, d.stride_up, d.stride_down = stride_gate, stride_up, stride_down
    keep = [gate, up, down]
    if shared is not None:
        d.has_shared = 1
        d.sh_gate, d.sh_up, d.sh_down = shared[0].desc, shared[1].desc, shared[2].desc
        keep += list(shared)
    return MoeLayer(d, keep)


def moe_route_gemv(layer: MoeLayer, X: torch.Tensor, logits: torch.Tensor, Y: torch.Tensor | None = None,
                   topk_ids: torch.Tensor | None = None, topk_w: torch.Tensor | None = None,
                   H: torch.Tensor | None = None, ws=None, stream=None):
    """One MoE layer for X bf16 [M, hidden] and router logits float32 [M, E].
    Returns (Y float32 [M, hidden], topk_ids int32 [M, k], topk_w float32 [M, k])."""
    d = layer.desc
    M = X.shape[0]
    dev = X.device
    if Y is None:
        Y = torch.empty((M, d.hidden), dtype=torch.float32, device=dev)
    if topk_ids is None:
        topk_ids = torch.empty((M, d.top_k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((M, d.top_k), dtype=torch.float32, device=dev)
    wsb, need = _workspace(OP_MOE, layer, M, dev, ws)
    assert logits.dtype == torch.float32 and logits.is_contiguous()
    _check(lib().moe_route_gemv(ctypes.byref(d), _bits(X), logits.data_ptr(), M, Y.data_ptr(), topk_ids.data_ptr(),
                                topk_w.data_ptr(), _ptr(H), _ptr(wsb), wsb.numel() if wsb is not None else 0,
                                _stream(stream)), "moe_route_gemv")
    return Y, topk_ids, topk_w
