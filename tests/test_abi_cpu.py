"""The C ABI library loads without a GPU, exports every declared symbol, and
refuses every bad argument before any HIP call.  CPU only: no call here reaches a
kernel launch (each one fails validation first)."""
import ctypes
import re
from pathlib import Path

import pytest

import bit_weight_gemv_fp4_amd as fg
from oracle import layout

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "fp4gemv.h"

OK, E_NULL, E_SHAPE, E_ALIGN, E_FORMAT, E_WORKSPACE, E_PATH, E_ALIAS, E_HIP = range(9)
FAKE = 0x7F0000000000  # a 256-B aligned address that is never dereferenced


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == 17, names
    L = fg.lib()
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_status_strings():
    assert fg.abi_version() == 1
    for s in range(9):
        assert fg.status_string(s) and fg.status_string(s) != "unknown status"
    assert fg.status_string(99) == "unknown status"


@pytest.mark.parametrize("fmt", [fg.NVFP4, fg.MXFP4, fg.FP8_ROW])
@pytest.mark.parametrize("shape", [(1, 32), (64, 256), (70, 288), (5120, 5120), (17408, 5120), (248320, 5120)])
def test_packed_bytes_match_layout_reference(fmt, shape):
    assert fg.packed_bytes(fmt, *shape) == layout.packed_bytes(fmt, *shape)


def test_packed_bytes_bad_shapes_are_zero():
    for fmt, d_out, d_in in [(1, 0, 32), (1, 5, 16), (1, 5, 48), (4, 5, 64), (0, 5, 64)]:
        assert fg.packed_bytes(fmt, d_out, d_in) == 0


def good_desc(fmt=fg.NVFP4, d_out=128, d_in=512):
    d = fg.WeightDesc()
    d.format, d.layout_tag, d.d_out, d.d_in = fmt, fg.LAYOUT_TILE64x256, d_out, d_in
    d.packed = FAKE
    d.packed_bytes = fg.packed_bytes(fmt, d_out, d_in)
    d.tensor_scale = 1.0
    return d


def call_gemv(d, x=FAKE + (1 << 30), y=FAKE + (2 << 30), ws=None, wsb=0):
    return fg.lib().fp4_gemv(ctypes.byref(d), x, y, ws, wsb, None)


def test_gemv_error_paths():
    L = fg.lib()
    assert L.fp4_gemv(None, FAKE, FAKE, None, 0, None) == E_NULL
    d = good_desc()
    assert call_gemv(d, x=None) == E_NULL
    assert call_gemv(d, y=None) == E_NULL
    d2 = good_desc(); d2.packed = None
    assert call_gemv(d2) == E_NULL
    d2 = good_desc(); d2.layout_tag = 0
    assert call_gemv(d2) == E_FORMAT
    d2 = good_desc(fmt=fg.FP8_ROW)
    assert call_gemv(d2) == E_FORMAT          # FP8 rows are not an fp4_gemv format
    d2 = good_desc(); d2.d_in = 48
    assert call_gemv(d2) == E_SHAPE
    d2 = good_desc(); d2.d_out = 0
    assert call_gemv(d2) == E_SHAPE
    d2 = good_desc(); d2.packed_bytes -= 1
    assert call_gemv(d2) == E_SHAPE
    d2 = good_desc(); d2.packed = FAKE + 16
    assert call_gemv(d2) == E_ALIGN
    assert call_gemv(d, x=FAKE + (1 << 30) + 2) == E_ALIGN
    d2 = good_desc(); d2.tensor_scale = float("nan")
    assert call_gemv(d2) == E_FORMAT
    d2 = good_desc(fmt=fg.MXFP4); d2.tensor_scale = 2.0
    assert call_gemv(d2) == E_FORMAT
    # output overlapping the weights
    assert call_gemv(d, y=FAKE + 256) == E_ALIAS
    # a shape that needs split-K workspace
    big = good_desc(d_out=5120, d_in=5120)
    need = fg.workspace_bytes(fg.OP_GEMV, big, 1)
    assert need > 0
    assert call_gemv(big, ws=None, wsb=0) == E_NULL
    assert call_gemv(big, ws=FAKE + (3 << 30), wsb=need - 1) == E_WORKSPACE
    assert call_gemv(big, ws=FAKE + (3 << 30) + 16, wsb=need) == E_ALIGN


def test_noalloc_error_paths_before_any_hip_call():
    """The allocation-free variant validates like fp4_skinny_gemm and refuses a
    product whose workspace would exceed its fixed scratch, all on the host."""
    L = fg.lib()
    X, Y = FAKE, FAKE + (1 << 30)
    assert L.fp4_skinny_gemm_noalloc(None, X, 1, Y, 0, None) == E_NULL
    d = good_desc()
    assert L.fp4_skinny_gemm_noalloc(ctypes.byref(d), None, 1, Y, 0, None) == E_NULL
    assert L.fp4_skinny_gemm_noalloc(ctypes.byref(d), X, 0, Y, 0, None) == E_SHAPE
    assert L.fp4_skinny_gemm_noalloc(ctypes.byref(d), X, 9, Y, fg.PATH_VALU, None) == E_PATH
    big = good_desc(fg.NVFP4, 248320, 5120)
    assert fg.workspace_bytes(fg.OP_GEMV, big, 12) > fg.NOALLOC_SCRATCH_BYTES
    assert L.fp4_skinny_gemm_noalloc(ctypes.byref(big), X, 12, Y, 0, None) == E_WORKSPACE
    f8 = good_desc(fg.FP8_ROW)
    assert L.fp4_skinny_gemm_noalloc(ctypes.byref(f8), X, 1, Y, 0, None) == E_FORMAT


def test_skinny_and_lmhead_error_paths():
    L = fg.lib()
    d = good_desc()
    X, Y = FAKE + (1 << 30), FAKE + (2 << 30)
    assert L.fp4_skinny_gemm(ctypes.byref(d), X, 0, Y, 0, None, 0, None) == E_SHAPE
    assert L.fp4_skinny_gemm(ctypes.byref(d), X, 17, Y, 0, None, 0, None) == E_SHAPE
    # 9..16 vectors run on the matrix cores only
    assert L.fp4_skinny_gemm(ctypes.byref(d), X, 9, Y, fg.PATH_VALU, None, 0, None) == E_PATH
    assert L.fp4_skinny_gemm(ctypes.byref(d), X, 16, Y, fg.PATH_VALU, None, 0, None) == E_PATH
    assert L.fp4_skinny_gemm(ctypes.byref(d), X, 4, Y, 7, None, 0, None) == E_PATH
    assert L.fp4_skinny_gemm(ctypes.byref(d), X, 4, Y, -1, None, 0, None) == E_PATH
    assert L.fp4_skinny_gemm(ctypes.byref(d), X, 4, Y, fg.PATH_A8, None, 0, None) == E_PATH  # A8: MXFP4 only
    assert L.fp8_lmhead_gemv(ctypes.byref(d), X, 1, Y, None, 0, None) == E_FORMAT  # NVFP4 given
    f8 = good_desc(fmt=fg.FP8_ROW)
    assert L.fp8_lmhead_gemv(ctypes.byref(f8), X, 17, Y, None, 0, None) == E_SHAPE  # 1..16
    assert L.fp8_lmhead_gemv(ctypes.byref(f8), None, 1, Y, None, 0, None) == E_NULL


def group_desc(*members):
    G = fg.GroupDesc()
    G.n = len(members)
    for i, d in enumerate(members):
        G.w[i] = d
    return G


def call_grouped(G, M=1, x=FAKE + (1 << 30), ys=None, ws=None, wsb=0, path=0):
    if ys is None:
        ys = [FAKE + ((2 + i) << 30) for i in range(max(G.n, 1))]
    arr = (ctypes.c_void_p * len(ys))(*ys)
    return fg.lib().fp4_gemv_grouped(ctypes.byref(G), x, M, arr, path, ws, wsb, None)


def test_grouped_error_paths():
    L = fg.lib()
    q = good_desc(d_out=128); k = good_desc(d_out=64); k.packed = FAKE + (8 << 30)
    assert L.fp4_gemv_grouped(None, FAKE, 1, None, 0, None, 0, None) == E_NULL
    assert call_grouped(group_desc()) == E_SHAPE                       # n = 0
    G = group_desc(q, k); G.n = 5
    assert call_grouped(G) == E_SHAPE                                  # n > 4
    assert call_grouped(group_desc(q, k), M=17) == E_SHAPE
    assert call_grouped(group_desc(q, k), M=9, path=fg.PATH_VALU) == E_PATH
    k2 = good_desc(fg.MXFP4, d_out=64); k2.packed = FAKE + (8 << 30)
    assert call_grouped(group_desc(q, k2)) == E_FORMAT                 # mixed formats
    k3 = good_desc(d_out=64, d_in=256); k3.packed = FAKE + (8 << 30)
    assert call_grouped(group_desc(q, k3)) == E_SHAPE                  # mixed d_in
    f8 = good_desc(fg.FP8_ROW); f8b = good_desc(fg.FP8_ROW, d_out=64); f8b.packed = FAKE + (8 << 30)
    assert call_grouped(group_desc(f8, k)) == E_FORMAT                 # FP8 rows with NVFP4
    assert call_grouped(group_desc(f8, f8b), path=fg.PATH_MFMA) == E_PATH  # FP8 rows: VALU only
    assert call_grouped(group_desc(f8, f8b), M=17) == E_SHAPE
    assert call_grouped(group_desc(q, k), ys=[FAKE + (2 << 30), 0]) == E_NULL
    assert call_grouped(group_desc(q, k), ys=[FAKE + (2 << 30), FAKE + (3 << 30) + 4]) == E_ALIGN
    assert call_grouped(group_desc(q, k), ys=[FAKE + (2 << 30), FAKE + (2 << 30) + 256]) == E_ALIAS
    assert call_grouped(group_desc(q, k), ys=[FAKE + (2 << 30), FAKE + (8 << 30) + 512]) == E_ALIAS  # into k's weights
    assert fg.lib().fp4_gemv_grouped(ctypes.byref(group_desc(q, k)), FAKE, 1, None, 0, None, 0, None) == E_NULL
    assert call_grouped(group_desc(q, k), path=7) == E_PATH
    # QKV-shaped group: more row groups than any member, so split-K workspace
    qq = good_desc(d_out=5120, d_in=5120); kk = good_desc(d_out=1024, d_in=5120); kk.packed = FAKE + (8 << 30)
    G = group_desc(qq, kk)
    need = L.fp4g_workspace_bytes(fg.OP_GROUPED, ctypes.byref(G), 1)
    assert need > 0
    assert call_grouped(G) == E_NULL
    assert call_grouped(G, ws=FAKE + (12 << 30), wsb=need - 8) == E_WORKSPACE
    assert L.fp4g_workspace_bytes(fg.OP_GROUPED, ctypes.byref(group_desc(q, k2)), 1) == 0


def test_lmhead_argmax_error_paths():
    L = fg.lib()
    f8 = good_desc(fmt=fg.FP8_ROW, d_out=300, d_in=512)
    X, I, V, LG = FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30), FAKE + (4 << 30)
    need = L.fp4g_workspace_bytes(fg.OP_LMHEAD_ARGMAX, ctypes.byref(f8), 1)
    assert 0 < need <= 8192
    assert L.fp4g_workspace_bytes(fg.OP_LMHEAD_ARGMAX, ctypes.byref(f8), 16) == need
    WS = FAKE + (5 << 30)

    def call(d=f8, M=1, rb=0, n=300, lg=LG, i=I, v=V, ws=WS, wsb=need):
        return L.fp8_lmhead_argmax(ctypes.byref(d), X, M, rb, n, lg, i, v, ws, wsb, None)

    assert call(d=good_desc()) == E_FORMAT        # NVFP4 is not a head format here
    assert call(M=17) == E_SHAPE
    assert call(rb=32) == E_SHAPE                 # row_begin not a multiple of 64
    assert call(n=0) == E_SHAPE
    assert call(rb=64, n=237) == E_SHAPE          # past d_out
    assert call(i=None) == E_NULL
    assert call(v=None) == E_NULL
    assert call(ws=None) == E_NULL
    assert call(wsb=need - 1) == E_WORKSPACE
    assert call(lg=LG + 4) == E_ALIGN
    assert call(lg=FAKE + 1024) == E_ALIAS        # logits over the weights
    assert call(i=V) == E_ALIAS                   # the two outputs overlap
    assert L.fp4g_workspace_bytes(fg.OP_LMHEAD_ARGMAX, ctypes.byref(good_desc()), 1) == 0


def test_quantize_error_paths():
    L = fg.lib()
    W, C, S, T, WS = FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30), FAKE + (4 << 30)

    def q(fmt=fg.NVFP4, d_out=64, d_in=256, w=W, c=C, s=S, t=T, ws=WS, wsb=256):
        return L.fp4g_quantize(fmt, d_out, d_in, w, c, s, t, ws, wsb, None)

    assert q(fmt=4) == E_FORMAT
    assert q(w=None) == E_NULL
    assert q(c=None) == E_NULL
    assert q(d_in=48) == E_SHAPE
    assert q(d_out=0) == E_SHAPE
    assert q(w=W + 2) == E_ALIGN
    assert q(ws=None) == E_NULL                   # NVFP4 needs the scratch
    assert q(wsb=255) == E_WORKSPACE
    assert q(c=W + 1024) == E_ALIAS               # codes over the input
    assert q(s=C) == E_ALIAS                      # scales over the codes


def test_gate_up_error_paths():
    L = fg.lib()
    g, u = good_desc(), good_desc()
    X, H = FAKE + (1 << 30), FAKE + (2 << 30)
    u2 = good_desc(d_out=256)
    assert L.fp4_gate_up_silu(ctypes.byref(g), ctypes.byref(u2), X, 1, H, 0, None, 0, None) == E_SHAPE
    u3 = good_desc(fmt=fg.MXFP4)
    assert L.fp4_gate_up_silu(ctypes.byref(g), ctypes.byref(u3), X, 1, H, 0, None, 0, None) == E_FORMAT
    assert L.fp4_gate_up_silu(ctypes.byref(g), ctypes.byref(u), X, 1, H, fg.PATH_A8, None, 0, None) == E_PATH  # A8: MXFP4 only
    assert L.fp4_gate_up_silu(ctypes.byref(g), ctypes.byref(u), X, 17, H, 0, None, 0, None) == E_SHAPE
    assert L.fp4_gate_up_silu(ctypes.byref(g), ctypes.byref(u), X, 9, H, fg.PATH_VALU, None, 0, None) == E_PATH
    # FP8 row pairs (a mixed layout's FP8 MLPs): VALU only, up to 8 vectors, one format per pair
    g8, u8 = good_desc(fg.FP8_ROW), good_desc(fg.FP8_ROW); u8.packed = FAKE + (8 << 30)
    assert L.fp4_gate_up_silu(ctypes.byref(g8), ctypes.byref(u), X, 1, H, 0, None, 0, None) == E_FORMAT
    assert L.fp4_gate_up_silu(ctypes.byref(g8), ctypes.byref(u8), X, 1, H, fg.PATH_MFMA, None, 0, None) == E_PATH
    assert L.fp4_gate_up_silu(ctypes.byref(g8), ctypes.byref(u8), X, 1, H, fg.PATH_A8, None, 0, None) == E_PATH
    assert L.fp4_gate_up_silu(ctypes.byref(g8), ctypes.byref(u8), X, 9, H, 0, None, 0, None) == E_SHAPE
    big8 = good_desc(fg.FP8_ROW, 17408, 5120)
    assert fg.workspace_bytes(fg.OP_GATE_UP, big8, 8) > 0 and fg.workspace_bytes(fg.OP_GATE_UP, big8, 9) == 0
    assert L.fp4_gate_up_silu(ctypes.byref(g), ctypes.byref(u), X, 1, None, 0, None, 0, None) == E_NULL
    assert L.fp4_gate_up_silu(ctypes.byref(g), ctypes.byref(u), X, 1, X, 0, None, 0, None) == E_ALIAS


def moe_desc(E=16, k=4, hidden=256, dff=128, shared=True):
    m = fg.MoeDesc()
    m.num_experts, m.top_k, m.hidden, m.d_ff = E, k, hidden, dff
    pg = fg.packed_bytes(fg.MXFP4, dff, hidden)
    pd = fg.packed_bytes(fg.MXFP4, hidden, dff)
    for name, (o, i, base, p) in {"gate": (dff, hidden, 0, pg), "up": (dff, hidden, 1, pg),
                                  "down": (hidden, dff, 2, pd)}.items():
        d = good_desc(fg.MXFP4, o, i)
        d.packed = FAKE + (base << 32)
        d.packed_bytes = p * E
        setattr(m, name, d)
    m.stride_gate = m.stride_up = pg
    m.stride_down = pd
    if shared:
        m.has_shared = 1
        m.sh_gate = good_desc(fg.MXFP4, dff, hidden); m.sh_gate.packed = FAKE + (3 << 32)
        m.sh_up = good_desc(fg.MXFP4, dff, hidden); m.sh_up.packed = FAKE + (4 << 32)
        m.sh_down = good_desc(fg.MXFP4, hidden, dff); m.sh_down.packed = FAKE + (5 << 32)
    return m


def call_moe(m, M=1, ws=FAKE + (9 << 32), wsb=None, **kw):
    if wsb is None:
        wsb = fg.workspace_bytes(fg.OP_MOE, m, M)
    a = dict(X=FAKE + (6 << 32), logits=FAKE + (7 << 32), Y=FAKE + (8 << 32), ids=FAKE + (10 << 32),
             w=FAKE + (11 << 32), H=None)
    a.update(kw)
    return fg.lib().moe_route_gemv(ctypes.byref(m), a["X"], a["logits"], M, a["Y"], a["ids"], a["w"], a["H"], ws,
                                   wsb, None)


def test_moe_error_paths():
    m = moe_desc()
    assert fg.workspace_bytes(fg.OP_MOE, m, 1) > 0
    assert fg.workspace_bytes(fg.OP_MOE, m, 16) > 0 and fg.workspace_bytes(fg.OP_MOE, m, 17) == 0
    assert call_moe(m, M=0) == E_SHAPE
    assert call_moe(m, M=17) == E_SHAPE
    m2 = moe_desc(); m2.top_k = 9
    assert call_moe(m2, wsb=1 << 30) == E_SHAPE
    m2 = moe_desc(); m2.top_k = 17; m2.num_experts = 16
    assert call_moe(m2, wsb=1 << 30) == E_SHAPE
    m2 = moe_desc(); m2.down.d_out = 128
    assert call_moe(m2, wsb=1 << 30) == E_SHAPE
    m2 = moe_desc(); m2.up.format = fg.NVFP4
    assert call_moe(m2, wsb=1 << 30) == E_FORMAT
    m2 = moe_desc(); m2.gate.packed_bytes -= 1
    assert call_moe(m2, wsb=1 << 30) == E_SHAPE
    m2 = moe_desc(); m2.stride_up += 16
    assert call_moe(m2, wsb=1 << 30) in (E_ALIGN, E_SHAPE)
    assert call_moe(m, ws=None) == E_NULL
    m2 = moe_desc(); m2.act = 2                                   # unknown activation format
    assert call_moe(m2, wsb=1 << 30) == E_PATH
    assert fg.workspace_bytes(fg.OP_MOE, m2, 1) == 0
    m2 = moe_desc(); m2.act = fg.ACT_MXFP8                        # W4A8 takes the same workspace
    assert fg.workspace_bytes(fg.OP_MOE, m2, 4) == fg.workspace_bytes(fg.OP_MOE, moe_desc(), 4)
    assert call_moe(m, wsb=fg.workspace_bytes(fg.OP_MOE, m, 1) - 1) == E_WORKSPACE
    assert call_moe(m, Y=FAKE + (6 << 32)) == E_ALIAS          # output on top of X
    assert call_moe(m, ids=FAKE + (8 << 32)) == E_ALIAS        # two outputs overlap
    assert call_moe(m, logits=FAKE + (7 << 32) + 4) == E_ALIGN


def test_moe_workspace_does_not_depend_on_m():
    """MoE tables sit after the exchange slots at an M-independent offset, so calls
    of any M on one layer shape can share a workspace."""
    m = moe_desc()
    sizes = {fg.lib().fp4g_workspace_bytes(fg.OP_MOE, ctypes.byref(m), M) for M in range(1, 9)}
    assert len(sizes) == 1 and sizes.pop() > 0


def test_pack_error_paths():
    L = fg.lib()
    out = fg.WeightDesc()
    C, S, P = FAKE, FAKE + (1 << 30), FAKE + (2 << 30)
    nb = fg.packed_bytes(fg.NVFP4, 64, 256)
    assert L.fp4g_pack(fg.NVFP4, 64, 256, None, S, 1.0, P, nb, ctypes.byref(out), None) == E_NULL
    assert L.fp4g_pack(9, 64, 256, C, S, 1.0, P, nb, ctypes.byref(out), None) == E_FORMAT
    assert L.fp4g_pack(fg.NVFP4, 64, 250, C, S, 1.0, P, nb, ctypes.byref(out), None) == E_SHAPE
    assert L.fp4g_pack(fg.NVFP4, 64, 256, C, S, 1.0, P, nb - 1, ctypes.byref(out), None) == E_SHAPE
    assert L.fp4g_pack(fg.NVFP4, 64, 256, C, S, 1.0, P + 16, nb, ctypes.byref(out), None) == E_ALIGN
    assert L.fp4g_pack(fg.NVFP4, 64, 256, C, S, float("inf"), P, nb, ctypes.byref(out), None) == E_FORMAT
    nb8 = fg.packed_bytes(fg.FP8_ROW, 64, 256)
    assert L.fp4g_pack(fg.FP8_ROW, 64, 256, C, S, 2.0, P, nb8, ctypes.byref(out), None) == E_FORMAT
    assert L.fp4g_pack(fg.NVFP4, 64, 256, C, S, 1.0, C + 256, nb, ctypes.byref(out), None) == E_ALIAS
    d = good_desc(); d.layout_tag = 3
    assert L.fp4g_unpack(ctypes.byref(d), C, S, None) == E_FORMAT
    assert L.fp4g_validate(ctypes.byref(d), FAKE, None) == E_FORMAT
    assert L.fp4g_validate(ctypes.byref(good_desc()), None, None) == E_NULL


def test_workspace_queries():
    assert fg.workspace_bytes(fg.OP_GEMV, good_desc(d_out=64, d_in=256), 1) == 0  # one row group, one chunk
    assert fg.workspace_bytes(99, good_desc(), 1) == 0
    assert fg.workspace_bytes(fg.OP_GEMV, good_desc(), 0) == 0
    # up to 16 vectors for the NVFP4/MXFP4 products, 8 for the FP8 head and MoE
    big = good_desc(d_out=5120, d_in=17408)
    assert fg.workspace_bytes(fg.OP_GEMV, big, 16) > 0
    assert fg.workspace_bytes(fg.OP_GATE_UP, good_desc(d_out=17408, d_in=5120), 16) > 0
    assert fg.workspace_bytes(fg.OP_GEMV, big, 17) == 0
    assert fg.workspace_bytes(fg.OP_LMHEAD, good_desc(fg.FP8_ROW, 5120, 17408), 8) > 0
    assert fg.workspace_bytes(fg.OP_LMHEAD, good_desc(fg.FP8_ROW, 5120, 17408), 16) > 0  # FP8 rows: up to 16
    assert fg.workspace_bytes(fg.OP_LMHEAD, good_desc(fg.FP8_ROW, 5120, 17408), 17) == 0
    assert fg.workspace_bytes(fg.OP_GATE_UP, good_desc(fg.FP8_ROW, 5120, 17408), 9) == 0  # FP8 pairs: up to 8
    assert fg.workspace_bytes(fg.OP_MOE, moe_desc(), 16) > 0 and fg.workspace_bytes(fg.OP_MOE, moe_desc(), 17) == 0
    assert fg.MAX_M == 8 and fg.MAX_M_WIDE == 16
    bad = good_desc(); bad.layout_tag = 0
    assert fg.workspace_bytes(fg.OP_GEMV, bad, 1) == 0


def test_workspace_check_error_paths():
    """The workspace check refuses bad arguments before touching the device."""
    L = fg.lib()
    d = good_desc(fg.NVFP4, 5120, 17408)
    need = L.fp4g_workspace_bytes(fg.OP_GEMV, ctypes.byref(d), 1)
    assert need > 0
    n = ctypes.c_uint64(7)
    assert L.fp4g_workspace_check(fg.OP_GEMV, None, 1, FAKE, need, ctypes.byref(n), None) == E_NULL
    assert L.fp4g_workspace_check(fg.OP_GEMV, ctypes.byref(d), 1, None, need, ctypes.byref(n), None) == E_NULL
    assert L.fp4g_workspace_check(fg.OP_GEMV, ctypes.byref(d), 1, FAKE, need, None, None) == E_NULL
    assert L.fp4g_workspace_check(fg.OP_GEMV, ctypes.byref(d), 1, FAKE, need - 8, ctypes.byref(n), None) == E_WORKSPACE
    assert L.fp4g_workspace_check(fg.OP_GEMV, ctypes.byref(d), 1, FAKE + 16, need, ctypes.byref(n), None) == E_ALIGN
    small = good_desc(fg.NVFP4, 64, 256)  # one tile column: no split-K, no workspace
    assert L.fp4g_workspace_bytes(fg.OP_GEMV, ctypes.byref(small), 1) == 0
    assert L.fp4g_workspace_check(fg.OP_GEMV, ctypes.byref(small), 1, FAKE, 256, ctypes.byref(n), None) == E_SHAPE
    assert L.fp4g_workspace_check(fg.OP_MOE, ctypes.byref(moe_desc()), 17, FAKE, 1 << 30, ctypes.byref(n),
                                  None) == E_SHAPE
    assert n.value == 7  # untouched


def test_moe_layer_timing_program_rejects_bad_arguments():
    """The MoE layer timing program (built with the library) links against it and
    refuses out-of-range arguments before touching a GPU."""
    import subprocess

    exe = Path(fg.__file__).resolve().parent / "moe_layer_timing"
    if not exe.exists():
        pytest.skip("timing program not built")
    for args in (["0"], ["17"], ["1", "0"], ["1", "65"], ["1", "4", "0"]):
        r = subprocess.run([str(exe), *args], capture_output=True, text=True, timeout=60)
        assert r.returncode == 2, (args, r.returncode, r.stderr)
        assert "usage" in r.stderr
