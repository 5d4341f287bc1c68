"""The workspace contract on the GPU: every call leaves the part of its
workspace that must start zero (exchange slots, running maxima) at zero, a
leftover word there is found by fp4g_workspace_check before a call (the caller
refuses or zero-fills), and a call on the zero-filled workspace gives the same
bits as before."""
import numpy as np
import pytest
import torch

import bit_weight_gemv_fp4_amd as fg
import datagen
from gpu_common import DEV, bits, build_moe, check_product, log, make, sample_rows

pytestmark = pytest.mark.gpu

# a partial sum as a split-K deposit encodes it: low word bits(a) + 1, high word bits(b)
LEFTOVER = int(np.array([1.0], dtype=np.float32).view(np.uint32)[0]) + 1 + (0x3F800000 << 32)


def _dirty(ws, word):
    ws.view(torch.int64)[word] = LEFTOVER - (1 << 64) if LEFTOVER >= 1 << 63 else LEFTOVER


@pytest.mark.parametrize("M", [1, 4])
def test_dense_product_workspace(M):
    log("workspace dense", M)
    W, host = make(fg.NVFP4, 5120, 17408, seed=71)
    X = datagen.bf16_normal((M, 17408), datagen.tensor_seed("wsx", M), device=DEV)
    need = fg.workspace_bytes(fg.OP_GEMV, W, M)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    assert fg.workspace_check(fg.OP_GEMV, W, M, ws) == 0
    Y = fg.fp4_skinny_gemm(W, X, ws=ws)
    torch.cuda.synchronize()
    assert fg.workspace_check(fg.OP_GEMV, W, M, ws) == 0  # the call left its slots at zero
    check_product(Y, host, bits(X), rows=sample_rows(5120, 64))
    for word in (0, need // 16, need // 8 - 1):
        _dirty(ws, word)
        assert fg.workspace_check(fg.OP_GEMV, W, M, ws) == 1  # found: refuse, or zero-fill
        ws.zero_()
    Y2 = fg.fp4_skinny_gemm(W, X, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)
    assert fg.workspace_check(fg.OP_GEMV, W, M, ws) == 0


def test_greedy_pick_workspace():
    log("workspace argmax")
    W, host = make(fg.FP8_ROW, 157184, 2560, seed=72)
    X = datagen.bf16_normal((2, 2560), 73, device=DEV)
    need = fg.workspace_bytes(fg.OP_LMHEAD_ARGMAX, W, 2)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    idx, val, _ = fg.fp8_lmhead_argmax(W, X, ws=ws)
    torch.cuda.synchronize()
    assert fg.workspace_check(fg.OP_LMHEAD_ARGMAX, W, 2, ws) == 0  # the running maxima were returned to zero
    _dirty(ws, 3)
    assert fg.workspace_check(fg.OP_LMHEAD_ARGMAX, W, 2, ws) == 1
    ws.zero_()
    idx2, val2, _ = fg.fp8_lmhead_argmax(W, X, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(val, val2)


@pytest.mark.parametrize("M", [1, 4])
def test_moe_workspace(M):
    """The MoE workspace: its slots must start zero, its tables (after them) need not."""
    log("workspace moe", M)
    layer, expert, sh = build_moe(fg.MXFP4, 512, 8, 2560, 768, seed=74)
    X = datagen.bf16_normal((M, 2560), datagen.tensor_seed("wmx", M), device=DEV)
    logits = datagen.router_logits(M, 512, datagen.tensor_seed("wml", M), device=DEV)
    need = fg.workspace_bytes(fg.OP_MOE, layer, M)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    Y, ids, _ = fg.moe_route_gemv(layer, X, logits, ws=ws)
    torch.cuda.synchronize()
    assert fg.workspace_check(fg.OP_MOE, layer, M, ws) == 0
    assert bool((ws != 0).any())  # the tables stay behind, outside the checked part
    _dirty(ws, 0)
    assert fg.workspace_check(fg.OP_MOE, layer, M, ws) == 1
    ws.zero_()
    Y2, ids2, _ = fg.moe_route_gemv(layer, X, logits, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(Y, Y2)
