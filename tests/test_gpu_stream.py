"""GPU parity of the one-launch decode stream (fp4g_stream_build / fp4_stream_run)
against the FP64 oracle, op by op.  Needs gfx950."""
import sys

import numpy as np
import pytest
import torch

import bit_weight_gemv_fp4_amd as fg
import datagen
import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 2e-3


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def make(fmt, d_out, d_in, seed):
    m = datagen.matrix(fmt, d_out, d_in, datagen.tensor_seed("stream", fmt, d_out, d_in, seed), device=DEV)
    W = fg.pack(fmt, m["codes"], m["scales"], m["tensor_scale"])
    return W, {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in m.items()}


def check_y(y, host, Xb, rows=None):
    Y, A = oracle.gemv(host["format"], host["codes"], host["scales"], host["tensor_scale"], Xb, rows=rows)
    g = y.detach().float().cpu().double().numpy().reshape(Y.shape[0], -1)
    if rows is not None:
        g = g[:, rows]
    bad = np.abs(g - Y) > TOL * A
    assert not bad.any(), f"{bad.sum()} outputs out of bound"


def check_h(H, gate, up, Xb, rows=None):
    r = oracle.gate_up_silu(gate, up, Xb, rows=rows)
    h = H.detach().float().cpu().double().numpy().reshape(r["h"].shape[0], -1)
    if rows is not None:
        h = h[:, rows]
    tg, tu = TOL * r["Ag"], TOL * r["Au"]
    sg = r["g"] / (1 + np.exp(-r["g"]))
    bound = 1.1 * tg * (np.abs(r["u"]) + tu) + np.abs(sg) * tu + 2.0 ** -8 * np.abs(r["h"])
    assert np.all(np.abs(h - r["h"]) <= bound)


def small_chain(M):
    x = datagen.bf16_normal((M, 512), datagen.tensor_seed("sx", M), device=DEV)
    Wg, hg = make(fg.NVFP4, 768, 512, 1)
    Wu, hu = make(fg.NVFP4, 768, 512, 2)
    Wd, hd = make(fg.NVFP4, 512, 768, 3)
    Wm, hm = make(fg.MXFP4, 256, 512, 4)
    Wh, hh = make(fg.FP8_ROW, 1024, 512, 5)
    h0 = torch.empty((M, 768), dtype=torch.bfloat16, device=DEV)
    y1 = torch.empty((M, 512), dtype=torch.float32, device=DEV)
    y2 = torch.empty((M, 256), dtype=torch.float32, device=DEV)
    y3 = torch.empty((M, 1024), dtype=torch.float32, device=DEV)
    ops = [
        {"kind": fg.OP_GATE_UP, "w": Wg, "w_up": Wu, "x": x, "out": h0, "wait_op": -1},
        {"kind": fg.OP_GEMV, "w": Wd, "x": h0, "out": y1, "wait_op": 0},
        {"kind": fg.OP_GEMV, "w": Wm, "x": x, "out": y2, "wait_op": 1},
        {"kind": fg.OP_LMHEAD, "w": Wh, "x": x, "out": y3, "wait_op": 2},
    ]
    return ops, (hg, hu, hd, hm, hh), x, (h0, y1, y2, y3)


@pytest.mark.parametrize("M", [1, 2, 3, 8])
def test_small_chain_matches_oracle(M):
    log("stream small", M)
    ops, (hg, hu, hd, hm, hh), x, (h0, y1, y2, y3) = small_chain(M)
    st = fg.Stream(ops, M)
    outs = []
    for rep in range(3):
        for t in (h0, y1, y2, y3):
            t.fill_(float("nan"))
        st.run()
        torch.cuda.synchronize()
        assert st.error() == 0
        outs.append([t.clone() for t in (h0, y1, y2, y3)])
    xb = bits(x)
    check_h(h0, hg, hu, xb)
    check_y(y1, hd, bits(h0))  # down, given the stream's own h
    check_y(y2, hm, xb)
    check_y(y3, hh, xb)
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a, b), "repeated runs differ"


def test_new_inputs_each_run():
    """Inputs change between runs (as activations do between decode steps): every
    run must read this run's inputs and intermediates, never a copy cached by the
    previous run."""
    log("stream new inputs")
    M = 2
    ops, (hg, hu, hd, hm, hh), x, (h0, y1, y2, y3) = small_chain(M)
    st = fg.Stream(ops, M)
    for rep in range(4):
        x.copy_(datagen.bf16_normal((M, 512), datagen.tensor_seed("sx-rep", rep), device=DEV))
        st.run()
        torch.cuda.synchronize()
        assert st.error() == 0
        xb = bits(x)
        check_h(h0, hg, hu, xb)
        check_y(y1, hd, bits(h0))
        check_y(y2, hm, xb)
        check_y(y3, hh, xb)


def test_graph_replays_match_eager():
    log("stream graph")
    M = 2
    ops, _, x, outs = small_chain(M)
    st = fg.Stream(ops, M)
    st.run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run()
    for rep in range(4):
        for t in outs:
            t.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, outs):
            assert torch.equal(a, b), rep
        # eager work between replays
        fg.fp4_gemv(ops[2]["w"], x[0])
    assert st.error() == 0


def test_dense_layers_full_size():
    """Two layers of the dense decode chain at full size: attention-shaped
    projections, then gate/up + SiLU, then down, each op waiting for the one before."""
    log("stream dense 2 layers")
    M = 1
    H, F = datagen.HIDDEN, datagen.FFN
    x = datagen.bf16_normal((M, H), 7, device=DEV)
    xa = datagen.bf16_normal((M, 12288), 8, device=DEV)
    ops, hosts = [], []
    for L in range(2):
        for j, (o, i) in enumerate(datagen.ATTN_SHAPES):
            W, h = make(fg.NVFP4, o, i, ("attn", L, j))
            out = torch.empty((M, o), dtype=torch.float32, device=DEV)
            ops.append({"kind": fg.OP_GEMV, "w": W, "x": x if i == H else xa, "out": out, "wait_op": len(ops) - 1})
            hosts.append(("y", h, x if i == H else xa))
        Wg, hg = make(fg.NVFP4, F, H, ("g", L))
        Wu, hu = make(fg.NVFP4, F, H, ("u", L))
        hbuf = torch.empty((M, F), dtype=torch.bfloat16, device=DEV)
        ops.append({"kind": fg.OP_GATE_UP, "w": Wg, "w_up": Wu, "x": x, "out": hbuf, "wait_op": len(ops) - 1})
        hosts.append(("h", (hg, hu), x))
        Wd, hd = make(fg.NVFP4, H, F, ("d", L))
        y = torch.empty((M, H), dtype=torch.float32, device=DEV)
        ops.append({"kind": fg.OP_GEMV, "w": Wd, "x": hbuf, "out": y, "wait_op": len(ops) - 1})
        hosts.append(("y", hd, hbuf))
    Wh, hh = make(fg.FP8_ROW, 248320, H, "head")
    logits = torch.empty((M, 248320), dtype=torch.float32, device=DEV)
    ops.append({"kind": fg.OP_LMHEAD, "w": Wh, "x": x, "out": logits, "wait_op": len(ops) - 1})
    hosts.append(("y", hh, x))
    st = fg.Stream(ops, M)
    st.run()
    torch.cuda.synchronize()
    assert st.error() == 0
    for op, (kind, h, xin) in zip(ops, hosts):
        rows = np.unique(np.concatenate([np.arange(0, op["out"].shape[1], 97), [op["out"].shape[1] - 1]]))
        if kind == "h":
            check_h(op["out"], h[0], h[1], bits(xin), rows=rows)
        else:
            check_y(op["out"], h, bits(xin), rows=rows)
