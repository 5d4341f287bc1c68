#!/usr/bin/env python3
"""Decode-GEMV benchmark on one MI355X.

Default workload (the one the metric's implied tok/s is defined on): the full
dense weight stream of one decoded token at M = 1 -- 64 layers, each an NVFP4 MLP
(gate and up 17408x5120 fused with SiLU*mul, down 5120x17408) and four NVFP4
attention projections (12288x5120, 12288x5120, 5120x12288, 7680x5120), then an
FP8 E4M3 LM head 248320x5120 with FP32 row scales: 19.11 GB of weights per token,
the figure the mdjawad.com DGX Spark feed counts (19.10 GB).  A step is one token:
257 kernel launches (per layer gate/up, down, the three projections of x as one
grouped launch, the output projection; then the head) replayed from one HIP
graph.  Inputs are seeded synthetic tensors already resident in HBM.

Prints ONE JSON line: achieved GB/s (algorithmic bytes / time), implied tok/s,
the roofline of the dominant kernel (timed live with HIP events), and the
FP64 CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload c3|c3m|c1|c2|c4|c5|head|copy]
                    [--M vectors] [--path auto|valu|mfma] [--router] [--no-breakdown]

Other workloads: c1 one 5120x5120 NVFP4 GEMV; c2 the NVFP4 MLP; c4 the MLP at a
verify block of M vectors (up to 16); c3m the dense stream in the checkpoint's
mixed NVFP4/FP8 layout; c5 the MoE decode (--router: router logits from an FP8
product of x); head the FP8 head with the fused greedy pick and a draft head;
copy a 1 GiB device copy (the reference for HBM counter calibration).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBPS = 8000.0
HEAD_DRAFT_ROWS = 100032  # the draft head's reduced vocabulary: the leading rows of the FP8 head


# The files the NVFP4 and FP8-row product kernels (and their launch planning) are
# built from; the committed counter summary is valid only while they are unchanged.
TRAFFIC_SOURCES = ("bit_weight_gemv_fp4_amd/build.py", "bit_weight_gemv_fp4_amd/csrc/common.hpp",
                   "bit_weight_gemv_fp4_amd/csrc/gemv_kernel.hpp", "bit_weight_gemv_fp4_amd/csrc/gemv_mfma.hpp",
                   "bit_weight_gemv_fp4_amd/csrc/gemv.hip", "bit_weight_gemv_fp4_amd/csrc/gemv_nvfp4.hip",
                   "bit_weight_gemv_fp4_amd/csrc/gemv_mfma_nvfp4.hip", "bit_weight_gemv_fp4_amd/csrc/gemv_mfma_nvfp4_silu.hip",
                   "bit_weight_gemv_fp4_amd/csrc/gemv_fp8.hip")


def traffic_sources_hash():
    """First 16 hex digits of a sha256 over the kernel sources' code: comments
    and runs of white space are dropped first, so that the committed counters
    stay valid across edits that cannot change a kernel."""
    import hashlib
    import re

    def code(text):
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        return " ".join(text.split())

    return hashlib.sha256("\n".join(code((ROOT / q).read_text()) for q in TRAFFIC_SOURCES).encode()).hexdigest()[:16]


def resolved_path(workload, path, M):
    """The kernel path a workload's products take: 'valu' or 'mfma' for the
    NVFP4/MXFP4 products of c4 and skinny ('auto': the matrix cores from M = 3
    on), 'auto' where the workload has a single kernel choice."""
    if workload not in ("c4", "skinny"):
        return "auto"
    if path == "auto":
        return "valu" if M <= 2 else "mfma"
    return path


def counter_traffic(workload, M, path, fmt, kind):
    """HBM bytes per launch of `kind` in this workload from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (profiles/counters.json): only for
    the (workload, M, path, format) the counters were taken on, and only while
    the kernel sources hash to the value recorded there; otherwise None."""
    p = ROOT / "profiles" / "counters.json"
    if not p.exists():
        return None
    d = json.loads(p.read_text())
    if d.get("source_sha256_16") != traffic_sources_hash():
        return None
    for e in d.get("entries", []):
        if (e["workload"], e["M"], e["path"], e["fmt"], e["kind"]) == (workload, M, path, fmt, kind):
            return round(e["fetch_bytes"] + e["write_bytes"])
    return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c3",
                    choices=["c1", "c2", "c3", "c3m", "c4", "c5", "head", "skinny", "copy"],
                    help="c3m: the dense stream in the checkpoint's mixed NVFP4/FP8 layout; skinny: one "
                         "17408x5120 product at M vectors (--fmt, --path)")
    ap.add_argument("--fmt", default="nvfp4", choices=["nvfp4", "mxfp4"], help="weight format of the skinny, c2 and c4 workloads")
    ap.add_argument("--M", type=int, default=None, help="vectors per step for c4/c5")
    ap.add_argument("--router", action="store_true",
                    help="c5: compute each layer's router logits with an FP8 512x2560 product of x")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true",
                    help="skip the per-kernel breakdown (each kind's launches timed alone, and its share of the step)")
    ap.add_argument("--path", default="auto", choices=["auto", "valu", "mfma", "a8"],
                    help="kernel path of the NVFP4/MXFP4 products (auto: MFMA from M = 3 on)")
    return ap.parse_args()


# ---- helpers -------------------------------------------------------------------------------


def algorithmic_gemv_bytes(fg, fmt, d_out, d_in, M, out_bytes=4):
    """Packed weights + activations read once + outputs written once."""
    return fg.packed_bytes(fmt, d_out, d_in) + M * d_in * 2 + M * d_out * out_bytes


class Step:
    """A list of launches (closures) plus byte accounting.  One graph replay runs
    `steps_per_replay` steps (several copies of a small workload, so that weights
    rotate through more memory than the 256 MB Infinity Cache holds)."""

    def __init__(self, steps_per_replay=1):
        self.calls = []  # (kind, fn, bytes)
        self.steps_per_replay = steps_per_replay

    def add(self, kind, fn, nbytes):
        self.calls.append((kind, fn, nbytes))

    def bytes(self):
        return sum(b for _, _, b in self.calls)

    def run(self, kinds=None):
        for kind, fn, _ in self.calls:
            if kinds is None or kind in kinds:
                fn()


# ---- workloads ------------------------------------------------------------------------------


def build_dense_stream(fg, datagen, torch, layers, with_head=True, M=1):
    """The dense decode chain; returns (step of separate launches, keep)."""
    dev = "cuda"
    H, F = datagen.HIDDEN, datagen.FFN
    step = Step()
    keep = []
    x = datagen.bf16_normal((M, H), datagen.tensor_seed("c3", "x"), device=dev)
    x_attn_in = datagen.bf16_normal((M, 12288), datagen.tensor_seed("c3", "x12288"), device=dev)
    h = torch.empty((M, F), dtype=torch.bfloat16, device=dev)
    y = torch.empty((M, H), dtype=torch.float32, device=dev)
    ya = torch.empty((M, 12288), dtype=torch.float32, device=dev)
    keep += [x, x_attn_in, h, y, ya]
    ws = None
    for L in range(layers):
        def mat(name, o, i):
            m = datagen.matrix(fg.NVFP4, o, i, datagen.tensor_seed("c3", L, name), device=dev)
            W = fg.pack(fg.NVFP4, m["codes"], m["scales"], m["tensor_scale"])
            del m
            return W
        Wg, Wu, Wd = mat("gate", F, H), mat("up", F, H), mat("down", H, F)
        att = [mat(f"attn{j}", o, i) for j, (o, i) in enumerate(datagen.ATTN_SHAPES)]
        keep += [Wg, Wu, Wd] + att
        gu_bytes = 2 * fg.packed_bytes(fg.NVFP4, F, H) + M * H * 2 + M * F * 2
        step.add("gate_up_silu", (lambda Wg=Wg, Wu=Wu: fg.fp4_gate_up_silu(Wg, Wu, x, h)), gu_bytes)
        if M == 1:
            step.add("down", (lambda Wd=Wd: fg.fp4_gemv(Wd, h.view(-1), y.view(-1))),
                     algorithmic_gemv_bytes(fg, fg.NVFP4, H, F, M))
        else:
            step.add("down", (lambda Wd=Wd: fg.fp4_skinny_gemm(Wd, h, y)), algorithmic_gemv_bytes(fg, fg.NVFP4, H, F, M))
        # the projections that read x go out as one grouped launch, the output
        # projection (reads the 12288-wide attention result) as its own
        qkv = [j for j, (o, i) in enumerate(datagen.ATTN_SHAPES) if i == H]
        G = fg.Group([att[j] for j in qkv])
        ys = [torch.empty((M, datagen.ATTN_SHAPES[j][0]), dtype=torch.float32, device=dev) for j in qkv]
        keep += [G, ys]
        step.add("qkv", (lambda G=G, ys=ys: fg.fp4_gemv_grouped(G, x, ys)),
                 sum(algorithmic_gemv_bytes(fg, fg.NVFP4, *datagen.ATTN_SHAPES[j], M) - M * H * 2 for j in qkv)
                 + M * H * 2)
        for j, (o, i) in enumerate(datagen.ATTN_SHAPES):
            if j in qkv:
                continue
            W = att[j]
            if M == 1:
                fn = (lambda W=W: fg.fp4_gemv(W, x_attn_in.view(-1), y.view(-1)))
            else:
                fn = (lambda W=W: fg.fp4_skinny_gemm(W, x_attn_in, y))
            step.add("o_proj", fn, algorithmic_gemv_bytes(fg, fg.NVFP4, o, i, M))
    if with_head:
        m = datagen.matrix(fg.FP8_ROW, datagen.VOCAB, H, datagen.tensor_seed("c3", "head"), device=dev)
        Wh = fg.pack(fg.FP8_ROW, m["codes"], m["scales"])
        del m
        logits = torch.empty((M, datagen.VOCAB), dtype=torch.float32, device=dev)
        keep += [Wh, logits]
        step.add("lm_head", (lambda: fg.fp8_lmhead_gemv(Wh, x, logits)),
                 algorithmic_gemv_bytes(fg, fg.FP8_ROW, datagen.VOCAB, H, M))
    return step, keep


def build_mixed_stream(fg, datagen, torch, M=1):
    """The dense decode chain in the checkpoint's mixed layout: FP8 row-scaled
    projections (linear attention in 48 layers, full attention in every fourth),
    NVFP4 MLPs in layers 0..55 and FP8 MLPs in the last 8, then the FP8 head."""
    dev = "cuda"
    H, F = datagen.HIDDEN, datagen.FFN
    step = Step()
    keep = []
    x = datagen.bf16_normal((M, H), datagen.tensor_seed("c3m", "x"), device=dev)
    wide = {i: datagen.bf16_normal((M, i), datagen.tensor_seed("c3m", "x", i), device=dev) for i in (6144, 10240)}
    h = torch.empty((M, F), dtype=torch.bfloat16, device=dev)
    y = torch.empty((M, H), dtype=torch.float32, device=dev)
    keep += [x, h, y, wide]

    def mat(fmt, L, name, o, i):
        m = datagen.matrix(fmt, o, i, datagen.tensor_seed("c3m", L, name), device=dev)
        W = fg.pack(fmt, m["codes"], m["scales"], m["tensor_scale"])
        del m
        keep.append(W)
        return W

    def product(fmt, W, xin, out):
        if fmt == fg.FP8_ROW:
            return lambda: fg.fp8_lmhead_gemv(W, xin, out)
        return lambda: fg.fp4_skinny_gemm(W, xin, out)

    for L in range(datagen.LAYERS):
        shapes = datagen.MIXED_ATTN_SHAPES if datagen.mixed_full_attention(L) else datagen.MIXED_GDN_SHAPES
        ws = [mat(fg.FP8_ROW, L, f"proj{j}", o, i) for j, (o, i) in enumerate(shapes)]
        into = [j for j, (o, i) in enumerate(shapes) if i == H]     # projections of x: one grouped launch
        G = fg.Group([ws[j] for j in into])
        ys = [torch.empty((M, shapes[j][0]), dtype=torch.float32, device=dev) for j in into]
        keep += [G, ys]
        step.add("proj_in", (lambda G=G, ys=ys: fg.fp4_gemv_grouped(G, x, ys)),
                 sum(fg.packed_bytes(fg.FP8_ROW, *shapes[j]) + 4 * M * shapes[j][0] for j in into) + 2 * M * H)
        for j, (o, i) in enumerate(shapes):
            if j not in into:
                step.add("proj_out", product(fg.FP8_ROW, ws[j], wide[i], y),
                         algorithmic_gemv_bytes(fg, fg.FP8_ROW, o, i, M))
        fmt = fg.NVFP4 if L < datagen.MIXED_FP8_MLP_FROM else fg.FP8_ROW
        Wg, Wu, Wd = mat(fmt, L, "gate", F, H), mat(fmt, L, "up", F, H), mat(fmt, L, "down", H, F)
        kind = "gate_up_silu" if fmt == fg.NVFP4 else "gate_up_silu_fp8"
        step.add(kind, (lambda Wg=Wg, Wu=Wu: fg.fp4_gate_up_silu(Wg, Wu, x, h)),
                 2 * fg.packed_bytes(fmt, F, H) + M * H * 2 + M * F * 2)
        step.add("down" if fmt == fg.NVFP4 else "down_fp8", product(fmt, Wd, h, y),
                 algorithmic_gemv_bytes(fg, fmt, H, F, M))
    Wh = mat(fg.FP8_ROW, "head", "head", datagen.VOCAB, H)
    logits = torch.empty((M, datagen.VOCAB), dtype=torch.float32, device=dev)
    keep.append(logits)
    step.add("lm_head", (lambda: fg.fp8_lmhead_gemv(Wh, x, logits)),
             algorithmic_gemv_bytes(fg, fg.FP8_ROW, datagen.VOCAB, H, M))
    return step, keep


def weights_only_bytes_dense(fg, datagen, layers, with_head=True):
    H, F = datagen.HIDDEN, datagen.FFN
    per_layer = 2 * fg.packed_bytes(fg.NVFP4, F, H) + fg.packed_bytes(fg.NVFP4, H, F)
    per_layer += sum(fg.packed_bytes(fg.NVFP4, o, i) for o, i in datagen.ATTN_SHAPES)
    total = layers * per_layer
    if with_head:
        total += fg.packed_bytes(fg.FP8_ROW, datagen.VOCAB, H)
    return total


def copies_for(nbytes, min_total=1 << 30):
    return max(1, -(-min_total // nbytes))


def build_other(name, M, fg, datagen, torch, path=0, router=False, fmt=None):
    dev = "cuda"
    H, F = datagen.HIDDEN, datagen.FFN
    keep = []
    if name == "skinny":
        fmt = fmt or fg.NVFP4
        nb = fg.packed_bytes(fmt, F, H)
        R = copies_for(nb)
        step = Step(R)
        X = datagen.bf16_normal((M, H), datagen.tensor_seed("skinny", "x", M), device=dev)
        Y = torch.empty((M, F), dtype=torch.float32, device=dev)
        keep += [X, Y]
        for r in range(R):
            m = datagen.matrix(fmt, F, H, datagen.tensor_seed("skinny", r), device=dev)
            W = fg.pack(fmt, m["codes"], m["scales"], m["tensor_scale"])
            keep.append(W)
            step.add("skinny", (lambda W=W: fg.fp4_skinny_gemm(W, X, Y, path=path)), algorithmic_gemv_bytes(fg, fmt, F, H, M))
        name_f = "NVFP4" if fmt == fg.NVFP4 else "MXFP4"
        return step, keep, f"one {name_f} product 17408x5120 at M={M} ({R} copies rotated)", "skinny"
    if name == "c1":
        nb = fg.packed_bytes(fg.NVFP4, H, H)
        R = copies_for(nb)
        step = Step(R)
        x = datagen.bf16_normal((H,), datagen.tensor_seed("c1", "x"), device=dev)
        y = torch.empty(H, dtype=torch.float32, device=dev)
        for r in range(R):
            m = datagen.matrix(fg.NVFP4, H, H, datagen.tensor_seed("c1", r), device=dev)
            W = fg.pack(fg.NVFP4, m["codes"], m["scales"])
            keep.append(W)
            step.add("gemv", (lambda W=W: fg.fp4_gemv(W, x, y)), algorithmic_gemv_bytes(fg, fg.NVFP4, H, H, 1))
        keep += [x, y]
        return step, keep, f"single NVFP4 GEMV 5120x5120, M=1 ({R} weight copies rotated)", "gemv"
    if name in ("c2", "c4"):
        fmt = fmt or fg.NVFP4
        nb = 3 * fg.packed_bytes(fmt, F, H)
        R = copies_for(nb)
        step = Step(R)
        X = datagen.bf16_normal((M, H), datagen.tensor_seed(name, "x", M), device=dev)
        h = torch.empty((M, F), dtype=torch.bfloat16, device=dev)
        y = torch.empty((M, H), dtype=torch.float32, device=dev)
        keep += [X, h, y]
        for r in range(R):
            ws = []
            for nm, (o, i) in (("gate", (F, H)), ("up", (F, H)), ("down", (H, F))):
                m = datagen.matrix(fmt, o, i, datagen.tensor_seed(name, r, nm), device=dev)
                ws.append(fg.pack(fmt, m["codes"], m["scales"]))
            keep += ws
            Wg, Wu, Wd = ws
            step.add("gate_up_silu", (lambda Wg=Wg, Wu=Wu: fg.fp4_gate_up_silu(Wg, Wu, X, h, path=path)),
                     2 * fg.packed_bytes(fmt, F, H) + M * H * 2 + M * F * 2)
            if M == 1 and path == fg.PATH_AUTO:
                fn = (lambda Wd=Wd: fg.fp4_gemv(Wd, h.view(-1), y.view(-1)))
            else:
                fn = (lambda Wd=Wd: fg.fp4_skinny_gemm(Wd, h, y, path=path))
            step.add("down", fn, algorithmic_gemv_bytes(fg, fmt, H, F, M))
        what = "dense MLP" if name == "c2" else "speculative-verify MLP"
        name_f = "NVFP4" if fmt == fg.NVFP4 else "MXFP4"
        return step, keep, f"{what}, {name_f} gate/up 17408x5120 + SiLU*mul, down 5120x17408, M={M} ({R} copies rotated)", \
            "gate_up_silu"
    if name == "head":
        # the dense model's FP8 head: plain logits, fused greedy pick, and a draft
        # head over the leading 100032 rows (the reduced vocabulary)
        V, DV = datagen.VOCAB, HEAD_DRAFT_ROWS
        m = datagen.matrix(fg.FP8_ROW, V, H, datagen.tensor_seed("c3", "head"), device=dev)
        Wh = fg.pack(fg.FP8_ROW, m["codes"], m["scales"])
        del m
        X = datagen.bf16_normal((M, H), datagen.tensor_seed("head", "x", M), device=dev)
        logits = torch.empty((M, V), dtype=torch.float32, device=dev)
        keep += [Wh, X, logits]
        step = Step()
        step.add("lm_head", (lambda: fg.fp8_lmhead_gemv(Wh, X, logits)), algorithmic_gemv_bytes(fg, fg.FP8_ROW, V, H, M))
        step.add("lm_head_argmax", (lambda: fg.fp8_lmhead_argmax(Wh, X)),
                 algorithmic_gemv_bytes(fg, fg.FP8_ROW, V, H, M, out_bytes=0) + 8 * M)
        step.add("draft_head_argmax", (lambda: fg.fp8_lmhead_argmax(Wh, X, 0, DV)),
                 DV * H + 4 * DV + 2 * M * H + 8 * M)
        return step, keep, f"FP8 LM head 248320x5120, M={M}: logits; fused greedy pick; pick over the first 100032 rows", \
            "lm_head_argmax"
    if name == "c5":
        E, K, Hm, Fm = datagen.MOE_EXPERTS, datagen.MOE_TOPK, datagen.MOE_HIDDEN, datagen.MOE_FF
        pg = fg.packed_bytes(fg.MXFP4, Fm, Hm)
        pd = fg.packed_bytes(fg.MXFP4, Hm, Fm)
        layers = []
        for L in range(datagen.MOE_LAYERS):
            descs = []
            for nm, (o, i), st in (("gate", (Fm, Hm), pg), ("up", (Fm, Hm), pg), ("down", (Hm, Fm), pd)):
                buf = torch.empty((E + 1) * st, dtype=torch.uint8, device=dev)  # expert E = shared
                first = None
                for e0 in range(0, E + 1, 64):
                    e1 = min(E + 1, e0 + 64)
                    m = datagen.matrix(fg.MXFP4, o, i, datagen.tensor_seed("c5", L, nm, e0), device=dev,
                                       batch=e1 - e0)
                    for e in range(e0, e1):
                        w = fg.pack(fg.MXFP4, m["codes"][e - e0], m["scales"][e - e0], 1.0, out=buf, offset=e * st)
                        if e == 0:
                            first = w
                    del m
                shared = first.view(E * st)
                first.desc.packed_bytes = E * st
                descs.append((first, shared))
                keep.append(buf)
            layer = fg.moe_layer(descs[0][0], descs[1][0], descs[2][0], E, K, pg, pg, pd,
                                 shared=(descs[0][1], descs[1][1], descs[2][1]))
            layers.append(layer)
        m = datagen.matrix(fg.FP8_ROW, datagen.MOE_VOCAB, Hm, datagen.tensor_seed("c5", "head"), device=dev)
        Wh = fg.pack(fg.FP8_ROW, m["codes"], m["scales"])
        del m
        keep += layers + [Wh]
        R = 4  # token steps per replay, each with its own router logits
        step = Step(R)
        X = datagen.bf16_normal((M, Hm), datagen.tensor_seed("c5", "x", M), device=dev)
        Y = torch.empty((M, Hm), dtype=torch.float32, device=dev)
        ids = torch.empty((M, K), dtype=torch.int32, device=dev)
        wts = torch.empty((M, K), dtype=torch.float32, device=dev)
        logits_out = torch.empty((M, datagen.MOE_VOCAB), dtype=torch.float32, device=dev)
        keep += [X, Y, ids, wts, logits_out]
        moe_bytes = 0
        routers = []
        if router:
            for L in range(len(layers)):
                m = datagen.matrix(fg.FP8_ROW, E, Hm, datagen.tensor_seed("c5", "router", L), device=dev)
                routers.append(fg.pack(fg.FP8_ROW, m["codes"], m["scales"]))
                del m
            keep += routers
        for r in range(R):
            for L, layer in enumerate(layers):
                if router:
                    lg = torch.empty((M, E), dtype=torch.float32, device=dev)
                    fg.fp8_lmhead_gemv(routers[L], X, lg)
                    step.add("router", (lambda Wr=routers[L], lg=lg: fg.fp8_lmhead_gemv(Wr, X, lg)),
                             algorithmic_gemv_bytes(fg, fg.FP8_ROW, E, Hm, M))
                else:
                    lg = datagen.router_logits(M, E, datagen.tensor_seed("c5", "logits", r, L), device=dev)
                keep.append(lg)
                # algorithmic bytes: the realised union of experts (+ shared), logits, x, y
                _, rid, _ = fg.moe_route_gemv(layer, X, lg, Y, ids, wts)
                n_union = len(set(rid.cpu().numpy().ravel().tolist())) + 1
                nbytes = n_union * (2 * pg + pd) + M * E * 4 + M * Hm * 2 + M * Hm * 4
                moe_bytes += nbytes
                step.add("moe", (lambda layer=layer, lg=lg: fg.moe_route_gemv(layer, X, lg, Y, ids, wts)), nbytes)
            step.add("lm_head", (lambda: fg.fp8_lmhead_gemv(Wh, X, logits_out)),
                     algorithmic_gemv_bytes(fg, fg.FP8_ROW, datagen.MOE_VOCAB, Hm, M))
        return step, keep, (f"MoE decode, M={M}: 40 layers x [{'FP8 router 512x2560, ' if router else ''}"
                            f"route top-8 of 512 + shared, MXFP4 experts "
                            f"gate/up 768x2560, down 2560x768] + FP8 LM head 157184x2560"), "moe"
    raise ValueError(name)


# ---- CPU oracle baseline ------------------------------------------------------------------------
# The FP64 oracle (oracle/, test infrastructure) timed on the host as a baseline:
# bounded samples of the workload, each run three times (median), at the box's
# thread share and at one thread.  The oracle is plain C in FP64 and is not
# tuned for speed: the ratio to the GPU says nothing about the kernels' quality.


def host_info():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"nproc": os.cpu_count(), "affinity_cpus": aff, "model": model}


def box_threads():
    """Threads for the multi-threaded baseline: the CPU share this process may use
    (OMP_NUM_THREADS when set, else the affinity mask), at most 16."""
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    env = os.environ.get("OMP_NUM_THREADS", "")
    n = int(env) if env.isdigit() and int(env) > 0 else aff
    return max(1, min(16, n, aff))


def median3(fn):
    ts = []
    for _ in range(3):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    ts.sort()
    return ts[1], ts


def baseline_entry(bytes_per_step, legs, per_token=True):
    """legs: list of (threads, seconds per step, sample text, run times).  The
    first leg (the box's thread share) is the reported value."""
    th, sec, sample, runs = legs[0]
    out = {"value": round(bytes_per_step / sec / 1e9, 4), "unit": "GB/s", "cores": th, "kind": "oracle",
           "sample": sample, "stat": "median of 3 runs", "host": host_info(), "legs": []}
    for th, sec, sample, runs in legs:
        leg = {"threads": th, "GB/s": round(bytes_per_step / sec / 1e9, 4), "s_per_step": round(sec, 3),
               "sample": sample, "sample_run_s": [round(t, 3) for t in runs]}
        if per_token:
            leg["implied_tok_s"] = round(1.0 / sec, 5)
        out["legs"].append(leg)
    return out


def cpu_baseline_dense(fg, datagen, torch, bytes_per_token, mt_layers=8, st_layers=1):
    """C3: mt_layers full layers + every 8th LM-head row at the box's thread
    share, st_layers + every 256th head row at one thread; scaled to one token."""
    import numpy as np

    import oracle

    H, F = datagen.HIDDEN, datagen.FFN
    x = datagen.bf16_normal((1, H), datagen.tensor_seed("c3", "x"), device="cuda")
    xb = x.cpu().view(torch.int16).numpy().view(np.uint16)
    xa = datagen.bf16_normal((1, 12288), datagen.tensor_seed("c3", "x12288"), device="cuda")
    xab = xa.cpu().view(torch.int16).numpy().view(np.uint16)
    layers = []
    for L in range(max(mt_layers, st_layers)):
        mats = []
        for name, (o, i) in [("gate", (F, H)), ("up", (F, H)), ("down", (H, F))] + [
                (f"attn{j}", sh) for j, sh in enumerate(datagen.ATTN_SHAPES)]:
            m = datagen.matrix(fg.NVFP4, o, i, datagen.tensor_seed("c3", L, name), device="cuda")
            mats.append((i, m["codes"].cpu().numpy(), m["scales"].cpu().numpy()))
            del m
        layers.append(mats)
    V = datagen.VOCAB
    m = datagen.matrix(fg.FP8_ROW, V, H, datagen.tensor_seed("c3", "head"), device="cuda")
    hc, hs = m["codes"].cpu().numpy(), m["scales"].cpu().numpy()
    del m

    def run(n_layers, head_every, th):
        for mats in layers[:n_layers]:
            g, _ = oracle.gemv(1, mats[0][1], mats[0][2], 1.0, xb, nthreads=th)
            u, _ = oracle.gemv(1, mats[1][1], mats[1][2], 1.0, xb, nthreads=th)
            oracle.gemv(1, mats[2][1], mats[2][2], 1.0, oracle.silu_mul(g, u), nthreads=th)
            for i, c, sc in mats[3:]:
                oracle.gemv(1, c, sc, 1.0, xb if i == H else xab, nthreads=th)
        rows = np.arange(0, V, head_every, dtype=np.int64)
        oracle.gemv(3, hc, hs, 1.0, xb, rows=rows, nthreads=th)

    legs = []
    for th, nl, every in ((box_threads(), mt_layers, 8), (1, st_layers, 256)):
        med, runs = median3(lambda: run(nl, every, th))
        # the sample's share of one token: nl / 64 of the layers' weights, 1/every of the head's
        Wl = 2 * F * H + H * F + sum(o * i for o, i in datagen.ATTN_SHAPES)
        frac_l, head_w = nl * Wl, V * H / every
        tok_w = datagen.LAYERS * Wl + V * H
        legs.append((th, med * tok_w / (frac_l + head_w), f"{nl} of 64 layers + every {every}th LM-head row "
                     f"({(frac_l + head_w) / tok_w:.3f} of a token's weights), scaled to one token", runs))
    return baseline_entry(bytes_per_token, legs)


def cpu_baseline_moe(fg, datagen, torch, bytes_per_step, M, mt_layers=4, st_layers=1):
    """C5: the oracle's MoE layer (routing, the picked experts and the shared
    one) on the bench's own logits for the first layers, plus every 8th (16th at
    one thread) LM-head row; scaled to one step of 40 layers."""
    import numpy as np

    import oracle

    E, K, Hm, Fm = datagen.MOE_EXPERTS, datagen.MOE_TOPK, datagen.MOE_HIDDEN, datagen.MOE_FF
    X = datagen.bf16_normal((M, Hm), datagen.tensor_seed("c5", "x", M), device="cuda")
    Xb = X.cpu().view(torch.int16).numpy().view(np.uint16)
    cases = []
    for L in range(max(mt_layers, st_layers)):
        lg = datagen.router_logits(M, E, datagen.tensor_seed("c5", "logits", 0, L), device="cuda").cpu().numpy()
        ids, _ = oracle.topk_softmax(lg, K)
        experts = {}
        for e in sorted(set(ids.ravel().tolist()) | {E}):   # expert E is the shared one
            e0 = (e // 64) * 64
            ex = {}
            for nm, (o, i) in (("gate", (Fm, Hm)), ("up", (Fm, Hm)), ("down", (Hm, Fm))):
                m = datagen.matrix(fg.MXFP4, o, i, datagen.tensor_seed("c5", L, nm, e0), device="cuda",
                                   batch=min(64, E + 1 - e0))
                ex[nm] = {"format": fg.MXFP4, "codes": m["codes"][e - e0].cpu().numpy(),
                          "scales": m["scales"][e - e0].cpu().numpy(), "tensor_scale": 1.0}
                del m
            experts[e] = ex
        cases.append((lg, experts))
    V = datagen.MOE_VOCAB
    m = datagen.matrix(fg.FP8_ROW, V, Hm, datagen.tensor_seed("c5", "head"), device="cuda")
    hc, hs = m["codes"].cpu().numpy(), m["scales"].cpu().numpy()
    del m

    def run(n_layers, head_every, th):
        for lg, experts in cases[:n_layers]:
            oracle.moe(lambda e: experts[e], experts[E], Xb, lg, K, nthreads=th)
        oracle.gemv(3, hc, hs, 1.0, Xb, rows=np.arange(0, V, head_every, dtype=np.int64), nthreads=th)

    legs = []
    for th, nl, every in ((box_threads(), mt_layers, 8), (1, st_layers, 16)):
        med, runs = median3(lambda: run(nl, every, th))
        # layer time and head time measured together: scale each part by its weights
        w_layer = (len(cases[0][1])) * 3 * Fm * Hm
        frac = nl * w_layer + V * Hm / every
        step_w = datagen.MOE_LAYERS * w_layer + V * Hm
        legs.append((th, med * step_w / frac, f"MoE layers 0..{nl - 1} at M={M} (oracle routing on the bench's "
                     f"logits, {len(cases[0][1])} experts read in layer 0) + every {every}th LM-head row, "
                     f"scaled to one step", runs))
    return baseline_entry(bytes_per_step, legs, per_token=M == 1)


def cpu_baseline_products(fg, datagen, torch, name, M, bytes_per_step):
    """C1 (one 5120x5120 GEMV), C2 / C4 (the MLP at M vectors): the oracle on one
    copy of the workload's matrices; the one-thread leg on every 8th output row
    of each product (the MLP's down on the oracle's own h), scaled."""
    import numpy as np

    import oracle

    H, F = datagen.HIDDEN, datagen.FFN
    if name == "c1":
        m = datagen.matrix(fg.NVFP4, H, H, datagen.tensor_seed("c1", 0), device="cuda")
        mats = [("gemv", m["codes"].cpu().numpy(), m["scales"].cpu().numpy())]
        x = datagen.bf16_normal((H,), datagen.tensor_seed("c1", "x"), device="cuda")
        X = x.view(1, -1).cpu().view(torch.int16).numpy().view(np.uint16)
    else:
        mats = []
        for nm, (o, i) in (("gate", (F, H)), ("up", (F, H)), ("down", (H, F))):
            m = datagen.matrix(fg.NVFP4, o, i, datagen.tensor_seed(name, 0, nm), device="cuda")
            mats.append((nm, m["codes"].cpu().numpy(), m["scales"].cpu().numpy()))
        X = datagen.bf16_normal((M, H), datagen.tensor_seed(name, "x", M), device="cuda").cpu().view(
            torch.int16).numpy().view(np.uint16)

    def run(th, every):
        rows = lambda n: None if every == 1 else np.arange(0, n, every, dtype=np.int64)  # noqa: E731
        if name == "c1":
            oracle.gemv(1, mats[0][1], mats[0][2], 1.0, X, rows=rows(H), nthreads=th)
            return
        g, _ = oracle.gemv(1, mats[0][1], mats[0][2], 1.0, X, rows=rows(F), nthreads=th)
        u, _ = oracle.gemv(1, mats[1][1], mats[1][2], 1.0, X, rows=rows(F), nthreads=th)
        h = oracle.silu_mul(g, u)
        if every != 1:  # down needs the whole h: the sampled rows' h, zeros elsewhere
            hf = np.zeros((X.shape[0], F))
            hf[:, ::every] = h
            h = hf
        oracle.gemv(1, mats[2][1], mats[2][2], 1.0, h, rows=rows(H), nthreads=th)

    legs = []
    for th, every in ((box_threads(), 1), (1, 8)):
        med, runs = median3(lambda: run(th, every))
        legs.append((th, med * every, "the whole product" if every == 1 else
                     f"every {every}th output row of each product, scaled", runs))
    return baseline_entry(bytes_per_step, legs, per_token=False)


def cpu_baseline_head(fg, datagen, torch, M, bytes_per_step, draft_rows):
    """The FP8 head: the oracle's logits over every 8th row (every 64th at one
    thread) and the greedy pick of those rows; scaled to one step (logits, the
    fused pick and the draft pick: 2 x 248320 + draft_rows rows)."""
    import numpy as np

    import oracle

    H, V = datagen.HIDDEN, datagen.VOCAB
    m = datagen.matrix(fg.FP8_ROW, V, H, datagen.tensor_seed("c3", "head"), device="cuda")
    hc, hs = m["codes"].cpu().numpy(), m["scales"].cpu().numpy()
    del m
    X = datagen.bf16_normal((M, H), datagen.tensor_seed("head", "x", M), device="cuda").cpu().view(
        torch.int16).numpy().view(np.uint16)

    def run(th, every):
        rows = np.arange(0, V, every, dtype=np.int64)
        y, _ = oracle.gemv(3, hc, hs, 1.0, X, rows=rows, nthreads=th)
        np.argmax(y, axis=1)

    legs = []
    for th, every in ((box_threads(), 8), (1, 64)):
        med, runs = median3(lambda: run(th, every))
        legs.append((th, med * every * (2 * V + draft_rows) / V,
                     f"every {every}th head row (logits and their greedy pick), scaled to one step", runs))
    return baseline_entry(bytes_per_step, legs, per_token=False)


# ---- main ---------------------------------------------------------------------------------------


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; multi-GPU runs are not part of it",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import bit_weight_gemv_fp4_amd as fg
    import datagen

    torch.cuda.set_device(0)
    if args.workload == "copy":
        return copy_calibration(torch)
    dev = "cuda"
    M = args.M or (4 if args.workload in ("c4", "skinny") else 1)
    t_setup = time.perf_counter()
    if args.workload == "c3":
        step, keep = build_dense_stream(fg, datagen, torch, datagen.LAYERS, True, M=M)
        workload = "full dense weight stream, M=1: 64 x [NVFP4 attention 12288x5120, 12288x5120, 5120x12288, " \
                   "7680x5120, gate/up 17408x5120 + SiLU*mul, down 5120x17408] + FP8 LM head 248320x5120"
        dominant = "gate_up_silu"
    elif args.workload == "c3m":
        step, keep = build_mixed_stream(fg, datagen, torch, M=M)
        workload = (f"full dense weight stream in the mixed layout, M={M}: 64 layers of FP8 projections (48 linear "
                    f"attention 12288x5120 + 5120x10240, 16 full attention 12288x5120 + 2 x 1024x5120 + 5120x6144), "
                    f"MLPs 17408x5120 x2 + 5120x17408 NVFP4 in layers 0-55 and FP8 in 56-63, + FP8 LM head 248320x5120")
        dominant = "gate_up_silu"
    else:
        path = {"auto": fg.PATH_AUTO, "valu": fg.PATH_VALU, "mfma": fg.PATH_MFMA, "a8": fg.PATH_A8}[args.path]
        fmt = {"nvfp4": fg.NVFP4, "mxfp4": fg.MXFP4}[args.fmt]
        step, keep, workload, dominant = build_other(args.workload, M, fg, datagen, torch, path, args.router, fmt)
    bytes_per_step = step.bytes() / step.steps_per_replay
    # one eager pass allocates the workspace and checks every launch
    step.run()
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    n_dom = sum(1 for k, _, _ in step.calls if k == dominant)
    dom_bytes = sum(b for k, _, b in step.calls if k == dominant) / n_dom
    # The timed graph holds one step (or steps_per_replay of them).
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.run()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    # one HIP event between consecutive replays (on the replay stream) gives each
    # step's own time for the statistics; the wall clock around all of them gives
    # the headline rate
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(args.steps):
        g.replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) / step.steps_per_replay for i in range(args.steps))
    gpu_ms = evs[0].elapsed_time(evs[-1]) / args.steps
    # The dominant kernel: a graph of only its launches (same weights, same order),
    # timed with HIP events on the replay stream; the average per launch includes
    # the gaps between back-to-back launches, so it is a lower bound on the
    # kernel's own bandwidth.
    dom_us = kind_avg_us(step, torch, dominant, reps=max(3, min(20, args.steps)))
    dom_how = "graph of the dominant kernel's launches, HIP events around the replays (includes launch gaps)"
    ms_per_step = wall * 1e3 / args.steps / step.steps_per_replay
    gpu_ms /= step.steps_per_replay
    value = bytes_per_step / (ms_per_step * 1e-3) / 1e9
    dom_avg = dom_us
    achieved = dom_bytes / (dom_avg * 1e-6) / 1e9
    out = {
        "metric": "achieved HBM GB/s (% of 8 TB/s) for FP4 decode GEMV; implied tok/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "pct_of_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "implied_tok_s": round(1e3 / ms_per_step, 2) if args.workload in ("c3", "c3m", "c5") else None,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "gpu_ms_per_step": round(gpu_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e2m1/e4m3 weights x bf16 -> f32",
        "data": "synthetic (seeded; weights and activations resident in HBM)",
        "config": {"workload": workload, "M": M, "path": args.path, "bytes_per_step": bytes_per_step,
                   "launches_per_step": len(step.calls), "setup_s": round(setup_s, 1)},
        "step_stats": {
            "runs": args.steps,
            "median_ms": round(per_step[len(per_step) // 2], 4),
            "min_ms": round(per_step[0], 4),
            "p90_ms": round(per_step[min(len(per_step) - 1, int(0.9 * len(per_step)))], 4),
            "median_GBps": round(bytes_per_step / (per_step[len(per_step) // 2] * 1e-3) / 1e9, 1),
            "timed_by": "HIP events between consecutive graph replays",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": dominant,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": counter_traffic(args.workload, M, resolved_path(args.workload, args.path, M), args.fmt, dominant),
            "avg_us": round(dom_avg, 3),
            "launches_timed": n_dom,
            "timed_by": dom_how,
            "algorithmic_bytes_per_launch": dom_bytes,
        },
    }
    if not args.no_breakdown:
        out["breakdown"] = breakdown(step, torch, ms_per_step)
    if not args.no_cpu_baseline:
        if args.workload == "c3":
            out["cpu_baseline"] = cpu_baseline_dense(fg, datagen, torch, bytes_per_step)
        elif args.workload == "c5" and not args.router:
            out["cpu_baseline"] = cpu_baseline_moe(fg, datagen, torch, bytes_per_step, M)
        elif args.workload in ("c1", "c2", "c4") and args.fmt == "nvfp4":
            out["cpu_baseline"] = cpu_baseline_products(fg, datagen, torch, args.workload, M, bytes_per_step)
        elif args.workload == "head":
            out["cpu_baseline"] = cpu_baseline_head(fg, datagen, torch, M, bytes_per_step, HEAD_DRAFT_ROWS)
    print(json.dumps(out), flush=True)


def copy_calibration(torch, nbytes=1 << 30):
    """A plain device-to-device copy of known size: the reference for scaling the
    FETCH_SIZE / WRITE_SIZE counters of rocprofv3 into HBM bytes."""
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"workload": "copy", "bytes_read": nbytes, "bytes_written": nbytes, "launches": 3}), flush=True)


def kind_avg_us(step, torch, kind, reps=5):
    """Average time per launch of one kernel kind: its launches alone in a graph."""
    n = sum(1 for k, _, _ in step.calls if k == kind)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.run(kinds={kind})
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * n)


def breakdown(step, torch, ms_per_step):
    """Per-kind average launch time (each kind's launches alone in a graph), its
    bandwidth, and the share of one step its launches account for."""
    agg = {}
    for kind, _, b in step.calls:
        a = agg.setdefault(kind, {"launches": 0, "bytes": 0})
        a["launches"] += 1
        a["bytes"] += b
    for kind, a in agg.items():
        us = kind_avg_us(step, torch, kind)
        a["avg_us"] = round(us, 3)
        a["GB/s"] = round(a["bytes"] / a["launches"] / (us * 1e-6) / 1e9, 1)
        a["share_of_step"] = round(a["launches"] * us / step.steps_per_replay / (ms_per_step * 1e3), 4)
    return agg


if __name__ == "__main__":
    main()
