"""Helpers shared by the GPU parity tests: seeded operands, the comparisons
against the FP64 oracle and the MoE layer builder.  Imported by tests only."""
import sys

import numpy as np
import torch

import bit_weight_gemv_fp4_amd as fg
import datagen
import oracle

DEV = "cuda"
TOL = 2e-3


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits(x_bf16: torch.Tensor) -> np.ndarray:
    return x_bf16.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def make(fmt, d_out, d_in, seed, tensor_scale=1.0):
    mat = datagen.matrix(fmt, d_out, d_in, datagen.tensor_seed("gpu", fmt, d_out, d_in, seed), device=DEV)
    W = fg.pack(fmt, mat["codes"], mat["scales"], tensor_scale)
    host = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in mat.items()}
    host["tensor_scale"] = tensor_scale
    return W, host


def sample_rows(d_out, n=192, seed=0):
    rng = np.random.default_rng(seed)
    fixed = {0, 1, 63, 64, d_out - 1, d_out // 2}
    rows = sorted(fixed | set(rng.integers(0, d_out, n).tolist()))
    return np.array([r for r in rows if 0 <= r < d_out], dtype=np.int64)


def check_product(y_gpu, host, X_bits, rows=None, tol=TOL):
    Y, A = oracle.gemv(host["format"], host["codes"], host["scales"], host["tensor_scale"], X_bits, rows=rows)
    y = y_gpu.detach().cpu().double().numpy().reshape(Y.shape[0], -1)
    if rows is not None:
        y = y[:, rows]
    err = np.abs(y - Y)
    bound = tol * A
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} outputs out of bound; worst ratio {np.max(err / np.maximum(bound, 1e-300)):.3g}"
    return float(np.max(err / np.maximum(A, 1e-300)))


def h_bound(r, h_ref):
    tg, tu = TOL * r["Ag"], TOL * r["Au"]
    silu_g = r["g"] / (1.0 + np.exp(-r["g"]))
    return 1.1 * tg * (np.abs(r["u"]) + tu) + np.abs(silu_g) * tu + 2.0 ** -8 * np.abs(h_ref)


def check_h(H_gpu, gate, up, X_bits, rows=None):
    r = oracle.gate_up_silu(gate, up, X_bits, rows=rows)
    h = H_gpu.detach().float().cpu().double().numpy().reshape(r["h"].shape[0], -1)
    if rows is not None:
        h = h[:, rows]
    err = np.abs(h - r["h"])
    bad = err > h_bound(r, r["h"])
    assert not bad.any(), f"{bad.sum()} h values out of bound"


def check_mlp_e2e(Y_gpu, H_gpu, gate, up, down, X_bits, rows):
    """Dense MLP end to end against the pure FP64 oracle (h kept in FP64): on the
    given output rows, |y - y_oracle| <= TOL sum_i |d[r][i] h^[i]| + sum_i
    |d[r][i]| hb[i] (1.0001 slack for the bound's own rounding), hb the h bound of
    every intermediate -- the bound the gate/up and down checks imply."""
    r = oracle.gate_up_silu(gate, up, X_bits)
    hb = h_bound(r, r["h"])
    assert np.all(np.abs(H_gpu.detach().float().cpu().double().numpy().reshape(r["h"].shape) - r["h"]) <= hb)
    y_ref, _ = oracle.gemv(down["format"], down["codes"], down["scales"], down["tensor_scale"], r["h"], rows=rows)
    _, A_h = oracle.gemv(down["format"], down["codes"], down["scales"], down["tensor_scale"],
                         bits(H_gpu).reshape(r["h"].shape), rows=rows)
    _, A_hb = oracle.gemv(down["format"], down["codes"], down["scales"], down["tensor_scale"], hb, rows=rows)
    y = Y_gpu.detach().cpu().double().numpy().reshape(y_ref.shape[0], -1)[:, rows]
    bound = TOL * A_h + A_hb
    ratio = float(np.max(np.abs(y - y_ref) / np.maximum(bound, 1e-300)))
    log(f"mlp end-to-end against the derived bound: worst ratio {ratio:.3g}")
    assert np.all(np.abs(y - y_ref) <= 1.0001 * bound)


def build_moe(fmt, E, k, hidden, dff, seed, shared=True, tscales=(1.0, 1.0, 1.0), sh_tscales=(1.0, 1.0, 1.0),
              scales=None, sh_scales=None, act=0):
    """An MoE layer of E routed experts (and a shared one if `shared`), packed
    back to back.  tscales: the routed gate/up/down tensor scales (one per kind,
    as the layer descriptor holds them; NVFP4 only); sh_tscales: the shared
    expert's.  scales: optional {"gate"|"up"|"down": uint8 [E][rows][blocks]}
    replacing the drawn block scales of the routed experts; sh_scales the same
    for the shared expert ([rows][blocks] each).  Returns (layer,
    expert(e) -> host operands, shared host operands or None)."""
    pg = fg.packed_bytes(fmt, dff, hidden)
    pd = fg.packed_bytes(fmt, hidden, dff)
    bufs = {n: torch.empty(E * (pd if n == "down" else pg), dtype=torch.uint8, device=DEV) for n in ("gate", "up", "down")}
    logical = {}
    descs = {}
    kinds = (("gate", (dff, hidden)), ("up", (dff, hidden)), ("down", (hidden, dff)))
    for j, (n, (o, i)) in enumerate(kinds):
        mats = datagen.matrix(fmt, o, i, datagen.tensor_seed("moe", seed, n), device=DEV, batch=E)
        if scales is not None and n in scales:
            mats["scales"] = scales[n].to(DEV).contiguous()
        stride = pd if n == "down" else pg
        first = None
        for e in range(E):
            w = fg.pack(fmt, mats["codes"][e].contiguous(), mats["scales"][e].contiguous(), tscales[j], out=bufs[n],
                        offset=e * stride)
            if first is None:
                first = w
        first.desc.packed_bytes = bufs[n].numel()
        descs[n] = first
        logical[n] = mats
    sh = None
    sh_host = None
    if shared:
        sh, sh_host = [], {}
        for j, (n, (o, i)) in enumerate(kinds):
            if sh_scales is not None and n in sh_scales:
                mat = datagen.matrix(fmt, o, i, datagen.tensor_seed("moe-shared", seed, n), device=DEV)
                mat["scales"] = sh_scales[n].to(DEV).contiguous()
                W = fg.pack(fmt, mat["codes"], mat["scales"], sh_tscales[j])
                host = {"format": fmt, "codes": mat["codes"].cpu(), "scales": mat["scales"].cpu(),
                        "tensor_scale": sh_tscales[j]}
            else:
                W, host = make(fmt, o, i, seed=("shared", seed, n), tensor_scale=sh_tscales[j])
            sh.append(W)
            sh_host[n] = host
    layer = fg.moe_layer(descs["gate"], descs["up"], descs["down"], E, k, pg, pg, pd, shared=sh, act=act)
    layer.keep.append(bufs)

    def expert(e):
        return {n: {"format": fmt, "codes": logical[n]["codes"][e].cpu(), "scales": logical[n]["scales"][e].cpu(),
                    "tensor_scale": tscales[j]} for j, (n, _) in enumerate(kinds)}

    return layer, expert, sh_host


def check_moe(layer, expert, sh_host, X, logits, k, e2e_max=0.05):
    """Stage-wise MoE parity: ids exact, gate weights to 1e-5, every (token,
    chosen expert) intermediate within the h bound, the output given the GPU's own
    h and gate weights within the product bound.  End to end against the pure
    FP64 oracle: with bf16 activations within the bound those stages imply,
    |y - y_oracle| <= sum_j c_j ((TOL + 1e-5) sum_i |d_j[r][i] h^_j[i]|
    + sum_i |d_j[r][i]| hb_j[i]), hb_j the h bound of expert j's intermediate
    (the GPU's h, its gate weights and its down product each within their own
    bounds); with 8-bit activations reported and held under e2e_max of the
    tolerance scale.  A layer with 8-bit activations is checked against the W4A8
    oracle: each product's input quantised to MXFP8 (x for gate and up, the GPU's
    own bf16 h for down)."""
    from oracle import w4a8
    a8 = layer.desc.act == fg.ACT_MXFP8

    def product(mat, xbits):
        if a8:
            return w4a8.gemv(mat["format"], mat["codes"], mat["scales"], mat["tensor_scale"], xbits)
        return oracle.gemv(mat["format"], mat["codes"], mat["scales"], mat["tensor_scale"], xbits)
    M = X.shape[0]
    has_shared = sh_host is not None
    dff = layer.desc.d_ff
    nh = k + (1 if has_shared else 0)
    H = torch.empty((M, nh, dff), dtype=torch.bfloat16, device=DEV)
    Y, ids, w = fg.moe_route_gemv(layer, X, logits, H=H)
    torch.cuda.synchronize()
    rid, rw = oracle.topk_softmax(logits.cpu().numpy(), k)
    assert np.array_equal(ids.cpu().numpy(), rid), "top-k ids differ"
    wg = w.cpu().double().numpy()
    assert np.all(np.abs(wg - rw) <= 1e-5 * rw), "gate weights"
    Xb = bits(X)
    Hb = bits(H.view(M * nh, dff)).reshape(M, nh, dff)
    hbs = {}
    # stage 1: every (token, expert) intermediate
    for m in range(M):
        for j in range(nh):
            ex = expert(int(rid[m, j])) if j < k else sh_host
            g, Ag = product(ex["gate"], Xb[m][None, :])
            u, Au = product(ex["up"], Xb[m][None, :])
            r = {"h": oracle.silu_mul(g, u), "g": g, "u": u, "Ag": Ag, "Au": Au}
            h = H[m, j].float().cpu().double().numpy()[None, :]
            hb = h_bound(r, r["h"])
            assert np.all(np.abs(h - r["h"]) <= hb), (m, j)
            hbs[(m, j)] = hb
    # stage 2: combine given the GPU's own h and gate weights
    yg = Y.cpu().double().numpy()
    assert np.all(np.isfinite(yg))
    e2e_bound = np.zeros((M, layer.desc.hidden))
    for m in range(M):
        ref = np.zeros(layer.desc.hidden)
        tol = np.zeros(layer.desc.hidden)
        for j in range(nh):
            ex = expert(int(rid[m, j])) if j < k else sh_host
            d, Ad = product(ex["down"], Hb[m, j][None, :])
            c = wg[m, j] if j < k else 1.0
            ref += c * d[0]
            tol += c * Ad[0]
            if not a8:
                dn = ex["down"]
                _, Ahb = oracle.gemv(dn["format"], dn["codes"], dn["scales"], dn["tensor_scale"], hbs[(m, j)])
                e2e_bound[m] += (rw[m, j] if j < k else 1.0) * ((TOL + 1e-5) * Ad[0] + Ahb[0])
        assert np.all(np.abs(yg[m] - ref) <= TOL * tol), m
    # end to end against the pure FP64 oracle
    full = (w4a8.moe if a8 else oracle.moe)(expert, sh_host, Xb, logits.cpu().numpy(), k)
    e2e = float(np.max(np.abs(yg - full["y"]) / np.maximum(full["tol"], 1e-300)))
    log(f"moe end-to-end max |y - y_oracle| / sum(g A_down) = {e2e:.3g}")
    if a8:
        assert e2e < e2e_max
    else:
        ratio = np.abs(yg - full["y"]) / np.maximum(e2e_bound, 1e-300)
        log(f"moe end-to-end against the derived bound: worst ratio {float(ratio.max()):.3g}")
        assert np.all(np.abs(yg - full["y"]) <= 1.0001 * e2e_bound), "end to end"
    return ids
