"""Every block-scale code through every kernel path, and the MoE layer's less
common configurations, against the FP64 oracle.  Needs gfx950.

The drawn test matrices only reach a narrow band of scale codes (|z|/6 gives
E4M3 codes up to about 0x35 and E8M0 codes of about 117-128), so here scales are
set explicitly:

  * E4M3 (NVFP4): all 254 finite codes, the sign-bit codes 0x80-0xFE (negative
    block scales, which the format allows) and the subnormals included;
  * E8M0 (MXFP4): all 255 finite codes 0..254, in three bands of 85 codes with
    the input scaled by 2^85, 1 and 2^-85 so that every product, partial sum and
    result stays inside the FP32 normal range (an FP32 output cannot hold more).

One scale code per row, with x in {-1, 0, 1} times a power of two: every
partial sum is then a multiple of half the row's scale times |x| and below 2^24
of them, so any summation order is exact and each row must equal the oracle bit
for bit -- a wrong decode of any single code shows.  Row r = 64 g + l gets code
number (g + l) mod n, so every code meets every lane position (row within a
64-row group).  A second layout mixes the codes inside each row (every code once
per row) and is held to the product bound.
"""
import numpy as np
import pytest
import torch

import bit_weight_gemv_fp4_amd as fg
import datagen
import oracle
from gpu_common import DEV, bits, build_moe, check_h, check_moe, check_product, h_bound, log
from oracle import w4a8 as oracle_a8

pytestmark = pytest.mark.gpu

E4M3_CODES = [c for c in range(256) if (c & 0x7F) != 0x7F]          # 254 finite codes
E8M0_BANDS = ((0, 85, 85.0), (85, 170, 0.0), (170, 255, -85.0))      # (first, end, log2 |x|)


@pytest.fixture(scope="module", autouse=True)
def _gpu_and_native_library():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert fg.LIB_PATH.exists(), "the HIP library must be built"
    fg.lib()
    yield
    torch.cuda.synchronize()


def row_codes(codes, d_in, blk):
    """[64 n][d_in / blk] uint8: row 64 g + l carries codes[(g + l) % n] in every block."""
    n = len(codes)
    r = np.arange(64 * n)
    idx = (r // 64 + r % 64) % n
    return torch.from_numpy(np.repeat(np.asarray(codes, np.uint8)[idx][:, None], d_in // blk, axis=1)).to(DEV)


def mixed_codes(codes, d_out, blk):
    """[d_out][n]: row r carries codes[(r + b) % n] in block b (every code once per row)."""
    n = len(codes)
    r = np.arange(d_out)[:, None]
    b = np.arange(n)[None, :]
    return torch.from_numpy(np.asarray(codes, np.uint8)[(r + b) % n]).to(DEV)


def ternary(M, d_in, seed, log2_mag=0.0):
    g = torch.Generator(DEV).manual_seed(seed)
    X = torch.randint(-1, 2, (M, d_in), generator=g, device=DEV).to(torch.float32) * (2.0 ** log2_mag)
    return X.to(torch.bfloat16)


def exact_check(fmt, codes, scales, X, got, a8=False):
    ref = oracle_a8 if a8 else oracle
    Y, _ = ref.gemv(fmt, codes.cpu(), scales.cpu(), 1.0, bits(X))
    g = got.detach().cpu().double().numpy()
    bad = g != Y
    assert not bad.any(), f"{bad.sum()} rows differ (first at {np.argwhere(bad)[0].tolist()})"


@pytest.mark.parametrize("path,Ms", [(fg.PATH_VALU, (1, 5)), (fg.PATH_MFMA, (1, 5, 12))])
def test_every_e4m3_scale_code_exact(path, Ms):
    log("e4m3 sweep", path, Ms)
    d_in = 544
    sc = row_codes(E4M3_CODES, d_in, 16)
    d_out = sc.shape[0]
    mat = datagen.matrix(fg.NVFP4, d_out, d_in, datagen.tensor_seed("sweep4", d_in), device=DEV)
    W = fg.pack(fg.NVFP4, mat["codes"], sc)
    for M in Ms:
        X = ternary(M, d_in, 100 + M)
        exact_check(fg.NVFP4, mat["codes"], sc, X, fg.fp4_skinny_gemm(W, X, path=path))


@pytest.mark.parametrize("path,Ms", [(fg.PATH_VALU, (1, 5)), (fg.PATH_MFMA, (1, 5, 12))])
def test_every_e4m3_scale_code_mixed_in_rows(path, Ms):
    log("e4m3 mixed sweep", path, Ms)
    d_out = 130
    sc = mixed_codes(E4M3_CODES, d_out, 16)
    d_in = 16 * sc.shape[1]
    mat = datagen.matrix(fg.NVFP4, d_out, d_in, datagen.tensor_seed("sweep4m"), device=DEV)
    W = fg.pack(fg.NVFP4, mat["codes"], sc)
    host = {"format": fg.NVFP4, "codes": mat["codes"].cpu(), "scales": sc.cpu(), "tensor_scale": 1.0}
    for M in Ms:
        X = datagen.bf16_normal((M, d_in), datagen.tensor_seed("sweep4mX", M), device=DEV)
        check_product(fg.fp4_skinny_gemm(W, X, path=path), host, bits(X))


@pytest.mark.parametrize("path,Ms", [(fg.PATH_VALU, (1, 5)), (fg.PATH_MFMA, (1, 5, 12))])
def test_every_e4m3_scale_code_gate_up(path, Ms):
    """Gate and up both carry the sweep's scales (rows shifted between the two)."""
    log("e4m3 sweep gate/up", path, Ms)
    d_in = 288
    sc = row_codes(E4M3_CODES, d_in, 16)
    d_out = sc.shape[0]
    gm = datagen.matrix(fg.NVFP4, d_out, d_in, datagen.tensor_seed("sweepg"), device=DEV)
    um = datagen.matrix(fg.NVFP4, d_out, d_in, datagen.tensor_seed("sweepu"), device=DEV)
    su = torch.roll(sc, 37, dims=0).contiguous()
    Wg = fg.pack(fg.NVFP4, gm["codes"], sc)
    Wu = fg.pack(fg.NVFP4, um["codes"], su)
    hg = {"format": fg.NVFP4, "codes": gm["codes"].cpu(), "scales": sc.cpu(), "tensor_scale": 1.0}
    hu = {"format": fg.NVFP4, "codes": um["codes"].cpu(), "scales": su.cpu(), "tensor_scale": 1.0}
    for M in Ms:
        X = datagen.bf16_normal((M, d_in), datagen.tensor_seed("sweepgX", M), device=DEV)
        check_h(fg.fp4_gate_up_silu(Wg, Wu, X, path=path), hg, hu, bits(X))


@pytest.mark.parametrize("path,Ms", [(fg.PATH_VALU, (1, 5)), (fg.PATH_MFMA, (1, 5, 12)), (fg.PATH_A8, (1, 5, 12))])
@pytest.mark.parametrize("band", [0, 1, 2])
def test_every_e8m0_scale_code_exact(band, path, Ms):
    lo, hi, lx = E8M0_BANDS[band]
    log("e8m0 sweep", lo, hi, path, Ms)
    d_in = 544
    sc = row_codes(list(range(lo, hi)), d_in, 32)
    d_out = sc.shape[0]
    mat = datagen.matrix(fg.MXFP4, d_out, d_in, datagen.tensor_seed("sweep8", band), device=DEV)
    W = fg.pack(fg.MXFP4, mat["codes"], sc)
    for M in Ms:
        X = ternary(M, d_in, 200 + M + band, lx)
        exact_check(fg.MXFP4, mat["codes"], sc, X, fg.fp4_skinny_gemm(W, X, path=path), a8=path == fg.PATH_A8)


@pytest.mark.parametrize("band", [0, 1, 2])
def test_every_e8m0_scale_code_a8_gate_up(band):
    """W4A8 fused gate/up over a band of codes (the activation scale then meets
    every weight scale of the band inside the scaled matrix-core instruction)."""
    lo, hi, lx = E8M0_BANDS[band]
    log("e8m0 sweep a8 gate/up", lo, hi)
    d_in = 288
    sc = row_codes(list(range(lo, hi)), d_in, 32)
    d_out = sc.shape[0]
    gm = datagen.matrix(fg.MXFP4, d_out, d_in, datagen.tensor_seed("sw8g", band), device=DEV)
    um = datagen.matrix(fg.MXFP4, d_out, d_in, datagen.tensor_seed("sw8u", band), device=DEV)
    Wg = fg.pack(fg.MXFP4, gm["codes"], sc)
    Wu = fg.pack(fg.MXFP4, um["codes"], sc)
    for M in (1, 5):
        X = (datagen.bf16_normal((M, d_in), datagen.tensor_seed("sw8X", M), device=DEV).float()
             * 2.0 ** (lx - 20)).to(torch.bfloat16)
        H = fg.fp4_gate_up_silu(Wg, Wu, X, path=fg.PATH_A8)
        g, Ag = oracle_a8.gemv(fg.MXFP4, gm["codes"].cpu(), sc.cpu(), 1.0, bits(X))
        u, Au = oracle_a8.gemv(fg.MXFP4, um["codes"].cpu(), sc.cpu(), 1.0, bits(X))
        r = {"h": oracle.silu_mul(g, u), "g": g, "u": u, "Ag": Ag, "Au": Au}
        h = H.detach().float().cpu().double().numpy().reshape(M, -1)
        bad = np.abs(h - r["h"]) > h_bound(r, r["h"])
        assert not bad.any(), f"{bad.sum()} h values out of bound"


def _moe_band_scales(E, dff, hidden, lo, hi, kind):
    """Scales of E experts (the last of E is the shared expert's): `kind`
    ("gate_up" or "down") sweeps the band, one code per row; the other kind keeps
    codes 124..130 (2^-3..2^3)."""
    n = hi - lo
    out = {}
    for name, (o, i) in (("gate", (dff, hidden)), ("up", (dff, hidden)), ("down", (hidden, dff))):
        sweep = (kind == "gate_up") == (name != "down")
        r = np.arange(E * o).reshape(E, o)
        code = lo + (r + (7 if name == "up" else 0)) % n if sweep else 124 + r % 7
        out[name] = torch.from_numpy(np.repeat(code.astype(np.uint8)[:, :, None], i // 32, axis=2))
    return out


@pytest.mark.parametrize("M", [1, 4, 6])
@pytest.mark.parametrize("kind", ["gate_up", "down"])
@pytest.mark.parametrize("band", [0, 1, 2])
def test_every_e8m0_scale_code_moe(band, kind, M):
    """moe_route_gemv with the experts' gate/up (or down) scales sweeping a band of
    E8M0 codes; the input is scaled so that h and y stay in range (M = 1: the
    VALU kernels; 4: matrix-core gate/up; 6: both halves on the matrix cores)."""
    lo, hi, lx = E8M0_BANDS[band]
    log("e8m0 sweep moe", lo, hi, kind, M)
    E, k, hidden, dff = 16, 8, 256, 128
    sc = _moe_band_scales(E + 1, dff, hidden, lo, hi, kind)
    layer, expert, sh = build_moe(fg.MXFP4, E, k, hidden, dff, seed=("sweep", band, kind),
                                  scales={n: v[:E] for n, v in sc.items()}, sh_scales={n: v[E] for n, v in sc.items()})
    xmag = lx if kind == "gate_up" else lx / 2 - 4
    X = (datagen.bf16_normal((M, hidden), datagen.tensor_seed("swmX", M), device=DEV).float()
         * 2.0 ** xmag).to(torch.bfloat16)
    logits = datagen.router_logits(M, E, datagen.tensor_seed("swml", M, band), device=DEV)
    check_moe(layer, expert, sh, X, logits, k)


# ---- MoE configurations beyond the drawn ones --------------------------------------------------


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8])
def test_moe_nvfp4_experts_tensor_scales_no_shared(M):
    """NVFP4 experts with routed tensor scales other than 1 and no shared expert
    (M = 1, 2: VALU halves; 3, 4: matrix-core gate/up; 5, 8: both on the matrix
    cores)."""
    log("moe nvfp4 no shared", M)
    layer, expert, sh = build_moe(fg.NVFP4, 16, 4, 256, 128, seed=31, shared=False, tscales=(0.5, 2.0, 0.75))
    assert sh is None
    X = datagen.bf16_normal((M, 256), datagen.tensor_seed("mnx", M), device=DEV)
    logits = datagen.router_logits(M, 16, datagen.tensor_seed("mnl", M), device=DEV)
    check_moe(layer, expert, sh, X, logits, 4)


@pytest.mark.parametrize("M", [1, 3, 6])
def test_moe_nvfp4_experts_with_scaled_shared(M):
    """NVFP4 experts and a shared expert whose own tensor scales differ from the
    routed ones."""
    log("moe nvfp4 shared", M)
    layer, expert, sh = build_moe(fg.NVFP4, 16, 4, 256, 128, seed=32, tscales=(1.25, 0.5, 3.0),
                                  sh_tscales=(1.5, 0.25, 0.375))
    X = datagen.bf16_normal((M, 256), datagen.tensor_seed("msx", M), device=DEV)
    logits = datagen.router_logits(M, 16, datagen.tensor_seed("msl", M), device=DEV)
    check_moe(layer, expert, sh, X, logits, 4)


@pytest.mark.parametrize("M", [1, 4, 8])
def test_moe_mxfp4_no_shared(M):
    log("moe mxfp4 no shared", M)
    layer, expert, sh = build_moe(fg.MXFP4, 16, 8, 256, 128, seed=33, shared=False)
    X = datagen.bf16_normal((M, 256), datagen.tensor_seed("mmx", M), device=DEV)
    logits = datagen.router_logits(M, 16, datagen.tensor_seed("mml", M), device=DEV)
    check_moe(layer, expert, sh, X, logits, 8)
