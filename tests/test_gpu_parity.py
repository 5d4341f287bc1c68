"""GPU parity of every C-ABI entry point against the FP64 oracle.  Needs gfx950.

Bars:
  * packing / unpacking and top-k ids: bit-exact;
  * products: |y_gpu - y_ref| <= 2e-3 * sum_k |w x| per row (every product w x is
    exact in FP32, so only the FP32 summation rounds; a decode or layout slip
    breaks the bound);
  * fused h = bf16(SiLU(g) u): |h - h_ref| <= 1.1 tg (|u| + tu) + |SiLU(g)| tu + 2^-8 |h_ref|,
    with tg, tu the product bounds of g and u;
  * MoE gate weights: relative 1e-5; MoE output given the GPU's own h and gate
    weights: 2e-3 * (sum_j g_j A_down,j + A_down,shared).
Inputs are seeded synthetic tensors from datagen, drawn on the GPU and copied to
the host for the oracle.
"""
import sys

import numpy as np
import pytest
import torch

import bit_weight_gemv_fp4_amd as fg
import datagen
import oracle
from gpu_common import (DEV, TOL, bits, check_mlp_e2e, build_moe, check_h, check_moe, check_product, h_bound, log, make,
                        sample_rows)
from oracle import layout

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_and_native_library():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert fg.LIB_PATH.exists(), "the HIP library must be built"
    fg.lib()
    yield
    torch.cuda.synchronize()


# ---- packing -------------------------------------------------------------------------


@pytest.mark.parametrize("fmt", [fg.NVFP4, fg.MXFP4, fg.FP8_ROW])
@pytest.mark.parametrize("shape", [(1, 32), (64, 256), (70, 288), (130, 544), (5120, 5120)])
def test_pack_is_bit_exact_and_invertible(fmt, shape):
    log("pack", fmt, shape)
    W, host = make(fmt, *shape, seed=1)
    img = W.buf.cpu().numpy()
    ref = layout.pack(fmt, host["codes"].numpy(), host["scales"].numpy())
    assert img.size == ref.size and np.array_equal(img, ref)
    codes, scales = fg.unpack(W)
    assert torch.equal(codes.cpu(), host["codes"])
    assert torch.equal(scales.cpu().view(torch.uint8), host["scales"].contiguous().view(torch.uint8))
    assert fg.validate(W) == 0


def test_validate_counts_nan_codes():
    log("validate")
    mat = datagen.matrix(fg.NVFP4, 70, 288, 5, device=DEV)
    sc = mat["scales"].clone()
    sc[3, 2] = 0x7F
    sc[69, 17] = 0xFF
    W = fg.pack(fg.NVFP4, mat["codes"], sc)
    assert fg.validate(W) == 2
    mx = datagen.matrix(fg.MXFP4, 64, 256, 6, device=DEV)
    s2 = mx["scales"].clone()
    s2[0, 0] = 0xFF
    assert fg.validate(fg.pack(fg.MXFP4, mx["codes"], s2)) == 1
    f8 = datagen.matrix(fg.FP8_ROW, 64, 256, 7, device=DEV)
    c3 = f8["codes"].clone()
    c3[5, 5] = 0x7F
    s3 = f8["scales"].clone()
    s3[9] = float("inf")
    assert fg.validate(fg.pack(fg.FP8_ROW, c3, s3)) == 2


# ---- single vector products ---------------------------------------------------------------


@pytest.mark.parametrize("fmt", [fg.NVFP4, fg.MXFP4])
@pytest.mark.parametrize("shape", [(1, 32), (64, 256), (70, 288), (200, 1056), (777, 4128), (5120, 5120)])
def test_gemv_matches_oracle(fmt, shape):
    log("gemv", fmt, shape)
    W, host = make(fmt, *shape, seed=2)
    x = datagen.bf16_normal((shape[1],), datagen.tensor_seed("x", shape), device=DEV)
    y = fg.fp4_gemv(W, x)
    check_product(y, host, bits(x)[None, :])


def test_gemv_tensor_scale():
    log("tensor scale")
    mat = datagen.matrix(fg.NVFP4, 130, 544, 8, device=DEV)
    x = datagen.bf16_normal((544,), 3, device=DEV)
    for ts in (0.5, 3.75, 1e-3):
        W = fg.pack(fg.NVFP4, mat["codes"], mat["scales"], ts)
        host = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in mat.items()}
        host["tensor_scale"] = ts
        check_product(fg.fp4_gemv(W, x), host, bits(x)[None, :])


PATHS = [fg.PATH_VALU, fg.PATH_MFMA]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("fmt", [fg.NVFP4, fg.MXFP4])
def test_skinny_matches_oracle(fmt, M, path):
    log("skinny", fmt, M, path)
    for shape in ((200, 1056), (5120, 5120)):
        W, host = make(fmt, *shape, seed=3)
        X = datagen.bf16_normal((M, shape[1]), datagen.tensor_seed("X", M, shape), device=DEV)
        Y = fg.fp4_skinny_gemm(W, X, path=path)
        check_product(Y, host, bits(X))


@pytest.mark.parametrize("M", [1, 4, 8])
def test_lmhead_matches_oracle(M):
    log("lmhead", M)
    for shape in ((300, 544), (1, 32), (2048, 2560)):
        W, host = make(fg.FP8_ROW, *shape, seed=4)
        X = datagen.bf16_normal((M, shape[1]), datagen.tensor_seed("Xh", M, shape), device=DEV)
        check_product(fg.fp8_lmhead_gemv(W, X), host, bits(X))


def f32_argmax(L):
    """Per row of L (float32), the column of the largest value, the lower column
    on ties (-0 == +0): the pick the kernel must make from its own FP32 logits."""
    L = np.where(L == 0, np.float32(0), L)
    return np.argmax(L, axis=1)


@pytest.mark.parametrize("M", [1, 4, 8])
def test_lmhead_argmax(M):
    """Fused greedy pick: logits within the bound, the pick is the FP32 arg-max of
    those very logits, its value is that logit, and the oracle's best row is
    within the bound of it; also on a row range (a draft head's rows)."""
    log("lmhead argmax", M)
    W, host = make(fg.FP8_ROW, 1000, 544, seed=40)
    X = datagen.bf16_normal((M, 544), datagen.tensor_seed("am", M), device=DEV)
    Y, A = oracle.gemv(fg.FP8_ROW, host["codes"], host["scales"], 1.0, bits(X))
    for rb, n in ((0, 1000), (128, 300), (960, 40), (0, 64)):
        idx, val, L = fg.fp8_lmhead_argmax(W, X, rb, n, logits=True)
        Lh = L.cpu().numpy()
        check_product(L, {**host, "codes": host["codes"][rb:rb + n], "scales": host["scales"][rb:rb + n]}, bits(X))
        pick = f32_argmax(Lh) + rb
        assert np.array_equal(idx.cpu().numpy(), pick), (rb, n)
        assert np.array_equal(val.cpu().numpy(), Lh[np.arange(M), pick - rb]), (rb, n)
        best = np.argmax(Y[:, rb:rb + n], axis=1)
        assert np.all(Y[np.arange(M), idx.cpu().numpy()] >= Y[np.arange(M), best + rb] - 2 * TOL * A.max()), (rb, n)
        # no logits requested: the same pick
        idx2, val2, _ = fg.fp8_lmhead_argmax(W, X, rb, n)
        assert torch.equal(idx2, idx) and torch.equal(val2, val)


def test_lmhead_argmax_ties_pick_the_lower_row():
    log("lmhead argmax ties")
    mat = datagen.matrix(fg.FP8_ROW, 320, 256, 41, device=DEV)
    codes = mat["codes"][:1].repeat(320, 1).contiguous()       # every row the same
    scales = torch.full((320,), 0.01, dtype=torch.float32, device=DEV)
    W = fg.pack(fg.FP8_ROW, codes, scales)
    X = datagen.bf16_normal((3, 256), 42, device=DEV)
    for rb in (0, 64, 192):
        idx, val, _ = fg.fp8_lmhead_argmax(W, X, rb, 320 - rb)
        assert idx.tolist() == [rb] * 3


@pytest.mark.parametrize("M", [1, 4])
def test_lmhead_argmax_full_vocabulary(M):
    """The dense model's 248320-row head (M = 1) and the MoE model's 157184-row head
    (M = 4) against the full FP64 oracle."""
    log("lmhead argmax full", M)
    V, d = (datagen.VOCAB, datagen.HIDDEN) if M == 1 else (datagen.MOE_VOCAB, datagen.MOE_HIDDEN)
    W, host = make(fg.FP8_ROW, V, d, seed=43)
    X = datagen.bf16_normal((M, d), datagen.tensor_seed("amf", M), device=DEV)
    idx, val, L = fg.fp8_lmhead_argmax(W, X, logits=True)
    Lh = L.cpu().numpy()
    assert np.array_equal(idx.cpu().numpy(), f32_argmax(Lh))
    Y, A = oracle.gemv(fg.FP8_ROW, host["codes"], host["scales"], 1.0, bits(X))
    assert np.all(np.abs(Lh.astype(np.float64) - Y) <= TOL * A)
    i = idx.cpu().numpy().astype(np.int64)
    assert np.all(Y[np.arange(M), i] >= Y.max(axis=1) - 2 * TOL * A.max(axis=1))


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("M", [1, 2, 4, 5, 8])
@pytest.mark.parametrize("fmt", [fg.NVFP4, fg.MXFP4])
def test_gate_up_silu_matches_oracle(fmt, M, path):
    log("gate_up", fmt, M, path)
    for shape in ((200, 1056), (130, 544)):
        Wg, hg = make(fmt, *shape, seed=5)
        Wu, hu = make(fmt, *shape, seed=6)
        X = datagen.bf16_normal((M, shape[1]), datagen.tensor_seed("Xg", M, shape), device=DEV)
        H = fg.fp4_gate_up_silu(Wg, Wu, X, path=path)
        check_h(H, hg, hu, bits(X))


# ---- load-time quantisers ------------------------------------------------------------------------
from oracle import quant as oq  # noqa: E402


def quant_inputs(d_out, d_in, seed):
    """Normal weights with outliers, an all-zero block, tiny values (E4M3/E8M0
    subnormal range) and mixed signs, as bf16."""
    g = torch.Generator("cpu").manual_seed(seed)
    w = torch.randn((d_out, d_in), generator=g)
    w[0, :32] = 0.0
    w[1, 5] = 300.0
    w[2, :64] *= 1e-5
    w[3] = torch.randn(d_in, generator=g) * 1e-30
    return w.to(torch.bfloat16)


def check_quant_exact(fmt, w_bf16, label):
    """The kernel's codes, scales and tensor scale against the exact-decision
    oracle, bit for bit.  The oracle's marks (decisions within 2^-22 of a
    midpoint, where an FP32-quotient order could differ) are counted and
    reported: the kernel decides those exactly too, so none may differ."""
    codes, scales, ts = fg.quantize(fmt, w_bf16.to(DEV))
    ref = oq.quantize_detail(fmt, w_bf16.cpu().view(torch.int16).numpy().view(np.uint16))
    n_marked = int(ref["el_amb"].sum()) + int(ref.get("scale_amb", np.zeros(1, bool)).sum())
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    n_diff = int((oq.elements_of(fmt, gc) != ref["el"]).sum())
    n_diff += int((gs.view(np.uint32) != np.asarray(ref["scales"]).view(np.uint32)).sum()) if fmt == fg.FP8_ROW \
        else int((gs != ref["scales"]).sum())
    log(f"quantize {label} fmt={fmt}: {ref['el'].size} elements, {n_marked} decisions near a midpoint, {n_diff} differ")
    assert np.float32(ts).view(np.uint32) == np.float32(ref["tensor_scale"]).view(np.uint32)
    assert n_diff == 0
    assert np.array_equal(gc, ref["codes"])
    return codes, scales, ts


@pytest.mark.parametrize("fmt", [fg.NVFP4, fg.MXFP4, fg.FP8_ROW])
@pytest.mark.parametrize("shape", [(130, 544), (256, 2048)])
def test_quantize_matches_exact_oracle(fmt, shape):
    log("quantize", fmt, shape)
    check_quant_exact(fmt, quant_inputs(*shape, seed=shape[0] + fmt), shape)


def midpoint_inputs(fmt, seed, d_out=64, d_in=512):
    """Weights placed exactly on rounding midpoints of the decoded scale (a
    power-of-two tensor / row scale makes every quotient exact in FP32 too) and
    one bf16 step either side of them, mixed with normal weights."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((d_out, d_in))
    mids2 = oq._MID_E2M1
    mids8 = oq._MID_E4M3
    if fmt == fg.FP8_ROW:
        for r in range(d_out):
            s = 2.0 ** int(rng.integers(-8, 3))
            w[r, 0] = 448.0 * s
            k = 1 + np.arange(128)
            w[r, k] = mids8[rng.integers(0, 125, 128)] * s * np.where(rng.random(128) < .5, -1, 1)
    else:
        blk = 16 if fmt == fg.NVFP4 else 32
        s_t = 2.0 ** -6 if fmt == fg.NVFP4 else 1.0
        for r in range(d_out):
            for b in range(d_in // blk):
                sb = oq._E4M3[int(rng.integers(48, 110))] if fmt == fg.NVFP4 else 2.0 ** int(rng.integers(-8, 8))
                w[r, blk * b] = 6.0 * sb * s_t
                k = blk * b + 1 + np.arange(blk // 2)
                w[r, k] = mids2[rng.integers(0, 7, blk // 2)] * sb * s_t * np.where(rng.random(blk // 2) < .5, -1, 1)
        if fmt == fg.NVFP4:
            w[0, 0] = 2688.0 * s_t
    wt = torch.from_numpy(w.astype(np.float32)).to(torch.bfloat16)
    # one bf16 step up or down on a quarter of the entries
    nudge = torch.from_numpy(rng.integers(-1, 2, w.shape).astype(np.int16)) * torch.from_numpy(rng.random(w.shape) < 0.25)
    bits = (wt.view(torch.int16).to(torch.int32) + nudge.to(torch.int32)).to(torch.int16)
    bits[0, 0] = wt.view(torch.int16)[0, 0]
    bits[:, 0] = wt.view(torch.int16)[:, 0]
    return bits.view(torch.bfloat16)


@pytest.mark.parametrize("fmt", [fg.NVFP4, fg.MXFP4, fg.FP8_ROW])
def test_quantize_midpoints_ties_to_even(fmt):
    """Exact midpoints go to the even code and their bf16 neighbours to the
    nearer side, bit-exact against the exact oracle."""
    log("quantize midpoints", fmt)
    check_quant_exact(fmt, midpoint_inputs(fmt, 20 + fmt), "midpoints")


def test_quantize_then_product():
    """Quantise -> pack -> product: within the product bound of the oracle's
    GEMV of the quantised matrix, and within the quantisation error of the bf16
    matrix's exact product: |y - W x| <= sum_k |x_k| e_k + bound, with e_k the
    largest rounding error of element k: half the widest E2M1 step (1) times the
    decoded block scale, or, where the block scale rounded down far enough that
    the block maximum saturates (a zero or subnormal E4M3 scale), the block
    maximum's excess over 6 times it; MXFP4 never saturates; for FP8 rows
    2^-4 |w| + half the smallest E4M3 step times the row scale."""
    log("quantize -> gemv")
    w = quant_inputs(192, 1024, 7).to(DEV)
    x = datagen.bf16_normal((1024,), 8, device=DEV)
    wd = w.double().cpu().numpy()
    xd = x.double().cpu().numpy()
    exact = wd @ xd
    for fmt in (fg.NVFP4, fg.MXFP4, fg.FP8_ROW):
        codes, scales, ts = check_quant_exact(fmt, w, "product")
        W = fg.pack(fmt, codes, scales, ts)
        y = (fg.fp8_lmhead_gemv(W, x) if fmt == fg.FP8_ROW else fg.fp4_gemv(W, x)).reshape(-1)
        host = {"format": fmt, "codes": codes.cpu(), "scales": scales.cpu(), "tensor_scale": ts}
        check_product(y, host, bits(x)[None, :])
        sc = scales.cpu().numpy()
        if fmt == fg.NVFP4:
            sb = oq._E4M3[sc] * ts
            amax_b = np.abs(wd).reshape(wd.shape[0], -1, 16).max(-1)
            e = np.repeat(np.maximum(sb, amax_b - 6.0 * sb), 16, axis=1)
        elif fmt == fg.MXFP4:
            e = np.repeat(np.exp2(sc.astype(np.float64) - 127), 32, axis=1)
        else:
            e = 2.0 ** -4 * np.abs(wd) + 2.0 ** -10 * sc.astype(np.float64)[:, None]
        _, A = oracle.gemv(fmt, codes.cpu(), scales.cpu(), ts, bits(x)[None, :])
        bound = e @ np.abs(xd) + TOL * A[0]
        err = np.abs(y.cpu().double().numpy() - exact)
        assert np.all(err <= bound), (fmt, float(np.max(err / bound)))


# ---- special cases: bit-exact ------------------------------------------------------------------


@pytest.mark.parametrize("fmt", [fg.NVFP4, fg.MXFP4, fg.FP8_ROW])
def test_one_hot_gives_exact_column(fmt):
    log("one-hot", fmt)
    d_out, d_in = 130, 544
    W, host = make(fmt, d_out, d_in, seed=9)
    Wd = oracle.dequant(fmt, host["codes"], host["scales"], host["tensor_scale"])
    for k in (0, 1, 31, 256, 543):
        x = torch.zeros(d_in, dtype=torch.bfloat16, device=DEV)
        x[k] = 1.0
        y = fg.fp8_lmhead_gemv(W, x) if fmt == fg.FP8_ROW else fg.fp4_gemv(W, x)
        # one exact product per output, rounded once to FP32 (FP8: code x row scale
        # can exceed 24 significant bits; FP4 products are exact in FP32)
        assert np.array_equal(y.cpu().double().numpy(), Wd[:, k].astype(np.float32).astype(np.float64)), k


def test_exact_sums_are_bit_exact():
    # scales all 1.0 (E4M3 0x38) and x in {-1, 0, 1}: every partial sum is a multiple
    # of 0.5 far below 2^24, so any summation order is exact
    log("exact sums")
    d_out, d_in = 640, 5120
    mat = datagen.matrix(fg.NVFP4, d_out, d_in, 10, device=DEV)
    sc = torch.full_like(mat["scales"], 0x38)
    W = fg.pack(fg.NVFP4, mat["codes"], sc)
    x = (torch.randint(-1, 2, (d_in,), generator=torch.Generator(DEV).manual_seed(4), device=DEV)).to(torch.bfloat16)
    Y, _ = oracle.gemv(fg.NVFP4, mat["codes"].cpu(), sc.cpu(), 1.0, bits(x)[None, :])
    assert np.array_equal(fg.fp4_gemv(W, x).cpu().double().numpy(), Y[0])


def test_sign_flip_and_determinism():
    log("sign flip")
    mat = datagen.matrix(fg.NVFP4, 5120, 5120, 11, device=DEV)
    x = datagen.bf16_normal((5120,), 12, device=DEV)
    W = fg.pack(fg.NVFP4, mat["codes"], mat["scales"])
    Wn = fg.pack(fg.NVFP4, mat["codes"] ^ 0x88, mat["scales"])
    y1 = fg.fp4_gemv(W, x).clone()
    y2 = fg.fp4_gemv(W, x).clone()
    yn = fg.fp4_gemv(Wn, x).clone()
    assert torch.equal(y1, y2)
    assert torch.equal(yn, -y1)
    assert torch.equal(fg.fp4_gemv(W, -x), -y1)


def exact_scales(fmt, shape, gen):
    """Power-of-two block scales (0.5, 1, 2 or 4): with x in {-1, 0, 1} every
    partial sum is a multiple of 1/4 below 2^19, so any summation order is exact
    and every path must return the oracle's value bit for bit -- also where a
    scale is applied to the wrong row or block."""
    n = shape[0] * (shape[1] // (16 if fmt == fg.NVFP4 else 32))
    pick = torch.randint(0, 4, (n,), generator=gen, device=DEV)
    if fmt == fg.NVFP4:  # E4M3 2^e: bits (e + 7) << 3
        codes = ((pick + 6) << 3).to(torch.uint8)
    else:  # E8M0 2^e: e + 127
        codes = (pick + 126).to(torch.uint8)
    return codes.view(shape[0], -1)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("fmt", [fg.NVFP4, fg.MXFP4])
def test_exact_sums_with_mixed_scales(fmt, path):
    log("exact mixed scales", fmt, path)
    for shape in ((130, 1056), (200, 5120), (64, 17408)):
        gen = torch.Generator(DEV).manual_seed(shape[0] + shape[1])
        mat = datagen.matrix(fmt, *shape, datagen.tensor_seed("exact", fmt, shape), device=DEV)
        sc = exact_scales(fmt, shape, gen)
        W = fg.pack(fmt, mat["codes"], sc)
        for M in (1, 3, 4, 5, 8):
            X = torch.randint(-1, 2, (M, shape[1]), generator=gen, device=DEV).to(torch.bfloat16)
            Y, _ = oracle.gemv(fmt, mat["codes"].cpu(), sc.cpu(), 1.0, bits(X))
            got = fg.fp4_skinny_gemm(W, X, path=path)
            assert np.array_equal(got.cpu().double().numpy(), Y), (shape, M)


# ---- full-size shapes on the VALU kernel, exact sums ---------------------------------------------
# The dense shapes and a few ragged and narrow ones: the launch plans they get
# (one to five workgroups per row group, 4 to 16 waves, ragged rows and columns,
# 18 workgroups on one row group for 1088x17408 at the wider vector counts)
# must all return the exact sums.


FULL_SHAPES = [(5120, 5120), (4160, 4096), (1088, 17408), (5152, 5152), (5120, 17408), (17408, 5120)]


@pytest.mark.parametrize("M", [1, 2, 5, 8])
@pytest.mark.parametrize("fmt", [fg.NVFP4, fg.MXFP4])
def test_full_size_exact_sums_valu(fmt, M):
    """Power-of-two block scales and x in {-1, 0, 1}: every row equals the oracle
    bit for bit on the VALU kernel (a row group summed by the wrong workgroups or
    waves, a partial added twice or lost breaks this), and a second call repeats
    the bits."""
    log("full-size exact", fmt, M)
    for shape in FULL_SHAPES:
        gen = torch.Generator(DEV).manual_seed(shape[0] * 7 + shape[1] + M)
        mat = datagen.matrix(fmt, *shape, datagen.tensor_seed("even", fmt, shape), device=DEV)
        sc = exact_scales(fmt, shape, gen)
        W = fg.pack(fmt, mat["codes"], sc)
        X = torch.randint(-1, 2, (M, shape[1]), generator=gen, device=DEV).to(torch.bfloat16)
        Y, _ = oracle.gemv(fmt, mat["codes"].cpu(), sc.cpu(), 1.0, bits(X))
        got = fg.fp4_skinny_gemm(W, X, path=fg.PATH_VALU).clone()
        assert np.array_equal(got.cpu().double().numpy(), Y), shape
        assert torch.equal(fg.fp4_skinny_gemm(W, X, path=fg.PATH_VALU), got), shape


@pytest.mark.parametrize("M", [1, 2, 3])
def test_grouped_exact_sums_ragged_members(M):
    """Members of 4000, 70 and 1000 rows in one launch (ragged member ends),
    exact sums bit for bit."""
    log("grouped exact", M)
    shapes = [(4000, 5120), (70, 5120), (1000, 5120)]
    gen = torch.Generator(DEV).manual_seed(91 + M)
    mats, Ws = [], []
    for j, shape in enumerate(shapes):
        mat = datagen.matrix(fg.NVFP4, *shape, datagen.tensor_seed("evg", j), device=DEV)
        sc = exact_scales(fg.NVFP4, shape, gen)
        mats.append((mat, sc))
        Ws.append(fg.pack(fg.NVFP4, mat["codes"], sc))
    X = torch.randint(-1, 2, (M, 5120), generator=gen, device=DEV).to(torch.bfloat16)
    Ys = fg.fp4_gemv_grouped(fg.Group(Ws), X, path=fg.PATH_VALU)
    for (mat, sc), Yg in zip(mats, Ys):
        Y, _ = oracle.gemv(fg.NVFP4, mat["codes"].cpu(), sc.cpu(), 1.0, bits(X))
        assert np.array_equal(Yg.cpu().double().numpy(), Y)


@pytest.mark.parametrize("M", [1, 2, 4])
def test_gate_up_and_fp8_ragged_full_size(M):
    """Fused gate/up (NVFP4 and FP8 pairs) and FP8 row products on the VALU
    kernel, against the oracle's bounds, on shapes with ragged rows and columns;
    repeated calls give the same bits."""
    log("gate/up, fp8 ragged", M)
    for fmt, shape in ((fg.NVFP4, (5152, 2080)), (fg.FP8_ROW, (2080, 2080))):
        Wg, hg = make(fmt, *shape, seed=("evgu", 0))
        Wu, hu = make(fmt, *shape, seed=("evgu", 1))
        X = datagen.bf16_normal((M, shape[1]), datagen.tensor_seed("evguX", M, fmt), device=DEV)
        H = fg.fp4_gate_up_silu(Wg, Wu, X, path=fg.PATH_VALU)
        check_h(H, hg, hu, bits(X))
        assert torch.equal(fg.fp4_gate_up_silu(Wg, Wu, X, path=fg.PATH_VALU), H)
    for shape in ((5120, 5120), (5152, 2080)):
        W, host = make(fg.FP8_ROW, *shape, seed="ev8")
        X = datagen.bf16_normal((M, shape[1]), datagen.tensor_seed("ev8X", M), device=DEV)
        check_product(fg.fp8_lmhead_gemv(W, X), host, bits(X))


# ---- split-K exchange tree and grouped launches ----------------------------------------------


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("M", [1, 2, 3, 8])
def test_split_k_tree_exact_for_every_split_count(M, path):
    """Exact-sum inputs (scales 1.0, x in {-1,0,1}) at widths that give 2..63
    workgroups per row group, power of two or not: every tree shape must return
    the exact sum, bit for bit, and a second call the same bits."""
    log("tree exact", M, path)
    for C in (8, 12, 20, 28, 36, 60, 124, 252):
        d_out, d_in = 130, 256 * C
        mat = datagen.matrix(fg.NVFP4, d_out, d_in, datagen.tensor_seed("tree", C), device=DEV)
        sc = torch.full_like(mat["scales"], 0x38)
        W = fg.pack(fg.NVFP4, mat["codes"], sc)
        g = torch.Generator(DEV).manual_seed(C * 10 + M)
        X = torch.randint(-1, 2, (M, d_in), generator=g, device=DEV).to(torch.bfloat16)
        Y, _ = oracle.gemv(fg.NVFP4, mat["codes"].cpu(), sc.cpu(), 1.0, bits(X))
        got = fg.fp4_skinny_gemm(W, X, path=path).clone()
        assert np.array_equal(got.cpu().double().numpy(), Y), C
        assert torch.equal(fg.fp4_skinny_gemm(W, X, path=path), got), C


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("M", [1, 3, 8])
@pytest.mark.parametrize("fmt", [fg.NVFP4, fg.MXFP4])
def test_grouped_matches_oracle(fmt, M, path):
    """Ragged members (1, 70, 200 and 64 rows) of one input in one launch."""
    log("grouped", fmt, M, path)
    shapes = [(70, 1056), (1, 1056), (200, 1056), (64, 1056)]
    mats = [make(fmt, o, i, seed=("grp", j)) for j, (o, i) in enumerate(shapes)]
    X = datagen.bf16_normal((M, 1056), datagen.tensor_seed("grpX", M), device=DEV)
    for n in (1, 2, 4):
        G = fg.Group([W for W, _ in mats[:n]])
        Ys = fg.fp4_gemv_grouped(G, X, path=path)
        for (W, host), Y in zip(mats[:n], Ys):
            check_product(Y, host, bits(X))


def test_grouped_qkv_full_size():
    """The three projections of the dense attention block that read the hidden
    vector (12288, 12288 and 7680 rows of 5120), sampled rows, M = 1 and 4; the
    grouped results agree with single-matrix calls and repeat bit for bit."""
    log("grouped qkv")
    shapes = [s for s in datagen.ATTN_SHAPES if s[1] == datagen.HIDDEN]
    mats = [make(fg.NVFP4, o, i, seed=("qkv", j)) for j, (o, i) in enumerate(shapes)]
    G = fg.Group([W for W, _ in mats])
    for M in (1, 4):
        X = datagen.bf16_normal((M, datagen.HIDDEN), datagen.tensor_seed("qkvX", M), device=DEV)
        Ys = [y.clone() for y in fg.fp4_gemv_grouped(G, X)]
        again = fg.fp4_gemv_grouped(G, X)
        for (W, host), Y, Y2 in zip(mats, Ys, again):
            assert torch.equal(Y, Y2)
            check_product(Y, host, bits(X), rows=sample_rows(W.d_out, 128, seed=M))
            single = fg.fp4_skinny_gemm(W, X)
            scale = single.abs().max().item()
            assert (single - Y).abs().max().item() <= 1e-5 * scale


# ---- the workloads at full size (sampled rows where the oracle would be slow) -----------


def test_config1_gemv_5120():
    log("C1")
    W, host = make(fg.NVFP4, 5120, 5120, seed=100)
    x = datagen.bf16_normal((5120,), 101, device=DEV)
    check_product(fg.fp4_gemv(W, x), host, bits(x)[None, :])


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_config2_and_4_mlp(M, path):
    """Dense MLP: gate/up 17408x5120 fused with SiLU*mul, then down 5120x17408."""
    log("C2/C4 MLP", M, path)
    Wg, hg = make(fg.NVFP4, 17408, 5120, seed=200)
    Wu, hu = make(fg.NVFP4, 17408, 5120, seed=201)
    Wd, hd = make(fg.NVFP4, 5120, 17408, seed=202)
    X = datagen.bf16_normal((M, 5120), datagen.tensor_seed("C2x", M), device=DEV)
    H = fg.fp4_gate_up_silu(Wg, Wu, X, path=path)
    Y = fg.fp4_skinny_gemm(Wd, H, path=path)
    rows = sample_rows(17408, 160, seed=M)
    check_h(H, hg, hu, bits(X), rows=rows)
    drows = sample_rows(5120, 160, seed=M + 10)
    check_product(Y, hd, bits(H), rows=drows)  # down, given the GPU's own h
    check_mlp_e2e(Y, H, hg, hu, hd, bits(X), drows)  # end to end, h in FP64


@pytest.mark.parametrize("shape", [(12288, 5120), (5120, 12288), (7680, 5120)])
def test_config3_attention_shapes(shape):
    log("C3 attn", shape)
    W, host = make(fg.NVFP4, *shape, seed=300)
    x = datagen.bf16_normal((shape[1],), 301, device=DEV)
    check_product(fg.fp4_gemv(W, x), host, bits(x)[None, :], rows=sample_rows(shape[0]))


def test_config3_lm_head():
    log("C3 head")
    W, host = make(fg.FP8_ROW, 248320, 5120, seed=310)
    x = datagen.bf16_normal((1, 5120), 311, device=DEV)
    check_product(fg.fp8_lmhead_gemv(W, x), host, bits(x), rows=sample_rows(248320, 400))


# ---- MoE --------------------------------------------------------------------------------------


@pytest.mark.parametrize("M", [1, 2, 3, 5, 8])
def test_moe_small(M):
    log("moe small", M)
    layer, expert, sh = build_moe(fg.MXFP4, 16, 4, 256, 128, seed=1)
    X = datagen.bf16_normal((M, 256), datagen.tensor_seed("mx", M), device=DEV)
    logits = datagen.router_logits(M, 16, datagen.tensor_seed("ml", M), device=DEV)
    check_moe(layer, expert, sh, X, logits, 4)


def test_moe_ties_and_repeat():
    log("moe ties")
    layer, expert, sh = build_moe(fg.MXFP4, 16, 4, 256, 128, seed=2)
    X = datagen.bf16_normal((3, 256), 1, device=DEV)
    logits = torch.zeros((3, 16), dtype=torch.float32, device=DEV)
    logits[1, 5] = 1.0
    logits[2] = torch.tensor([0.5, -1, 0.5, 0.25] * 4, device=DEV)
    logits[0, 3] = -0.0  # a negative zero ties with the positive zeros
    ids = check_moe(layer, expert, sh, X, logits, 4)
    assert ids[0].tolist() == [0, 1, 2, 3]
    Y1, _, _ = fg.moe_route_gemv(layer, X, logits)
    Y2, _, _ = fg.moe_route_gemv(layer, X, logits)
    assert torch.equal(Y1, Y2)


@pytest.mark.parametrize("M", [1, 3, 4, 6, 8])
def test_config5_moe_layer(M):
    """Ling-3.0-flash-shaped MoE layer: 512 MXFP4 experts 768x2560 / 2560x768, top-8 + shared
    (M = 1: VALU gate/up and down; 3, 4: matrix-core gate/up whose workgroups route the
    tokens themselves; 6, 8: a routing launch, then both halves on the matrix cores)."""
    log("C5 moe", M)
    layer, expert, sh = build_moe(fg.MXFP4, 512, 8, 2560, 768, seed=5)
    X = datagen.bf16_normal((M, 2560), datagen.tensor_seed("C5x", M), device=DEV)
    logits = datagen.router_logits(M, 512, datagen.tensor_seed("C5l", M), device=DEV)
    check_moe(layer, expert, sh, X, logits, 8)


@pytest.mark.parametrize("M", [4, 6])
def test_config5_moe_layer_nvfp4(M):
    """The same layer with NVFP4 experts and tensor scales other than 1 (the
    matrix-core gate/up without a K split once the union's row groups fill the
    CUs; at M = 4 the VALU down with one chunk per wave)."""
    log("C5 moe nvfp4", M)
    layer, expert, sh = build_moe(fg.NVFP4, 512, 8, 2560, 768, seed=6, tscales=(0.5, 2.0, 1.5),
                                  sh_tscales=(1.25, 0.75, 2.0))
    X = datagen.bf16_normal((M, 2560), datagen.tensor_seed("C5nx", M), device=DEV)
    logits = datagen.router_logits(M, 512, datagen.tensor_seed("C5nl", M), device=DEV)
    check_moe(layer, expert, sh, X, logits, 8)


def test_config5_lm_head():
    log("C5 head")
    W, host = make(fg.FP8_ROW, 157184, 2560, seed=500)
    X = datagen.bf16_normal((4, 2560), 501, device=DEV)
    check_product(fg.fp8_lmhead_gemv(W, X), host, bits(X), rows=sample_rows(157184, 300))


def test_workspace_reuse_across_shapes():
    """One workspace shared by calls of different shapes (split-K counters must
    start at zero for each)."""
    log("workspace reuse")
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
    for shape in ((777, 4128), (5120, 5120), (200, 1056), (5120, 17408), (777, 4128)):
        W, host = make(fg.NVFP4, *shape, seed=20)
        x = datagen.bf16_normal((shape[1],), 21, device=DEV)
        y = fg.fp4_gemv(W, x, ws=ws)
        check_product(y, host, bits(x)[None, :], rows=sample_rows(shape[0], 64))
        X = datagen.bf16_normal((3, shape[1]), 22, device=DEV)
        Y = fg.fp4_skinny_gemm(W, X, ws=ws)
        check_product(Y, host, bits(X), rows=sample_rows(shape[0], 64))


# ---- wider verify blocks: 9..16 vectors on the matrix-core kernel -----------------------------


@pytest.mark.parametrize("path", [fg.PATH_AUTO, fg.PATH_MFMA])
@pytest.mark.parametrize("M", [9, 11, 16])
@pytest.mark.parametrize("fmt", [fg.NVFP4, fg.MXFP4])
def test_wide_verify_skinny_matches_oracle(fmt, M, path):
    """A verify block of K + 1 = 9..16 positions (the feed verifies up to 11)."""
    log("wide skinny", fmt, M, path)
    for shape in ((200, 1056), (70, 288), (5120, 5120)):
        W, host = make(fmt, *shape, seed=3)
        X = datagen.bf16_normal((M, shape[1]), datagen.tensor_seed("Xw", M, shape), device=DEV)
        Y = fg.fp4_skinny_gemm(W, X, path=path)
        check_product(Y, host, bits(X))


@pytest.mark.parametrize("M", [9, 11, 16])
@pytest.mark.parametrize("fmt", [fg.NVFP4, fg.MXFP4])
def test_wide_verify_gate_up_and_grouped(fmt, M):
    log("wide gate_up/grouped", fmt, M)
    for shape in ((200, 1056), (130, 544)):
        Wg, hg = make(fmt, *shape, seed=5)
        Wu, hu = make(fmt, *shape, seed=6)
        X = datagen.bf16_normal((M, shape[1]), datagen.tensor_seed("Xgw", M, shape), device=DEV)
        check_h(fg.fp4_gate_up_silu(Wg, Wu, X), hg, hu, bits(X))
    shapes = [(70, 1056), (1, 1056), (200, 1056)]
    mats = [make(fmt, o, i, seed=("grpw", j)) for j, (o, i) in enumerate(shapes)]
    X = datagen.bf16_normal((M, 1056), datagen.tensor_seed("grpXw", M), device=DEV)
    for (W, host), Y in zip(mats, fg.fp4_gemv_grouped(fg.Group([W for W, _ in mats]), X)):
        check_product(Y, host, bits(X))


@pytest.mark.parametrize("fmt", [fg.NVFP4, fg.MXFP4])
def test_wide_verify_exact_sums(fmt):
    """Power-of-two scales mixed per block with x in {-1, 0, 1}: every partial sum
    is representable, so 9..16 vectors must give the oracle's sums bit for bit
    (a token or row mapped to the wrong output column breaks this); split counts
    up to 63 across the tree."""
    log("wide exact", fmt)
    for shape in ((130, 1056), (64, 17408), (70, 256 * 63)):
        gen = torch.Generator(DEV).manual_seed(shape[0] + shape[1] + 7)
        mat = datagen.matrix(fmt, *shape, datagen.tensor_seed("exactw", fmt, shape), device=DEV)
        sc = exact_scales(fmt, shape, gen)
        W = fg.pack(fmt, mat["codes"], sc)
        for M in (9, 12, 16):
            X = torch.randint(-1, 2, (M, shape[1]), generator=gen, device=DEV).to(torch.bfloat16)
            Y, _ = oracle.gemv(fmt, mat["codes"].cpu(), sc.cpu(), 1.0, bits(X))
            got = fg.fp4_skinny_gemm(W, X).clone()
            assert np.array_equal(got.cpu().double().numpy(), Y), (shape, M)
            assert torch.equal(fg.fp4_skinny_gemm(W, X), got), (shape, M)


@pytest.mark.parametrize("M", [11, 16])
def test_wide_verify_config4_mlp(M):
    """The dense MLP (gate/up 17408x5120 + SiLU*mul, down 5120x17408) at a verify
    block of 11 (K = 10) and 16 positions, sampled rows."""
    log("wide C4 MLP", M)
    Wg, hg = make(fg.NVFP4, 17408, 5120, seed=200)
    Wu, hu = make(fg.NVFP4, 17408, 5120, seed=201)
    Wd, hd = make(fg.NVFP4, 5120, 17408, seed=202)
    X = datagen.bf16_normal((M, 5120), datagen.tensor_seed("C2x", M), device=DEV)
    H = fg.fp4_gate_up_silu(Wg, Wu, X)
    Y = fg.fp4_skinny_gemm(Wd, H)
    check_h(H, hg, hu, bits(X), rows=sample_rows(17408, 160, seed=M))
    check_product(Y, hd, bits(H), rows=sample_rows(5120, 160, seed=M + 10))


def test_wide_verify_refuses_the_valu_path():
    W, _ = make(fg.NVFP4, 200, 1056, seed=3)
    X = datagen.bf16_normal((9, 1056), 5, device=DEV)
    with pytest.raises(fg.Fp4gError):
        fg.fp4_skinny_gemm(W, X, path=fg.PATH_VALU)
    with pytest.raises(fg.Fp4gError):
        fg.fp4_skinny_gemm(W, datagen.bf16_normal((17, 1056), 5, device=DEV))


# ---- wider verify blocks on the FP8 head and the MoE layer ---------------------------------------


@pytest.mark.parametrize("M", [9, 11, 16])
def test_wide_verify_lmhead(M):
    """FP8 rows at a verify block of 9..16 positions in one read of the matrix
    (ragged shapes and the dense head's sampled rows)."""
    log("wide lmhead", M)
    for shape in ((300, 544), (1, 32), (2048, 2560)):
        W, host = make(fg.FP8_ROW, *shape, seed=4)
        X = datagen.bf16_normal((M, shape[1]), datagen.tensor_seed("Xhw", M, shape), device=DEV)
        check_product(fg.fp8_lmhead_gemv(W, X), host, bits(X))
    W, host = make(fg.FP8_ROW, datagen.VOCAB, datagen.HIDDEN, seed=310)
    X = datagen.bf16_normal((M, datagen.HIDDEN), datagen.tensor_seed("Xhw", M), device=DEV)
    check_product(fg.fp8_lmhead_gemv(W, X), host, bits(X), rows=sample_rows(datagen.VOCAB, 200, seed=M))


@pytest.mark.parametrize("M", [11, 16])
def test_wide_verify_lmhead_argmax_full_vocabulary(M):
    """The greedy pick for 11 and 16 positions over the MoE model's whole
    157184-row head: logits within the bound on every row, the pick the FP32
    arg-max of those logits, the oracle's best row within twice the bound; and a
    row range (a draft head)."""
    log("wide lmhead argmax", M)
    V, d = datagen.MOE_VOCAB, datagen.MOE_HIDDEN
    W, host = make(fg.FP8_ROW, V, d, seed=44)
    X = datagen.bf16_normal((M, d), datagen.tensor_seed("amw", M), device=DEV)
    idx, val, L = fg.fp8_lmhead_argmax(W, X, logits=True)
    Lh = L.cpu().numpy()
    assert np.array_equal(idx.cpu().numpy(), f32_argmax(Lh))
    assert np.array_equal(val.cpu().numpy(), Lh[np.arange(M), idx.cpu().numpy()])
    Y, A = oracle.gemv(fg.FP8_ROW, host["codes"], host["scales"], 1.0, bits(X))
    assert np.all(np.abs(Lh.astype(np.float64) - Y) <= TOL * A)
    i = idx.cpu().numpy().astype(np.int64)
    assert np.all(Y[np.arange(M), i] >= Y.max(axis=1) - 2 * TOL * A.max(axis=1))
    idx2, _, _ = fg.fp8_lmhead_argmax(W, X, 64 * 100, 100032)
    sub = Lh[:, 6400:6400 + 100032]
    assert np.array_equal(idx2.cpu().numpy(), f32_argmax(sub) + 6400)


@pytest.mark.parametrize("M", [9, 12, 16])
def test_wide_verify_moe_small(M):
    log("wide moe small", M)
    for fmt, shared in ((fg.MXFP4, True), (fg.NVFP4, False)):
        layer, expert, sh = build_moe(fmt, 16, 4, 256, 128, seed=("wide", M), shared=shared,
                                      tscales=(1.0, 1.0, 1.0) if fmt == fg.MXFP4 else (0.5, 2.0, 1.5))
        X = datagen.bf16_normal((M, 256), datagen.tensor_seed("mxw", M), device=DEV)
        logits = datagen.router_logits(M, 16, datagen.tensor_seed("mlw", M), device=DEV)
        check_moe(layer, expert, sh, X, logits, 4)


@pytest.mark.parametrize("M", [11, 16])
def test_wide_verify_config5_moe_layer(M):
    """The Ling-3.0-flash-shaped MoE layer (512 MXFP4 experts, top-8 + shared) at
    11 and 16 tokens: up to 129 experts in the union."""
    log("wide C5 moe", M)
    layer, expert, sh = build_moe(fg.MXFP4, 512, 8, 2560, 768, seed=5)
    X = datagen.bf16_normal((M, 2560), datagen.tensor_seed("C5xw", M), device=DEV)
    logits = datagen.router_logits(M, 512, datagen.tensor_seed("C5lw", M), device=DEV)
    check_moe(layer, expert, sh, X, logits, 8)


# ---- W4A8 mixture-of-experts layer (8-bit activations, MXFP4 experts) -----------------------------


@pytest.mark.parametrize("M", [1, 2, 3, 8, 16])
def test_moe_a8_small(M):
    log("moe a8 small", M)
    for shared in (True, False):
        layer, expert, sh = build_moe(fg.MXFP4, 16, 4, 256, 128, seed=("a8moe", M), shared=shared, act=fg.ACT_MXFP8)
        X = datagen.bf16_normal((M, 256), datagen.tensor_seed("a8mx", M), device=DEV)
        logits = datagen.router_logits(M, 16, datagen.tensor_seed("a8ml", M), device=DEV)
        check_moe(layer, expert, sh, X, logits, 4)


@pytest.mark.parametrize("M", [4, 8, 11, 16])
def test_moe_a8_config5_layer(M):
    """The Ling-3.0-flash-shaped layer on the article's measured W4A8
    configuration (Table 1, sec. 3): 512 MXFP4 experts 768x2560 / 2560x768,
    top-8 + shared, x and h quantised to MXFP8, at 4, 8, 11 and 16 tokens."""
    log("moe a8 C5", M)
    layer, expert, sh = build_moe(fg.MXFP4, 512, 8, 2560, 768, seed=5, act=fg.ACT_MXFP8)
    X = datagen.bf16_normal((M, 2560), datagen.tensor_seed("C5x8", M), device=DEV)
    logits = datagen.router_logits(M, 512, datagen.tensor_seed("C5l8", M), device=DEV)
    check_moe(layer, expert, sh, X, logits, 8)


def test_moe_a8_refuses_nvfp4_experts():
    layer, _, _ = build_moe(fg.NVFP4, 16, 4, 256, 128, seed=("a8nv",), act=fg.ACT_MXFP8)
    X = datagen.bf16_normal((2, 256), 1, device=DEV)
    logits = datagen.router_logits(2, 16, 2, device=DEV)
    with pytest.raises(fg.Fp4gError) as e:
        fg.moe_route_gemv(layer, X, logits)
    assert e.value.status == 6  # FP4G_E_PATH


# ---- mixed layout: FP8 row-scaled MLPs and projections, the MoE router ---------------------


@pytest.mark.parametrize("M", [1, 3, 8])
def test_fp8_gate_up_silu_matches_oracle(M):
    """The FP8 MLPs of a mixed layout: gate and up as FP8 rows, each with its own
    row scales, fused with SiLU * mul (ragged shapes, tails of 32 columns)."""
    log("fp8 gate_up", M)
    for shape in ((200, 1056), (130, 544), (64, 256)):
        Wg, hg = make(fg.FP8_ROW, *shape, seed=15)
        Wu, hu = make(fg.FP8_ROW, *shape, seed=16)
        X = datagen.bf16_normal((M, shape[1]), datagen.tensor_seed("X8g", M, shape), device=DEV)
        check_h(fg.fp4_gate_up_silu(Wg, Wu, X), hg, hu, bits(X))


def test_fp8_mlp_full_size():
    """One FP8 MLP of the dense model (gate/up 17408x5120, down 5120x17408), sampled rows."""
    log("fp8 MLP full")
    Wg, hg = make(fg.FP8_ROW, 17408, 5120, seed=300)
    Wu, hu = make(fg.FP8_ROW, 17408, 5120, seed=301)
    Wd, hd = make(fg.FP8_ROW, 5120, 17408, seed=302)
    x = datagen.bf16_normal((1, 5120), 303, device=DEV)
    H = fg.fp4_gate_up_silu(Wg, Wu, x)
    check_h(H, hg, hu, bits(x), rows=sample_rows(17408, 160, seed=3))
    check_product(fg.fp8_lmhead_gemv(Wd, H), hd, bits(H), rows=sample_rows(5120, 160, seed=4))


@pytest.mark.parametrize("M", [1, 4])
def test_fp8_grouped_projections(M):
    """FP8 projections of one input in one launch (members with their own row
    scales): equal to the single-matrix products up to the FP32 summation order."""
    log("fp8 grouped", M)
    shapes = [(300, 1056), (64, 1056), (128, 1056)]
    mats = [make(fg.FP8_ROW, o, i, seed=("g8", j)) for j, (o, i) in enumerate(shapes)]
    X = datagen.bf16_normal((M, 1056), datagen.tensor_seed("g8X", M), device=DEV)
    Ys = fg.fp4_gemv_grouped(fg.Group([W for W, _ in mats]), X)
    for (W, host), Y in zip(mats, Ys):
        check_product(Y, host, bits(X))


@pytest.mark.parametrize("M", [1, 4])
def test_router_gemv_feeds_moe(M):
    """The MoE router as an FP8 row-scaled 512x2560 product in front of
    moe_route_gemv: its logits within the product bound, then the full layer
    (512 MXFP4 experts, top-8 + shared) routed on those very logits, checked
    stage by stage against the oracle (ids exact)."""
    log("router -> moe", M)
    Wr, hr = make(fg.FP8_ROW, datagen.MOE_EXPERTS, datagen.MOE_HIDDEN, seed=310)
    X = datagen.bf16_normal((M, datagen.MOE_HIDDEN), datagen.tensor_seed("rX", M), device=DEV)
    logits = fg.fp8_lmhead_gemv(Wr, X)
    check_product(logits, hr, bits(X))
    layer, expert, sh = build_moe(fg.MXFP4, datagen.MOE_EXPERTS, datagen.MOE_TOPK, datagen.MOE_HIDDEN,
                                  datagen.MOE_FF, seed=311)
    check_moe(layer, expert, sh, X, logits, datagen.MOE_TOPK)


# ---- W4A8: MXFP4 weights x MXFP8 activations on the scaled matrix cores ------------------------
from oracle import w4a8 as oracle_a8  # noqa: E402


def check_a8(Y, host, X_bits, rows=None):
    Yr, A = oracle_a8.gemv(fg.MXFP4, host["codes"], host["scales"], host["tensor_scale"], X_bits)
    y = Y.detach().cpu().double().numpy().reshape(Yr.shape[0], -1)
    if rows is not None:
        y, Yr, A = y[:, rows], Yr[:, rows], A[:, rows]
    bad = np.abs(y - Yr) > TOL * A
    assert not bad.any(), f"{bad.sum()} outputs out of bound"


@pytest.mark.parametrize("M", [1, 3, 8, 16])
def test_a8_matches_w4a8_oracle(M):
    """The input quantised to MXFP8 inside the kernel, then the exact product:
    within the product bound of the W4A8 oracle (ragged shapes, tails)."""
    log("a8", M)
    for shape in ((200, 1056), (70, 288), (96, 5120)):
        W, host = make(fg.MXFP4, *shape, seed=60)
        X = datagen.bf16_normal((M, shape[1]), datagen.tensor_seed("a8X", M, shape), device=DEV)
        X[0, :32] = 0.0           # an all-zero block
        X[-1, 32:64] *= 1e-6      # tiny values (the block's scale follows them)
        X[0, 64] = 100.0          # block scale 2^-2: below it E4M3 subnormals and,
        X[0, 65:80] = -1e-3       # under half the smallest step, negatives that
        X[0, 80:96] = -1e-5       # round to zero (the -0 code on the device)
        check_a8(fg.fp4_skinny_gemm(W, X, path=fg.PATH_A8), host, bits(X))


def test_a8_exact_sums():
    """Power-of-two weight scales and x in {-1, 0, 1}: the activations quantise
    without loss and every partial sum is representable, so the W4A8 product
    equals the oracle bit for bit, and repeats bit for bit."""
    log("a8 exact")
    for shape in ((130, 1056), (64, 5120)):
        gen = torch.Generator(DEV).manual_seed(shape[0] + 77)
        mat = datagen.matrix(fg.MXFP4, *shape, datagen.tensor_seed("a8exact", shape), device=DEV)
        sc = exact_scales(fg.MXFP4, shape, gen)
        W = fg.pack(fg.MXFP4, mat["codes"], sc)
        for M in (1, 5, 16):
            X = torch.randint(-1, 2, (M, shape[1]), generator=gen, device=DEV).to(torch.bfloat16)
            Yr, _ = oracle_a8.gemv(fg.MXFP4, mat["codes"].cpu(), sc.cpu(), 1.0, bits(X))
            got = fg.fp4_skinny_gemm(W, X, path=fg.PATH_A8).clone()
            assert np.array_equal(got.cpu().double().numpy(), Yr), (shape, M)
            assert torch.equal(fg.fp4_skinny_gemm(W, X, path=fg.PATH_A8), got)


def test_a8_grouped_and_refusals():
    log("a8 grouped")
    shapes = [(70, 1056), (1, 1056), (200, 1056)]
    mats = [make(fg.MXFP4, o, i, seed=("a8g", j)) for j, (o, i) in enumerate(shapes)]
    X = datagen.bf16_normal((4, 1056), datagen.tensor_seed("a8gX"), device=DEV)
    for (W, host), Y in zip(mats, fg.fp4_gemv_grouped(fg.Group([W for W, _ in mats]), X, path=fg.PATH_A8)):
        check_a8(Y, host, bits(X))
    Wn, _ = make(fg.NVFP4, 64, 256, seed=61)
    with pytest.raises(fg.Fp4gError):
        fg.fp4_skinny_gemm(Wn, datagen.bf16_normal((2, 256), 1, device=DEV), path=fg.PATH_A8)
    with pytest.raises(fg.Fp4gError):
        fg.fp4_gate_up_silu(Wn, Wn, datagen.bf16_normal((2, 256), 1, device=DEV), path=fg.PATH_A8)


@pytest.mark.parametrize("M", [1, 3, 8, 16])
def test_a8_gate_up_silu_matches_oracle(M):
    """Fused gate/up on the W4A8 path: both products of the once-quantised
    input, then bf16(SiLU(g) u), within the bound of the bf16 path with the W4A8
    oracle's products and magnitude sums."""
    log("a8 gate_up", M)
    for shape in ((200, 1056), (70, 288), (96, 5120)):
        Wg, hg = make(fg.MXFP4, *shape, seed=("a8gu", 0))
        Wu, hu = make(fg.MXFP4, *shape, seed=("a8gu", 1))
        X = datagen.bf16_normal((M, shape[1]), datagen.tensor_seed("a8guX", M, shape), device=DEV)
        X[0, 64] = 100.0
        X[0, 65:96] = -1e-5
        H = fg.fp4_gate_up_silu(Wg, Wu, X, path=fg.PATH_A8)
        g, Ag = oracle_a8.gemv(fg.MXFP4, hg["codes"], hg["scales"], hg["tensor_scale"], bits(X))
        u, Au = oracle_a8.gemv(fg.MXFP4, hu["codes"], hu["scales"], hu["tensor_scale"], bits(X))
        r = {"h": oracle.silu_mul(g, u), "g": g, "u": u, "Ag": Ag, "Au": Au}
        h = H.detach().float().cpu().double().numpy().reshape(M, -1)
        bad = np.abs(h - r["h"]) > h_bound(r, r["h"])
        assert not bad.any(), f"{bad.sum()} h values out of bound ({shape})"
