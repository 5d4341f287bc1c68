"""The seeded input generator draws what its docstring says.  CPU only."""
import math

import numpy as np
import scipy.stats
import torch

import datagen


def test_e4m3_scale_cast_is_round_to_nearest_even():
    # every finite non-negative E4M3FN value, brute-force nearest with ties to even
    vals = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    z = datagen.normal_f32((20000,), 123).abs().double().numpy() / 6.0
    z = np.concatenate([z, (vals[1:] + vals[:-1]) / 2])  # exact midpoints
    got = torch.from_numpy(z.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    zf = z.astype(np.float32).astype(np.float64)
    for v, code in zip(zf, got):
        d = np.abs(vals - v)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert code == want, (v, code, want)


def test_e4m3_scale_fractions():
    n = 400000
    s = datagen.e4m3_block_scales((n,), 77).numpy()
    # zero when |z|/6 < 2^-10 (half the smallest subnormal, tie goes to even 0)
    p_zero = 2 * scipy.stats.norm.cdf(6 * 2.0 ** -10) - 1
    # nonzero subnormal when 2^-10 <= |z|/6 < 15 * 2^-10 (midpoint to 2^-6 ties up)
    p_sub = 2 * (scipy.stats.norm.cdf(6 * 15 * 2.0 ** -10) - scipy.stats.norm.cdf(6 * 2.0 ** -10))
    for frac, p in (((s == 0).mean(), p_zero), (((s > 0) & (s < 8)).mean(), p_sub)):
        sd = math.sqrt(p * (1 - p) / n)
        assert abs(frac - p) < 5 * sd, (frac, p)
    assert abs(p_zero - 0.004675) < 1e-5


def test_codes_uniform():
    c = datagen.uniform_bytes((200000,), 5).numpy()
    nib = np.concatenate([c & 15, c >> 4])
    counts = np.bincount(nib, minlength=16)
    assert scipy.stats.chisquare(counts).pvalue > 1e-4


def test_fp8_codes_finite_and_all_present():
    c = datagen.fp8_finite_codes((300000,), 6).numpy()
    assert not np.any((c & 0x7F) == 0x7F)
    assert len(np.unique(c)) == 254
    counts = np.bincount(c, minlength=256)
    counts = counts[(np.arange(256) & 0x7F) != 0x7F]
    assert scipy.stats.chisquare(counts).pvalue > 1e-4


def test_e8m0_scales_nearest_power_of_two():
    v = datagen.normal_f32((5000,), 17).abs().double().numpy() / 6.0
    codes = datagen.e8m0_block_scales((5000,), 17).numpy().astype(np.int64)
    for vi, ci in zip(v.astype(np.float32).astype(np.float64), codes):
        lo = 2.0 ** math.floor(math.log2(vi))
        want = lo if (vi - lo) < (2 * lo - vi) else 2 * lo
        assert 2.0 ** (ci - 127) == want


def test_bf16_activation_is_rne_of_normal():
    z = datagen.normal_f32((1000,), 9)
    x = datagen.bf16_normal((1000,), 9)
    assert torch.equal(x, z.to(torch.bfloat16))


def test_seeds_are_stable_and_distinct():
    assert datagen.tensor_seed(1, "a") == datagen.tensor_seed(1, "a")
    assert datagen.tensor_seed(1, "a") != datagen.tensor_seed(1, "b")
    a = datagen.matrix(datagen.NVFP4, 64, 256, 3)
    b = datagen.matrix(datagen.NVFP4, 64, 256, 3)
    assert torch.equal(a["codes"], b["codes"]) and torch.equal(a["scales"], b["scales"])


def test_mixed_layout_reproduces_the_pages_byte_split():
    """The mixed-layout workload (FP8 projections, NVFP4 MLPs in layers 0..55, FP8
    MLPs in 56..63) is a reading of the pages' shapes: it must reproduce their
    layer bytes (17.83 GB), step bytes with the head (19.10 GB) and the shares of
    MLP / linear attention / full attention (59 / 31 / 9%)."""
    import json
    from pathlib import Path

    import bit_weight_gemv_fp4_amd as fg

    page = json.loads((Path(__file__).parent / "golden" / "page_numbers.json").read_text())
    H, F = datagen.HIDDEN, datagen.FFN
    nv = lambda o, i: fg.packed_bytes(fg.NVFP4, o, i)
    f8 = lambda o, i: fg.packed_bytes(fg.FP8_ROW, o, i)
    full = [L for L in range(datagen.LAYERS) if datagen.mixed_full_attention(L)]
    assert len(full) == datagen.LAYERS // page["byte_shares_of_layers"]["full_attention_every"]
    assert datagen.LAYERS - len(full) == page["byte_shares_of_layers"]["linear_attention_layers"]
    assert datagen.MIXED_FP8_MLP_FROM == page["mixed_layout"]["nvfp4_mlp_layers"][1] + 1
    assert max(o * i for o, i in datagen.MIXED_GDN_SHAPES + datagen.MIXED_ATTN_SHAPES) == 12288 * 5120
    mlp = sum(3 * (nv if L < datagen.MIXED_FP8_MLP_FROM else f8)(F, H) for L in range(datagen.LAYERS))
    gdn = sum(f8(o, i) for L in range(datagen.LAYERS) if L not in full for o, i in datagen.MIXED_GDN_SHAPES)
    att = sum(f8(o, i) for L in full for o, i in datagen.MIXED_ATTN_SHAPES)
    layers = mlp + gdn + att
    shares = page["byte_shares_of_layers"]
    assert abs(mlp / layers - shares["mlp"]) < 0.01
    assert abs(gdn / layers - shares["linear_attention"]) < 0.01
    assert abs(att / layers - shares["full_attention"]) < 0.01
    assert abs(layers / 1e9 - page["bytes_per_step_gb"]["layers_gb"]) / page["bytes_per_step_gb"]["layers_gb"] < 0.005
    step = layers + f8(datagen.VOCAB, H)
    assert abs(step / 1e9 - page["bytes_per_step_gb"]["value"]) / page["bytes_per_step_gb"]["value"] < 0.005
