"""Seeded synthetic inputs for the tests, smoke() and bench.py.

This module only draws numbers: it holds none of the arithmetic of the product
(no decoding, no dot products, no routing).  Both the CPU oracle and the GPU
library consume what it returns; it imports neither.

Distributions (the pages publish no weights; the inputs stand in for the
checkpoints and prompt sets the pages measure on):

* NVFP4 matrix: E2M1 codes uniform over all 16 codes (each code byte uniform over
  0..255); one E4M3FN scale per 16 weights equal to |z|/6 rounded to nearest-even
  E4M3 (z ~ N(0,1) drawn in FP32; values below half the smallest subnormal become
  0); tensor scale 1.0.
* MXFP4 matrix: codes as above; one E8M0 scale per 32 weights equal to |z|/6
  rounded to the nearest power of two in the linear domain (v >= 0.75 * 2^e
  rounds up to 2^e, where 2^(e-1) <= v < 2^e), clamped to codes 0..254.
* FP8 rows: E4M3FN codes uniform over the 254 finite codes (0x7F and 0xFF, the
  NaNs, excluded); one FP32 scale per row equal to |z|/448.
* Activations: bf16 round-to-nearest-even of z ~ N(0,1).
* Router logits: FP32 z ~ N(0,1).

Every tensor is drawn from its own torch.Generator seeded by tensor_seed(...), on
the device it is asked for.  The same call on the same device type gives the same
bits; CUDA/HIP and CPU generators give different (equally distributed) streams.
"""
from __future__ import annotations

import hashlib

import torch

SEED_BASE = 0xF4E50000

NVFP4, MXFP4, FP8_ROW = 1, 2, 3


def tensor_seed(*ids) -> int:
    """A 63-bit seed from a tuple of ints/strings (stable across runs)."""
    h = hashlib.blake2b(repr((SEED_BASE,) + tuple(ids)).encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(int(seed))
    return g


def uniform_bytes(shape, seed, device="cpu") -> torch.Tensor:
    return torch.randint(0, 256, tuple(shape), dtype=torch.uint8, generator=_gen(seed, device), device=device)


def normal_f32(shape, seed, device="cpu") -> torch.Tensor:
    return torch.randn(tuple(shape), dtype=torch.float32, generator=_gen(seed, device), device=device)


def e4m3_block_scales(shape, seed, device="cpu") -> torch.Tensor:
    """E4M3FN bytes of |z|/6 (torch's float8_e4m3fn cast rounds to nearest even)."""
    z = normal_f32(shape, seed, device)
    return (z.abs() / 6.0).to(torch.float8_e4m3fn).view(torch.uint8)


def e8m0_block_scales(shape, seed, device="cpu") -> torch.Tensor:
    """E8M0 bytes of |z|/6 rounded to the nearest power of two (linear distance)."""
    v = normal_f32(shape, seed, device).abs() / 6.0
    mant, ex = torch.frexp(v)  # v = mant * 2^ex, mant in [0.5, 1)
    e = torch.where(mant >= 0.75, ex, ex - 1).to(torch.int32)
    code = torch.clamp(e + 127, 0, 254)
    code = torch.where(v > 0, code, torch.zeros_like(code))
    return code.to(torch.uint8)


def fp8_finite_codes(shape, seed, device="cpu") -> torch.Tensor:
    r = torch.randint(0, 254, tuple(shape), dtype=torch.int32, generator=_gen(seed, device), device=device)
    return (r + (r >= 127).to(torch.int32)).to(torch.uint8)


def bf16_normal(shape, seed, device="cpu") -> torch.Tensor:
    """bf16 activations, returned as a torch.bfloat16 tensor."""
    return normal_f32(shape, seed, device).to(torch.bfloat16)


def router_logits(M, E, seed, device="cpu") -> torch.Tensor:
    return normal_f32((M, E), seed, device)


def matrix(fmt: int, d_out: int, d_in: int, seed: int, device="cpu", batch: int | None = None) -> dict:
    """Logical operands of one matrix (or `batch` matrices stacked in front).

    Returns {"format", "d_out", "d_in", "codes", "scales", "tensor_scale"} with
    codes u8[..., d_out, d_in/2] (FP4) or u8[..., d_out, d_in] (FP8) and scales
    u8[..., d_out, d_in/16] (NVFP4), u8[..., d_out, d_in/32] (MXFP4) or
    f32[..., d_out] (FP8)."""
    lead = () if batch is None else (batch,)
    if fmt == NVFP4:
        codes = uniform_bytes(lead + (d_out, d_in // 2), tensor_seed(seed, "codes"), device)
        scales = e4m3_block_scales(lead + (d_out, d_in // 16), tensor_seed(seed, "scales"), device)
    elif fmt == MXFP4:
        codes = uniform_bytes(lead + (d_out, d_in // 2), tensor_seed(seed, "codes"), device)
        scales = e8m0_block_scales(lead + (d_out, d_in // 32), tensor_seed(seed, "scales"), device)
    elif fmt == FP8_ROW:
        codes = fp8_finite_codes(lead + (d_out, d_in), tensor_seed(seed, "codes"), device)
        scales = normal_f32(lead + (d_out,), tensor_seed(seed, "scales"), device).abs() / 448.0
    else:
        raise ValueError(f"unknown format {fmt}")
    return {"format": fmt, "d_out": d_out, "d_in": d_in, "codes": codes, "scales": scales, "tensor_scale": 1.0}


# ---- the workloads' shapes (from the pages) ----

HIDDEN = 5120          # dense model hidden size
FFN = 17408            # dense MLP intermediate size
ATTN_SHAPES = ((12288, 5120), (12288, 5120), (5120, 12288), (7680, 5120))
LAYERS = 64
VOCAB = 248320

# The mixed layout of the dense checkpoint (feed, section "Fewer bytes per weight:
# NVFP4": the MLPs of layers 0..55 are NVFP4; the attention and linear-attention
# projections, the output layer and the MLPs of the last 8 layers are FP8;
# section "Decode speed is bytes divided by bandwidth" puts full attention in
# every fourth layer, linear attention in the other 48).  The pages give only the
# largest projection, 12288x5120, and the byte shares (MLP 59%, linear attention
# 31%, full attention 9% of 17.83 GB): these projection shapes are a reading that
# reproduces both (17.78 GB for 64 layers, 19.05 GB with the head).
MIXED_FP8_MLP_FROM = 56                                        # first layer with an FP8 MLP
MIXED_GDN_SHAPES = ((12288, 5120), (5120, 10240))              # linear attention: in, out
MIXED_ATTN_SHAPES = ((12288, 5120), (1024, 5120), (1024, 5120), (5120, 6144))  # q, k, v, out


def mixed_full_attention(layer: int) -> bool:
    return layer % 4 == 3


MOE_HIDDEN = 2560
MOE_FF = 768
MOE_EXPERTS = 512
MOE_TOPK = 8
MOE_LAYERS = 40
MOE_VOCAB = 157184


def config_seed(config: int) -> int:
    return SEED_BASE + config
