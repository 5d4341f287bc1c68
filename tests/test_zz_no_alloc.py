"""fp4_skinny_gemm_noalloc -- the allocation-free variant of fp4_skinny_gemm,
called through the C ABI: its split-K workspace is the library's fixed scratch
array.  Its results must equal fp4_skinny_gemm's bit for bit (same kernels and
plan) and stay within the product bound of the FP64 oracle, over two calls in a
row where the second has the smaller input (the array keeps what the first
left)."""
import numpy as np
import pytest
import torch

import bit_weight_gemv_fp4_amd as fg
import datagen
from gpu_common import DEV, bits, check_product, log, make

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_and_native_library():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert fg.LIB_PATH.exists(), "the HIP library must be built"
    fg.lib()
    yield
    torch.cuda.synchronize()


CASES = [  # (format, d_out, d_in, M, path): a large call, then smaller ones
    (fg.NVFP4, 5120, 17408, 16, fg.PATH_MFMA),
    (fg.NVFP4, 200, 1056, 3, fg.PATH_AUTO),
    (fg.MXFP4, 17408, 5120, 8, fg.PATH_VALU),
    (fg.MXFP4, 70, 288, 2, fg.PATH_A8),
    (fg.NVFP4, 5120, 5120, 1, fg.PATH_AUTO),
]


@pytest.mark.parametrize("first", [0, 2])
def test_noalloc_matches_the_workspace_entry_point(first):
    """Two calls in a row, the second with a smaller input; each equals
    fp4_skinny_gemm bit for bit and the oracle within the product bound (sampled
    rows on the large shapes)."""
    for fmt, d_out, d_in, M, path in (CASES[first], CASES[first + 1], CASES[4]):
        log("noalloc", fmt, d_out, d_in, M, path)
        W, host = make(fmt, d_out, d_in, seed=("noalloc", d_out))
        X = datagen.bf16_normal((M, d_in), datagen.tensor_seed("noallocX", M, d_in), device=DEV)
        Y = torch.empty((M, d_out), dtype=torch.float32, device=DEV)
        fg.fp4_skinny_gemm_noalloc(W, X, Y, path=path)
        ref = fg.fp4_skinny_gemm(W, X, path=path)
        torch.cuda.synchronize()
        assert torch.equal(Y, ref)
        rows = None if d_out <= 256 else np.array(sorted({0, 1, 63, 64, d_out - 1} | set(range(0, d_out, 97))))
        if path == fg.PATH_A8:
            from oracle import w4a8
            Yr, A = w4a8.gemv(fmt, host["codes"], host["scales"], 1.0, bits(X))
            assert np.all(np.abs(Y.cpu().double().numpy() - Yr) <= 2e-3 * A)
        else:
            check_product(Y, host, bits(X), rows=rows)


def test_noalloc_refuses_a_product_beyond_its_scratch():
    W, _ = make(fg.NVFP4, 248320, 5120, seed="noalloc-big")
    need = fg.workspace_bytes(fg.OP_GEMV, W, 12)
    X = torch.zeros((12, 5120), dtype=torch.bfloat16, device=DEV)
    Y = torch.empty((12, 248320), dtype=torch.float32, device=DEV)
    if need <= fg.NOALLOC_SCRATCH_BYTES:
        pytest.skip(f"this shape needs only {need} bytes")
    with pytest.raises(fg.Fp4gError) as e:
        fg.fp4_skinny_gemm_noalloc(W, X, Y)
    assert e.value.status == 5  # FP4G_E_WORKSPACE
