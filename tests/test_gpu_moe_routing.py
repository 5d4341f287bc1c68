"""MoE routing on the gate/up kernel of M = 1, 2 (every workgroup routes the
tokens itself; at M = 1 the slots follow the pick order and each workgroup picks
only as far as its own slot): ties, expert counts on both pick paths (up to 512
experts: sorted keys per lane; above: a scan per pick), a single pick, and
repeated calls on one workspace.  Parity as in test_gpu_parity: ids exact,
stage-wise bounds against the FP64 oracle."""
import pytest
import torch

import bit_weight_gemv_fp4_amd as fg
import datagen
from gpu_common import DEV, build_moe, check_moe, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M", [1, 2])
def test_routing_ties(M):
    """Equal logits (zeros of both signs, repeated values): lower expert index first."""
    log("routing ties", M)
    layer, expert, sh = build_moe(fg.MXFP4, 16, 4, 256, 128, seed=21)
    X = datagen.bf16_normal((M, 256), datagen.tensor_seed("ftx", M), device=DEV)
    logits = torch.zeros((M, 16), dtype=torch.float32, device=DEV)
    logits[0, 3] = -0.0
    logits[0, 9] = 0.75
    if M > 1:
        logits[1] = torch.tensor([0.5, -1, 0.5, 0.25] * 4, device=DEV)
    ids = check_moe(layer, expert, sh, X, logits, 4)
    assert ids[0].tolist() == [9, 0, 1, 2]
    if M > 1:
        assert ids[1].tolist() == [0, 2, 4, 6]


@pytest.mark.parametrize("E,k", [(100, 8), (512, 1), (640, 8), (1024, 6)])
@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_routing_expert_counts(E, k, M):
    """Partial last lane of keys (100), a single pick, and the scan path above 512
    (M = 1, 2: the VALU gate/up's routing; 3, 4: the matrix-core gate/up
    workgroups routing for themselves)."""
    log("routing experts", E, k, M)
    layer, expert, sh = build_moe(fg.MXFP4, E, k, 256, 128, seed=22)
    X = datagen.bf16_normal((M, 256), datagen.tensor_seed("fex", E, k, M), device=DEV)
    logits = datagen.router_logits(M, E, datagen.tensor_seed("fel", E, k, M), device=DEV)
    check_moe(layer, expert, sh, X, logits, k)


@pytest.mark.parametrize("M", [1, 2, 4])
def test_config5_repeated_calls(M):
    """The C5 layer three times in a row on one workspace, new inputs each time."""
    log("C5 repeat", M)
    layer, expert, sh = build_moe(fg.MXFP4, 512, 8, 2560, 768, seed=23)
    for rep in range(3):
        X = datagen.bf16_normal((M, 2560), datagen.tensor_seed("frx", M, rep), device=DEV)
        logits = datagen.router_logits(M, 512, datagen.tensor_seed("frl", M, rep), device=DEV)
        check_moe(layer, expert, sh, X, logits, 8)


@pytest.mark.parametrize("M", [1, 3])
def test_no_shared_expert_pick_order(M):
    """Without a shared expert: at M = 1 the slots are exactly the K picks; at
    M = 3 the union alone (the matrix-core workgroups' own routing)."""
    log("no shared", M)
    layer, expert, sh = build_moe(fg.MXFP4, 64, 8, 256, 128, seed=25, shared=False)
    X = datagen.bf16_normal((M, 256), 251 + M, device=DEV)
    logits = datagen.router_logits(M, 64, 252 + M, device=DEV)
    check_moe(layer, expert, sh, X, logits, 8)


@pytest.mark.parametrize("M", [1, 4])
def test_layer_timing_program_picks(M):
    """The C++ layer timing program drives moe_route_gemv through the C ABI on
    C5-shaped layers and checks every token's picks against a host top-8 of the
    same logits (it exits non-zero on the first mismatch)."""
    import subprocess
    from pathlib import Path

    log("layer timing program", M)
    exe = Path(fg.__file__).resolve().parent / "moe_layer_timing"
    assert exe.exists(), "moe_layer_timing is built with the library"
    r = subprocess.run([str(exe), str(M), "2", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "picks match the host top-8" in r.stdout
