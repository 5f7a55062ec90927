"""GPU GEMV engine through the isolated-GEMV probe entry point (kie_gemv_probe)."""
import pytest
import torch

import oracle
from persistent_decode_monokernel_amd import kie, synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,cols", [(64, 256), (300, 2048), (257, 8192), (1000, 14336), (96, 4096)])
def test_integer_inputs_bit_exact(rows, cols):
    # entries in {-2..2}: every product and partial sum is an exact fp32 integer
    W, x = synth.make_gemv(rows, cols, 3, seed=rows + cols, integer=True, device="cuda")
    y, _ = kie.gemv_probe(W, x)
    ref = oracle.matvec(W[0].cpu(), x.cpu())
    assert torch.equal(y.cpu().double(), ref)


@pytest.mark.parametrize("rows,cols", synth.GEMV_SHAPES)
def test_gaussian_parity_probe_shapes(rows, cols):
    W, x = synth.make_gemv(rows, cols, 16, seed=synth.GEMV_SEEDS[0], device="cuda")
    y, _ = kie.gemv_probe(W, x)
    ref = oracle.matvec(W[0].cpu(), x.cpu())
    # fp16 products are exact in fp32; only fp32 summation order differs
    tol = 1e-5 * (cols ** 0.5) * 8
    err = (y.cpu().double() - ref).abs().max().item()
    assert err < tol, err


def test_bf16_parity():
    W, x = synth.make_gemv(512, 2048, 4, seed=7, device="cuda", dtype=torch.bfloat16)
    y, _ = kie.gemv_probe(W, x)
    ref = oracle.matvec(W[0].cpu(), x.cpu())
    assert (y.cpu().double() - ref).abs().max().item() < 1e-3


def test_rotating_copies():
    W, x = synth.make_gemv(256, 2048, 6, seed=9, n_copies=3, device="cuda")
    y, _ = kie.gemv_probe(W, x)
    for i in range(6):
        ref = oracle.matvec(W[i % 3].cpu(), x[i:i + 1].cpu())[0]
        assert (y[i].cpu().double() - ref).abs().max().item() < 1e-3
