"""GPU GEMV engine through the isolated-GEMV probe entry point (kie_gemv_probe),
in both orders: a decode stage's (each product's first weight block, then its
input vector) and input first (the input vector, then the weights)."""
import pytest
import torch

import oracle
from persistent_decode_monokernel_amd import kie, synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("input_first", [False, True])
@pytest.mark.parametrize("rows,cols", [(64, 256), (300, 2048), (257, 8192), (1000, 14336), (96, 4096)])
def test_integer_inputs_bit_exact(rows, cols, input_first):
    # entries in {-2..2}: every product and partial sum is an exact fp32 integer
    W, x = synth.make_gemv(rows, cols, 3, seed=rows + cols, integer=True, device="cuda")
    y, _ = kie.gemv_probe(W, x, input_first=input_first)
    ref = oracle.matvec(W[0].cpu(), x.cpu())
    assert torch.equal(y.cpu().double(), ref)


@pytest.mark.parametrize("input_first", [False, True])
@pytest.mark.parametrize("rows,cols", synth.GEMV_SHAPES)
def test_gaussian_parity_probe_shapes(rows, cols, input_first):
    W, x = synth.make_gemv(rows, cols, 16, seed=synth.GEMV_SEEDS[0], device="cuda")
    y, _ = kie.gemv_probe(W, x, input_first=input_first)
    ref = oracle.matvec(W[0].cpu(), x.cpu())
    # fp16 products are exact in fp32; only fp32 summation order differs
    tol = 1e-5 * (cols ** 0.5) * 8
    err = (y.cpu().double() - ref).abs().max().item()
    assert err < tol, err


@pytest.mark.parametrize("n_vec", [1, 2, 37])
@pytest.mark.parametrize("rows,cols", list(synth.GEMV_SHAPES) + [(300, 14336)])
def test_input_first_equals_stage_order(rows, cols, n_vec):
    # the two orders run the same arithmetic: bit-identical, over rotating
    # copies, with one vector and a ragged count
    W, x = synth.make_gemv(rows, cols, n_vec, seed=11 + n_vec, n_copies=3, device="cuda")
    a, _ = kie.gemv_probe(W, x, input_first=False)
    b, _ = kie.gemv_probe(W, x, input_first=True)
    assert torch.equal(a, b)
    ref = oracle.matvec(W[(n_vec - 1) % 3].cpu(), x[-1:].cpu())[0]
    assert (b[-1].cpu().double() - ref).abs().max().item() < 1e-5 * (cols ** 0.5) * 8


def test_probe_argument_checks():
    W, x = synth.make_gemv(64, 256, 2, seed=3, device="cuda")
    with pytest.raises(kie.KieError):
        kie.gemv_probe(W.cpu(), x.cpu())
    with pytest.raises(kie.KieError):
        kie.gemv_probe(W, x.to(torch.bfloat16))
    with pytest.raises(kie.KieError):
        kie.gemv_probe(W, x[:, :128])


@pytest.mark.parametrize("input_first", [False, True])
def test_bf16_parity(input_first):
    W, x = synth.make_gemv(512, 2048, 4, seed=7, device="cuda", dtype=torch.bfloat16)
    y, _ = kie.gemv_probe(W, x, input_first=input_first)
    ref = oracle.matvec(W[0].cpu(), x.cpu())
    assert (y.cpu().double() - ref).abs().max().item() < 1e-3


def test_rotating_copies():
    W, x = synth.make_gemv(256, 2048, 6, seed=9, n_copies=3, device="cuda")
    y, _ = kie.gemv_probe(W, x)
    for i in range(6):
        ref = oracle.matvec(W[i % 3].cpu(), x[i:i + 1].cpu())[0]
        assert (y[i].cpu().double() - ref).abs().max().item() < 1e-3
