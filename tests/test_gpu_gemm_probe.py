"""The prompt path's matrix-core GEMMs through kie_gemm_probe.

Host side (no GPU): argument and capacity errors the call rejects before it
touches the device.  GPU: C = A W^T, C += A W^T and silu(A Wg^T) * (A Wu^T) for
fp16 (fp16 activations) and bf16 (fp32 activations split into three bf16
terms) against a float64 product of the same inputs on the CPU: ragged row
counts, split-K shapes (fewer than 512 output tiles) and an unsplit one; the
fp16 GEMMs on grids that fill the GPU with 256 x 256 tiles (the long-prompt
kernel: store and add from 256 tiles, gate/up + SwiGLU from 512), with a
ragged last row tile.
"""
import ctypes

import pytest
import torch

from persistent_decode_monokernel_amd import kie

DEV = "cuda:0"
FAKE = 0x10000


def _call(op=kie.KIE_GEMM_STORE, dtype=kie.KIE_F16, A=FAKE, M=256, K=256, W=FAKE, W2=FAKE, N=256, out=FAKE,
          part=FAKE, pbytes=1 << 30, reps=1):
    return kie.lib().kie_gemm_probe(op, dtype, ctypes.c_void_p(A), M, K, ctypes.c_void_p(W), ctypes.c_void_p(W2), N,
                                    ctypes.c_void_p(out), ctypes.c_void_p(part), pbytes, reps, None, None, None)


@pytest.mark.parametrize("kw", [
    {"op": 3}, {"op": -1}, {"dtype": 0}, {"dtype": 3},
    {"A": 0}, {"W": 0}, {"out": 0}, {"op": kie.KIE_GEMM_SWIGLU, "W2": 0},
    {"M": 0}, {"M": 65537}, {"K": 0}, {"K": 96}, {"N": 0}, {"N": 192}, {"op": kie.KIE_GEMM_SWIGLU, "N": 96},
    {"M": 65536, "N": 65536}, {"reps": 0}, {"A": FAKE + 8}, {"out": FAKE + 4}, {"part": FAKE + 8},
], ids=lambda kw: ",".join(f"{k}={v}" for k, v in kw.items()))
def test_argument_errors_before_any_device_call(kw):
    assert _call(**kw) == kie.KIE_ERR_ARG


def test_split_k_needs_partial_buffer():
    # one output tile: four slices of M * N floats each
    assert _call(M=1, N=128, K=1024, part=0, pbytes=0) == kie.KIE_ERR_CAPACITY
    assert _call(M=1, N=128, K=1024, pbytes=4 * 128 * 4 - 1) == kie.KIE_ERR_CAPACITY


# (1024, 8192, 128): unsplit 128 x 128 tiles; the last two: fp16 on 256 x 256 tiles (256 and 320 of them,
# the second with a ragged last row tile)
SHAPES = [(1, 128, 128), (77, 256, 512), (300, 384, 256), (512, 256, 2048), (1024, 8192, 128), (2048, 8192, 64),
          (1100, 16384, 64)]


def _inputs(M, N, K, dt, seed):
    g = torch.Generator().manual_seed(seed)
    a = torch.randn(M, K, generator=g)
    w = torch.randn(N, K, generator=g) / K ** 0.5
    w2 = torch.randn(N, K, generator=g) / K ** 0.5
    if dt == torch.float16:
        a = a.half()
    else:
        a = a.float()  # bf16 models hand fp32 activations to the GEMMs
    return a, w.to(dt), w2.to(dt)


@pytest.mark.gpu
@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16], ids=["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SHAPES])
def test_gemm_store_and_add(dt, M, N, K):
    a, w, _ = _inputs(M, N, K, dt, 11)
    ref = a.double() @ w.double().t()
    A, W = a.to(DEV), w.to(DEV)
    part = torch.empty(4 * M * N, dtype=torch.float32, device=DEV)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    _, S = kie.gemm_probe(kie.KIE_GEMM_STORE, A, W, C, part=part)
    err = (C.cpu().double() - ref).abs().max().item() / ref.abs().max().item()
    print(f"store {M}x{N}x{K} {dt}: split {S}, max rel err {err:.2e}", flush=True)
    assert err < 5e-5
    assert (S == 1) == ((N // 128) * ((M + 127) // 128) >= 512)
    c0 = torch.randn(M, N, generator=torch.Generator().manual_seed(12))
    C = c0.to(DEV)
    kie.gemm_probe(kie.KIE_GEMM_ADD, A, W, C, part=part, reps=3)
    want = c0.double() + 3 * ref
    err = (C.cpu().double() - want).abs().max().item() / want.abs().max().item()
    assert err < 5e-5


@pytest.mark.gpu
@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16], ids=["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (77, 192, 512), (300, 128, 256), (640, 1024, 128),
                                   (1100, 16384, 64), (2048, 8192, 128)],
                         ids=["1x64x128", "77x192x512", "300x128x256", "640x1024x128",
                              "1100x16384x64", "2048x8192x128"])  # the last two: fp16 takes the 256 x 256 tiles
def test_gemm_swiglu(dt, M, N, K):
    a, w, w2 = _inputs(M, N, K, dt, 13)
    gt = a.double() @ w.double().t()
    up = a.double() @ w2.double().t()
    ref = gt / (1 + torch.exp(-gt)) * up
    H = torch.empty(M, N, dtype=torch.float16 if dt == torch.float16 else torch.float32, device=DEV)
    kie.gemm_probe(kie.KIE_GEMM_SWIGLU, a.to(DEV), w.to(DEV), H, W2=w2.to(DEV))
    d = (H.cpu().double() - ref).abs()
    if dt == torch.float16:  # fp16 output: half an ulp of each value
        bound = 1e-3 * ref.abs() + 1e-5 * ref.abs().max()
    else:
        bound = 5e-5 * ref.abs().max() + 0 * ref
    print(f"swiglu {M}x{N}x{K} {dt}: max err {d.max().item():.2e}", flush=True)
    assert bool((d <= bound).all())
