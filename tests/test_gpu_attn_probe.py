"""The prompt path's matrix-core causal attention through kie_attn_probe.

Host side (no GPU): argument errors the call rejects before it touches the
device.  GPU: query rows p0 .. p0+M-1 against cache rows 0 .. p0+m, fp16 and
bf16 caches, head widths 64 and 128, 1 / 2 / 4 / 8 query heads per KV head,
ragged row counts (up to 2100) and a nonzero start position, grids with one
query block per work-group and grids large enough for pairs of blocks,
against plain softmax attention in float64 on the CPU over the same (stored)
cache values.
"""
import ctypes
import math

import pytest
import torch

from persistent_decode_monokernel_amd import kie

DEV = "cuda:0"
FAKE = 0x10000


def _call(dtype=kie.KIE_F16, qkv=FAKE, M=16, hq=4, hkv=1, hd=128, p0=0, max_seq=64, kc=FAKE, vc=FAKE, out=FAKE,
          reps=1):
    return kie.lib().kie_attn_probe(dtype, ctypes.c_void_p(qkv), M, hq, hkv, hd, p0, max_seq, ctypes.c_void_p(kc),
                                    ctypes.c_void_p(vc), ctypes.c_void_p(out), reps, None, None)


@pytest.mark.parametrize("kw", [
    {"dtype": 0}, {"qkv": 0}, {"kc": 0}, {"vc": 0}, {"out": 0}, {"reps": 0},
    {"hd": 96}, {"hd": 256}, {"hkv": 0}, {"hq": 3, "hkv": 2}, {"hq": 16, "hkv": 1}, {"hq": 6, "hkv": 2},
    {"M": 0}, {"p0": -1}, {"p0": 60, "M": 5}, {"max_seq": 0}, {"qkv": FAKE + 4}, {"out": FAKE + 8},
], ids=lambda kw: ",".join(f"{k}={v}" for k, v in kw.items()))
def test_argument_errors_before_any_device_call(kw):
    assert _call(**kw) == kie.KIE_ERR_ARG


CASES = [  # (hq, hkv, hd, p0, M)
    (4, 1, 128, 0, 1), (4, 1, 128, 0, 77), (8, 2, 64, 37, 130), (2, 2, 128, 5, 40), (8, 1, 64, 0, 200),
    (16, 4, 128, 100, 64), (16, 4, 128, 0, 2100), (8, 1, 64, 64, 2048), (2, 2, 128, 3, 2077),
    # 63 query blocks x 16 head groups: work-groups take pairs of blocks (the middle one alone)
    (64, 16, 64, 0, 2010), (64, 16, 64, 40, 2010),
]


@pytest.mark.gpu
@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16], ids=["f16", "bf16"])
@pytest.mark.parametrize("hq,hkv,hd,p0,M", CASES, ids=[f"h{c[0]}x{c[1]}_d{c[2]}_p{c[3]}_m{c[4]}" for c in CASES])
def test_causal_attention(dt, hq, hkv, hd, p0, M):
    g = torch.Generator().manual_seed(hq * 1000 + hd + p0 + M)
    max_seq = p0 + M + 3
    ldq = (hq + 2 * hkv) * hd
    qkv = torch.randn(M, ldq, generator=g)
    kc = torch.randn(hkv, max_seq, hd, generator=g).to(dt)
    vc = torch.randn(hkv, max_seq, hd, generator=g).to(dt)
    out = torch.full((M, hq * hd), float("nan"), dtype=torch.float16 if dt == torch.float16 else torch.float32,
                     device=DEV)
    kie.attn_probe(qkv.to(DEV), kc.to(DEV), vc.to(DEV), out, hq, p0)
    # plain softmax attention in float64 over the stored cache values: query m
    # (position p0 + m) sees cache rows 0 .. p0 + m
    q = qkv[:, :hq * hd].double().view(M, hq, hd)
    K, V = kc.double(), vc.double()
    n = p0 + M
    visible = torch.arange(n)[None, :] <= (p0 + torch.arange(M))[:, None]
    ref = torch.empty(M, hq, hd, dtype=torch.float64)
    G = hq // hkv
    for h in range(hq):
        sc = (q[:, h] @ K[h // G, :n].t()) / math.sqrt(hd)
        sc = sc.masked_fill(~visible, float("-inf"))
        ref[:, h] = torch.softmax(sc, 1) @ V[h // G, :n]
    got = out.cpu().double().view(M, hq, hd)
    err = (got - ref).abs().max().item()
    print(f"attention h{hq}/{hkv} d{hd} p0 {p0} M {M} {dt}: max |d| {err:.2e}", flush=True)
    # fp16 operands (queries, softmax weights; bf16: two terms each) and, for
    # fp16 models, a half-precision output: a few 2^-11 of the output scale
    assert err < 4e-3
