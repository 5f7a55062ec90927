"""Shared helpers for the GPU parity tests (GPU path vs the CPU oracle)."""
import math

import torch

import oracle
from persistent_decode_monokernel_amd import kie, synth

LOGIT_TOL = 2e-2     # max |logit_gpu - logit_oracle| over vocab and steps
MARGIN = 0.05        # tokens must agree where the oracle's top1 - top2 exceeds this


KV_TOL = 2e-2        # max |cache row - oracle row| beyond one storage ulp (values ~N(0, 1))


def stored_rows_excess(gpu: torch.Tensor, ora: torch.Tensor) -> float:
    """How far two caches of rows stored in a 16-bit format differ beyond one
    ulp of that format: max(|g - o| - ulp) over elements, ulp the format's
    spacing at the larger of |g|, |o|.  Each side rounds its own unrounded
    value (fp32 on the GPU, fp64 in the oracle) to the format; when those lie
    on either side of a rounding boundary the stored values differ by one ulp
    however close the unrounded values were, so correctly rounded rows of
    values within e of each other differ by at most e + 1 ulp."""
    mant = {torch.float16: 10, torch.bfloat16: 7}[gpu.dtype]
    g = gpu.detach().to("cpu", torch.float64)
    o = ora.detach().to("cpu", torch.float64)
    _, e = torch.frexp(torch.maximum(g.abs(), o.abs()))  # |x| in [2^(e-1), 2^e)
    ulp = torch.ldexp(torch.ones_like(g), e - 1 - mant)
    return float(((g - o).abs() - ulp).max())


def top2_margin(logits: torch.Tensor) -> torch.Tensor:
    """top1 - top2 per row."""
    v = torch.topk(logits, 2, dim=-1).values
    return v[..., 0] - v[..., 1]


def weights_on(shape, seed, device, **kw):
    return synth.make_weights(shape, seed, device=device, **kw)


def cpu_copy(w):
    return synth.weights_to(w, "cpu")


def check_tokens_and_logits(gpu_tokens, gpu_logits, ora_logits, what=""):
    """Compare a GPU run with the oracle run teacher-forced on the GPU's own tokens.

    gpu_logits / ora_logits: [n][V]; gpu_tokens[i] is the GPU's choice at row i.
    """
    g = gpu_logits.detach().to("cpu", torch.float64)
    o = ora_logits.detach().to("cpu", torch.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    err = (g - o).abs().max().item()
    assert math.isfinite(err) and err <= LOGIT_TOL, f"{what}: max |dlogit| = {err:.3e} > {LOGIT_TOL}"
    marg = top2_margin(o)
    ora_tok = torch.tensor([oracle.greedy_token(o[i]) for i in range(o.shape[0])])
    gt = torch.tensor(gpu_tokens[: o.shape[0]])
    decisive = marg > MARGIN
    bad = (ora_tok != gt) & decisive
    assert not bad.any(), f"{what}: token mismatch at rows {torch.nonzero(bad).flatten().tolist()[:10]}"
    return err, int(decisive.sum())


def error_curve(gpu_logits, ora_logits, bucket: int = 128):
    """Per-step max |logit_gpu - logit_oracle|, summarised per bucket of
    `bucket` consecutive steps: (first step, last step, max, median).  Shows
    whether the error drifts along a long decode or stays level."""
    g = gpu_logits.detach().to("cpu", torch.float64)
    o = ora_logits.detach().to("cpu", torch.float64)
    per_step = (g - o).abs().amax(dim=1)
    out = []
    for s0 in range(0, per_step.numel(), bucket):
        b = per_step[s0:s0 + bucket]
        out.append((s0, s0 + b.numel() - 1, b.max().item(), b.median().item()))
    return out


def print_error_curve(curve, what=""):
    print(f"{what}: per-step max |dlogit| by bucket (steps: max / median)", flush=True)
    for s0, s1, mx, med in curve:
        print(f"  {s0:5d}-{s1:5d}: {mx:.2e} / {med:.2e}", flush=True)


def check_logits(gpu_logits, ora_logits, what=""):
    """max |logit_gpu - logit_oracle| <= LOGIT_TOL over all rows and vocabulary entries."""
    g = gpu_logits.detach().to("cpu", torch.float64)
    o = ora_logits.detach().to("cpu", torch.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    err = (g - o).abs().max().item()
    assert math.isfinite(err) and err <= LOGIT_TOL, f"{what}: max |dlogit| = {err:.3e} > {LOGIT_TOL}"
    return err


DRAW_MARGIN = 1e-4   # sampled decisions closer than this (relative mass) to a boundary may differ


def check_sampled(gpu_tokens, gpu_logits, positions, temperature, top_k, top_p, seed, what=""):
    """Each sampled token equals the oracle sampler's choice on the GPU's own fp32 logits
    and the same Philox uniform, except where the decision lies within DRAW_MARGIN of a
    boundary of the cumulative weights (fp32 on the device, float64 in the oracle).
    Returns (agreeing, borderline)."""
    g = gpu_logits.detach().to("cpu", torch.float32)
    agree = border = 0
    for row, (tok, pos) in enumerate(zip(gpu_tokens, positions)):
        u = oracle.sampling.uniform_for_position(seed, pos)
        ref, m = oracle.sampling.sample_detail(g[row], temperature, top_k, top_p, u)
        if ref == tok:
            agree += 1
            continue
        assert m is not None and min(m["draw"], m["nucleus"]) < DRAW_MARGIN, \
            f"{what}: row {row} (pos {pos}) token {tok} != oracle {ref}, margins {m}"
        border += 1
    return agree, border
