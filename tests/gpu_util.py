"""Shared helpers for the GPU parity tests (GPU path vs the CPU oracle)."""
import math

import torch

import oracle
from persistent_decode_monokernel_amd import kie, synth

LOGIT_TOL = 2e-2     # max |logit_gpu - logit_oracle| over vocab and steps
MARGIN = 0.05        # tokens must agree where the oracle's top1 - top2 exceeds this


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
