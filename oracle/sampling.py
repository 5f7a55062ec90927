"""Oracle: token sampling beyond greedy, and the counter-based generator it draws from.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module;
only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code with the GPU path.

What the pages fix.  The engine's per-request loop ends each token with
LM-head sampling and the end-of-sequence check, on the device (revietech.ru,
"Kog vyzhimayet maksimum iz GPU: 3000 tokenov/s", section "Chto takoye
monokernel").  They do not say which sampling rule.  Greedy decoding is the
oracle's ``decoder`` module.  This module is the reading taken for sampling
beyond greedy; each step is plain and written in the order below.

Sampling rule (reading; the same definition is implemented on the device):
  1. Candidates: the vocabulary ordered by logit, larger first, ties to the
     lower token index; keep the first ``top_k`` (1 <= top_k <= 64).
  2. Weights w_j = exp((z_j - z_0) / temperature) over the kept candidates
     (z_0 the largest logit), temperature > 0; cumulative sums S_j in that
     order, S_j = w_0 + ... + w_j.
  3. Nucleus: keep the first n candidates, n the smallest count whose mass
     reaches the fraction top_p of the total: S_{n-1} >= top_p * S_{k-1}
     (0 < top_p <= 1; n >= 1).
  4. Draw: r = u * S_{n-1} for a uniform u in [0, 1); the token is candidate
     j, the first with S_j > r (inverse of the cumulative distribution).
  temperature <= 0 means greedy: the first index of the largest logit.

Uniform numbers (reading): the draw for the token that follows position p
(the position of the token fed to that step) takes u from Philox4x32-10 (J.
K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random numbers: as
easy as 1, 2, 3", SC'11): counter (p, 0, 0, 0), key (seed mod 2^32,
floor(seed / 2^32)), u = (first output word >> 8) * 2^-24, exact in fp32 and
fp64.  The position alone picks the number, so the tokens of a sequence do not
depend on how decoding is split into calls.

Arithmetic: logits come in as given (the engine's fp32 values; ordering
compares them exactly); weights, sums and the draw threshold are float64.

Pins (tests/test_oracle_sampling.py): the published Philox4x32-10 known-answer
vectors (tests/golden/philox4x32_10_kat.txt); the same round function at 64-bit
words against numpy's independent Philox4x64-10; the output distribution over a
uniform grid of u equal to the renormalised softmax of the kept set; the kept
set against brute force; top_k = 1 and temperature -> 0 equal to greedy.
"""
from __future__ import annotations

import numpy as np
import torch

from .decoder import argmax_first

# Philox constants (Salmon et al., SC'11): round multipliers and the key
# increments (Weyl sequence) per word width.
PHILOX = {
    32: dict(mult=(0xD2511F53, 0xCD9E8D57), weyl=(0x9E3779B9, 0xBB67AE85)),
    64: dict(mult=(0xD2E7470EE14C6C93, 0xCA5A826395121157), weyl=(0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)),
}
MAX_TOP_K = 64


def philox4(counter, key, width: int = 32, rounds: int = 10):
    """Philox4xW-R block function: 4 counter words, 2 key words -> 4 words.

    Each round multiplies counter words 0 and 2 by the two constants, and the
    new words are (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1,
    lo(M0*c0)); the key is incremented by the Weyl constants before every
    round after the first (Salmon et al., SC'11, section on Philox)."""
    mask = (1 << width) - 1
    m0, m1 = PHILOX[width]["mult"]
    w0, w1 = PHILOX[width]["weyl"]
    c = [int(x) & mask for x in counter]
    k0, k1 = int(key[0]) & mask, int(key[1]) & mask
    for r in range(rounds):
        if r > 0:
            k0, k1 = (k0 + w0) & mask, (k1 + w1) & mask
        p0, p1 = m0 * c[0], m1 * c[2]
        c = [(p1 >> width) ^ c[1] ^ k0, p1 & mask, (p0 >> width) ^ c[3] ^ k1, p0 & mask]
    return c


def uniform_for_position(seed: int, pos: int) -> float:
    """u in [0, 1) for the draw after position `pos`: top 24 bits of the first
    Philox4x32-10 word, counter (pos, 0, 0, 0), key from the 64-bit seed."""
    seed = int(seed) & ((1 << 64) - 1)
    x0 = philox4([int(pos), 0, 0, 0], [seed & 0xFFFFFFFF, seed >> 32], 32, 10)[0]
    return (x0 >> 8) * 2.0 ** -24


def candidate_order(logits) -> np.ndarray:
    """Token indices by logit, larger first, ties to the lower index."""
    z = np.asarray(torch.as_tensor(logits).double().numpy())
    return np.lexsort((np.arange(z.size), -z))


def sample_detail(logits, temperature: float, top_k: int, top_p: float, u: float):
    """Apply the sampling rule; returns (token, margins).  `margins` measures
    how far the decision is from a boundary, relative to the kept mass: the
    distance of r from the nearest cumulative sum (`draw`) and of top_p from
    the nearest normalised cumulative sum (`nucleus`).  Greedy: margins None."""
    z = torch.as_tensor(logits).double()
    if temperature <= 0:
        return int(argmax_first(z)), None
    if not 1 <= top_k <= MAX_TOP_K or not 0 < top_p <= 1:
        raise ValueError("top_k in [1, 64], top_p in (0, 1]")
    order = candidate_order(z)[:top_k]
    zc = z.numpy()[order]
    w = np.exp((zc - zc[0]) / temperature)
    S = np.cumsum(w)
    total = S[-1]
    n = int(np.argmax(S >= top_p * total)) + 1  # first index reaching the mass (S[-1] always does)
    r = u * S[n - 1]
    j = int(np.argmax(S[:n] > r))
    margins = {"draw": float(np.min(np.abs(S[:n] - r)) / S[n - 1]),
               "nucleus": float(np.min(np.abs(S / total - top_p)))}
    return int(order[j]), margins


def sample_token(logits, temperature: float, top_k: int, top_p: float, u: float) -> int:
    return sample_detail(logits, temperature, top_k, top_p, u)[0]

