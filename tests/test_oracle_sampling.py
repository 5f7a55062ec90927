"""Pins of the oracle's sampler and generator (oracle/sampling.py), CPU only.

Generator: the published Philox4x32-10 known-answer vectors; the same round
function at 64-bit words against numpy's own Philox4x64-10 (an independent
implementation; numpy advances its counter by one before each block).
Sampler: the distribution it draws from, enumerated over a uniform grid of u,
equals the renormalised softmax of the nucleus computed here by brute force
(sorted with Python's sort, exponentials with math.exp, the cut by trying every
prefix length); top_k = 1 and tiny temperatures reduce to greedy; a planted
mistake (the wrong candidate order) is caught.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import sampling

HERE = os.path.dirname(__file__)


def kat_vectors():
    rows = []
    with open(os.path.join(HERE, "golden", "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                w = [int(x, 16) for x in line.split()]
                rows.append((w[0:4], w[4:6], w[6:10]))
    return rows


@pytest.mark.parametrize("ctr,key,out", kat_vectors())
def test_philox4x32_10_known_answers(ctr, key, out):
    assert sampling.philox4(ctr, key, 32, 10) == out


@pytest.mark.parametrize("key,start", [((0, 0), 0), ((0x0123456789ABCDEF, 0xFEDCBA9876543210), 0),
                                       ((2**64 - 1, 12345), 7)])
def test_philox4x64_10_matches_numpy(key, start):
    bg = np.random.Philox(counter=np.array([start, 0, 0, 0], dtype=np.uint64),
                          key=np.array(key, dtype=np.uint64))
    raw = [int(x) for x in bg.random_raw(12)]
    for blk in range(3):
        assert sampling.philox4([start + 1 + blk, 0, 0, 0], key, 64, 10) == raw[4 * blk:4 * blk + 4]


def test_uniform_is_24_bit_and_position_keyed():
    us = [sampling.uniform_for_position(99, p) for p in range(200)]
    assert all(0.0 <= u < 1.0 and (u * 2**24).is_integer() for u in us)
    assert len(set(us)) == 200
    assert sampling.uniform_for_position(99, 5) != sampling.uniform_for_position(100, 5)
    # the key takes both 32-bit halves of the seed
    assert sampling.uniform_for_position(1, 5) != sampling.uniform_for_position(1 + 2**32, 5)
    x0 = sampling.philox4([5, 0, 0, 0], [7, 3], 32, 10)[0]
    assert sampling.uniform_for_position(7 + (3 << 32), 5) == (x0 >> 8) / 2**24


def brute_nucleus(z, temperature, top_k, top_p):
    """{token: probability}: candidates by Python's sort on (-logit, index),
    weights exp((z - max) / T), the shortest prefix with mass >= top_p."""
    cand = sorted(range(len(z)), key=lambda i: (-float(z[i]), i))[:top_k]
    w = [math.exp((float(z[i]) - float(z[cand[0]])) / temperature) for i in cand]
    total = sum(w)
    for n in range(1, len(w) + 1):
        if sum(w[:n]) >= top_p * total:
            break
    kept = sum(w[:n])
    return {cand[i]: w[i] / kept for i in range(n)}


CASES = [(1.0, 64, 1.0), (0.7, 40, 0.9), (1.3, 8, 0.5), (0.5, 64, 0.95), (2.0, 20, 1.0), (1.0, 3, 0.01)]


@pytest.mark.parametrize("temperature,top_k,top_p", CASES)
def test_draw_distribution_equals_nucleus_softmax(temperature, top_k, top_p):
    g = torch.Generator().manual_seed(int(temperature * 100) + top_k)
    z = (torch.randn(300, generator=g) * 2).float()
    z[17] = z[3]  # a tie: the lower index comes first
    target = brute_nucleus(z, temperature, top_k, top_p)
    N = 20000
    counts = {}
    for j in range(N):
        t = sampling.sample_token(z, temperature, top_k, top_p, (j + 0.5) / N)
        counts[t] = counts.get(t, 0) + 1
    assert set(counts) <= set(target)
    for tok, p in target.items():
        assert abs(counts.get(tok, 0) / N - p) <= 1.0 / N + 1e-12, (tok, p)


def test_top_k_one_and_cold_temperature_are_greedy():
    g = torch.Generator().manual_seed(5)
    for _ in range(20):
        z = torch.randn(1000, generator=g).float()
        cold_best = int(torch.argmax(z))  # continuous draws: no tie at the maximum
        for u in (0.0, 0.3, 0.999999):
            assert sampling.sample_token(z, 1e-4, 64, 1.0, u) == cold_best
        z[int(torch.randint(0, 1000, (1,), generator=g))] = z.max()  # tie at the maximum
        best = int(torch.nonzero(z == z.max())[0, 0])
        for u in (0.0, 0.3, 0.999999):
            assert sampling.sample_token(z, 0.8, 1, 1.0, u) == best
        assert sampling.sample_token(z, 0.0, 64, 1.0, 0.5) == best


def test_small_top_p_keeps_one_candidate_and_extremes_of_u():
    z = torch.tensor([0.0, 2.0, 1.0, 2.0, -1.0])
    # ordered candidates: 1, 3 (tie, lower index first), 2, 0, 4
    assert sampling.sample_token(z, 1.0, 5, 1e-6, 0.99) == 1
    assert sampling.sample_token(z, 1.0, 5, 1.0, 0.0) == 1
    assert sampling.sample_token(z, 1.0, 5, 1.0, 1 - 2**-24) == 4
    assert sampling.sample_token(z, 1.0, 2, 1.0, 0.49) == 1 and sampling.sample_token(z, 1.0, 2, 1.0, 0.51) == 3


def test_rejects_out_of_range_arguments():
    z = torch.zeros(10)
    for k, p in ((0, 1.0), (65, 1.0), (5, 0.0), (5, 1.5)):
        with pytest.raises(ValueError):
            sampling.sample_token(z, 1.0, k, p, 0.5)


def test_planted_wrong_order_is_caught(monkeypatch):
    """Candidates taken in increasing logit order: the distribution pin fails."""
    monkeypatch.setattr(sampling, "candidate_order",
                        lambda logits: np.lexsort((np.arange(len(logits)), np.asarray(torch.as_tensor(logits)))))
    with pytest.raises(AssertionError):
        test_draw_distribution_equals_nucleus_softmax(1.0, 8, 0.9)
