"""Pins of the fp32 C++ CPU decoder (oracle/cpu_decoder.cpp) against the
float64 oracle, which is itself pinned by brute force and closed forms
(test_oracle_pins.py).  The two are independent implementations of the same
definition; on tiny shapes their logits agree within 1e-4 (fp32 rounding)."""
import pytest
import torch

import oracle
from oracle.cpu_decoder import CpuDecoder
from persistent_decode_monokernel_amd import synth

TOL = 1e-4

SMALL = synth.small_shape(n_layers=3, d_model=64, n_heads=8, n_kv_heads=2, head_dim=16, d_ffn=96, vocab=101)
MHA = synth.small_shape(n_layers=2, d_model=32, n_heads=4, n_kv_heads=4, head_dim=8, d_ffn=48, vocab=57)


@pytest.mark.parametrize("shape,seed", [(SMALL, 3), (MHA, 4)])
def test_full_causal_pass_matches_float64(shape, seed):
    w = synth.make_weights(shape, seed, gain_jitter=0.2, std=0.15)
    toks = synth.make_prompt(shape, 40, seed + 10).tolist()
    ref = oracle.forward(w, shape, toks)
    dec = CpuDecoder(shape, w, max_seq=64, n_threads=3)
    got = dec.feed(toks).double()
    assert dec.position == len(toks)
    err = float((got - ref).abs().max())
    assert err <= TOL, err


def test_greedy_token_is_first_argmax_of_its_logits():
    w = synth.make_weights(SMALL, 5, std=0.15)
    dec = CpuDecoder(SMALL, w, max_seq=32)
    toks = synth.make_prompt(SMALL, 12, 6).tolist()
    for t in toks:
        g, lg = dec.step(t)
        assert g == oracle.argmax_first(lg)


def test_thread_count_changes_no_bit():
    w = synth.make_weights(SMALL, 7, std=0.15)
    toks = synth.make_prompt(SMALL, 16, 8).tolist()
    a = CpuDecoder(SMALL, w, max_seq=32, n_threads=1).feed(toks)
    b = CpuDecoder(SMALL, w, max_seq=32, n_threads=7).feed(toks)
    assert torch.equal(a, b)


@pytest.mark.parametrize("n_pos", [1, 700, 5000])
def test_imported_cache_and_far_positions_match_float64(n_pos):
    """A cache imported at n_pos positions, then tokens teacher-forced: the
    rotation angles at positions in the thousands must still be accurate."""
    shape = synth.small_shape(n_layers=2, d_model=32, n_heads=4, n_kv_heads=2, head_dim=16, d_ffn=48, vocab=61)
    w = synth.make_weights(shape, 9, std=0.2)
    k, v = synth.make_kv(shape, n_pos, seed=10)
    fed = [3, 14, 15, 9, 26]
    ref = oracle.teacher_forced(w, shape, oracle.KVCache.from_tensors(k, v), fed)
    dec = CpuDecoder(shape, w, max_seq=n_pos + len(fed), n_threads=2)
    dec.set_cache(k, v)
    assert dec.position == n_pos
    got = dec.feed(fed).double()
    err = float((got - ref).abs().max())
    assert err <= TOL, err


def test_errors():
    w = synth.make_weights(MHA, 1, std=0.2)
    dec = CpuDecoder(MHA, w, max_seq=2)
    with pytest.raises(ValueError):
        dec.step(MHA.vocab)
    dec.step(1)
    dec.step(2)
    with pytest.raises(ValueError):  # cache full
        dec.step(3)
    k, v = synth.make_kv(MHA, 2, seed=1)
    with pytest.raises(ValueError):  # no room left for a step
        dec.set_cache(k, v)
