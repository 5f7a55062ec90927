"""Races and ties of the hand-off protocol, on the GPU.

  * Argmax ties: two LM-head rows made identical give bit-identical logits
    (every row's dot product is reduced in the same order), so whenever they
    hold the largest logit the device must emit the lower index -- across
    work-groups, since the rows sit in different vocabulary slices.
  * A delayed producer: one work-group holds back every hand-off publication
    (kie_set_delay), so every consumer of its words polls them late; tokens and
    logits must not change by a single bit, for a work-group at the start,
    middle and end of the grid.
  * Exchange-set recycling: after a launch, the two sets the last step did not
    use must hold the NaN pattern in every word (kie_check_idle_sets).
  * Determinism at the ~2B size: two identical runs give bit-identical logits.
"""
import pytest
import torch

from persistent_decode_monokernel_amd import kie, synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _tiny():
    wl = synth.WORKLOADS["tiny"]
    w = synth.make_weights(wl.shape, wl.weight_seed, device=DEV)
    prompt = synth.make_prompt(wl.shape, wl.n_prompt, wl.prompt_seed).tolist()
    return wl.shape, w, prompt


def _run(shape, w, prompt, n, max_seq=64, delay=None, sampling=None):
    eng = kie.Engine(shape, max_seq=max_seq, device=DEV)
    try:
        eng.load_weights(w)
        if delay is not None:
            eng.set_delay(*delay)
        if sampling is not None:
            eng.set_sampling(*sampling)
        tok0, lg0 = eng.prefill(prompt, want_logits=True)
        toks, lgs, st = eng.decode(n, want_logits=True)
        assert st == kie.KIE_OK
        return [tok0] + toks, torch.cat([lg0[None], lgs]).cpu()
    finally:
        eng.close()


def test_argmax_tie_goes_to_the_lower_index():
    s, w, prompt = _tiny()
    print("[race] tie: natural first token", flush=True)
    (a, *_), _ = _run(s, w, prompt, 1)
    grid_rows = max(1, s.vocab // 256)  # vocabulary rows per work-group at a 256-wide grid
    b = a - grid_rows - 1 if a > grid_rows else a + grid_rows + 1
    lo, hi = min(a, b), max(a, b)
    w["lm_head"][b].copy_(w["lm_head"][a])  # rows a and b identical
    print(f"[race] tie: rows {a} and {b} identical, decode 24", flush=True)
    seq, lg = _run(s, w, prompt, 24)
    assert torch.equal(lg[:, a], lg[:, b])  # bit-identical logits
    assert seq[0] == lo, (seq[0], a, b)  # the first step's maximum is the tied pair
    ties = 0
    for i, t in enumerate(seq):
        row = lg[i]
        top = row.max()
        if row[a] == top:  # the tied pair holds the maximum: the lower index wins
            assert t == lo, (i, t, lo, hi)
            ties += 1
        else:
            assert t == int(torch.nonzero(row == top)[0])  # first index of the maximum
    assert ties >= 1


@pytest.mark.parametrize("wg,sampled", [(0, False), (101, False), (255, False), (0, True), (200, True)])
def test_delayed_producer_changes_nothing(wg, sampled):
    s, w, prompt = _tiny()
    samp = (0.9, 40, 0.9, 11) if sampled else None
    print(f"[race] delay: reference, then work-group {wg} held back 30 us per publication "
          f"({'sampled' if sampled else 'greedy'})", flush=True)
    ref_t, ref_l = _run(s, w, prompt, 16, sampling=samp)
    t, l = _run(s, w, prompt, 16, delay=(wg, 3000), sampling=samp)
    assert t == ref_t
    assert torch.equal(l, ref_l)


@pytest.mark.parametrize("steps", [2, 3, 13])
def test_idle_exchange_sets_are_recycled(steps):
    s, w, prompt = _tiny()
    print(f"[race] idle sets after decode({steps})", flush=True)
    eng = kie.Engine(s, max_seq=64, device=DEV)
    try:
        eng.load_weights(w)
        eng.prefill(prompt)
        toks, _, st = eng.decode(steps)
        assert st == kie.KIE_OK and len(toks) == steps
        assert eng.idle_sets_dirty_words() == 0
        # and after a sampled launch (its candidate lists live in the sets too)
        eng.set_sampling(0.8, 40, 0.95, 3)
        toks, _, st = eng.decode(steps)
        assert st == kie.KIE_OK
        assert eng.idle_sets_dirty_words() == 0
    finally:
        eng.close()


def test_2b_runs_are_bit_identical():
    s = synth.M2B
    wl = synth.WORKLOADS["2b"]
    w = synth.make_weights(s, wl.weight_seed, device=DEV)
    prompt = synth.make_prompt(s, 128, wl.prompt_seed).tolist()
    print("[race] 2b determinism: two runs of prompt 128 + decode 24", flush=True)
    t1, l1 = _run(s, w, prompt, 24, max_seq=160)
    t2, l2 = _run(s, w, prompt, 24, max_seq=160)
    assert t1 == t2
    assert torch.equal(l1, l2)
    del w
    torch.cuda.empty_cache()
