"""The arrival-counter hand-off (kie_set_handoff, the comparison protocol)
against the default NaN-polled hand-off: the same kernels do the same
arithmetic in the same order, only the way consumers learn that their inputs
are complete differs, so tokens and logits must agree bit for bit -- greedy and
sampled, on the full-depth ~2B decoder and reduced-depth ~2B and ~8B-shaped
ones (the shapes the counter instance is built for) -- and the exchange sets
must still be recycled to the NaN pattern."""
import dataclasses

import pytest
import torch

from persistent_decode_monokernel_amd import kie, synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run(shape, w, prompt, n, handoff, max_seq, sampling=None):
    eng = kie.Engine(shape, max_seq=max_seq, device=DEV)
    try:
        eng.load_weights(w)
        eng.set_handoff(handoff)
        if sampling is not None:
            eng.set_sampling(*sampling)
        tok0, lg0 = eng.prefill(prompt, want_logits=True)
        toks, lgs, st = eng.decode(n, want_logits=True)
        assert st == kie.KIE_OK and len(toks) == n
        dirty = eng.idle_sets_dirty_words()
        return [tok0] + toks, torch.cat([lg0[None], lgs]).cpu(), dirty
    finally:
        eng.close()


@pytest.mark.parametrize("name,layers,n_prompt,n_decode,sampled", [("2b", None, 64, 16, False),
                                                                  ("2b", 4, 40, 16, True),
                                                                  ("8b", 2, 40, 12, False)])
def test_counters_match_nan_polls_bit_for_bit(name, layers, n_prompt, n_decode, sampled):
    wl = synth.WORKLOADS[name]
    s = wl.shape if layers is None else dataclasses.replace(wl.shape, n_layers=layers)
    w = synth.make_weights(s, wl.weight_seed, device=DEV)
    prompt = synth.make_prompt(s, n_prompt, wl.prompt_seed).tolist()
    samp = (0.8, 32, 0.9, 5) if sampled else None
    print(f"[handoff] {name}: prompt {n_prompt}, decode {n_decode}, {'sampled' if sampled else 'greedy'}", flush=True)
    ref_t, ref_l, d0 = _run(s, w, prompt, n_decode, kie.KIE_HANDOFF_NAN_POLL, n_prompt + n_decode + 1, samp)
    t, l, d1 = _run(s, w, prompt, n_decode, kie.KIE_HANDOFF_COUNTERS, n_prompt + n_decode + 1, samp)
    assert t == ref_t
    assert torch.equal(l, ref_l)
    assert d0 == 0 and d1 == 0


def test_handoff_argument_checks():
    s = dataclasses.replace(synth.M2B, n_layers=1)
    eng = kie.Engine(s, max_seq=8, device=DEV)
    try:
        for bad in (-1, 2, 7):
            assert kie.lib().kie_set_handoff(eng._h, bad) == kie.KIE_ERR_ARG
        eng.set_handoff(kie.KIE_HANDOFF_COUNTERS)
        eng.set_handoff(kie.KIE_HANDOFF_NAN_POLL)
    finally:
        eng.close()
    eng = kie.Engine(synth.TINY, max_seq=8, device=DEV)  # no counter instance for this shape
    try:
        assert kie.lib().kie_set_handoff(eng._h, kie.KIE_HANDOFF_COUNTERS) == kie.KIE_ERR_UNSUPPORTED
        eng.set_handoff(kie.KIE_HANDOFF_NAN_POLL)
    finally:
        eng.close()
