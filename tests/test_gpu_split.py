"""Role split (kie_set_split): the attention block on one half of the grid,
the feed-forward block on the other.  Every output row is still reduced in
the same order (the reduction depends only on the row width), so tokens and
logits must equal the unsplit kernel's bit for bit: greedy and sampled, the
tiny decoder, the full-depth ~2B one, a bf16 8B-shaped model with two layers,
an 8192-position context; and the exchange sets must still be recycled."""
import dataclasses

import pytest
import torch

from persistent_decode_monokernel_amd import kie, synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run(shape, w, prompt, n, split, max_seq, sampling=None, kv=None):
    eng = kie.Engine(shape, max_seq=max_seq, device=DEV)
    try:
        eng.load_weights(w)
        eng.set_split(split)
        if sampling is not None:
            eng.set_sampling(*sampling)
        if kv is None:
            tok0, lg0 = eng.prefill(prompt, want_logits=True)
            head_t, head_l = [tok0], [lg0[None]]
        else:
            eng.import_kv(kv[0], kv[1], kv[2])
            head_t, head_l = [], []
        toks, lgs, st = eng.decode(n, want_logits=True)
        assert st == kie.KIE_OK and len(toks) == n
        dirty = eng.idle_sets_dirty_words()
        return head_t + toks, torch.cat(head_l + [lgs]).cpu(), dirty
    finally:
        eng.close()


CASES = [("tiny", None, 16, 24, False), ("tiny", None, 16, 24, True), ("2b", None, 64, 20, False),
         ("8b", 2, 48, 12, False), ("8b", 2, 48, 12, True)]


@pytest.mark.parametrize("name,layers,n_prompt,n_decode,sampled", CASES)
def test_split_matches_unsplit_bit_for_bit(name, layers, n_prompt, n_decode, sampled):
    wl = synth.WORKLOADS[name]
    s = wl.shape if layers is None else dataclasses.replace(wl.shape, n_layers=layers)
    w = synth.make_weights(s, wl.weight_seed, device=DEV)
    prompt = synth.make_prompt(s, n_prompt, wl.prompt_seed).tolist()
    samp = (0.8, 32, 0.9, 5) if sampled else None
    print(f"[split] {s.name} L={s.n_layers}: prompt {n_prompt}, decode {n_decode}, "
          f"{'sampled' if sampled else 'greedy'}", flush=True)
    ms = n_prompt + n_decode + 1
    ref_t, ref_l, d0 = _run(s, w, prompt, n_decode, False, ms, samp)
    t, l, d1 = _run(s, w, prompt, n_decode, True, ms, samp)
    assert t == ref_t
    assert torch.equal(l, ref_l)
    assert d0 == 0 and d1 == 0


def test_split_long_context():
    """8192 cached positions: attention units wrap the half grid twice."""
    s = dataclasses.replace(synth.M2B, n_layers=3)
    w = synth.make_weights(s, 5, device=DEV)
    k, v = synth.make_kv(s, 8192, seed=7, device=DEV)
    print("[split] 2b L=3: 8192 cached positions, decode 8", flush=True)
    ref_t, ref_l, _ = _run(s, w, None, 8, False, 8200, kv=(k, v, 17))
    t, l, _ = _run(s, w, None, 8, True, 8200, kv=(k, v, 17))
    assert t == ref_t
    assert torch.equal(l, ref_l)


def test_split_argument_checks():
    s = synth.TINY
    eng = kie.Engine(s, max_seq=16, device=DEV)
    try:
        assert kie.lib().kie_set_split(eng._h, 2) == kie.KIE_ERR_ARG
        eng.set_split(True)
        with pytest.raises(kie.KieError):  # a grid that is not a multiple of 16
            eng.set_grid(200)
        eng.set_grid(128)
        eng.set_split(False)
        eng.set_grid(200)
        with pytest.raises(kie.KieError):
            eng.set_split(True)
    finally:
        eng.close()
