"""One launch per stage (kie_set_launch_mode) against the persistent kernel.
The per-stage launches run the same stage code on the same tiling, so tokens
and logits must agree bit for bit -- from a host loop and from a HIP graph --
on the tiny decoder and the full-depth ~2B one; the modes reject what they do
not support."""
import pytest
import torch

from persistent_decode_monokernel_amd import kie, synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run(shape, w, prompt, n, mode, max_seq):
    eng = kie.Engine(shape, max_seq=max_seq, device=DEV)
    try:
        eng.load_weights(w)
        tok0, _ = eng.prefill(prompt)
        eng.set_launch_mode(mode)
        toks, lgs, st = eng.decode(n, want_logits=True)
        assert st == kie.KIE_OK and len(toks) == n
        toks2, lgs2, st2 = eng.decode(3, want_logits=True)  # a second call continues the sequence
        assert st2 == kie.KIE_OK
        dirty = eng.idle_sets_dirty_words()
        return [tok0] + toks + toks2, torch.cat([lgs, lgs2]).cpu(), dirty
    finally:
        eng.close()


@pytest.mark.parametrize("name,n_prompt,n_decode", [("tiny", 16, 12), ("2b", 32, 6)])
def test_per_stage_launches_match_persistent(name, n_prompt, n_decode):
    wl = synth.WORKLOADS[name]
    s = wl.shape
    w = synth.make_weights(s, wl.weight_seed, device=DEV)
    prompt = synth.make_prompt(s, n_prompt, wl.prompt_seed).tolist()
    ms = n_prompt + n_decode + 4
    print(f"[launch modes] {name}: persistent", flush=True)
    ref_t, ref_l, _ = _run(s, w, prompt, n_decode, kie.KIE_LAUNCH_PERSISTENT, ms)
    for mode in (kie.KIE_LAUNCH_PER_STAGE, kie.KIE_LAUNCH_PER_STAGE_GRAPH):
        print(f"[launch modes] {name}: mode {mode}", flush=True)
        t, l, dirty = _run(s, w, prompt, n_decode, mode, ms)
        assert t == ref_t
        assert torch.equal(l, ref_l)
        assert dirty == 0


def test_per_stage_rejects_what_it_does_not_support():
    s = synth.TINY
    w = synth.make_weights(s, 1, device=DEV)
    eng = kie.Engine(s, max_seq=32, device=DEV)
    try:
        eng.load_weights(w)
        eng.prefill([1, 2, 3])
        for bad in (-1, 3):
            with pytest.raises(kie.KieError):
                eng.set_launch_mode(bad)
        eng.set_launch_mode(kie.KIE_LAUNCH_PER_STAGE)
        toks, _, st = eng.decode(2, eos_id=5, raise_on_error=False)
        assert st == kie.KIE_ERR_UNSUPPORTED and toks == []
        eng.set_sampling(0.8, 8, 0.9, 1)
        _, _, st = eng.decode(2, raise_on_error=False)
        assert st == kie.KIE_ERR_UNSUPPORTED
        eng.set_sampling(0.0)
        eng.set_launch_mode(kie.KIE_LAUNCH_PERSISTENT)
        toks, _, st = eng.decode(2)
        assert st == kie.KIE_OK and len(toks) == 2
    finally:
        eng.close()
