"""kie_create_static: an engine on the library's static device workspace (no
allocation) gives the same tokens and logits as an engine on a caller
workspace (kie_create), call after call, the second call on a smaller input."""
import pytest
import torch

import oracle
from persistent_decode_monokernel_amd import kie, synth
from tests.gpu_util import LOGIT_TOL

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run(shape, w, prompt, n_decode, max_seq, static):
    print(f"[no_alloc] {'static' if static else 'caller'} engine: max_seq {max_seq}, prompt {len(prompt)}, "
          f"decode {n_decode}", flush=True)
    eng = kie.Engine(shape, max_seq=max_seq, device=DEV, static=static)
    try:
        eng.load_weights(w)
        tok0, lg0 = eng.prefill(prompt, want_logits=True)
        toks, lgs, st = eng.decode(n_decode, want_logits=True)
        assert st == kie.KIE_OK
        return [tok0] + toks, torch.cat([lg0[None], lgs]).cpu()
    finally:
        eng.close()


def test_static_workspace_matches_caller_workspace():
    wl = synth.WORKLOADS["tiny"]
    s = wl.shape
    w = synth.make_weights(s, wl.weight_seed, device=DEV)
    wc = synth.weights_to(w, "cpu")
    prompt = synth.make_prompt(s, wl.n_prompt, wl.prompt_seed).tolist()
    # two calls in a row on the static workspace, the second on a smaller input
    for max_seq, n_prompt, n_decode in ((64, 16, 12), (24, 8, 6)):
        p = prompt[:n_prompt]
        ts, ls = _run(s, w, p, n_decode, max_seq, static=True)
        tc, lc = _run(s, w, p, n_decode, max_seq, static=False)
        assert ts == tc, (ts, tc)
        assert torch.equal(ls, lc), (ls - lc).abs().max().item()
        # and both match the oracle (teacher-forced on the emitted tokens)
        ora = oracle.forward(wc, s, p + ts[:-1])[n_prompt - 1:]
        err = (ls.double() - ora).abs().max().item()
        assert err <= LOGIT_TOL, err


def test_static_workspace_limits():
    s = synth.WORKLOADS["tiny"].shape
    big = kie.make_config(s, 4096)
    assert kie.workspace_bytes(big) > kie.KIE_STATIC_WORKSPACE_BYTES
    with pytest.raises(kie.KieError) as ei:
        kie.Engine(s, max_seq=4096, device=DEV, static=True)
    assert ei.value.status == kie.KIE_ERR_CAPACITY
    # one static engine per GPU at a time
    e1 = kie.Engine(s, max_seq=32, device=DEV, static=True)
    try:
        with pytest.raises(kie.KieError) as ei:
            kie.Engine(s, max_seq=32, device=DEV, static=True)
        assert ei.value.status == kie.KIE_ERR_STATE
    finally:
        e1.close()
    e2 = kie.Engine(s, max_seq=32, device=DEV, static=True)  # released: available again
    e2.close()
