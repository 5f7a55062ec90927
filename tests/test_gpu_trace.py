"""GPU test of the per-token trace (kie_set_trace): the buffer layout the
timeline reader assumes and the order of the stamps.

The trace is work-group-major: buf[(w * S + s) * 4 + j] for work-group w,
slot s (S = n_layers * 6 + 3) and stamp j (entry, input arrived, arithmetic
done, exit).  On the traced step every work-group stamps every GEMV stage it
runs, so within a slot its non-zero stamps never go back in time, and a
work-group leaves one GEMV stage before it enters the next.  A wrong layout
(slot-major read as work-group-major, or the reverse) mixes stamps of
different work-groups and breaks these orders.  Tracing must not change the
tokens or the logits.
"""
import numpy as np
import pytest
import torch

from persistent_decode_monokernel_amd import kie, synth

pytestmark = pytest.mark.gpu

GEMV_STAGES = (0, 3, 4, 5)  # qkv, wo, gate/up, down: every work-group runs them


def _decode(shape, prompt, w, n, trace_step=None):
    eng = kie.Engine(shape, max_seq=len(prompt) + n + 1)
    eng.load_weights(w)
    buf = None
    if trace_step is not None:
        buf = torch.zeros(eng.trace_words(), dtype=torch.int64, device="cuda")
        eng.set_trace(buf, trace_step)
    tok0, _ = eng.prefill(prompt, want_logits=True)
    toks, lgs, st = eng.decode(n, want_logits=True)
    grid = eng.info().grid
    eng.close()
    assert st == kie.KIE_OK
    return [tok0] + toks, lgs.cpu(), buf, grid


@pytest.mark.parametrize("name", ["tiny", "2b_2layers"])
def test_trace_layout_and_order(name):
    import dataclasses

    shape = synth.TINY if name == "tiny" else dataclasses.replace(synth.M2B, name=name, n_layers=2)
    wl = synth.WORKLOADS["tiny"] if name == "tiny" else synth.WORKLOADS["2b"]
    w = synth.make_weights(shape, wl.weight_seed, device="cuda")
    prompt = synth.make_prompt(shape, 24, wl.prompt_seed).tolist()
    print(f"[trace] {name}: plain and traced decode of 6 steps", flush=True)
    seq0, lg0, _, _ = _decode(shape, prompt, w, 6)
    seq1, lg1, buf, grid = _decode(shape, prompt, w, 6, trace_step=3)
    assert seq0 == seq1 and torch.equal(lg0, lg1)  # tracing changes nothing
    L = shape.n_layers
    S = L * 6 + 3
    assert buf.numel() == grid * S * 4
    tr = buf.cpu().numpy().reshape(grid, S, 4).astype(np.int64)  # [work-group][slot][stamp]
    for wg in range(grid):
        for s in range(L * 6 + 1):  # the stages and the LM head
            x = tr[wg, s][tr[wg, s] > 0]
            assert np.all(np.diff(x) >= 0), (wg, s, tr[wg, s])
        for l in range(L):
            for k in GEMV_STAGES:
                assert tr[wg, 6 * l + k, 0] > 0 and tr[wg, 6 * l + k, 3] > 0, (wg, l, k)
        seq_slots = [6 * l + k for l in range(L) for k in GEMV_STAGES] + [6 * L]
        ex = [tr[wg, s, 3] for s in seq_slots[:-1]]
        en = [tr[wg, s, 0] for s in seq_slots[1:]]
        assert all(a <= b for a, b in zip(ex, en)), (wg, ex, en)
    # every work-group stamped the same traced step: its QKV entries lie within
    # a few hundred microseconds of each other (100 MHz ticks)
    q0 = tr[:, 0, 0]
    assert q0.max() - q0.min() < 100 * 300, (q0.min(), q0.max())
