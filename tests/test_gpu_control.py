"""Control paths of the persistent decode on the tiny decoder: on-device EOS,
abort and resume, a forced poll timeout and the restart after it, state and
capacity errors, and the KV-cache checkpoint round trip.

The timeout is forced from the host: one work-group withholds its end-of-step
partial and the poll deadline is shortened, so every work-group's bounded wait
ends and the kernel exits normally with KIE_ERR_TIMEOUT.
"""
import pytest
import torch

from persistent_decode_monokernel_amd import kie, synth

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS["tiny"]
S = W.shape
N = W.n_decode


@pytest.fixture(scope="module")
def eng():
    w = synth.make_weights(S, W.weight_seed, device="cuda")
    e = kie.Engine(S, max_seq=W.n_prompt + 2 * N)
    e.load_weights(w)
    e._w = w  # keep the borrowed weights alive
    yield e
    e.close()


@pytest.fixture(scope="module")
def prompt():
    return synth.make_prompt(S, W.n_prompt, W.prompt_seed).tolist()


@pytest.fixture(scope="module")
def ref(eng, prompt):
    tok0, _ = eng.prefill(prompt)
    toks, _, st = eng.decode(N)
    assert st == kie.KIE_OK
    return tok0, toks


def test_eos_stops_after_emitting_it(eng, prompt, ref):
    _, toks = ref
    for k in (0, 5, N - 1):
        eos = toks[k]
        first = toks.index(eos)
        eng.prefill(prompt)
        out, _, st = eng.decode(N, eos_id=eos)
        assert st == kie.KIE_OK
        assert out == toks[: first + 1], (k, eos)
        assert eng.info().pos == W.n_prompt + first + 1


def test_abort_keeps_the_sequence(eng, prompt, ref):
    _, toks = ref
    eng.prefill(prompt)
    eng.set_abort_after(7)
    out, _, st = eng.decode(N, raise_on_error=False)
    assert st == kie.KIE_ERR_ABORTED and out == toks[:7]
    assert eng.info().pos == W.n_prompt + 7
    rest, _, st = eng.decode(N - 7)  # the request was consumed; decoding goes on
    assert st == kie.KIE_OK and out + rest == toks


def test_abort_before_any_step(eng, prompt, ref):
    eng.prefill(prompt)
    eng.set_abort_after(0)
    out, _, st = eng.decode(4, raise_on_error=False)
    assert st == kie.KIE_ERR_ABORTED and out == []
    assert eng.info().pos == W.n_prompt


def test_forced_timeout_then_restart(eng, prompt, ref):
    tok0, toks = ref
    eng.prefill(prompt)
    eng.set_withhold(5)
    eng.set_poll_timeout(2_000_000)  # 20 ms of the 100 MHz counter
    try:
        out, _, st = eng.decode(4, raise_on_error=False)
    finally:
        eng.set_withhold(-1)
        eng.set_poll_timeout(0)
    assert st == kie.KIE_ERR_TIMEOUT and out == []
    # the step that timed out may have left a partial cache row
    with pytest.raises(kie.KieError) as ei:
        eng.decode(1)
    assert ei.value.status == kie.KIE_ERR_STATE
    t, _ = eng.prefill(prompt)
    again, _, st = eng.decode(N)
    assert st == kie.KIE_OK and t == tok0 and again == toks


def test_state_and_capacity_errors(prompt):
    w = synth.make_weights(S, W.weight_seed, device="cuda")
    e = kie.Engine(S, max_seq=W.n_prompt + 4)
    with pytest.raises(kie.KieError) as ei:
        e.prefill(prompt)  # no weights yet
    assert ei.value.status == kie.KIE_ERR_STATE
    e.load_weights(w)
    with pytest.raises(kie.KieError) as ei:
        e.decode(1)  # no sequence yet
    assert ei.value.status == kie.KIE_ERR_STATE
    with pytest.raises(kie.KieError) as ei:
        e.prefill([S.vocab] + prompt[1:])  # token out of range
    assert ei.value.status == kie.KIE_ERR_ARG
    e.prefill(prompt)
    with pytest.raises(kie.KieError) as ei:
        e.decode(5)  # pos 16 + 5 > max_seq 20
    assert ei.value.status == kie.KIE_ERR_CAPACITY
    out, _, st = e.decode(0)
    assert st == kie.KIE_OK and out == []
    out, _, st = e.decode(4)
    assert st == kie.KIE_OK and len(out) == 4
    with pytest.raises(kie.KieError) as ei:
        e.decode(1)
    assert ei.value.status == kie.KIE_ERR_CAPACITY
    e.close()


def test_kv_export_import_resumes(eng, prompt, ref):
    tok0, toks = ref
    eng.prefill(prompt)
    a, _, _ = eng.decode(10)
    k, v, pending = eng.export_kv()
    assert k.shape == (S.n_layers, S.n_kv_heads, W.n_prompt + 10, S.head_dim) and pending == a[-1]
    b, _, _ = eng.decode(N - 10)
    assert a + b == toks
    # a second engine resumes from the checkpoint
    e2 = kie.Engine(S, max_seq=W.n_prompt + 2 * N)
    e2.load_weights(eng._w)
    e2.import_kv(k, v, pending)
    c, _, _ = e2.decode(N - 10)
    assert c == b
    k2, v2, _ = e2.export_kv()
    assert torch.equal(k2[:, :, : k.shape[2]], k) and torch.equal(v2[:, :, : v.shape[2]], v)
    e2.close()
