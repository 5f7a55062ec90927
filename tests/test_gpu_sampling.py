"""GPU parity of on-device sampling (kie_set_sampling): temperature, top-k and
nucleus draws with Philox4x32-10 uniforms, inside the persistent kernel.

Every emitted token -- the prompt's next token and each decode step's -- is
checked against the oracle sampler applied to the GPU's own fp32 logits with
the same uniform (counter = position of the fed token); the logits themselves
against the oracle teacher-forced on the GPU's tokens (2e-2).  A decision that
lies within 1e-4 of a boundary of the cumulative weights may go either way
(fp32 sums on the device, float64 in the oracle).  Shapes: the tiny decoder
(16 vocabulary rows per work-group: padded candidate lists) and a one-layer
model with a 128256-entry vocabulary (~500 rows per work-group).  Also: top_k
= 1 equals greedy, tokens do not depend on how decoding is split into calls,
and the argument checks.
"""
import pytest
import torch

import oracle
from persistent_decode_monokernel_amd import kie, synth
from tests.gpu_util import check_logits, check_sampled, cpu_copy

pytestmark = pytest.mark.gpu

BIGV = synth.ModelShape("bigvocab", 1, 256, 4, 4, 64, 512, 128256, synth.F16)


def run(shape, T, k, p, seed, P=12, n=40, wseed=3):
    w = synth.make_weights(shape, wseed, device="cuda", gain_jitter=0.1)
    prompt = synth.make_prompt(shape, P, wseed + 1).tolist()
    eng = kie.Engine(shape, max_seq=P + n + 1)
    eng.load_weights(w)
    eng.set_sampling(T, k, p, seed)
    tok0, lg0 = eng.prefill(prompt, want_logits=True)
    toks, lgs, st = eng.decode(n, want_logits=True)
    assert st == kie.KIE_OK and len(toks) == n
    eng.close()
    seq = [tok0] + toks
    gpu = torch.cat([lg0[None].cpu(), lgs.cpu()])
    return w, prompt, seq, gpu


@pytest.mark.parametrize("shape,T,k,p,seed", [
    (synth.TINY, 1.0, 64, 1.0, 7),
    (synth.TINY, 0.7, 40, 0.9, 8),
    (BIGV, 1.2, 50, 0.95, 9),
    (BIGV, 0.5, 8, 0.5, 10),
])
def test_sampled_tokens_match_oracle(shape, T, k, p, seed):
    w, prompt, seq, gpu = run(shape, T, k, p, seed)
    P = len(prompt)
    positions = list(range(P - 1, P - 1 + len(seq)))  # position of the token fed to each step
    agree, border = check_sampled(seq, gpu, positions, T, k, p, seed, shape.name)
    cache = oracle.KVCache(shape.n_layers, shape.n_kv_heads, shape.head_dim)
    ora = oracle.forward(cpu_copy(w), shape, prompt + seq[:-1], cache, logits_rows=list(range(P - 1, P - 1 + len(seq))))
    err = check_logits(gpu, ora, shape.name)
    distinct = len(set(seq))
    print(f"{shape.name} T={T} k={k} p={p}: {agree} agree, {border} borderline, {distinct} distinct tokens, "
          f"max |dlogit| {err:.2e}")
    assert border <= 1
    if k > 1 and T >= 1.0:
        assert distinct > 1  # a sampled sequence, not a greedy one


def test_top_k_one_is_greedy():
    s = synth.TINY
    w = synth.make_weights(s, 5, device="cuda")
    prompt = synth.make_prompt(s, 10, 6).tolist()
    out = []
    for samp in (False, True):
        eng = kie.Engine(s, max_seq=64)
        eng.load_weights(w)
        if samp:
            eng.set_sampling(1.0, 1, 1.0, 1234)
        t0, _ = eng.prefill(prompt)
        toks, _, st = eng.decode(30)
        assert st == kie.KIE_OK
        out.append([t0] + toks)
        eng.close()
    assert out[0] == out[1]


def test_split_calls_give_the_same_sequence():
    s = synth.TINY
    w = synth.make_weights(s, 11, device="cuda")
    prompt = synth.make_prompt(s, 9, 12).tolist()
    seqs = []
    for parts in ((24,), (5, 7, 12)):
        eng = kie.Engine(s, max_seq=64)
        eng.load_weights(w)
        eng.set_sampling(1.0, 64, 1.0, 99)
        seq = [eng.prefill(prompt)[0]]
        for n in parts:
            toks, _, st = eng.decode(n)
            assert st == kie.KIE_OK
            seq += toks
        seqs.append(seq)
        eng.close()
    assert seqs[0] == seqs[1]
    assert len(set(seqs[0])) > 1


def test_sampling_arguments_checked():
    eng = kie.Engine(synth.TINY, max_seq=32)
    for args in ((1.0, 0, 1.0), (1.0, 65, 1.0), (1.0, 8, 0.0), (1.0, 8, 1.5), (float("nan"), 8, 1.0),
                 (1e-45, 8, 1.0)):
        with pytest.raises(kie.KieError) as ei:
            eng.set_sampling(*args, seed=1)
        assert ei.value.status == kie.KIE_ERR_ARG, args
    eng.set_sampling(0.0, 0, 0.0)  # greedy: the other arguments are ignored
    eng.set_sampling(0.8, 64, 1.0, 2**64 - 1)
    eng.close()


@pytest.mark.parametrize("shape,grid", [(synth.TINY, 60), (synth.TINY, 97), (BIGV, 255)])
def test_sampling_on_subset_grids(shape, grid):
    """Work-group 0's merge of the group lists takes a different branch for <= 8,
    <= 16 and <= 32 groups, and a grid that 8 does not divide leaves padding
    lists in the last group."""
    T, k, p, seed = 1.0, 64, 0.97, 21
    w = synth.make_weights(shape, 17, device="cuda", gain_jitter=0.1)
    prompt = synth.make_prompt(shape, 10, 18).tolist()
    eng = kie.Engine(shape, max_seq=40)
    eng.load_weights(w)
    eng.set_grid(grid)
    eng.set_sampling(T, k, p, seed)
    tok0, lg0 = eng.prefill(prompt, want_logits=True)
    toks, lgs, st = eng.decode(24, want_logits=True)
    assert st == kie.KIE_OK
    eng.close()
    seq = [tok0] + toks
    gpu = torch.cat([lg0[None].cpu(), lgs.cpu()])
    positions = list(range(len(prompt) - 1, len(prompt) - 1 + len(seq)))
    agree, border = check_sampled(seq, gpu, positions, T, k, p, seed, f"{shape.name} grid {grid}")
    print(f"{shape.name} grid {grid}: {agree} agree, {border} borderline, {len(set(seq))} distinct")
    assert border <= 1 and len(set(seq)) > 1


BF16_SHAPE = synth.ModelShape("g2_hd128_bf16", 3, 1024, 8, 4, 128, 2048, 2048, synth.BF16)


def test_sampled_tokens_match_oracle_bf16():
    """bf16 kernel instances (three-term activations), oracle cache stored in bf16."""
    T, k, p, seed = 0.9, 32, 0.9, 5
    w, prompt, seq, gpu = run(BF16_SHAPE, T, k, p, seed, P=20, n=30)
    P = len(prompt)
    positions = list(range(P - 1, P - 1 + len(seq)))
    agree, border = check_sampled(seq, gpu, positions, T, k, p, seed, "bf16")
    cache = oracle.KVCache(BF16_SHAPE.n_layers, BF16_SHAPE.n_kv_heads, BF16_SHAPE.head_dim, store_dtype=torch.bfloat16)
    ora = oracle.forward(cpu_copy(w), BF16_SHAPE, prompt + seq[:-1], cache, logits_rows=positions)
    err = check_logits(gpu, ora, "bf16")
    print(f"bf16: {agree} agree, {border} borderline, max |dlogit| {err:.2e}")
    assert border <= 1 and len(set(seq)) > 1


def test_sampled_eos_stops_after_emitting_it():
    """The stop test applies to the drawn token: with the k-th drawn token as
    EOS id, the run emits exactly k+1 tokens (the EOS token included)."""
    s = synth.TINY
    w = synth.make_weights(s, 23, device="cuda")
    prompt = synth.make_prompt(s, 8, 24).tolist()
    eng = kie.Engine(s, max_seq=64)
    eng.load_weights(w)
    eng.set_sampling(1.0, 64, 1.0, 77)
    eng.prefill(prompt)
    ref, _, _ = eng.decode(20)
    k = next(i for i in range(3, 20) if ref[i] not in ref[:i])  # first fresh token from the 4th on
    eng.prefill(prompt)
    toks, _, st = eng.decode(20, eos_id=ref[k])
    eng.close()
    assert st == kie.KIE_OK and toks == ref[:k + 1]


def test_sampling_with_decode_loop_prefill():
    """In the decode-loop prompt mode only the last prompt step draws; the
    token and its continuation equal the matrix-core mode's."""
    s = synth.TINY
    w = synth.make_weights(s, 29, device="cuda")
    prompt = synth.make_prompt(s, 30, 30).tolist()
    out = []
    for mode in (kie.KIE_PREFILL_AUTO, kie.KIE_PREFILL_DECODE_LOOP):
        eng = kie.Engine(s, max_seq=64)
        eng.load_weights(w)
        eng.set_prefill_mode(mode)
        eng.set_sampling(0.8, 40, 0.95, 3)
        t0, lg = eng.prefill(prompt, want_logits=True)
        toks, lgs, st = eng.decode(12, want_logits=True)
        assert st == kie.KIE_OK
        out.append(([t0] + toks, torch.cat([lg[None].cpu(), lgs.cpu()])))
        eng.close()
    (sa, la), (sb, lb) = out
    positions = list(range(len(prompt) - 1, len(prompt) + 12))
    for seq, lg in out:  # each mode's draws follow the rule on its own logits
        check_sampled(seq, lg, positions, 0.8, 40, 0.95, 3, "decode-loop prefill")
    assert (la - lb).abs().max().item() <= 2e-2
