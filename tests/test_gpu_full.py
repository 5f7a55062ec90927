"""GPU parity at full model sizes, in the launch configurations the benchmark times.

~2B decoder (28 layers, d 2048, GQA 16/4 x 128, SwiGLU 8192, vocab 32000, fp16):
  * prefill of the seeded 512-token prompt, then ONE kie_decode(1024) launch;
    every one of the 1025 greedy steps is compared with the oracle run
    teacher-forced on the GPU's own tokens (logits within 2e-2, tokens equal
    where the oracle's top-1/top-2 margin exceeds 0.05);
  * long context: an 8192-position KV cache (seeded synthetic rows, imported
    through kie_import_kv) followed by ONE kie_decode(512) launch, all 512
    steps compared the same way.  The synthetic cache stands in for the
    8192-token prompt: the decode launch sees the same shapes, chunking and
    byte counts, and the oracle reads the identical cache values.
"""
import time

import pytest
import torch

import oracle
from persistent_decode_monokernel_amd import kie, synth
from tests.gpu_util import check_tokens_and_logits, cpu_copy, error_curve, print_error_curve

pytestmark = pytest.mark.gpu

S = synth.M2B


@pytest.fixture(scope="module")
def m2b():
    wl = synth.WORKLOADS["2b"]
    w = synth.make_weights(S, wl.weight_seed, device="cuda")
    wc = cpu_copy(w)
    yield w, wc
    del w, wc
    torch.cuda.empty_cache()


def test_2b_prefill512_decode1024(m2b):
    w, wc = m2b
    wl = synth.WORKLOADS["2b"]
    prompt = synth.make_prompt(S, wl.n_prompt, wl.prompt_seed).tolist()
    eng = kie.Engine(S, max_seq=wl.n_prompt + wl.n_decode)
    eng.load_weights(w)
    tok0, lg0 = eng.prefill(prompt, want_logits=True)
    toks, lgs, st = eng.decode(wl.n_decode, want_logits=True)
    assert st == kie.KIE_OK and len(toks) == wl.n_decode
    seq = [tok0] + toks
    gpu = torch.cat([lg0[None].cpu(), lgs.cpu()])
    eng.close()
    t0 = time.time()
    P = len(prompt)
    ora = oracle.forward(wc, S, prompt + seq[:-1], logits_rows=list(range(P - 1, P + wl.n_decode)))
    print(f"oracle teacher-forced pass: {time.time() - t0:.1f}s", flush=True)
    err, dec = check_tokens_and_logits(seq, gpu, ora, "2b prefill 512 + decode 1024")
    print(f"2b: max |dlogit| {err:.2e}, decisive steps {dec}/{len(seq)}")
    print_error_curve(error_curve(gpu, ora), "2b prefill 512 + decode 1024")


def test_2b_long_context_decode512(m2b):
    w, wc = m2b
    wl = synth.WORKLOADS["2b_long"]
    n_ctx = wl.n_prompt
    k, v = synth.make_kv(S, n_ctx, seed=wl.prompt_seed)
    pending = int(synth.make_prompt(S, n_ctx, wl.prompt_seed)[-1])
    eng = kie.Engine(S, max_seq=n_ctx + wl.n_decode)
    eng.load_weights(w)
    eng.import_kv(k.cuda(), v.cuda(), pending)
    toks, lgs, st = eng.decode(wl.n_decode, want_logits=True)
    assert st == kie.KIE_OK and len(toks) == wl.n_decode
    assert eng.info().pos == n_ctx + wl.n_decode
    gpu = lgs.cpu()
    eng.close()
    t0 = time.time()
    cache = oracle.KVCache.from_tensors(k, v)
    fed = [pending] + toks[:-1]
    ora = torch.cat([oracle.teacher_forced(wc, S, cache, fed[i:i + 128]) for i in range(0, len(fed), 128)])
    print(f"oracle teacher-forced pass: {time.time() - t0:.1f}s", flush=True)
    err, dec = check_tokens_and_logits(toks, gpu, ora, "2b ctx 8192 + decode 512")
    print(f"2b long: max |dlogit| {err:.2e}, decisive steps {dec}/{len(toks)}")
    print_error_curve(error_curve(gpu, ora), "2b ctx 8192 + decode 512")
