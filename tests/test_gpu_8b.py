"""GPU parity on the ~8B-shaped decoder (32 layers, d 4096, GQA 32/8 x 128,
SwiGLU 14336, vocab 128256, bf16), one kie_decode(512) launch.

The context is a seeded synthetic 1024-position KV cache imported through
kie_import_kv (standing in for the 1024-token prompt; same shapes and byte
counts for the decode launch).  All 512 steps are compared with the oracle
teacher-forced on the GPU's tokens, within the 2e-2 logit bound stated for
fp16, applied unchanged.

The model runs at bf16 precision, so its KV cache is stored in bf16: the
oracle's cache rounds each appended key/value row to bf16 as the engine's
does (everything else in the oracle stays float64).  bf16 keeps 8 significant
bits, and against an exact float64 cache that one storage rounding alone moves
the logits by ~0.15 over 512 steps: a property of the storage format, not an
error of the kernel.  The engine feeds bf16 activations to the dot2 unit as
three bf16 terms (value and two rounding residuals), so the GEMVs see ~24
bits of each activation.
"""
import time

import pytest
import torch

import oracle
from persistent_decode_monokernel_amd import kie, synth
from tests.gpu_util import check_tokens_and_logits, cpu_copy

pytestmark = pytest.mark.gpu

S = synth.M8B


def test_8b_bf16_decode512():
    wl = synth.WORKLOADS["8b"]
    w = synth.make_weights(S, wl.weight_seed, device="cuda")
    k, v = synth.make_kv(S, wl.n_prompt, seed=wl.prompt_seed)
    pending = int(synth.make_prompt(S, wl.n_prompt, wl.prompt_seed)[-1])
    eng = kie.Engine(S, max_seq=wl.n_prompt + wl.n_decode)
    eng.load_weights(w)
    eng.import_kv(k.cuda(), v.cuda(), pending)
    toks, lgs, st = eng.decode(wl.n_decode, want_logits=True)
    assert st == kie.KIE_OK and len(toks) == wl.n_decode
    gpu = lgs.cpu()
    eng.close()
    wc = cpu_copy(w)
    del w, lgs
    torch.cuda.empty_cache()
    t0 = time.time()
    cache = oracle.KVCache.from_tensors(k, v, store_dtype=torch.bfloat16)
    fed = [pending] + toks[:-1]
    ora = torch.cat([oracle.teacher_forced(wc, S, cache, fed[i:i + 128]) for i in range(0, len(fed), 128)])
    print(f"oracle teacher-forced pass: {time.time() - t0:.1f}s", flush=True)
    err, dec = check_tokens_and_logits(toks, gpu, ora, "8b bf16 ctx 1024 + decode 512")
    print(f"8b: max |dlogit| {err:.2e}, decisive steps {dec}/{len(toks)}")
