"""GPU parity of the seeded long and bf16 prompts through the prompt path, on
reduced-depth models of the stated shapes.

The ~2B decoder at long context takes a seeded 8192-token prompt, and the
~8B-shaped bf16 decoder a seeded 1024-token prompt.  Here both prompts (the
workloads' own seeds) run through kie_prefill in the default mode: 8192
positions as one 8192-row matrix-core chunk (the default; the fp16 GEMMs on
256 x 256 tiles) and as two 4096-row chunks (set by kie_set_prefill_chunk),
1024 bf16 positions as one chunk with three-term activations.  The models have the exact
widths of the stated configurations (d 2048, GQA 16/4 x 128, SwiGLU 8192,
vocab 32000, fp16; d 4096, GQA 32/8 x 128, SwiGLU 14336, vocab 128256, bf16)
and two layers, so the float64 oracle finishes the whole prompt in seconds.
Checked against the oracle:
  * the logits of the last prompt position and the first token;
  * every key and value row the prompt path wrote, in both layers;
  * a continued decode in ONE kie_decode launch, teacher-forced.
(The full-depth decode launches at these context lengths are checked in
test_gpu_full.py and test_gpu_8b.py.)
"""
import dataclasses
import time

import pytest
import torch

import oracle
from persistent_decode_monokernel_amd import kie, synth
from tests.gpu_util import KV_TOL, check_tokens_and_logits, cpu_copy, stored_rows_excess

pytestmark = pytest.mark.gpu


S2 = dataclasses.replace(synth.M2B, name="2b_2layers", n_layers=2)
S8 = dataclasses.replace(synth.M8B, name="8b_2layers", n_layers=2)


def run_prompt(shape, workload: str, n_decode: int, seg: int = 1024, chunk: int = 0):
    wl = synth.WORKLOADS[workload]
    w = synth.make_weights(shape, wl.weight_seed, device="cuda")
    prompt = synth.make_prompt(shape, wl.n_prompt, wl.prompt_seed).tolist()
    P = len(prompt)
    print(f"[prompt shapes] {shape.name}: prompt {P}, decode {n_decode}, chunk {chunk or 'default'}", flush=True)
    eng = kie.Engine(shape, max_seq=P + n_decode + 1)
    eng.load_weights(w)
    if chunk:
        eng.set_prefill_chunk(chunk)
    tok0, lg0 = eng.prefill(prompt, want_logits=True)
    k, v, pend = eng.export_kv()
    assert pend == tok0 and k.shape[2] == P
    toks, lgs, st = eng.decode(n_decode, want_logits=True)
    assert st == kie.KIE_OK and len(toks) == n_decode
    eng.close()
    gpu = torch.cat([lg0[None].cpu(), lgs.cpu()])
    k, v = k.cpu(), v.cpu()
    wc = cpu_copy(w)
    del w
    torch.cuda.empty_cache()
    bf16 = shape.dtype == synth.BF16
    cache = oracle.KVCache(shape.n_layers, shape.n_kv_heads, shape.head_dim,
                           store_dtype=torch.bfloat16 if bf16 else None)
    seq = [tok0] + toks
    fed = prompt + seq[:-1]
    t0 = time.time()
    rows = []
    for a in range(0, len(fed), seg):  # the oracle's causal pass in segments (bounded score matrices)
        b = min(len(fed), a + seg)
        want = [i - a for i in range(max(a, P - 1), b)]
        lg = oracle.forward(wc, shape, fed[a:b], cache, logits_rows=want)
        if want:
            rows.append(lg)
    ora = torch.cat(rows)
    print(f"[prompt shapes] oracle pass {time.time() - t0:.1f}s", flush=True)
    err, dec = check_tokens_and_logits(seq, gpu, ora, f"{shape.name} P={P}")
    # the oracle's cache holds the rows rounded to the storage format as well
    kerr = max(stored_rows_excess(k[l], cache.k[l][:, :P]) for l in range(shape.n_layers))
    verr = max(stored_rows_excess(v[l], cache.v[l][:, :P]) for l in range(shape.n_layers))
    print(f"{shape.name} P={P}: max |dlogit| {err:.2e} (decisive {dec}/{len(seq)}), "
          f"cache |dk|, |dv| beyond one storage ulp {kerr:.2e}, {verr:.2e}")
    assert kerr <= KV_TOL and verr <= KV_TOL, (kerr, verr)


@pytest.mark.parametrize("chunk", [0, 4096], ids=["one_chunk", "two_chunks"])
def test_2b_shape_8192_token_prompt(chunk):
    run_prompt(S2, "2b_long", 128, chunk=chunk)


def test_8b_shape_bf16_1024_token_prompt():
    run_prompt(S8, "8b", 64)
