"""GPU parity of the matrix-core prompt path (kie_prefill, KIE_PREFILL_AUTO).

Positions 0 .. P-2 run as dense products on the matrix cores, the last
position as one forced step of the persistent kernel.  Checked against the
oracle: the logits of the last prompt position and the first token, the KV
cache rows the prompt path wrote (the oracle's keys/values rounded to fp16,
the cache format), and the decode that continues from them.  Prompts cover a
ragged tail (not a multiple of the 64-row tiles), several chunks (1100
positions in chunks of 512), the one-token prompt (no matrix-core part), and
every query-head grouping (1, 2, 4, 8 query heads per KV head) at head_dim 64
and 128 over several 32-row attention tiles, and bf16 models (fp32
activations split into bf16 terms on the matrix cores; the oracle's cache then
stores each row in bf16, the engine's format).
"""
import pytest
import torch

import oracle
from persistent_decode_monokernel_amd import kie, synth
from tests.gpu_util import LOGIT_TOL, check_tokens_and_logits, cpu_copy

pytestmark = pytest.mark.gpu

MID = synth.ModelShape("mid", 2, 512, 8, 2, 64, 1024, 1000, synth.F16)
MID_BF16 = synth.ModelShape("mid_bf16", 2, 512, 8, 2, 64, 1024, 1000, synth.BF16)
KV_TOL = 2e-2  # max |cache row - oracle row| (values ~N(0, 1); fp16 storage 2^-11 relative)


GROUPINGS = {
    "g1_hd128": synth.ModelShape("g1_hd128", 2, 512, 4, 4, 128, 1024, 1000, synth.F16),
    "g2_hd64": synth.ModelShape("g2_hd64", 2, 512, 8, 4, 64, 1024, 1000, synth.F16),
    "g4_hd128": synth.ModelShape("g4_hd128", 1, 1024, 8, 2, 128, 2048, 1000, synth.F16),
    "g8_hd64": synth.ModelShape("g8_hd64", 2, 512, 8, 1, 64, 1024, 1000, synth.F16),
    "g2_hd128_bf16": synth.ModelShape("g2_hd128_bf16", 3, 1024, 8, 4, 128, 2048, 2048, synth.BF16),
    "g8_hd64_bf16": synth.ModelShape("g8_hd64_bf16", 2, 512, 8, 1, 64, 1024, 1000, synth.BF16),
}


def run_case(s, P, n_dec, seed=31, chunk=0):
    w = synth.make_weights(s, seed, device="cuda", gain_jitter=0.1)
    prompt = synth.make_prompt(s, P, seed + 1).tolist()
    eng = kie.Engine(s, max_seq=P + n_dec + 1)
    eng.load_weights(w)
    eng.set_prefill_chunk(chunk)
    tok0, lg0 = eng.prefill(prompt, want_logits=True)
    k, v, pend = eng.export_kv()
    toks, lgs, st = eng.decode(n_dec, want_logits=True)
    assert st == kie.KIE_OK and pend == tok0
    eng.close()
    wc = cpu_copy(w)
    cache = oracle.KVCache(s.n_layers, s.n_kv_heads, s.head_dim,
                           store_dtype=torch.bfloat16 if s.dtype == synth.BF16 else None)
    seq = [tok0] + toks
    ora = oracle.forward(wc, s, prompt + seq[:-1], cache, logits_rows=list(range(P - 1, P + n_dec)))
    gpu = torch.cat([lg0[None].cpu(), lgs.cpu()])
    err, dec = check_tokens_and_logits(seq, gpu, ora, f"{s.name} P={P}")
    kerr = max((k[l].cpu().double() - cache.k[l][:, :P]).abs().max().item() for l in range(s.n_layers))
    verr = max((v[l].cpu().double() - cache.v[l][:, :P]).abs().max().item() for l in range(s.n_layers))
    print(f"{s.name} P={P}: max |dlogit| {err:.2e} (decisive {dec}/{len(seq)}), cache |dk| {kerr:.2e} |dv| {verr:.2e}")
    assert kerr <= KV_TOL and verr <= KV_TOL, (kerr, verr)


@pytest.mark.parametrize("P", [16, 77])
def test_tiny_prompt_path(P):
    run_case(synth.TINY, P, 24)


@pytest.mark.parametrize("shape", [MID, MID_BF16])
def test_three_chunks_ragged(shape):
    run_case(shape, 1100, 16, chunk=512)


@pytest.mark.parametrize("name", list(GROUPINGS))
def test_query_head_groupings(name):
    run_case(GROUPINGS[name], 300, 8)


def test_one_token_prompt():
    run_case(MID, 1, 8)


@pytest.mark.parametrize("s", [MID, MID_BF16])
def test_modes_agree(s):
    w = synth.make_weights(s, 41, device="cuda")
    prompt = synth.make_prompt(s, 200, 42).tolist()
    out = {}
    for mode in (kie.KIE_PREFILL_AUTO, kie.KIE_PREFILL_DECODE_LOOP):
        eng = kie.Engine(s, max_seq=256)
        eng.load_weights(w)
        eng.set_prefill_mode(mode)
        tok0, lg0 = eng.prefill(prompt, want_logits=True)
        k, v, _ = eng.export_kv()
        out[mode] = (tok0, lg0.cpu(), k.cpu().float(), v.cpu().float())
        eng.close()
    a, b = out[kie.KIE_PREFILL_AUTO], out[kie.KIE_PREFILL_DECODE_LOOP]
    assert (a[1] - b[1]).abs().max().item() <= LOGIT_TOL
    assert (a[2] - b[2]).abs().max().item() <= KV_TOL and (a[3] - b[3]).abs().max().item() <= KV_TOL
    top = torch.topk(b[1].double(), 2).values
    if float(top[0] - top[1]) > 0.05:
        assert a[0] == b[0]


def test_mode_argument_checked():
    eng = kie.Engine(synth.TINY, max_seq=32)
    with pytest.raises(kie.KieError) as ei:
        eng.set_prefill_mode(7)
    assert ei.value.status == kie.KIE_ERR_ARG
    for bad, code in ((-1, kie.KIE_ERR_ARG), (33, kie.KIE_ERR_CAPACITY)):  # workspace chunk = max_seq = 32
        with pytest.raises(kie.KieError) as ei:
            eng.set_prefill_chunk(bad)
        assert ei.value.status == code
    eng.set_prefill_chunk(32)
    eng.set_prefill_chunk(0)
    eng.close()
