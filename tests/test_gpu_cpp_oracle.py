"""GPU decode against the fp32 C++ CPU oracle (oracle/cpu_decoder.cpp), the
plain fp32 decoder written independently of the float64 one: the tiny decoder
over its whole workload, and the full-depth ~2B decoder (28 layers, fp16) over
a short prompt and decode, teacher-forced on the GPU's tokens, to the same bar
(logits within 2e-2; tokens equal wherever the oracle's top-1/top-2 margin
exceeds 0.05)."""
import pytest
import torch

from oracle.cpu_decoder import CpuDecoder
from persistent_decode_monokernel_amd import kie, synth
from tests.gpu_util import check_tokens_and_logits

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,n_prompt,n_decode", [("tiny", 16, 32), ("2b", 32, 32)])
def test_decode_matches_fp32_cpp_oracle(name, n_prompt, n_decode):
    wl = synth.WORKLOADS[name]
    s = wl.shape
    print(f"[cpp oracle] {name}: prompt {n_prompt}, decode {n_decode}", flush=True)
    w = synth.make_weights(s, wl.weight_seed, device="cuda")
    prompt = synth.make_prompt(s, n_prompt, wl.prompt_seed).tolist()
    eng = kie.Engine(s, max_seq=n_prompt + n_decode + 1)
    eng.load_weights(w)
    tok0, lg0 = eng.prefill(prompt, want_logits=True)
    toks, lgs, st = eng.decode(n_decode, want_logits=True)
    assert st == kie.KIE_OK
    eng.close()
    gpu = torch.cat([lg0[None], lgs]).cpu()
    seq = [tok0] + toks
    dec = CpuDecoder(s, w, max_seq=n_prompt + n_decode + 1, n_threads=8)
    del w
    torch.cuda.empty_cache()
    ora = dec.feed(prompt + seq[:-1])[n_prompt - 1:]
    dec.close()
    err, decisive = check_tokens_and_logits(seq, gpu, ora, f"{name} vs fp32 C++")
    print(f"{name}: max |dlogit| vs fp32 C++ oracle {err:.2e} (decisive {decisive}/{len(seq)})")
