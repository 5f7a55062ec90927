"""GPU parity on a subset of the compute units (kie_set_grid): the persistent
kernel on 97, 160 and 255 work-groups (uneven row splits, attention units
wrapping over the grid, fewer sampling groups) against the oracle teacher-forced
on the GPU's tokens, and the argument checks."""
import pytest
import torch

import oracle
from persistent_decode_monokernel_amd import kie, synth
from tests.gpu_util import check_tokens_and_logits, cpu_copy

pytestmark = pytest.mark.gpu

MID = synth.ModelShape("mid", 2, 512, 8, 2, 64, 1024, 1000, synth.F16)


@pytest.mark.parametrize("shape,grid", [(synth.TINY, 97), (MID, 160), (MID, 255)])
def test_subset_grid_parity(shape, grid):
    w = synth.make_weights(shape, 13, device="cuda", gain_jitter=0.1)
    prompt = synth.make_prompt(shape, 20, 14).tolist()
    eng = kie.Engine(shape, max_seq=64)
    eng.load_weights(w)
    eng.set_grid(grid)
    assert eng.info().grid == grid
    tok0, lg0 = eng.prefill(prompt, want_logits=True)
    toks, lgs, st = eng.decode(24, want_logits=True)
    assert st == kie.KIE_OK
    eng.close()
    seq = [tok0] + toks
    gpu = torch.cat([lg0[None].cpu(), lgs.cpu()])
    cache = oracle.KVCache(shape.n_layers, shape.n_kv_heads, shape.head_dim)
    ora = oracle.forward(cpu_copy(w), shape, prompt + seq[:-1], cache,
                         logits_rows=list(range(len(prompt) - 1, len(prompt) + 24)))
    err, dec = check_tokens_and_logits(seq, gpu, ora, f"{shape.name} grid {grid}")
    print(f"{shape.name} grid {grid}: max |dlogit| {err:.2e}, decisive {dec}/{len(seq)}")


def test_grid_arguments_checked():
    eng = kie.Engine(synth.TINY, max_seq=32)
    cus = eng.info().cu_count
    for bad, code in ((-1, kie.KIE_ERR_ARG), (cus + 1, kie.KIE_ERR_ARG)):
        with pytest.raises(kie.KieError) as ei:
            eng.set_grid(bad)
        assert ei.value.status == code
    with pytest.raises(kie.KieError) as ei:  # 4096 vocabulary rows on one work-group exceed the LDS rows
        eng.set_grid(1)
    assert ei.value.status == kie.KIE_ERR_UNSUPPORTED
    eng.set_grid(4)
    assert eng.info().grid == 4
    eng.set_grid(0)
    assert eng.info().grid == cus
    eng.close()
