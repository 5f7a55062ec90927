"""Host-side checks of the C ABI, the binding and the benchmark's byte model.

No GPU: the library is loaded and only its host-only entry points are called
(configuration checks, workspace sizing, the tiling coverage check).
"""
import ctypes
import os
import re
import subprocess
import sys

import pytest
import torch

from persistent_decode_monokernel_amd import kie, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kie.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kie_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ("kie_create", "kie_load_weights", "kie_prefill", "kie_decode", "kie_destroy"):
        assert f in names


def test_library_exports_every_declared_function():
    out = subprocess.run(["nm", "-D", "--defined-only", kie.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing
    L = kie.lib()
    for f in declared_functions():
        assert getattr(L, f) is not None
    # the binding declares a signature for every function of the header
    assert set(declared_functions()) <= set(kie.SIGNATURES)


def test_status_strings():
    for s in range(0, -8, -1):
        txt = kie.status_string(s)
        assert isinstance(txt, str) and txt
    assert kie.status_string(-99)


def cfg_of(shape, max_seq=64, **kw):
    c = kie.make_config(shape, max_seq)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("name", ["tiny", "2b", "2b_long", "8b"])
def test_workload_configs_are_supported(name):
    wl = synth.WORKLOADS[name]
    c = kie.make_config(wl.shape, wl.n_prompt + wl.n_decode)
    assert kie.validate(c) == kie.KIE_OK
    ws = kie.workspace_bytes(c)
    s = wl.shape
    kv = 2 * s.n_layers * s.n_kv_heads * (wl.n_prompt + wl.n_decode) * s.head_dim * 2
    assert ws >= kv
    assert ws % 256 == 0


@pytest.mark.parametrize("change,expect", [
    (dict(head_dim=96), kie.KIE_ERR_UNSUPPORTED),
    (dict(n_heads=6), kie.KIE_ERR_UNSUPPORTED),            # not a multiple of n_kv_heads
    (dict(n_heads=64, n_kv_heads=4), kie.KIE_ERR_UNSUPPORTED),  # 16 query heads per KV head
    (dict(d_model=3000), kie.KIE_ERR_UNSUPPORTED),
    (dict(d_model=8192), kie.KIE_ERR_UNSUPPORTED),         # above the compiled width classes
    (dict(d_ffn=4100), kie.KIE_ERR_UNSUPPORTED),
    (dict(dtype=3), kie.KIE_ERR_ARG),
    (dict(max_seq=0), kie.KIE_ERR_ARG),
    (dict(vocab=0), kie.KIE_ERR_ARG),
    (dict(rms_eps=0.0), kie.KIE_ERR_ARG),
    (dict(rope_base=float("nan")), kie.KIE_ERR_ARG),
    (dict(n_layers=0), kie.KIE_ERR_ARG),
])
def test_validate_rejects(change, expect):
    c = cfg_of(synth.M2B, **change)
    assert kie.validate(c) == expect
    assert kie.workspace_bytes(c) == 0


def test_validate_null():
    assert kie.lib().kie_config_validate(None) == kie.KIE_ERR_ARG


def test_workspace_grows_with_max_seq():
    a = kie.workspace_bytes(cfg_of(synth.M2B, max_seq=1024))
    b = kie.workspace_bytes(cfg_of(synth.M2B, max_seq=2048))
    s = synth.M2B
    assert b - a >= 2 * s.n_layers * s.n_kv_heads * 1024 * s.head_dim * 2


@pytest.mark.parametrize("name", ["tiny", "2b", "8b"])
@pytest.mark.parametrize("grid", [160, 201, 255, 256, 304])
def test_tiling_covers_every_row_once(name, grid):
    """Every GEMV stage's rows are split over the grid without gap or overlap,
    every vector a thread loads lies inside its matrix (host check; every
    work-group and thread at the MI355X's 256 CUs, sampled work-groups else)."""
    c = kie.make_config(synth.WORKLOADS[name].shape, 64)
    assert kie.check_tiling(c, grid, grid == 256) == kie.KIE_OK


def test_tiling_rejects_grids_too_small_for_lds():
    # one work-group would own all 32000 LM-head rows: more than its LDS holds
    assert kie.check_tiling(kie.make_config(synth.M2B, 64), 1, False) == kie.KIE_ERR_UNSUPPORTED
    assert kie.check_tiling(kie.make_config(synth.TINY, 64), 0, False) == kie.KIE_ERR_ARG


def test_odd_shapes_tile():
    for kw in (dict(d_ffn=5376), dict(d_ffn=14336, d_model=4096, n_heads=32, n_kv_heads=8),
               dict(d_model=512, n_heads=8, n_kv_heads=8, head_dim=64, d_ffn=2048, vocab=50257)):
        c = cfg_of(synth.M2B, **kw)
        assert kie.validate(c) == kie.KIE_OK, kw
        assert kie.check_tiling(c, 256, False) == kie.KIE_OK, kw
    # below 4096 an FFN width must be a power of two
    assert kie.validate(cfg_of(synth.M2B, d_ffn=1536)) == kie.KIE_ERR_UNSUPPORTED


def test_entry_points_reject_null_handles():
    L = kie.lib()
    n = ctypes.c_int32(0)
    toks = (ctypes.c_int32 * 4)()
    assert L.kie_decode(None, 1, -1, toks, ctypes.byref(n), None) == kie.KIE_ERR_ARG
    assert L.kie_prefill(None, toks, 1, ctypes.byref(n), None) == kie.KIE_ERR_ARG
    assert L.kie_load_weights(None, None) == kie.KIE_ERR_ARG
    assert L.kie_import_kv(None, None, None, 0, 0) == kie.KIE_ERR_ARG
    assert L.kie_get_info(None, None) == kie.KIE_ERR_ARG
    out = ctypes.c_void_p(1)
    assert L.kie_create(None, None, 0, None, ctypes.byref(out)) == kie.KIE_ERR_ARG
    L.kie_destroy(None)


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(kie, "_lib", None)
    monkeypatch.setattr(kie, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libkie.so"))
    with pytest.raises(RuntimeError, match="missing"):
        kie.lib()


# ---- the benchmark's byte model (algorithmic bytes per token) ---------------

sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_bytes_per_token_2b():
    s = synth.M2B
    assert synth.param_count(s) == 1_834_076_160
    assert bench.weight_bytes_per_token(s) == 3_537_084_416
    assert bench.kv_bytes_per_position(s) == 57_344
    # mean over 1024 steps after 512 prompt positions: context 1024.5
    assert bench.bytes_per_launch(s, 512, 1024) == 1024 * 3_595_890_688
    assert bench.bytes_per_launch(s, 8192, 512) == 512 * 4_021_612_544


def test_bytes_per_token_8b():
    s = synth.M8B
    assert synth.param_count(s) == 8_030_261_248
    assert bench.weight_bytes_per_token(s) == 15_009_857_536
    assert bench.bytes_per_launch(s, 1024, 512) == 512 * 15_177_826_304


def test_measured_traffic_tracks_sources():
    assert bench.MEASURED_TRAFFIC
    for (wl, steps), m in bench.MEASURED_TRAFFIC.items():
        assert bench.measured_traffic(wl, steps + 1) is None  # another launch size
        if m["src_sha"] == bench.kernel_source_hash():
            assert bench.measured_traffic(wl, steps) == m["fetch_bytes"] + m["write_bytes"]
        else:
            assert bench.measured_traffic(wl, steps) is None


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stdout


# ---- seeded inputs ----------------------------------------------------------

def test_synthetic_inputs_are_seeded():
    s = synth.TINY
    a = synth.make_weights(s, 1)
    b = synth.make_weights(s, 1)
    c = synth.make_weights(s, 2)
    assert torch.equal(a["tok_emb"], b["tok_emb"]) and torch.equal(a["layers"][1]["w_down"], b["layers"][1]["w_down"])
    assert not torch.equal(a["tok_emb"], c["tok_emb"])
    assert a["tok_emb"].dtype == torch.float16 and a["tok_emb"].shape == (s.vocab, s.d_model)
    std = a["layers"][0]["wq"].float().std().item()
    assert 0.018 < std < 0.022
    p = synth.make_prompt(s, 16, 2)
    assert torch.equal(p, synth.make_prompt(s, 16, 2))
    assert int(p.min()) >= 0 and int(p.max()) < s.vocab
    k, v = synth.make_kv(s, 8, 3)
    assert k.shape == (s.n_layers, s.n_kv_heads, 8, s.head_dim) and not torch.equal(k, v)

