"""Pins of the CPU oracle against facts fixed by mathematics, not by the oracle.

The pages print no worked example (no model values, no token sequences), so
the oracle is pinned by: closed forms, invariants, special cases that reduce to
a known answer, and a brute-force scalar-loop model on tiny shapes.  The last
group plants plausible mistakes into the oracle and checks that a pin fails.
"""
import math

import pytest
import torch

import oracle
from oracle import decoder as D
from persistent_decode_monokernel_amd import synth
from tests import bruteforce as BF

F64 = torch.float64


# ---------------------------------------------------------------- GEMV
def test_matvec_bruteforce_random():
    W, x = synth.make_gemv(7, 40, 3, seed=11)
    y = oracle.matvec(W[0], x)
    for n in range(3):
        ref = BF.mv(W[0].double().tolist(), x[n].double().tolist())
        assert max(abs(a - b) for a, b in zip(y[n].tolist(), ref)) < 1e-12


def test_matvec_integer_exact():
    W, x = synth.make_gemv(33, 512, 4, seed=12, integer=True)
    y = oracle.matvec(W[0], x)
    exact = torch.tensor([[sum(int(W[0, r, c]) * int(x[n, c]) for c in range(512)) for r in range(33)]
                          for n in range(4)], dtype=F64)
    assert torch.equal(y, exact)


def test_matvec_selector_rows():
    # W = identity-like selector rows -> y = x (closed form).
    cols = 64
    W = torch.zeros(cols, cols, dtype=torch.float16)
    perm = torch.randperm(cols, generator=torch.Generator().manual_seed(3))
    W[torch.arange(cols), perm] = 1
    x = torch.randn(cols, generator=torch.Generator().manual_seed(4)).to(torch.float16)
    assert torch.equal(oracle.matvec(W, x), x.double()[perm])


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_energy_closed_form():
    x = torch.randn(5, 128, dtype=F64, generator=torch.Generator().manual_seed(1)) * 3
    eps = 1e-5
    y = oracle.rmsnorm(x, torch.ones(128, dtype=F64), eps)
    ms = (x * x).mean(-1)
    assert torch.allclose((y * y).mean(-1), ms / (ms + eps), rtol=1e-13, atol=0)


def test_rmsnorm_gain_and_bruteforce():
    x = torch.randn(64, dtype=F64, generator=torch.Generator().manual_seed(2))
    g = torch.randn(64, dtype=F64, generator=torch.Generator().manual_seed(3))
    y = oracle.rmsnorm(x, g, 1e-5)
    ref = BF.rms(x.tolist(), g.tolist(), 1e-5)
    assert max(abs(a - b) for a, b in zip(y.tolist(), ref)) < 1e-13
    # eps only matters through the mean square: a vector of all-c has
    # y = c / sqrt(c^2 + eps).
    c = 0.003
    y2 = oracle.rmsnorm(torch.full((16,), c, dtype=F64), torch.ones(16, dtype=F64), 1e-5)
    assert torch.allclose(y2, torch.full((16,), c / math.sqrt(c * c + 1e-5), dtype=F64), rtol=1e-14)


# ---------------------------------------------------------------- RoPE
def _rope(x, pos, base=10000.0):
    cos, sin = oracle.rope_cos_sin(torch.tensor([pos]), x.shape[-1], base)
    return oracle.apply_rope(x[None, None, :], cos, sin)[0, 0]


def test_rope_position_zero_is_identity():
    x = torch.randn(128, dtype=F64, generator=torch.Generator().manual_seed(5))
    assert torch.equal(_rope(x, 0), x)


def test_rope_known_angles():
    # hd = 2: one pair, angle = pos rad. (1, 0) at pos 1 -> (cos 1, sin 1).
    y = _rope(torch.tensor([1.0, 0.0], dtype=F64), 1)
    assert torch.allclose(y, torch.tensor([math.cos(1.0), math.sin(1.0)], dtype=F64), rtol=0, atol=1e-15)
    # hd = 4, base 100: pair 1 turns by pos * 100^(-1/2) = pos / 10.
    # Pairs are (x0, x2) and (x1, x3).
    y = _rope(torch.tensor([0.0, 1.0, 0.0, 0.0], dtype=F64), 5, base=100.0)
    assert torch.allclose(y, torch.tensor([0.0, math.cos(0.5), 0.0, math.sin(0.5)], dtype=F64), atol=1e-15)
    # pi/2 turn: pos = pi/2 with hd = 2 maps (a, b) -> (-b, a).
    cos, sin = oracle.rope_cos_sin(torch.tensor([math.pi / 2]), 2, 10000.0)
    y = oracle.apply_rope(torch.tensor([[[3.0, 4.0]]], dtype=F64), cos, sin)[0, 0]
    assert torch.allclose(y, torch.tensor([-4.0, 3.0], dtype=F64), atol=1e-14)


def test_rope_preserves_pair_norms():
    x = torch.randn(128, dtype=F64, generator=torch.Generator().manual_seed(6))
    y = _rope(x, 777)
    nx = x[:64] ** 2 + x[64:] ** 2
    ny = y[:64] ** 2 + y[64:] ** 2
    assert torch.allclose(nx, ny, rtol=1e-13)


def test_rope_relative_position():
    g = torch.Generator().manual_seed(7)
    q = torch.randn(64, dtype=F64, generator=g)
    k = torch.randn(64, dtype=F64, generator=g)
    a = torch.dot(_rope(q, 10), _rope(k, 3))
    b = torch.dot(_rope(q, 1010), _rope(k, 1003))
    assert abs(float(a - b)) < 1e-11


def test_rope_bruteforce():
    x = torch.randn(16, dtype=F64, generator=torch.Generator().manual_seed(8))
    y = _rope(x, 37, 500.0)
    ref = BF.rot(x.tolist(), 37, 500.0)
    assert max(abs(a - b) for a, b in zip(y.tolist(), ref)) < 1e-13


# ---------------------------------------------------------------- softmax / silu / argmax
def test_softmax_known_values_and_rows():
    p = oracle.softmax(torch.tensor([0.0, math.log(2.0)], dtype=F64))
    assert torch.allclose(p, torch.tensor([1 / 3, 2 / 3], dtype=F64), atol=1e-15)
    s = torch.randn(6, 50, dtype=F64, generator=torch.Generator().manual_seed(9)) * 20
    p = oracle.softmax(s)
    assert torch.allclose(p.sum(-1), torch.ones(6, dtype=F64), atol=1e-14)
    assert torch.allclose(oracle.softmax(s + 1234.5), p, atol=1e-14)  # shift invariance


def test_silu_closed_forms():
    z = torch.tensor([0.0, 1.0, -1.0, 40.0, -40.0], dtype=F64)
    y = oracle.silu(z)
    assert y[0] == 0.0
    assert abs(float(y[1]) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    assert abs(float(y[2]) + 1.0 / (1.0 + math.e)) < 1e-15
    assert abs(float(y[3]) - 40.0) < 1e-15
    assert abs(float(y[4])) < 1e-15


def test_argmax_ties_first_index():
    v = torch.tensor([0.5, 2.0, -1.0, 2.0, 2.0], dtype=F64)
    assert oracle.argmax_first(v) == 1
    assert oracle.argmax_first(torch.zeros(9, dtype=F64)) == 0
    v = torch.randn(1000, dtype=F64, generator=torch.Generator().manual_seed(10))
    assert oracle.argmax_first(v) == int(max(range(1000), key=lambda i: (float(v[i]), -i)))


# ---------------------------------------------------------------- attention
def test_attention_single_key_returns_value():
    g = torch.Generator().manual_seed(12)
    q = torch.randn(1, 4, 16, dtype=F64, generator=g)
    K = torch.randn(2, 1, 16, dtype=F64, generator=g)
    V = torch.randn(2, 1, 16, dtype=F64, generator=g)
    o = oracle.attention(q, K, V, 0)
    assert torch.allclose(o[0], V[:, 0].repeat_interleave(2, dim=0), atol=1e-15)


def test_attention_zero_query_is_mean_of_values():
    g = torch.Generator().manual_seed(13)
    n, m = 3, 9
    q = torch.zeros(n, 2, 8, dtype=F64)
    K = torch.randn(1, m, 8, dtype=F64, generator=g)
    V = torch.randn(1, m, 8, dtype=F64, generator=g)
    o = oracle.attention(q, K, V, m - n)
    for i in range(n):
        ref = V[0, : m - n + i + 1].mean(0)
        assert torch.allclose(o[i, 0], ref, atol=1e-14) and torch.allclose(o[i, 1], ref, atol=1e-14)


def test_attention_bruteforce_gqa():
    g = torch.Generator().manual_seed(14)
    hq, hkv, hd, m = 6, 2, 8, 7
    q = torch.randn(1, hq, hd, dtype=F64, generator=g)
    K = torch.randn(hkv, m, hd, dtype=F64, generator=g)
    V = torch.randn(hkv, m, hd, dtype=F64, generator=g)
    o = oracle.attention(q, K, V, m - 1)
    for h in range(hq):
        kv = h // (hq // hkv)
        sc = [BF.dot(q[0, h].tolist(), K[kv, j].tolist()) / math.sqrt(hd) for j in range(m)]
        mx = max(sc)
        e = [math.exp(s - mx) for s in sc]
        ref = [sum(e[j] / sum(e) * float(V[kv, j, i]) for j in range(m)) for i in range(hd)]
        assert max(abs(a - b) for a, b in zip(o[0, h].tolist(), ref)) < 1e-13


# ---------------------------------------------------------------- whole model
MINI = synth.small_shape(n_layers=2, d_model=16, n_heads=4, n_kv_heads=2, head_dim=4, d_ffn=24, vocab=23)


def _mini_weights(seed=21, jitter=0.3, std=0.3):
    return synth.make_weights(MINI, seed, gain_jitter=jitter, std=std)


def test_forward_matches_bruteforce_loops():
    w = _mini_weights()
    toks = [3, 17, 0, 22, 5, 5, 9]
    lg = oracle.forward(w, MINI, toks)
    ref = torch.tensor(BF.model_logits(w, MINI, toks), dtype=F64)
    assert torch.allclose(lg, ref, rtol=0, atol=1e-11), float((lg - ref).abs().max())


def test_incremental_decode_equals_full_forward():
    shape = synth.small_shape(n_layers=3, d_model=64, n_heads=8, n_kv_heads=2, head_dim=8, d_ffn=96, vocab=101)
    w = synth.make_weights(shape, 5, gain_jitter=0.2, std=0.1)
    prompt = synth.make_prompt(shape, 9, 6).tolist()
    tok0, lg0, cache = oracle.prefill(w, shape, prompt)
    toks, lgs = oracle.greedy_decode(w, shape, cache, tok0, 12)
    full = oracle.forward(w, shape, prompt + [tok0] + toks[:-1])
    assert torch.allclose(full[len(prompt) - 1], lg0, atol=1e-12)
    assert torch.allclose(full[len(prompt):], lgs, atol=1e-12)
    # the greedy sequence is consistent with the full pass
    seq = [tok0] + toks
    for i in range(len(seq)):
        assert oracle.greedy_token(full[len(prompt) - 1 + i]) == seq[i]


@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16])
def test_cache_storage_dtype_rounds_each_appended_row(dt):
    """A cache stored in a 16-bit format holds exactly the rounded rows: layer 0's
    keys and values depend on no attention output, so they must equal the
    exact cache's layer-0 rows rounded to that format; incremental decode must
    still equal the full causal pass under the same storage."""
    shape = synth.small_shape(n_layers=2, d_model=32, n_heads=4, n_kv_heads=2, head_dim=8, d_ffn=64, vocab=61)
    w = synth.make_weights(shape, 12, std=0.2)
    prompt = synth.make_prompt(shape, 7, 13).tolist()
    exact = oracle.KVCache(shape.n_layers, shape.n_kv_heads, shape.head_dim)
    stored = oracle.KVCache(shape.n_layers, shape.n_kv_heads, shape.head_dim, store_dtype=dt)
    oracle.forward(w, shape, prompt, exact)
    oracle.forward(w, shape, prompt, stored)
    assert torch.equal(stored.k[0], exact.k[0].to(dt).to(torch.float64))
    assert torch.equal(stored.v[0], exact.v[0].to(dt).to(torch.float64))
    assert not torch.equal(stored.k[0], exact.k[0])  # the rounding did happen
    # later layers see rounded keys: close to, not equal to, the exact ones
    assert torch.allclose(stored.k[1], exact.k[1], rtol=0, atol=0.05)
    tok0, lg0, c = oracle.prefill(w, shape, prompt,
                                  oracle.KVCache(shape.n_layers, shape.n_kv_heads, shape.head_dim, store_dtype=dt))
    toks, lgs = oracle.greedy_decode(w, shape, c, tok0, 6)
    full = oracle.forward(w, shape, prompt + [tok0] + toks[:-1],
                          oracle.KVCache(shape.n_layers, shape.n_kv_heads, shape.head_dim, store_dtype=dt))
    assert torch.allclose(full[len(prompt) - 1], lg0, atol=1e-12)
    assert torch.allclose(full[len(prompt):], lgs, atol=1e-12)


@pytest.mark.parametrize("dt,fmt", [(torch.float16, "f16"), (torch.bfloat16, "bf16")])
def test_bruteforce_storage_rounding_matches_torch(dt, fmt):
    """The scalar model's 16-bit rounding (float64 -> float32 -> 16 bits, ties to
    even) agrees with PyTorch's conversion, including values that round
    differently directly and through float32."""
    g = torch.Generator().manual_seed(0)
    xs = (torch.randn(20000, dtype=F64, generator=g) * 10).tolist()
    xs += [1 + 2**-8 + 2**-30, 1 + 2**-11 + 2**-40, 65504.0, 1e-8, -0.0]
    ref = torch.tensor(xs, dtype=F64).to(dt).to(F64).tolist()
    assert [BF.round_store(x, fmt) for x in xs] == ref


@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16])
def test_cache_storage_dtype_matches_bruteforce(dt):
    """The 16-bit cache mode rounds exactly the cached keys (after rotation) and
    values, and nothing else: the scalar-loop model rounding only those
    elements gives the same logits at every position.  Rounding the query, the
    attention output or the key before rotation moves them well past 1e-11."""
    w = _mini_weights(seed=23, std=0.5)
    toks = [4, 11, 0, 19, 7, 7, 2, 13]
    assert _store_pin_error(w, toks, dt) < 1e-11


def _store_pin_error(w, toks, dt):
    fmt = "bf16" if dt == torch.bfloat16 else "f16"
    lg = oracle.forward(w, MINI, toks, oracle.KVCache(MINI.n_layers, MINI.n_kv_heads, MINI.head_dim, store_dtype=dt))
    ref = torch.tensor(BF.model_logits(w, MINI, toks, store=fmt), dtype=F64)
    return float((lg - ref).abs().max())


def _rounded(t):
    return t.to(torch.bfloat16).to(F64)


def _attention_rounds_query(q, K, V, q_pos0):
    return _ORIG_ATT(_rounded(q), K, V, q_pos0)


def _attention_rounds_output(q, K, V, q_pos0):
    return _rounded(_ORIG_ATT(q, K, V, q_pos0))


def _rope_rounds_key_input(x, cos, sin):
    if x.shape[-2] == MINI.n_kv_heads:  # the key projection (the query has more heads)
        x = _rounded(x)
    return _ORIG_ROPE(x, cos, sin)


_ORIG_ROPE = D.apply_rope
STORE_MUTATIONS = {
    "query_rounded": ("attention", _attention_rounds_query),
    "attention_output_rounded": ("attention", _attention_rounds_output),
    "key_rounded_before_rotation": ("apply_rope", _rope_rounds_key_input),
}


@pytest.mark.parametrize("name", sorted(STORE_MUTATIONS))
def test_cache_storage_pin_catches_extra_rounding(name, monkeypatch):
    w = _mini_weights(seed=23, std=0.5)
    toks = [4, 11, 0, 19, 7, 7, 2, 13]
    assert _store_pin_error(w, toks, torch.bfloat16) < 1e-11
    attr, fn = STORE_MUTATIONS[name]
    monkeypatch.setattr(D, attr, fn)
    monkeypatch.setattr(oracle, attr, fn, raising=False)
    assert _store_pin_error(w, toks, torch.bfloat16) > 1e-6, f"planted mistake {name} went unnoticed"


def test_teacher_forced_from_imported_cache():
    shape = synth.small_shape(n_layers=2, d_model=32, n_heads=4, n_kv_heads=4, head_dim=8, d_ffn=64, vocab=50)
    w = synth.make_weights(shape, 8, std=0.2)
    k, v = synth.make_kv(shape, 6, seed=9)
    fed = [1, 2, 3, 4]
    a = oracle.teacher_forced(w, shape, oracle.KVCache.from_tensors(k, v), fed)
    c = oracle.KVCache.from_tensors(k, v)
    b = torch.stack([oracle.forward(w, shape, [t], c)[0] for t in fed])
    assert torch.allclose(a, b, atol=1e-12)


def test_gqa_equals_mha_with_replicated_kv_heads():
    # A GQA model equals the MHA model whose KV projection rows are the GQA
    # rows replicated per query head in the group (head h -> KV head h // G).
    gqa = synth.small_shape(n_layers=1, d_model=32, n_heads=4, n_kv_heads=2, head_dim=8, d_ffn=32, vocab=40)
    mha = synth.small_shape(n_layers=1, d_model=32, n_heads=4, n_kv_heads=4, head_dim=8, d_ffn=32, vocab=40)
    w = synth.make_weights(gqa, 31, std=0.3)
    w2 = {k: v for k, v in w.items()}
    lw = dict(w["layers"][0])
    for key in ("wk", "wv"):
        lw[key] = lw[key].reshape(2, 8, 32).repeat_interleave(2, dim=0).reshape(32, 32)
    w2["layers"] = [lw]
    toks = [1, 5, 9, 13, 2]
    assert torch.allclose(oracle.forward(w, gqa, toks), oracle.forward(w2, mha, toks), atol=1e-12)


def _echo_model(shape, seed):
    """Wo = W_down = 0, gains 1, lm_head = tok_emb: the residual stays at E[t],
    so logits_j = E_j . E_t / rms(E_t) and the greedy token is t itself
    whenever |E_t|^2 exceeds every cross term E_j . E_t."""
    w = synth.make_weights(shape, seed, std=0.02)
    for lw in w["layers"]:
        lw["wo"] = torch.zeros_like(lw["wo"])
        lw["w_down"] = torch.zeros_like(lw["w_down"])
    w["lm_head"] = w["tok_emb"].clone()
    return w


def test_closed_form_echo_model():
    shape = synth.small_shape(n_layers=2, d_model=256, n_heads=4, n_kv_heads=2, head_dim=64, d_ffn=64, vocab=300)
    w = _echo_model(shape, 41)
    E = w["tok_emb"].double()
    prompt = [7, 123, 42]
    t = prompt[-1]
    # closed form of the logits at the last prompt position
    e = E[t]
    expect = E @ e / torch.sqrt((e * e).mean() + shape.rms_eps)
    tok0, lg, cache = oracle.prefill(w, shape, prompt)
    assert torch.allclose(lg, expect, atol=1e-12)
    assert tok0 == t
    toks, _ = oracle.greedy_decode(w, shape, cache, tok0, 5)
    assert toks == [t] * 5
    toks, _ = oracle.greedy_decode(w, shape, cache, tok0, 5, eos_id=t)
    assert toks == [t]


# ---------------------------------------------------------------- planted mistakes
def _pins_pass():
    try:
        test_forward_matches_bruteforce_loops()
        test_closed_form_echo_model()
        test_rope_known_angles()
        test_attention_bruteforce_gqa()
        test_rmsnorm_energy_closed_form()
        test_softmax_known_values_and_rows()
        test_silu_closed_forms()
    except AssertionError:
        return False
    return True


def _rope_sign_flip(x, cos, sin):
    h = x.shape[-1] // 2
    a, b = x[..., :h], x[..., h:]
    c, s = cos[:, None, :], sin[:, None, :]
    return torch.cat([a * c + b * s, -a * s + b * c], dim=-1)


def _rope_interleaved(x, cos, sin):
    a, b = x[..., 0::2], x[..., 1::2]
    c, s = cos[:, None, :], sin[:, None, :]
    out = torch.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def _attention_gqa_modulo(q, K, V, q_pos0):
    g = q.shape[1] // K.shape[0]
    # head h -> KV head h % Hkv (the wrong mapping)
    return _att_full(q, K.repeat(g, 1, 1), V.repeat(g, 1, 1), q_pos0)


def _att_full(q, Kh, Vh, q_pos0):
    n, hq, hd = q.shape
    m = Kh.shape[1]
    s = torch.matmul(q.transpose(0, 1), Kh.transpose(1, 2)) / math.sqrt(hd)
    qpos = torch.arange(n)[:, None] + q_pos0
    s = s.masked_fill((torch.arange(m)[None, :] > qpos)[None], float("-inf"))
    return torch.matmul(D.softmax(s, -1), Vh).transpose(0, 1)


def _attention_no_scale(q, K, V, q_pos0):
    return _ORIG_ATT(q * math.sqrt(q.shape[-1]), K, V, q_pos0)


def _attention_not_causal(q, K, V, q_pos0):
    n, hq, hd = q.shape
    g = hq // K.shape[0]
    s = torch.matmul(q.transpose(0, 1), K.repeat_interleave(g, 0).transpose(1, 2)) / math.sqrt(hd)
    return torch.matmul(D.softmax(s, -1), V.repeat_interleave(g, 0)).transpose(0, 1)


def _rmsnorm_no_eps(x, g, eps):
    return x / torch.sqrt((x * x).mean(-1, keepdim=True)) * g


def _rmsnorm_std(x, g, eps):
    return (x - x.mean(-1, keepdim=True)) / torch.sqrt(x.var(-1, unbiased=False, keepdim=True) + eps) * g


def _silu_as_sigmoid(z):
    return 1.0 / (1.0 + torch.exp(-z))


def _softmax_no_max(s, dim=-1):
    e = torch.exp(s)
    return e / e.sum(dim=dim, keepdim=True) * (1 + 1e-6)


_ORIG_ATT = D.attention

MUTATIONS = {
    "rope_sign": ("apply_rope", _rope_sign_flip),
    "rope_interleaved_pairs": ("apply_rope", _rope_interleaved),
    "gqa_modulo_mapping": ("attention", _attention_gqa_modulo),
    "attention_unscaled": ("attention", _attention_no_scale),
    "attention_not_causal": ("attention", _attention_not_causal),
    "rmsnorm_without_eps": ("rmsnorm", _rmsnorm_no_eps),
    "layernorm_instead_of_rmsnorm": ("rmsnorm", _rmsnorm_std),
    "sigmoid_instead_of_silu": ("silu", _silu_as_sigmoid),
    "softmax_scaled": ("softmax", _softmax_no_max),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    assert _pins_pass()
    monkeypatch.setattr(D, attr, fn)
    monkeypatch.setattr(oracle, attr, fn, raising=False)
    assert not _pins_pass(), f"planted mistake {name} went unnoticed"
