"""Oracle: slow, plain float64 CPU reference of greedy batch-1 decoding.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module;
only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code with the GPU path.

What it computes.  The pages describe one thing the engine does per request:
the LLM decode loop -- prompt processing, token-by-token decode, LM-head
sampling and the end-of-sequence check -- for one request at batch 1, on a
~2B-parameter FP16 model, without speculative decoding (revietech.ru, "Kog
vyzhimayet maksimum iz GPU: 3000 tokenov/s", section "Chto takoye monokernel";
remio.ai, "Kog stawia na glebsza optymalizacje GPU...", section "Dlaczego Kog
idzie glebiej w wnioskowanie GPU").  The monokernel changes how fast that
result is reached, not the result: the engine's output is exactly the greedy
decode of the model.  So this oracle is the plain definition of that decode.

The pages name no architecture beyond "~2B, FP16".  The reading taken (and
used by the workloads) is a standard dense pre-norm decoder:
  x = E[token]
  per layer:  xn = RMSNorm(x) * g_attn
              q, k, v = Wq xn, Wk xn, Wv xn ; rotary embedding on q and k
              attention of q over all cached k, v (causal, incl. self)
              x = x + Wo concat_heads(o)
              xn = RMSNorm(x) * g_ffn
              x = x + W_down( silu(W_gate xn) * (W_up xn) )
  logits = W_lm (RMSNorm(x) * g_final);  next token = argmax (first index on ties)
with RMSNorm(x) = x / sqrt(mean(x^2) + eps); rotate-half RoPE pairing element
i with i + hd/2 at angle pos * base^(-2i/hd); head h reads KV head
floor(h / (Hq/Hkv)); scores scaled by 1/sqrt(hd); silu(z) = z / (1 + e^-z); no
biases, no embedding scaling, untied LM head.

Arithmetic: weights stay in their storage dtype and are converted exactly to
float64 at use; every sum, product, exp and square root is float64.  Matrix
products use torch's float64 matmul (a library primitive) with no blocking or
reordering beyond what the definition states.

KV cache storage: exact float64 by default.  A cache may instead be given the
model's 16-bit storage dtype (KVCache(store_dtype=...)): every appended key and
value row is then rounded to that format once, as a model run at 16-bit
precision keeps it (the pages state the 2B model's precision as FP16 as a
whole: remio.ai, section "Dlaczego Kog idzie glebiej w wnioskowanie GPU").
Everything else stays float64.

Pins (tests/test_oracle_pins.py): brute-force scalar loops on tiny shapes,
closed forms (RMSNorm energy, RoPE rotation values, softmax of known scores,
silu values), invariants (RoPE norm preservation and relative-position
property, softmax rows summing to 1, incremental decode == full causal forward),
special models with closed-form greedy output, and argmax ties.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import torch

F64 = torch.float64


def to64(t: torch.Tensor) -> torch.Tensor:
    """Exact conversion of a stored tensor (fp16/bf16/fp32) to CPU float64."""
    return t.detach().to("cpu").to(F64)


def rmsnorm(x: torch.Tensor, g: torch.Tensor, eps: float) -> torch.Tensor:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * g."""
    ms = (x * x).mean(dim=-1, keepdim=True)
    return x / torch.sqrt(ms + eps) * g


def rope_cos_sin(positions: torch.Tensor, head_dim: int, base: float) -> Tuple[torch.Tensor, torch.Tensor]:
    """cos and sin of the rotary angles, float64, shape [n, head_dim/2].

    Angle of pair i at position p: p * base^(-2i/head_dim).
    """
    i = torch.arange(head_dim // 2, dtype=F64)
    inv_freq = torch.pow(torch.tensor(float(base), dtype=F64), -2.0 * i / head_dim)
    ang = positions.to(F64)[:, None] * inv_freq[None, :]
    return torch.cos(ang), torch.sin(ang)


def apply_rope(x: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor) -> torch.Tensor:
    """Rotate-half rotary embedding of x [n, H, hd] with cos/sin [n, hd/2].

    Element i and element i + hd/2 form a pair (a, b) -> (a c - b s, a s + b c).
    """
    h = x.shape[-1] // 2
    a, b = x[..., :h], x[..., h:]
    c, s = cos[:, None, :], sin[:, None, :]
    return torch.cat([a * c - b * s, a * s + b * c], dim=-1)


def silu(z: torch.Tensor) -> torch.Tensor:
    """silu(z) = z / (1 + exp(-z))."""
    return z / (1.0 + torch.exp(-z))


def softmax(s: torch.Tensor, dim: int = -1) -> torch.Tensor:
    """Max-subtracted softmax along ``dim``."""
    m = s.max(dim=dim, keepdim=True).values
    e = torch.exp(s - m)
    return e / e.sum(dim=dim, keepdim=True)


def argmax_first(v: torch.Tensor) -> int:
    """Index of the largest entry; the lowest such index on ties."""
    m = v.max()
    return int(torch.nonzero(v == m)[0, 0])


def greedy_token(logits: torch.Tensor) -> int:
    """Greedy choice, decided in float32 (the precision of the GPU's logits)."""
    return argmax_first(logits.to(torch.float32))


def matvec(W: torch.Tensor, x: torch.Tensor) -> torch.Tensor:
    """y = W x in float64 (W stored [rows][cols]); x may be [n][cols] -> [n][rows]."""
    return to64(x) @ to64(W).T


class KVCache:
    """Per-layer keys (already rotated) and values, [Hkv][n][hd] each, held as
    float64.  store_dtype None keeps appended rows exact; a 16-bit dtype rounds
    each appended row to it (the cache's storage format)."""

    def __init__(self, n_layers: int, n_kv_heads: int, head_dim: int, store_dtype: Optional[torch.dtype] = None):
        self.k: List[torch.Tensor] = [torch.zeros((n_kv_heads, 0, head_dim), dtype=F64) for _ in range(n_layers)]
        self.v: List[torch.Tensor] = [torch.zeros((n_kv_heads, 0, head_dim), dtype=F64) for _ in range(n_layers)]
        self.store_dtype = store_dtype

    @property
    def length(self) -> int:
        return int(self.k[0].shape[1])

    def append(self, l: int, k: torch.Tensor, v: torch.Tensor):
        """Append rows k, v [Hkv][n][hd] to layer l."""
        if self.store_dtype is not None:
            k = k.to(self.store_dtype).to(F64)
            v = v.to(self.store_dtype).to(F64)
        self.k[l] = torch.cat([self.k[l], k], dim=1)
        self.v[l] = torch.cat([self.v[l], v], dim=1)

    @classmethod
    def from_tensors(cls, k: torch.Tensor, v: torch.Tensor, store_dtype: Optional[torch.dtype] = None) -> "KVCache":
        """From stored K, V arrays [n_layers][Hkv][n][hd] (converted exactly)."""
        L, hkv, _, hd = k.shape
        c = cls(L, hkv, hd, store_dtype)
        c.k = [to64(k[l]) for l in range(L)]
        c.v = [to64(v[l]) for l in range(L)]
        return c


def attention(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, q_pos0: int) -> torch.Tensor:
    """Causal grouped-query attention.

    q [n, Hq, hd]: queries at absolute positions q_pos0 .. q_pos0+n-1.
    K, V [Hkv, m, hd]: keys/values of positions 0 .. m-1 (m = q_pos0 + n).
    Query i attends to keys j <= q_pos0 + i; head h reads KV head h // (Hq/Hkv).
    Returns o [n, Hq, hd].
    """
    n, hq, hd = q.shape
    hkv, m, _ = K.shape
    group = hq // hkv
    Kh = K.repeat_interleave(group, dim=0)  # [Hq, m, hd]: head h -> KV head h // group
    Vh = V.repeat_interleave(group, dim=0)
    s = torch.matmul(q.transpose(0, 1), Kh.transpose(1, 2)) / math.sqrt(hd)  # [Hq, n, m]
    qpos = torch.arange(n)[:, None] + q_pos0
    kpos = torch.arange(m)[None, :]
    s = s.masked_fill((kpos > qpos)[None, :, :], float("-inf"))
    p = softmax(s, dim=-1)
    o = torch.matmul(p, Vh)  # [Hq, n, hd]
    return o.transpose(0, 1)


def forward(w: Dict[str, object], shape, tokens: Sequence[int], cache: Optional[KVCache] = None,
            logits_rows: Optional[Sequence[int]] = None) -> torch.Tensor:
    """Run tokens through the model at positions cache.length .. cache.length+n-1.

    Appends the new keys/values to ``cache`` (a fresh cache when None).  Returns
    float64 logits [len(logits_rows)][vocab] for the segment rows listed in
    ``logits_rows`` (default: every row).
    """
    s = shape
    if cache is None:
        cache = KVCache(s.n_layers, s.n_kv_heads, s.head_dim)
    toks = torch.as_tensor(list(tokens), dtype=torch.int64)
    n = int(toks.numel())
    p0 = cache.length
    pos = torch.arange(p0, p0 + n)
    cos, sin = rope_cos_sin(pos, s.head_dim, s.rope_base)
    x = to64(w["tok_emb"][toks.to(w["tok_emb"].device)])  # [n, d]
    for l, lw in enumerate(w["layers"]):
        xn = rmsnorm(x, to64(lw["attn_norm"]), s.rms_eps)
        q = (xn @ to64(lw["wq"]).T).reshape(n, s.n_heads, s.head_dim)
        k = (xn @ to64(lw["wk"]).T).reshape(n, s.n_kv_heads, s.head_dim)
        v = (xn @ to64(lw["wv"]).T).reshape(n, s.n_kv_heads, s.head_dim)
        q = apply_rope(q, cos, sin)
        k = apply_rope(k, cos, sin)
        cache.append(l, k.transpose(0, 1), v.transpose(0, 1))
        o = attention(q, cache.k[l], cache.v[l], p0).reshape(n, s.n_heads * s.head_dim)
        x = x + o @ to64(lw["wo"]).T
        xn = rmsnorm(x, to64(lw["ffn_norm"]), s.rms_eps)
        h = silu(xn @ to64(lw["w_gate"]).T) * (xn @ to64(lw["w_up"]).T)
        x = x + h @ to64(lw["w_down"]).T
    rows = list(range(n)) if logits_rows is None else list(logits_rows)
    xf = rmsnorm(x[rows], to64(w["final_norm"]), s.rms_eps)
    return xf @ to64(w["lm_head"]).T


def prefill(w, shape, prompt: Sequence[int], cache: Optional[KVCache] = None):
    """Prompt pass: returns (first greedy token, logits of the last prompt position, cache)."""
    if cache is None:
        cache = KVCache(shape.n_layers, shape.n_kv_heads, shape.head_dim)
    lg = forward(w, shape, prompt, cache, logits_rows=[len(prompt) - 1])[0]
    return greedy_token(lg), lg, cache


def greedy_decode(w, shape, cache: KVCache, pending: int, n_steps: int, eos_id: int = -1):
    """Incremental greedy decode: step i feeds the pending token, emits token i.

    Stops after emitting eos_id when eos_id >= 0.  Returns (tokens, logits [k][V]).
    """
    toks: List[int] = []
    logits: List[torch.Tensor] = []
    tok = pending
    for _ in range(n_steps):
        lg = forward(w, shape, [tok], cache)[0]
        tok = greedy_token(lg)
        toks.append(tok)
        logits.append(lg)
        if eos_id >= 0 and tok == eos_id:
            break
    return toks, (torch.stack(logits) if logits else torch.zeros((0, shape.vocab), dtype=F64))


def teacher_forced(w, shape, cache: KVCache, fed: Sequence[int]) -> torch.Tensor:
    """Logits after feeding the tokens ``fed`` in one causal pass from ``cache``.

    Row i holds the logits at position cache.length + i, i.e. the distribution
    decode step i chooses from when step i is fed fed[i].
    """
    return forward(w, shape, fed, cache)
