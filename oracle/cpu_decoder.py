"""ctypes binding of the plain fp32 C++ CPU decoder (cpu_decoder.cpp).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: the tests, the smoke
check and the benchmark's CPU-baseline leg use it; the product path never does.
It shares no code with the GPU path.  The library is built with g++ by
``build()`` (called by the repository's build step); ``CpuDecoder`` builds it
on first use when it is missing.
"""
import ctypes
import os
import subprocess
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "cpu_decoder.cpp")
LIB = os.path.join(_HERE, "libkie_oracle_cpu.so")

_lib = None


def build(verbose: bool = False) -> str:
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


class _Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n_layers", "d_model", "n_heads", "n_kv_heads", "head_dim",
                                              "d_ffn", "vocab")] + [("rms_eps", ctypes.c_float),
                                                                    ("rope_base", ctypes.c_float)]


_PF = ctypes.POINTER(ctypes.c_float)
LAYER_KEYS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")


class _Layer(ctypes.Structure):
    _fields_ = [(k, _PF) for k in LAYER_KEYS]


class _Weights(ctypes.Structure):
    _fields_ = [("tok_emb", _PF), ("final_norm", _PF), ("lm_head", _PF), ("layers", ctypes.POINTER(_Layer))]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(LIB)
        L.oc_create.restype = ctypes.c_void_p
        L.oc_create.argtypes = [ctypes.POINTER(_Shape), ctypes.POINTER(_Weights), ctypes.c_int32, ctypes.c_int32]
        L.oc_destroy.restype = None
        L.oc_destroy.argtypes = [ctypes.c_void_p]
        L.oc_set_cache.restype = ctypes.c_int32
        L.oc_set_cache.argtypes = [ctypes.c_void_p, _PF, _PF, ctypes.c_int32]
        L.oc_step.restype = ctypes.c_int32
        L.oc_step.argtypes = [ctypes.c_void_p, ctypes.c_int32, _PF]
        L.oc_position.restype = ctypes.c_int32
        L.oc_position.argtypes = [ctypes.c_void_p]
        _lib = L
    return _lib


def _f32(t) -> torch.Tensor:
    """Host fp32 contiguous copy (16-bit values widen exactly)."""
    return t.detach().to(dtype=torch.float32).to("cpu").contiguous()


def _ptr(t: torch.Tensor):
    return ctypes.cast(t.data_ptr(), _PF)


class CpuDecoder:
    """fp32 C++ decoder over the weights ``w`` (synth layout, any device or
    16-bit dtype: widened to host fp32 once and kept alive here)."""

    def __init__(self, shape, w, max_seq: int, n_threads: Optional[int] = None):
        self.shape = shape
        self.n_threads = int(n_threads or 1)
        self._arrs = {"tok_emb": _f32(w["tok_emb"]), "final_norm": _f32(w["final_norm"]),
                      "lm_head": _f32(w["lm_head"]),
                      "layers": [{k: _f32(lw[k]) for k in LAYER_KEYS} for lw in w["layers"]]}
        layers = (_Layer * shape.n_layers)(*[_Layer(*[_ptr(a[k]) for k in LAYER_KEYS])
                                              for a in self._arrs["layers"]])
        ws = _Weights(_ptr(self._arrs["tok_emb"]), _ptr(self._arrs["final_norm"]), _ptr(self._arrs["lm_head"]),
                      layers)
        sh = _Shape(shape.n_layers, shape.d_model, shape.n_heads, shape.n_kv_heads, shape.head_dim, shape.d_ffn,
                    shape.vocab, shape.rms_eps, shape.rope_base)
        self._h = lib().oc_create(ctypes.byref(sh), ctypes.byref(ws), int(max_seq), self.n_threads)
        if not self._h:
            raise ValueError("oc_create: invalid shape or out of memory")

    @property
    def position(self) -> int:
        return int(lib().oc_position(self._h))

    def set_cache(self, k: torch.Tensor, v: torch.Tensor):
        """k, v [n_layers][n_kv_heads][n_pos][head_dim] (rotated keys)."""
        s = self.shape
        assert k.shape == v.shape and k.dim() == 4 and tuple(k.shape[:2]) == (s.n_layers, s.n_kv_heads)
        assert k.shape[3] == s.head_dim
        k32, v32 = _f32(k), _f32(v)
        if lib().oc_set_cache(self._h, _ptr(k32), _ptr(v32), int(k.shape[2])) != 0:
            raise ValueError("oc_set_cache: invalid arguments")

    def step(self, token: int, want_logits: bool = True):
        """Feed one token; returns (greedy token, fp32 logits [vocab] or None)."""
        lg = torch.empty(self.shape.vocab, dtype=torch.float32) if want_logits else None
        t = lib().oc_step(self._h, int(token), _ptr(lg) if lg is not None else None)
        if t < 0:
            raise ValueError("oc_step: cache full or token out of range")
        return int(t), lg

    def feed(self, tokens: Sequence[int]) -> torch.Tensor:
        """Feed tokens one by one; returns their logits [n][vocab] (row i = after tokens[i])."""
        return torch.stack([self.step(t)[1] for t in tokens])

    def close(self):
        if getattr(self, "_h", None):
            lib().oc_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
