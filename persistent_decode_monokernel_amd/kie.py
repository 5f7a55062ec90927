"""ctypes binding of libkie.so (include/kie.h): argument marshalling only.

Every step of the decode path runs in the HIP library; PyTorch only provides
device memory (weights, workspace, logits) and the stream.  Importing this
module does not load the library; the first call does, and raises if the
library is missing (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os
import sys
from typing import Dict, List, Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkie.so")

KIE_OK = 0
KIE_ERR_ARG = -1
KIE_ERR_STATE = -2
KIE_ERR_CAPACITY = -3
KIE_ERR_UNSUPPORTED = -4
KIE_ERR_HIP = -5
KIE_ERR_TIMEOUT = -6
KIE_ERR_ABORTED = -7
KIE_F16 = 1
KIE_BF16 = 2
KIE_PREFILL_AUTO = 0
KIE_PREFILL_DECODE_LOOP = 1
KIE_HANDOFF_NAN_POLL = 0
KIE_HANDOFF_COUNTERS = 1
KIE_LAUNCH_PERSISTENT = 0
KIE_LAUNCH_PER_STAGE = 1
KIE_LAUNCH_PER_STAGE_GRAPH = 2
KIE_STATIC_WORKSPACE_BYTES = 64 << 20  # include/kie.h
KIE_GEMM_STORE = 0
KIE_GEMM_ADD = 1
KIE_GEMM_SWIGLU = 2
KIE_PROBE_PING = 0
KIE_PROBE_ALL_TO_ALL = 1
KIE_PROBE_STREAM_NONE = 0
KIE_PROBE_STREAM_OTHERS = 1
KIE_PROBE_STREAM_OWN = 2
KIE_HANDOFF_PROBE_SCRATCH_BYTES = 192 * 1024  # include/kie.h


class KieError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class kie_config(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("d_ffn", ctypes.c_int32),
        ("vocab", ctypes.c_int32), ("max_seq", ctypes.c_int32), ("rms_eps", ctypes.c_float),
        ("rope_base", ctypes.c_float), ("dtype", ctypes.c_int32),
    ]


_PP = ctypes.POINTER(ctypes.c_void_p)


class kie_weights(ctypes.Structure):
    _fields_ = [
        ("tok_emb", ctypes.c_void_p), ("final_norm", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
        ("attn_norm", _PP), ("wq", _PP), ("wk", _PP), ("wv", _PP), ("wo", _PP), ("ffn_norm", _PP),
        ("w_gate", _PP), ("w_up", _PP), ("w_down", _PP),
    ]


class kie_info(ctypes.Structure):
    _fields_ = [
        ("grid", ctypes.c_int32), ("block", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
        ("cu_count", ctypes.c_int32), ("attn_max_chunks", ctypes.c_int32), ("pos", ctypes.c_int32),
        ("last_kernel_ms", ctypes.c_float), ("last_steps", ctypes.c_int32),
    ]


class kie_handoff_probe_result(ctypes.Structure):
    _fields_ = [
        ("exchange_us", ctypes.c_double), ("exchange_max_us", ctypes.c_double), ("stream_gbps", ctypes.c_double),
        ("xcc_a", ctypes.c_int32), ("xcc_b", ctypes.c_int32), ("completed", ctypes.c_int32),
        ("grid", ctypes.c_int32),
    ]


# name -> (restype, argtypes); mirrors include/kie.h
SIGNATURES = {
    "kie_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "kie_config_validate": (ctypes.c_int, [ctypes.POINTER(kie_config)]),
    "kie_set_prefill_mode": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]),
    "kie_set_prefill_chunk": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]),
    "kie_set_grid": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]),
    "kie_set_sampling": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_float, ctypes.c_int32, ctypes.c_float,
                                        ctypes.c_uint64]),
    "kie_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(kie_config)]),
    "kie_create": (ctypes.c_int, [ctypes.POINTER(kie_config), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                  ctypes.POINTER(ctypes.c_void_p)]),
    "kie_create_static": (ctypes.c_int, [ctypes.POINTER(kie_config), ctypes.c_void_p,
                                         ctypes.POINTER(ctypes.c_void_p)]),
    "kie_load_weights": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(kie_weights)]),
    "kie_prefill": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), ctypes.c_int32,
                                   ctypes.POINTER(ctypes.c_int32), ctypes.c_void_p]),
    "kie_decode": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                  ctypes.POINTER(ctypes.c_int32), ctypes.c_void_p]),
    "kie_destroy": (None, [ctypes.c_void_p]),
    "kie_import_kv": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                     ctypes.c_int32]),
    "kie_export_kv": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]),
    "kie_get_info": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(kie_info)]),
    "kie_set_poll_timeout": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_uint64]),
    "kie_set_abort_after": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]),
    "kie_set_withhold": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]),
    "kie_set_delay": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64]),
    "kie_set_handoff": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]),
    "kie_set_launch_mode": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]),
    "kie_check_idle_sets": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint64)]),
    "kie_trace_words": (ctypes.c_size_t, [ctypes.c_void_p]),
    "kie_set_trace": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]),
    "kie_check_tiling": (ctypes.c_int, [ctypes.POINTER(kie_config), ctypes.c_int32, ctypes.c_int32]),
    "kie_stream_probe": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)]),
    "kie_gemv_probe": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)]),
    "kie_gemm_probe": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_float)]),
    "kie_attn_probe": (ctypes.c_int, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.POINTER(ctypes.c_float)]),
    "kie_handoff_probe": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_size_t,
                                         ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                         ctypes.POINTER(kie_handoff_probe_result)]),
}

_lib = None


def lib():
    """Load libkie.so (once).  Raises if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m persistent_decode_monokernel_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().kie_status_string(int(s)).decode()


def _check(status: int, what: str):
    if status != KIE_OK:
        raise KieError(status, what)


def make_config(shape, max_seq: int) -> kie_config:
    """kie_config from a ModelShape-like object (n_layers, d_model, ... dtype)."""
    return kie_config(shape.n_layers, shape.d_model, shape.n_heads, shape.n_kv_heads, shape.head_dim,
                      shape.d_ffn, shape.vocab, max_seq, shape.rms_eps, shape.rope_base, shape.dtype)


def validate(cfg: kie_config) -> int:
    return lib().kie_config_validate(ctypes.byref(cfg))


def check_tiling(cfg: kie_config, grid: int, full: bool) -> int:
    return lib().kie_check_tiling(ctypes.byref(cfg), int(grid), 1 if full else 0)


def workspace_bytes(cfg: kie_config) -> int:
    return lib().kie_workspace_bytes(ctypes.byref(cfg))


def _dptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream or None


class Engine:
    """One decode engine: workspace (torch uint8 tensor), borrowed weights.

    Calls are synchronous on the engine stream (torch's current stream at
    construction unless given).
    """

    def __init__(self, shape, max_seq: int, device="cuda", stream=None, static: bool = False):
        """static=True: the engine runs on the library's static workspace
        (kie_create_static), and no workspace tensor is allocated."""
        self.shape = shape
        self.cfg = make_config(shape, max_seq)
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        nbytes = workspace_bytes(self.cfg)
        if nbytes == 0:
            raise KieError(validate(self.cfg), "kie_workspace_bytes")
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        h = ctypes.c_void_p()
        if static:
            self.workspace = None
            with torch.cuda.device(self.device):
                _check(lib().kie_create_static(ctypes.byref(self.cfg), ctypes.c_void_p(_stream_handle(self.stream)),
                                               ctypes.byref(h)), "kie_create_static")
        else:
            self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            with torch.cuda.device(self.device):
                _check(lib().kie_create(ctypes.byref(self.cfg), ctypes.c_void_p(_dptr(self.workspace)), nbytes,
                                        ctypes.c_void_p(_stream_handle(self.stream)), ctypes.byref(h)),
                       "kie_create")
        self._h = h
        self._weights = None

    # ---- lifecycle
    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().kie_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        # At interpreter exit the HIP runtime and any profiler attached to it
        # may already be shutting down: release the handle only while the
        # interpreter is alive (call close() explicitly before exit).
        if sys.is_finalizing():
            return
        try:
            self.close()
        except Exception:
            pass

    def load_weights(self, w: Dict[str, object]):
        """w: dict from synth.make_weights (device tensors of the engine dtype)."""
        layers = w["layers"]
        L = len(layers)
        s = self.shape
        if L != s.n_layers:
            raise KieError(KIE_ERR_ARG, f"load_weights: {L} layers for a {s.n_layers}-layer shape")
        d, qd, kvd, F, V = s.d_model, s.n_heads * s.head_dim, s.n_kv_heads * s.head_dim, s.d_ffn, s.vocab
        numel = {"tok_emb": V * d, "final_norm": d, "lm_head": V * d, "attn_norm": d, "ffn_norm": d,
                 "wq": qd * d, "wk": kvd * d, "wv": kvd * d, "wo": d * qd, "w_gate": F * d, "w_up": F * d,
                 "w_down": d * F}
        self._check_tensor("tok_emb", w["tok_emb"], numel["tok_emb"])
        self._check_tensor("final_norm", w["final_norm"], numel["final_norm"])
        self._check_tensor("lm_head", w["lm_head"], numel["lm_head"])
        arrs = {}
        keep: List[torch.Tensor] = [w["tok_emb"], w["final_norm"], w["lm_head"]]
        for key in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down"):
            ts = [lw[key].contiguous() for lw in layers]
            for t in ts:
                self._check_tensor(key, t, numel[key])
            keep.extend(ts)
            arrs[key] = (ctypes.c_void_p * L)(*[_dptr(t) for t in ts])
        kw = kie_weights(_dptr(w["tok_emb"].contiguous()), _dptr(w["final_norm"].contiguous()),
                         _dptr(w["lm_head"].contiguous()),
                         *[ctypes.cast(arrs[k], _PP) for k in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm",
                                                               "w_gate", "w_up", "w_down")])
        _check(lib().kie_load_weights(self._h, ctypes.byref(kw)), "kie_load_weights")
        self._weights = keep  # borrowed by the library: keep alive

    def prefill(self, prompt: Sequence[int], want_logits: bool = False) -> Tuple[int, Optional[torch.Tensor]]:
        p = (ctypes.c_int32 * len(prompt))(*[int(x) for x in prompt])
        tok = ctypes.c_int32(-1)
        lg = torch.empty(self.cfg.vocab, dtype=torch.float32, device=self.device) if want_logits else None
        st = lib().kie_prefill(self._h, p, len(prompt), ctypes.byref(tok),
                               ctypes.c_void_p(_dptr(lg)) if lg is not None else None)
        _check(st, "kie_prefill")
        return tok.value, lg

    def decode(self, n_steps: int, eos_id: int = -1, want_logits: bool = False, raise_on_error: bool = True):
        """Returns (tokens, logits [n][V] or None, status)."""
        toks = (ctypes.c_int32 * max(1, n_steps))()
        n = ctypes.c_int32(0)
        lg = (torch.empty((max(1, n_steps), self.cfg.vocab), dtype=torch.float32, device=self.device)
              if want_logits else None)
        st = lib().kie_decode(self._h, n_steps, eos_id, toks, ctypes.byref(n),
                              ctypes.c_void_p(_dptr(lg)) if lg is not None else None)
        if raise_on_error:
            _check(st, "kie_decode")
        out = [toks[i] for i in range(n.value)]
        return out, (lg[: n.value] if lg is not None else None), st

    def _check_tensor(self, what: str, t: torch.Tensor, numel: int, shape=None):
        """The library reads device memory through raw pointers: reject a tensor
        on another device, of another dtype or of another size before it does."""
        if not isinstance(t, torch.Tensor) or t.device != self.device:
            raise KieError(KIE_ERR_ARG, f"{what}: not a tensor on {self.device}")
        if t.dtype != self.shape.torch_dtype:
            raise KieError(KIE_ERR_ARG, f"{what}: dtype {t.dtype}, engine dtype {self.shape.torch_dtype}")
        if t.numel() != numel or (shape is not None and tuple(t.shape) != tuple(shape)):
            raise KieError(KIE_ERR_ARG, f"{what}: shape {tuple(t.shape)} does not match the engine's")

    def import_kv(self, k: torch.Tensor, v: torch.Tensor, pending: int):
        s = self.shape
        if k.dim() != 4:
            raise KieError(KIE_ERR_ARG, "import_kv: k must be [n_layers][n_kv_heads][n_pos][head_dim]")
        n_pos = int(k.shape[2])
        want = (s.n_layers, s.n_kv_heads, n_pos, s.head_dim)
        self._check_tensor("import_kv k", k, int(torch.Size(want).numel()), want)
        self._check_tensor("import_kv v", v, int(torch.Size(want).numel()), want)
        k = k.contiguous()
        v = v.contiguous()
        _check(lib().kie_import_kv(self._h, ctypes.c_void_p(_dptr(k)), ctypes.c_void_p(_dptr(v)), n_pos,
                                   int(pending)), "kie_import_kv")

    def export_kv(self):
        s = self.shape
        cap = self.info().pos
        k = torch.empty((s.n_layers, s.n_kv_heads, max(cap, 1), s.head_dim), dtype=s.torch_dtype,
                        device=self.device)
        v = torch.empty_like(k)
        n = ctypes.c_int32(max(cap, 1))
        pend = ctypes.c_int32(-1)
        _check(lib().kie_export_kv(self._h, ctypes.c_void_p(_dptr(k)), ctypes.c_void_p(_dptr(v)),
                                   ctypes.byref(n), ctypes.byref(pend)), "kie_export_kv")
        return k[:, :, : n.value], v[:, :, : n.value], pend.value

    def info(self) -> kie_info:
        i = kie_info()
        _check(lib().kie_get_info(self._h, ctypes.byref(i)), "kie_get_info")
        return i

    def set_poll_timeout(self, ticks: int):
        _check(lib().kie_set_poll_timeout(self._h, int(ticks)), "kie_set_poll_timeout")

    def set_abort_after(self, steps: int):
        _check(lib().kie_set_abort_after(self._h, int(steps)), "kie_set_abort_after")

    def trace_words(self) -> int:
        return int(lib().kie_trace_words(self._h))

    def set_trace(self, buf: Optional[torch.Tensor], step: int = 0):
        """buf: int64 device tensor of trace_words() entries, or None to stop."""
        _check(lib().kie_set_trace(self._h, ctypes.c_void_p(_dptr(buf)) if buf is not None else None, int(step)),
               "kie_set_trace")
        self._trace_buf = buf

    def set_prefill_mode(self, mode: int):
        """KIE_PREFILL_AUTO (matrix-core prompt path where supported) or KIE_PREFILL_DECODE_LOOP."""
        _check(lib().kie_set_prefill_mode(self._h, int(mode)), "kie_set_prefill_mode")

    def set_sampling(self, temperature: float, top_k: int = 64, top_p: float = 1.0, seed: int = 0):
        """Token choice: greedy for temperature <= 0, else temperature / top-k (<= 64) /
        nucleus sampling with Philox4x32-10 uniforms keyed by seed and position."""
        _check(lib().kie_set_sampling(self._h, float(temperature), int(top_k), float(top_p),
                                      int(seed) & (2**64 - 1)), "kie_set_sampling")

    def set_grid(self, grid: int):
        """Work-groups of the persistent kernel (0 = one per compute unit)."""
        _check(lib().kie_set_grid(self._h, int(grid)), "kie_set_grid")

    def set_prefill_chunk(self, positions: int):
        """Prompt positions per matrix-core chunk (0 = as many as the workspace holds)."""
        _check(lib().kie_set_prefill_chunk(self._h, int(positions)), "kie_set_prefill_chunk")

    def set_withhold(self, wg: int):
        _check(lib().kie_set_withhold(self._h, int(wg)), "kie_set_withhold")

    def set_delay(self, wg: int, ticks: int):
        """Race test: work-group wg holds back each hand-off publication by ticks (100 MHz)."""
        _check(lib().kie_set_delay(self._h, int(wg), int(ticks)), "kie_set_delay")

    def set_handoff(self, mode: int):
        """KIE_HANDOFF_NAN_POLL (default) or KIE_HANDOFF_COUNTERS (comparison protocol)."""
        _check(lib().kie_set_handoff(self._h, int(mode)), "kie_set_handoff")

    def set_launch_mode(self, mode: int):
        """KIE_LAUNCH_PERSISTENT (default), KIE_LAUNCH_PER_STAGE or KIE_LAUNCH_PER_STAGE_GRAPH."""
        _check(lib().kie_set_launch_mode(self._h, int(mode)), "kie_set_launch_mode")

    def idle_sets_dirty_words(self) -> int:
        """Words of the two idle exchange sets that are not the NaN pattern after the last launch."""
        n = ctypes.c_uint64(0)
        _check(lib().kie_check_idle_sets(self._h, ctypes.byref(n)), "kie_check_idle_sets")
        return int(n.value)


def gemv_probe(W: torch.Tensor, x: torch.Tensor, stream=None, input_first: bool = False) -> Tuple[torch.Tensor, float]:
    """y[i] = W[i % n_copies] @ x[i] in one persistent launch.  input_first:
    each product reads its input vector before its weights (else after its
    first weight block, a decode stage's order).  Returns (y fp32, kernel ms)."""
    if not (isinstance(W, torch.Tensor) and isinstance(x, torch.Tensor) and W.dim() == 3 and x.dim() == 2
            and W.shape[2] == x.shape[1]):
        raise KieError(KIE_ERR_ARG, "gemv_probe: W must be [n_copies][rows][cols] and x [n_vec][cols]")
    if W.device.type != "cuda" or x.device != W.device or not (W.is_contiguous() and x.is_contiguous()):
        raise KieError(KIE_ERR_ARG, "gemv_probe: W and x must be contiguous tensors on one GPU")
    if W.dtype not in (torch.float16, torch.bfloat16) or x.dtype != W.dtype:
        raise KieError(KIE_ERR_ARG, f"gemv_probe: dtypes {W.dtype}, {x.dtype} (float16 or bfloat16, both alike)")
    n_copies, rows, cols = W.shape
    dtype = KIE_F16 if W.dtype == torch.float16 else KIE_BF16
    y = torch.empty((x.shape[0], rows), dtype=torch.float32, device=W.device)
    ms = ctypes.c_float(0)
    _check(lib().kie_gemv_probe(ctypes.c_void_p(_dptr(W)), rows, cols, n_copies, ctypes.c_void_p(_dptr(x)),
                                ctypes.c_void_p(_dptr(y)), x.shape[0], dtype, int(bool(input_first)),
                                ctypes.c_void_p(_stream_handle(stream)), ctypes.byref(ms)), "kie_gemv_probe")
    return y, ms.value


def stream_probe(buf: torch.Tensor, depth: int = 3, reps: int = 4, stream=None) -> Tuple[float, int]:
    """Read-stream probe over the bytes of a device tensor.  Returns (kernel ms,
    bytes read)."""
    sink = torch.zeros(1024, dtype=torch.int32, device=buf.device)
    ms = ctypes.c_float(0)
    nbytes = buf.numel() * buf.element_size()
    _check(lib().kie_stream_probe(ctypes.c_void_p(_dptr(buf)), nbytes, int(depth), int(reps),
                                  ctypes.c_void_p(_dptr(sink)), ctypes.c_void_p(_stream_handle(stream)),
                                  ctypes.byref(ms)), "kie_stream_probe")
    grid = torch.cuda.get_device_properties(buf.device).multi_processor_count
    grid = min(grid, 1024)
    npass = nbytes // 16 // grid // 512
    read = grid * 512 * 16 * (npass // depth * depth) * reps  # whole rounds of `depth` passes
    return ms.value, read


def handoff_probe(kind: int, rounds: int = 200, wg_a: int = 0, wg_b: int = 1, where: int = KIE_PROBE_STREAM_NONE,
                  depth: int = 3, buf: Optional[torch.Tensor] = None, scratch: Optional[torch.Tensor] = None,
                  stride: int = 1, stream=None) -> kie_handoff_probe_result:
    """Hand-off latency probe (ping between work-groups wg_a and wg_b, or an
    all-to-all round over the grid), optionally beside streaming of `buf`."""
    if scratch is None:
        scratch = torch.zeros(KIE_HANDOFF_PROBE_SCRATCH_BYTES // 8, dtype=torch.int64, device="cuda")
    nbytes = 0 if buf is None else buf.numel() * buf.element_size()
    r = kie_handoff_probe_result()
    _check(lib().kie_handoff_probe(int(kind), int(wg_a), int(wg_b), int(rounds), int(stride), int(depth), int(where),
                                   ctypes.c_void_p(0 if buf is None else _dptr(buf)), nbytes,
                                   ctypes.c_void_p(_dptr(scratch)), scratch.numel() * scratch.element_size(),
                                   ctypes.c_void_p(_stream_handle(stream)), ctypes.byref(r)), "kie_handoff_probe")
    return r


def gemm_probe(op: int, A: torch.Tensor, W: torch.Tensor, out: torch.Tensor, W2: Optional[torch.Tensor] = None,
               part: Optional[torch.Tensor] = None, reps: int = 1, stream=None) -> Tuple[float, int]:
    """One matrix-core GEMM of the prompt path (kie_gemm_probe) into `out`.
    Returns (mean ms per product, split-K slices)."""
    M, K = A.shape
    N = W.shape[0]
    dtype = KIE_F16 if W.dtype == torch.float16 else KIE_BF16
    ms = ctypes.c_float(0)
    sl = ctypes.c_int32(0)
    pbytes = 0 if part is None else part.numel() * part.element_size()
    _check(lib().kie_gemm_probe(int(op), dtype, ctypes.c_void_p(_dptr(A)), M, K, ctypes.c_void_p(_dptr(W)),
                                ctypes.c_void_p(0 if W2 is None else _dptr(W2)), N, ctypes.c_void_p(_dptr(out)),
                                ctypes.c_void_p(0 if part is None else _dptr(part)), pbytes, int(reps),
                                ctypes.c_void_p(_stream_handle(stream)), ctypes.byref(sl), ctypes.byref(ms)),
           "kie_gemm_probe")
    return ms.value, sl.value


def attn_probe(qkv: torch.Tensor, kc: torch.Tensor, vc: torch.Tensor, out: torch.Tensor, n_heads: int, p0: int,
               reps: int = 1, stream=None) -> float:
    """One causal flash attention of the prompt path (kie_attn_probe) into
    `out`.  qkv fp32 [M][ldq]; kc, vc [n_kv_heads][max_seq][head_dim].
    Returns the mean ms per launch."""
    n_kv, max_seq, hd = kc.shape
    M = qkv.shape[0]
    dtype = KIE_F16 if kc.dtype == torch.float16 else KIE_BF16
    ms = ctypes.c_float(0)
    _check(lib().kie_attn_probe(dtype, ctypes.c_void_p(_dptr(qkv)), M, int(n_heads), n_kv, hd, int(p0), max_seq,
                                ctypes.c_void_p(_dptr(kc)), ctypes.c_void_p(_dptr(vc)), ctypes.c_void_p(_dptr(out)),
                                int(reps), ctypes.c_void_p(_stream_handle(stream)), ctypes.byref(ms)),
           "kie_attn_probe")
    return ms.value
