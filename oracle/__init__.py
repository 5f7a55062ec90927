"""CPU oracle (test infrastructure only; never imported by the product path).

Float64 PyTorch-CPU reference of greedy batch-1 decoding of a dense decoder
and of the isolated matrix-vector product (``oracle.decoder``), and of token
sampling beyond greedy with its counter-based generator (``oracle.sampling``).
"""
from . import sampling
from .decoder import (KVCache, apply_rope, argmax_first, attention, forward, greedy_decode,
                      greedy_token, matvec, prefill, rmsnorm, rope_cos_sin, silu, softmax,
                      teacher_forced, to64)

__all__ = ["sampling", "KVCache", "apply_rope", "argmax_first", "attention", "forward", "greedy_decode",
           "greedy_token", "matvec", "prefill", "rmsnorm", "rope_cos_sin", "silu", "softmax",
           "teacher_forced", "to64"]
