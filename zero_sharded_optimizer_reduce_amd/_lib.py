"""ctypes loader for libzero.so, the C-ABI library (include/zero.h).

The library is built in-tree by zero_sharded_optimizer_reduce_amd/csrc/build.py.
If it is missing, load() raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libzero.so")

ZERO_OK, ZERO_ERR_ARG, ZERO_ERR_ALIGN, ZERO_ERR_SIZE, ZERO_ERR_HIP, ZERO_ERR_STATE = 0, -1, -2, -3, -4, -5
ZERO_MAX_RANKS = 16
ZERO_NORM_BLOCKS = 1024
ZERO_OFFLOAD_MAX_CHUNKS = 65536
ZERO_OFFLOAD_REDUCE, ZERO_OFFLOAD_ADAM, ZERO_OFFLOAD_REDUCE_ADAM = 0, 1, 2


class AdamHparams(C.Structure):
    _fields_ = [("lr", C.c_float), ("beta1", C.c_float), ("beta2", C.c_float), ("eps", C.c_float),
                ("weight_decay", C.c_float), ("step", C.c_int64)]


class AdamScalars(C.Structure):
    _fields_ = [(n, C.c_float) for n in (
        "lr", "beta1", "beta2", "one_minus_beta1", "one_minus_beta2",
        "bias_correction1", "bias_correction2", "eps", "weight_decay")]


P = C.c_void_p
I64 = C.c_int64
PP = C.POINTER(C.c_void_p)
FP = C.POINTER(C.c_float)
I64P = C.POINTER(C.c_int64)

# name -> (restype, argtypes); mirrors include/zero.h
SIGNATURES = {
    "zero_adam_scalars_compute": (C.c_int, [C.POINTER(AdamHparams), C.POINTER(AdamScalars)]),
    "zero_rank_weights": (C.c_int, [I64P, C.c_int, FP]),
    "zero_shard_layout": (C.c_int, [I64P, C.c_int, C.c_int, I64P, I64P, I64P]),
    "zero_reduce_scatter": (C.c_int, [PP, FP, C.c_int, I64, PP, C.c_int, C.c_int, P]),
    "zero_reduce_scatter_f32": (C.c_int, [PP, FP, C.c_int, I64, PP, C.c_int, C.c_int, P]),
    "zero_adam_shard_step": (C.c_int, [P, P, P, P, P, I64, C.POINTER(AdamHparams), P]),
    "zero_adam_shard_step_scaled": (C.c_int, [P, P, P, P, P, P, I64, C.POINTER(AdamHparams), P]),
    "zero_grad_norm_sq": (C.c_int, [PP, C.c_int, I64, P, I64, P, C.c_float, P, P]),
    "zero_grad_norm_sq_no_alloc": (C.c_int, [PP, C.c_int, I64, P, C.c_float, P, P]),
    "zero_reduce_scatter_adam": (C.c_int, [PP, FP, C.c_int, I64, C.c_int, PP, PP, PP, PP, PP, PP,
                                           C.POINTER(AdamHparams), P]),
    "zero_adam_shard_step_dev": (C.c_int, [P, P, P, P, P, P, I64, P, P]),
    "zero_reduce_scatter_adam_dev": (C.c_int, [PP, FP, C.c_int, I64, C.c_int, PP, PP, PP, PP, PP, PP, P, P]),
    "zero_adam_scalars_fetch": (C.c_int, [P, C.c_int, P, P, P]),
    "zero_all_gather_layer": (C.c_int, [PP, C.c_int, I64, P, P]),
    "zero_offload_create": (C.c_int, [C.c_int, I64, I64, P, PP, PP, C.POINTER(C.c_void_p)]),
    "zero_offload_stream": (C.c_int, [P, C.c_int, I64, C.c_int, FP, P, P, P, P,
                                      C.POINTER(AdamHparams), P]),
    "zero_offload_sync": (C.c_int, [P]),
    "zero_offload_destroy": (C.c_int, [P]),
    "zero_status_string": (C.c_char_p, [C.c_int]),
    "zero_last_error": (C.c_char_p, []),
    "zero_last_path_vectorized": (C.c_int, []),
    "zero_tracing_enabled": (C.c_int, []),
}

_LIB = None


def load() -> C.CDLL:
    """Load libzero.so (once).  Raises RuntimeError if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: the HIP library has not been built "
            "(run `python -c 'import __graft_entry__ as g; g.build()'`). "
            "There is no CPU fallback.")
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


class ZeroError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        msg = lib.zero_last_error().decode(errors="replace")
        super().__init__(f"{where}: {lib.zero_status_string(status).decode()} ({msg})")
        self.status = status


def check(status: int, where: str) -> None:
    if status != ZERO_OK:
        raise ZeroError(status, where)
