"""The C-ABI library on a machine without a GPU: it loads, exports every
function include/zero.h declares, computes its host-side metadata exactly like
the oracle, and rejects bad arguments before touching the device."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zero.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(zero_\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported(libzero):
    names = _declared()
    assert len(names) >= 13, names
    for n in names:
        assert hasattr(libzero, n), f"{n} declared in zero.h but not exported"
    from zero_sharded_optimizer_reduce_amd import _lib
    assert set(_lib.SIGNATURES) == set(names)


def test_binding_constants_match_the_header():
    from zero_sharded_optimizer_reduce_amd import _lib
    src = open(HEADER).read()
    defines = dict(re.findall(r"^#define\s+(ZERO_\w+)\s+(\d+)", src, flags=re.M))
    assert {"ZERO_MAX_RANKS", "ZERO_NORM_BLOCKS", "ZERO_OFFLOAD_MAX_CHUNKS"} <= set(defines)
    for name, value in defines.items():
        assert getattr(_lib, name) == int(value), name
    enums = dict(re.findall(r"\b(ZERO_(?:OK|ERR_\w+|OFFLOAD_\w+))\s*=\s*(-?\d+)", src))
    for name, value in enums.items():
        assert getattr(_lib, name) == int(value), name


def test_status_strings(libzero):
    for st in (0, -1, -2, -3, -4, -5):
        assert libzero.zero_status_string(st).startswith(b"ZERO_")


def test_adam_scalars_match_oracle(libzero):
    from zero_sharded_optimizer_reduce_amd import api
    for step in (1, 2, 3, 10, 1000, 123456):
        for wd in (0.0, 0.1):
            hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=wd, step=step)
            lib = api.zero_adam_scalars_compute(hp)
            ref = oracle.adam_scalars(1e-3, 0.9, 0.999, 1e-8, wd, step)
            for k in ref:
                assert lib[k].view(np.uint32) == ref[k].view(np.uint32), (k, step)


def test_rank_weights_and_layout_match_oracle(libzero):
    from zero_sharded_optimizer_reduce_amd import api
    for counts in ([4096, 3072, 4096, 2048], [1, 2, 3], [5], [10 ** 9, 1, 7, 3]):
        lib = api.zero_rank_weights(counts, len(counts))
        assert np.array_equal(lib.view(np.uint32), oracle.weights_from_counts(counts).view(np.uint32))
    for n in (1, 2, 3, 4, 8, 16):
        lib = api.zero_rank_weights(None, n)
        assert np.array_equal(lib.view(np.uint32), oracle.weights_mean(n).view(np.uint32))
    for numels, n in (([202_375_168], 4), ([5, 7], 4), ([0], 3), ([1023, 1, 1], 4), ([10 ** 10], 16)):
        assert api.zero_shard_layout(numels, n) == oracle.shard_layout(numels, n)


def test_rank_weights_argument_errors(libzero):
    from zero_sharded_optimizer_reduce_amd import api
    from zero_sharded_optimizer_reduce_amd._lib import ZeroError
    with pytest.raises(ValueError, match="len"):
        api.zero_rank_weights([1, 2, 3], 2)          # more counts than ranks
    with pytest.raises(ValueError, match="len"):
        api.zero_rank_weights([1], 2)
    with pytest.raises(ValueError, match="at least 1"):
        api.zero_rank_weights(None, 0)
    with pytest.raises(ZeroError):
        api.zero_rank_weights(None, 17)              # the C ABI's limit
    with pytest.raises(ZeroError):
        api.zero_rank_weights([0, 0], 2)             # counts summing to 0
    with pytest.raises(ZeroError):
        api.zero_rank_weights([3, -1], 2)


def _pp(*vals):
    return (C.c_void_p * len(vals))(*vals)


def _w(n):
    return (C.c_float * n)(*([1.0 / n] * n))


def test_reduce_scatter_validation(libzero):
    L = libzero
    g = _pp(0x10000, 0x20000, 0x30000, 0x40000)
    o = _pp(0x100000, 0x110000, 0x120000, 0x130000)
    assert L.zero_reduce_scatter(g, _w(4), 0, 1024, o, 4, 0, None) == -1          # n_ranks
    assert L.zero_reduce_scatter(g, _w(4), 17, 1024, o, 4, 0, None) == -1
    assert L.zero_reduce_scatter(g, _w(4), 4, 1024, o, 0, 0, None) == -1          # n_shards
    assert L.zero_reduce_scatter(g, _w(4), 4, -1, o, 4, 0, None) == -1            # numel
    assert L.zero_reduce_scatter(g, _w(4), 4, 1023, o, 4, 0, None) == -3          # divisibility
    assert L.zero_reduce_scatter(g, _w(4), 4, 1024, o, 4, 2, None) == -1          # accumulate flag
    assert L.zero_reduce_scatter(_pp(0x10001, 0x20000, 0x30000, 0x40000), _w(4), 4, 1024, o, 4, 0, None) == -2
    assert L.zero_reduce_scatter(g, _w(4), 4, 1024, _pp(0x100002, 0x110000, 0x120000, 0x130000), 4, 0, None) == -2
    assert L.zero_reduce_scatter(_pp(0, 0x20000, 0x30000, 0x40000), _w(4), 4, 1024, o, 4, 0, None) == -1
    assert L.zero_reduce_scatter(_pp(0, 0, 0, 0), _w(4), 4, 0, _pp(0, 0, 0, 0), 4, 0, None) == 0
    assert L.zero_reduce_scatter(None, _w(4), 4, 1024, o, 4, 0, None) == -1
    # an output shard overlapping a rank buffer, and two overlapping outputs
    assert L.zero_reduce_scatter(g, _w(4), 4, 1024, _pp(0x10100, 0x110000, 0x120000, 0x130000), 4, 0, None) == -1
    assert L.zero_reduce_scatter(g, _w(4), 4, 1024, _pp(0x100000, 0x100100, 0x120000, 0x130000), 4, 0, None) == -1
    assert b"overlap" in L.zero_last_error()
    # zero elements: valid, nothing launched
    assert L.zero_reduce_scatter(g, _w(4), 4, 0, o, 4, 0, None) == 0


def test_adam_validation(libzero):
    from zero_sharded_optimizer_reduce_amd._lib import AdamHparams
    L = libzero
    hp = AdamHparams(1e-3, 0.9, 0.999, 1e-8, 0.0, 1)
    bufs = [0x100000, 0x200000, 0x300000, 0x400000, 0x500000]
    assert L.zero_adam_shard_step(*bufs[:4], bufs[4], 0, C.byref(hp), None) == 0
    assert L.zero_adam_shard_step(0, 0, 0, 0, 0, 0, C.byref(hp), None) == 0
    assert L.zero_adam_shard_step(*bufs[:4], bufs[4], -5, C.byref(hp), None) == -1
    assert L.zero_adam_shard_step(0, *bufs[1:4], bufs[4], 16, C.byref(hp), None) == -1
    assert L.zero_adam_shard_step(bufs[0] + 2, *bufs[1:4], bufs[4], 16, C.byref(hp), None) == -2
    assert L.zero_adam_shard_step(*bufs[:3], bufs[3] + 1, bufs[4], 16, C.byref(hp), None) == -2
    assert L.zero_adam_shard_step(bufs[0], bufs[0] + 8, *bufs[2:4], bufs[4], 16, C.byref(hp), None) == -1
    assert L.zero_adam_shard_step(*bufs[:4], bufs[4], 16, None, None) == -1
    for bad in (AdamHparams(1e-3, 0.9, 0.999, 1e-8, 0.0, 0), AdamHparams(1e-3, 1.0, 0.999, 1e-8, 0.0, 1),
                AdamHparams(1e-3, 0.9, -0.1, 1e-8, 0.0, 1)):
        assert L.zero_adam_shard_step(*bufs[:4], bufs[4], 16, C.byref(bad), None) == -1


def test_all_gather_validation(libzero):
    L = libzero
    s = _pp(0x10000, 0x20000)
    assert L.zero_all_gather_layer(s, 0, 64, 0x100000, None) == -1
    assert L.zero_all_gather_layer(s, 2, -1, 0x100000, None) == -1
    assert L.zero_all_gather_layer(s, 2, 64, 0, None) == -1
    assert L.zero_all_gather_layer(_pp(0, 0), 2, 0, 0, None) == 0
    assert L.zero_all_gather_layer(_pp(0x10000, 0x100010), 2, 64, 0x100000, None) == -1
    assert L.zero_all_gather_layer(s, 2, 0, 0x100000, None) == 0


def test_offload_validation(libzero):
    L = libzero
    h = C.c_void_p()
    slots = _pp(0x100000, 0x200000)
    stage = _pp(0x300000, 0x400000)
    assert L.zero_offload_create(0, 100, 10, 0x1000, slots, stage, C.byref(h)) == -1
    assert L.zero_offload_create(4, 0, 10, 0x1000, slots, stage, C.byref(h)) == -1
    assert L.zero_offload_create(4, 100, 10, 0, slots, stage, C.byref(h)) == -1
    assert L.zero_offload_create(4, 100, 10, 0x1000, _pp(0x100000, 0x100008), stage, C.byref(h)) == -1
    assert L.zero_offload_create(4, 100, 10, 0x1002, slots, stage, C.byref(h)) == -2
    assert L.zero_offload_create(4, 100, 10, 0x1000, slots, stage, None) == -1
    assert L.zero_offload_stream(None, 0, 0, 0, None, None, None, None, None, None, None) == -1
    assert L.zero_offload_sync(None) == -1
    assert L.zero_offload_destroy(None) == 0


def test_fused_validation_alias_rules(libzero):
    from zero_sharded_optimizer_reduce_amd._lib import AdamHparams
    L = libzero
    hp = AdamHparams(1e-3, 0.9, 0.999, 1e-8, 0.0, 1)
    g = _pp(0x10000000)                       # one rank, numel 1024 BF16
    P, M, V, B = _pp(0x100000), _pp(0x200000), _pp(0x300000), _pp(0x400000)
    acc = _pp(0x500000)
    # (grad_out identical to grad_acc is allowed; the GPU tests run that case)
    # grad_out overlapping grad_acc partially: rejected before any launch
    assert L.zero_reduce_scatter_adam(g, _w(1), 1, 1024, 1, P, M, V, B, acc, _pp(0x500010), C.byref(hp), None) == -1
    # grad_acc overlapping the master: rejected
    assert L.zero_reduce_scatter_adam(g, _w(1), 1, 1024, 1, P, M, V, B, _pp(0x100100), None, C.byref(hp), None) == -1
    # a rank buffer equal to grad_out == grad_acc: rejected
    assert L.zero_reduce_scatter_adam(_pp(0x500000), _w(1), 1, 1024, 1, P, M, V, B, acc, acc, C.byref(hp),
                                      None) == -1


def test_roctx_tracing_switch():
    # ZERO_ROCTX=1 loads ROCm's roctx library at the first use; without it the
    # library emits nothing.  Each case runs in a fresh interpreter (no GPU use).
    import os
    import subprocess
    import sys
    code = ("import ctypes, sys; sys.path.insert(0, %r); "
            "from zero_sharded_optimizer_reduce_amd import _lib; "
            "print(_lib.load().zero_tracing_enabled())") % ROOT
    for flag, want in (("1", "1"), ("0", "0"), (None, "0")):
        env = dict(os.environ)
        env.pop("ZERO_ROCTX", None)
        if flag is not None:
            env["ZERO_ROCTX"] = flag
        r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=120)
        assert r.returncode == 0, r.stderr
        assert r.stdout.strip() == want, (flag, r.stdout)
