"""Thin Python binding of libzero's C ABI (include/zero.h), same names.

Argument marshalling only: tensors are checked for device, dtype, layout and
size (the C ABI sees raw pointers and cannot), their data pointers and the
current HIP stream are passed through, and every computation runs in the HIP
kernels.  PyTorch provides device memory and streams.
"""
from __future__ import annotations

import ctypes as C
from typing import Mapping, Optional, Sequence

import numpy as np
import torch

from . import _lib
from ._lib import AdamHparams, check, load

_BF16_LIKE = (torch.bfloat16, torch.int16, torch.uint16)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dev(t: torch.Tensor, what: str, dtypes) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor")
    d = t.get_device() if t.is_cuda else -1
    if d < 0:
        raise ValueError(f"{what}: must be a device tensor, got {t.device}")
    if d != torch.cuda.current_device():
        raise ValueError(f"{what}: on {t.device}, but the current device is cuda:{torch.cuda.current_device()}")
    if t.dtype not in dtypes:
        raise TypeError(f"{what}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")
    return t.data_ptr()


def _ptrs(ptrs) -> C.Array:
    return (C.c_void_p * len(ptrs))(*ptrs)


def hparams(hp) -> AdamHparams:
    if isinstance(hp, AdamHparams):
        return hp
    return AdamHparams(float(hp["lr"]), float(hp["beta1"]), float(hp["beta2"]), float(hp["eps"]),
                       float(hp.get("weight_decay", 0.0)), int(hp["step"]))


# ------------------------------------------------------------ host metadata
def zero_adam_scalars_compute(hp) -> dict:
    out = _lib.AdamScalars()
    check(load().zero_adam_scalars_compute(C.byref(hparams(hp)), C.byref(out)), "zero_adam_scalars_compute")
    return {name: np.float32(getattr(out, name)) for name, _ in _lib.AdamScalars._fields_}


def zero_rank_weights(counts: Optional[Sequence[int]], n_ranks: int) -> np.ndarray:
    if counts is not None and len(counts) != n_ranks:
        raise ValueError("zero_rank_weights: len(counts) != n_ranks")
    if n_ranks < 1:
        raise ValueError("zero_rank_weights: n_ranks must be at least 1")
    out = (C.c_float * n_ranks)()
    arr = None if counts is None else (C.c_int64 * n_ranks)(*[int(c) for c in counts])
    check(load().zero_rank_weights(arr, n_ranks, out), "zero_rank_weights")
    return np.array(list(out), dtype=np.float32)


def zero_shard_layout(numels: Sequence[int], n_shards: int):
    arr = (C.c_int64 * max(1, len(numels)))(*[int(n) for n in numels])
    psi, pad, s = C.c_int64(), C.c_int64(), C.c_int64()
    check(load().zero_shard_layout(arr, len(numels), n_shards, C.byref(psi), C.byref(pad), C.byref(s)),
          "zero_shard_layout")
    return psi.value, pad.value, s.value


# ------------------------------------------------------------ device calls
def zero_reduce_scatter(rank_grads: Sequence[torch.Tensor], rank_weights, shards_out: Sequence[torch.Tensor],
                        accumulate: bool = False, stream=None) -> None:
    """Owner k's shard = sum_r w_r * float(rank_grads[r][k*S:(k+1)*S]) (rank order),
    or shard += that sum when accumulate.  rank_grads: BF16 (zero_reduce_scatter)
    or FP32 (zero_reduce_scatter_f32) device tensors of equal numel; shards_out:
    FP32 device tensors of numel/len(shards_out) each."""
    _reduce_scatter(rank_grads, rank_weights, shards_out, accumulate, stream, f32=False)


def zero_reduce_scatter_f32(rank_grads, rank_weights, shards_out, accumulate: bool = False, stream=None) -> None:
    _reduce_scatter(rank_grads, rank_weights, shards_out, accumulate, stream, f32=True)


def _reduce_scatter(rank_grads, rank_weights, shards_out, accumulate, stream, f32):
    name = "zero_reduce_scatter_f32" if f32 else "zero_reduce_scatter"
    n_ranks, n_shards = len(rank_grads), len(shards_out)
    if n_ranks < 1 or n_shards < 1:
        raise ValueError(f"{name}: need at least one rank and one shard")
    numel = rank_grads[0].numel()
    gp = [_dev(g, f"rank_grads[{r}]", (torch.float32,) if f32 else _BF16_LIKE) for r, g in enumerate(rank_grads)]
    if any(g.numel() != numel for g in rank_grads):
        raise ValueError("zero_reduce_scatter: rank contributions differ in size")
    if numel % n_shards:
        raise ValueError("zero_reduce_scatter: numel not divisible by the number of shards")
    op = [_dev(s, f"shards_out[{k}]", (torch.float32,)) for k, s in enumerate(shards_out)]
    if any(s.numel() != numel // n_shards for s in shards_out):
        raise ValueError("zero_reduce_scatter: each shard must hold numel/n_shards elements")
    w = np.ascontiguousarray(np.asarray(rank_weights, dtype=np.float32))
    if w.size != n_ranks:
        raise ValueError("zero_reduce_scatter: one weight per rank")
    check(getattr(load(), name)(_ptrs(gp), w.ctypes.data_as(_lib.FP), n_ranks, numel, _ptrs(op),
                                n_shards, int(bool(accumulate)), _stream(stream)), name)


def zero_adam_shard_step(master: torch.Tensor, exp_avg: torch.Tensor, exp_avg_sq: torch.Tensor,
                         bf16_out: torch.Tensor, grad: torch.Tensor, hp, stream=None) -> None:
    """Fused Adam/AdamW owner update in place (master, m, v FP32; bf16_out written)."""
    n = master.numel()
    ptrs = [_dev(master, "master", (torch.float32,)), _dev(exp_avg, "exp_avg", (torch.float32,)),
            _dev(exp_avg_sq, "exp_avg_sq", (torch.float32,)), _dev(bf16_out, "bf16_out", _BF16_LIKE),
            _dev(grad, "grad", (torch.float32,))]
    if any(t.numel() != n for t in (exp_avg, exp_avg_sq, bf16_out, grad)):
        raise ValueError("zero_adam_shard_step: all buffers must have the same numel")
    h = hparams(hp)
    check(load().zero_adam_shard_step(*ptrs, n, C.byref(h), _stream(stream)), "zero_adam_shard_step")


def zero_adam_shard_step_scaled(master, exp_avg, exp_avg_sq, bf16_out, grad, grad_scale: torch.Tensor, hp,
                                stream=None) -> None:
    """zero_adam_shard_step on grad * grad_scale[0] (a one-element FP32 device
    tensor, e.g. the clip coefficient from zero_grad_norm_sq)."""
    n = master.numel()
    ptrs = [_dev(master, "master", (torch.float32,)), _dev(exp_avg, "exp_avg", (torch.float32,)),
            _dev(exp_avg_sq, "exp_avg_sq", (torch.float32,)), _dev(bf16_out, "bf16_out", _BF16_LIKE),
            _dev(grad, "grad", (torch.float32,)), _dev(grad_scale, "grad_scale", (torch.float32,))]
    if any(t.numel() != n for t in (exp_avg, exp_avg_sq, bf16_out, grad)) or grad_scale.numel() < 1:
        raise ValueError("zero_adam_shard_step_scaled: size mismatch")
    h = hparams(hp)
    check(load().zero_adam_shard_step_scaled(*ptrs, n, C.byref(h), _stream(stream)),
          "zero_adam_shard_step_scaled")


def _norm_args(name, shards, norm_sq_out, clip_coef_out):
    n = len(shards)
    if n < 1:
        raise ValueError(f"{name}: no shards")
    numel = shards[0].numel()
    sp = [_dev(t, f"shards[{k}]", (torch.float32,)) for k, t in enumerate(shards)]
    if any(t.numel() != numel for t in shards):
        raise ValueError(f"{name}: shards differ in size")
    op = _dev(norm_sq_out, "norm_sq_out", (torch.float64,))
    if norm_sq_out.numel() < 1:
        raise ValueError(f"{name}: norm_sq_out needs one element")
    cp = None
    if clip_coef_out is not None:
        cp = _dev(clip_coef_out, "clip_coef_out", (torch.float32,))
        if clip_coef_out.numel() < 1:
            raise ValueError(f"{name}: clip_coef_out needs one element")
    return _ptrs(sp), n, numel, op, cp


def zero_grad_norm_sq(shards: Sequence[torch.Tensor], workspace: torch.Tensor, norm_sq_out: torch.Tensor,
                      max_norm: float = 0.0, clip_coef_out: Optional[torch.Tensor] = None, stream=None) -> None:
    """norm_sq_out[0] (FP64 device tensor) = sum of squares of all shards
    (deterministic order); clip_coef_out[0] (FP32) = min(1, max_norm/(norm+1e-6))
    when given.  workspace: FP64 device tensor of >= len(shards)*1024 elements."""
    sp, n, numel, op, cp = _norm_args("zero_grad_norm_sq", shards, norm_sq_out, clip_coef_out)
    wp = _dev(workspace, "workspace", (torch.float64,))
    check(load().zero_grad_norm_sq(sp, n, numel, wp, workspace.numel(), op, float(max_norm), cp,
                                   _stream(stream)), "zero_grad_norm_sq")


def zero_grad_norm_sq_no_alloc(shards: Sequence[torch.Tensor], norm_sq_out: torch.Tensor, max_norm: float = 0.0,
                               clip_coef_out: Optional[torch.Tensor] = None, stream=None) -> None:
    """zero_grad_norm_sq with the partial sums in the library's own per-GPU
    array instead of a caller workspace: nothing is allocated.  Calls that
    overlap in time on one GPU race on that array."""
    sp, n, numel, op, cp = _norm_args("zero_grad_norm_sq_no_alloc", shards, norm_sq_out, clip_coef_out)
    check(load().zero_grad_norm_sq_no_alloc(sp, n, numel, op, float(max_norm), cp, _stream(stream)),
          "zero_grad_norm_sq_no_alloc")


def _fused_args(name, rank_grads, rank_weights, master, exp_avg, exp_avg_sq, bf16_out, grad_out, grad_acc):
    n_ranks, n_shards = len(rank_grads), len(master)
    if n_ranks < 1 or n_shards < 1:
        raise ValueError(f"{name}: need at least one rank and one owner")
    numel = rank_grads[0].numel()
    gp = [_dev(g, f"rank_grads[{r}]", _BF16_LIKE) for r, g in enumerate(rank_grads)]
    if any(g.numel() != numel for g in rank_grads):
        raise ValueError(f"{name}: rank contributions differ in size")
    if numel % n_shards:
        raise ValueError(f"{name}: numel not divisible by the number of owners")
    s = numel // n_shards
    tables = []
    for tname, ts, dt in (("master", master, (torch.float32,)), ("exp_avg", exp_avg, (torch.float32,)),
                          ("exp_avg_sq", exp_avg_sq, (torch.float32,)), ("bf16_out", bf16_out, _BF16_LIKE)):
        if len(ts) != n_shards or any(t.numel() != s for t in ts):
            raise ValueError(f"{name}: {tname} needs {n_shards} tensors of {s} elements")
        tables.append(_ptrs([_dev(t, f"{tname}[{k}]", dt) for k, t in enumerate(ts)]))
    go = None
    if grad_out is not None:
        if len(grad_out) != n_shards or any(t.numel() != s for t in grad_out):
            raise ValueError(f"{name}: grad_out needs one tensor per owner")
        go = _ptrs([_dev(t, f"grad_out[{k}]", (torch.float32,)) for k, t in enumerate(grad_out)])
    ga = None
    if grad_acc is not None:
        if len(grad_acc) != n_shards or any(t.numel() != s for t in grad_acc):
            raise ValueError(f"{name}: grad_acc needs one tensor per owner")
        ga = _ptrs([_dev(t, f"grad_acc[{k}]", (torch.float32,)) for k, t in enumerate(grad_acc)])
    w = np.ascontiguousarray(np.asarray(rank_weights, dtype=np.float32))
    if w.size != n_ranks:
        raise ValueError(f"{name}: one weight per rank")
    return (_ptrs(gp), w, n_ranks, numel, n_shards, tables, ga, go)


def zero_reduce_scatter_adam(rank_grads: Sequence[torch.Tensor], rank_weights, master, exp_avg, exp_avg_sq,
                             bf16_out, hp, grad_out=None, grad_acc=None, stream=None) -> None:
    """Fused reduce-scatter + owner Adam update: for each owner k, the reduced
    shard k of the rank contributions (plus grad_acc[k] when given) updates
    (master[k], exp_avg[k], exp_avg_sq[k]) and writes bf16_out[k]; grad_out
    (optional list) receives the gradient used.  Bit-identical to
    zero_reduce_scatter (accumulate mode with grad_acc) followed by
    zero_adam_shard_step on every owner."""
    gp, w, n_ranks, numel, n_shards, tables, ga, go = _fused_args(
        "zero_reduce_scatter_adam", rank_grads, rank_weights, master, exp_avg, exp_avg_sq, bf16_out, grad_out,
        grad_acc)
    h = hparams(hp)
    check(load().zero_reduce_scatter_adam(gp, w.ctypes.data_as(_lib.FP), n_ranks, numel, n_shards,
                                          *tables, ga, go, C.byref(h), _stream(stream)),
          "zero_reduce_scatter_adam")


# ------------------------------------------------------------ graph-capturable forms
ADAM_SCALARS_FLOATS = len(_lib.AdamScalars._fields_)


def adam_scalars_tensor(hp, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The step's scalars (zero_adam_scalars_compute) as a float32 tensor in the
    struct's field order, ready to be copied into the device struct that the
    _dev calls read.  out: an existing CPU float32 tensor to fill (e.g. pinned)."""
    sc = _lib.AdamScalars()
    check(load().zero_adam_scalars_compute(C.byref(hparams(hp)), C.byref(sc)), "zero_adam_scalars_compute")
    vals = [getattr(sc, f) for f, _ in _lib.AdamScalars._fields_]
    if out is None:
        return torch.tensor(vals, dtype=torch.float32)
    if out.device.type != "cpu" or out.dtype != torch.float32 or out.numel() < ADAM_SCALARS_FLOATS:
        raise ValueError(f"adam_scalars_tensor: out must be a CPU float32 tensor of >= {ADAM_SCALARS_FLOATS} elements")
    out.numpy()[:ADAM_SCALARS_FLOATS] = np.array(vals, dtype=np.float32)
    return out


def _scalars_dev(scalars_dev: torch.Tensor) -> int:
    ptr = _dev(scalars_dev, "scalars_dev", (torch.float32,))
    if scalars_dev.numel() < ADAM_SCALARS_FLOATS:
        raise ValueError(f"scalars_dev: needs {ADAM_SCALARS_FLOATS} float32 elements")
    return ptr


def zero_adam_shard_step_dev(master, exp_avg, exp_avg_sq, bf16_out, grad, scalars_dev: torch.Tensor,
                             grad_scale: Optional[torch.Tensor] = None, stream=None) -> None:
    """zero_adam_shard_step with the step's scalars read from scalars_dev (a
    device float32 tensor holding adam_scalars_tensor(hp)) when the kernel runs,
    so that a captured graph replays with new scalars; grad_scale as in
    zero_adam_shard_step_scaled, or None."""
    n = master.numel()
    ptrs = [_dev(master, "master", (torch.float32,)), _dev(exp_avg, "exp_avg", (torch.float32,)),
            _dev(exp_avg_sq, "exp_avg_sq", (torch.float32,)), _dev(bf16_out, "bf16_out", _BF16_LIKE),
            _dev(grad, "grad", (torch.float32,))]
    if any(t.numel() != n for t in (exp_avg, exp_avg_sq, bf16_out, grad)):
        raise ValueError("zero_adam_shard_step_dev: all buffers must have the same numel")
    gs = None
    if grad_scale is not None:
        gs = _dev(grad_scale, "grad_scale", (torch.float32,))
    check(load().zero_adam_shard_step_dev(*ptrs, gs, n, _scalars_dev(scalars_dev), _stream(stream)),
          "zero_adam_shard_step_dev")


def zero_reduce_scatter_adam_dev(rank_grads, rank_weights, master, exp_avg, exp_avg_sq, bf16_out,
                                 scalars_dev: torch.Tensor, grad_out=None, grad_acc=None, stream=None) -> None:
    """zero_reduce_scatter_adam with the step's scalars read from scalars_dev
    when the kernels run (see zero_adam_shard_step_dev)."""
    gp, w, n_ranks, numel, n_shards, tables, ga, go = _fused_args(
        "zero_reduce_scatter_adam_dev", rank_grads, rank_weights, master, exp_avg, exp_avg_sq, bf16_out,
        grad_out, grad_acc)
    check(load().zero_reduce_scatter_adam_dev(gp, w.ctypes.data_as(_lib.FP), n_ranks, numel, n_shards,
                                              *tables, ga, go, _scalars_dev(scalars_dev), _stream(stream)),
          "zero_reduce_scatter_adam_dev")


def zero_adam_scalars_fetch(ring_host: torch.Tensor, cursor_dev: torch.Tensor, scalars_dev: torch.Tensor,
                            stream=None) -> None:
    """One kernel on the stream: scalars_dev <- slot (cursor mod ring length)
    of ring_host, then cursor + 1.  ring_host: a pinned CPU float32 tensor of
    ring_len * ADAM_SCALARS_FLOATS elements (ring_len a power of two), one
    adam_scalars_tensor per slot; cursor_dev: a one-element int32 device tensor,
    zero before the first replay; scalars_dev: as for the _dev calls."""
    if ring_host.device.type != "cpu" or ring_host.dtype != torch.float32 or not ring_host.is_contiguous():
        raise ValueError("zero_adam_scalars_fetch: ring_host must be a contiguous CPU float32 tensor")
    if not ring_host.is_pinned():
        raise ValueError("zero_adam_scalars_fetch: ring_host must be pinned (pin_memory=True)")
    if ring_host.numel() == 0 or ring_host.numel() % ADAM_SCALARS_FLOATS:
        raise ValueError(f"zero_adam_scalars_fetch: ring_host must hold a multiple of {ADAM_SCALARS_FLOATS} floats")
    cur = _dev(cursor_dev, "cursor_dev", (torch.int32,))
    if cursor_dev.numel() != 1:
        raise ValueError("zero_adam_scalars_fetch: cursor_dev must have one element")
    check(load().zero_adam_scalars_fetch(ring_host.data_ptr(), ring_host.numel() // ADAM_SCALARS_FLOATS, cur,
                                         _scalars_dev(scalars_dev), _stream(stream)), "zero_adam_scalars_fetch")


def zero_all_gather_layer(shards: Sequence[torch.Tensor], full_view: torch.Tensor, stream=None) -> None:
    """full_view = concatenation of the shards' bytes in owner order."""
    n = len(shards)
    if n < 1:
        raise ValueError("zero_all_gather_layer: no shards")
    nbytes = shards[0].numel() * shards[0].element_size()
    sp = [_dev(s, f"shards[{k}]", (s.dtype,)) for k, s in enumerate(shards)]
    if any(s.numel() * s.element_size() != nbytes for s in shards):
        raise ValueError("zero_all_gather_layer: shards differ in size")
    vp = _dev(full_view, "full_view", (full_view.dtype,))
    if full_view.numel() * full_view.element_size() != n * nbytes:
        raise ValueError("zero_all_gather_layer: full_view must hold exactly n_shards*shard_bytes bytes")
    check(load().zero_all_gather_layer(_ptrs(sp), n, nbytes, vp, _stream(stream)), "zero_all_gather_layer")


def zero_last_path_vectorized() -> int:
    return int(load().zero_last_path_vectorized())


# ------------------------------------------------------------ offload engine
class ZeroOffload:
    """Two-slot host-offloaded gradient shard (zero_offload_* in include/zero.h).

    host_shard: pinned FP32 CPU tensor [shard_numel]; slot_contrib: two BF16
    device tensors [n_ranks*chunk_numel]; slot_f32: two FP32 device tensors
    [chunk_numel].  The tensors must outlive the handle."""

    def __init__(self, n_ranks: int, shard_numel: int, chunk_numel: int, host_shard: torch.Tensor,
                 slot_contrib: Sequence[torch.Tensor], slot_f32: Sequence[torch.Tensor]):
        if host_shard.device.type != "cpu" or host_shard.dtype != torch.float32 or not host_shard.is_contiguous():
            raise ValueError("host_shard: contiguous float32 CPU tensor required")
        if not host_shard.is_pinned():
            raise ValueError("host_shard: must be pinned host memory")
        if host_shard.numel() != shard_numel:
            raise ValueError("host_shard: numel != shard_numel")
        if len(slot_contrib) != 2 or len(slot_f32) != 2:
            raise ValueError("two slots required")
        cp = [_dev(t, f"slot_contrib[{s}]", _BF16_LIKE) for s, t in enumerate(slot_contrib)]
        fp = [_dev(t, f"slot_f32[{s}]", (torch.float32,)) for s, t in enumerate(slot_f32)]
        if any(t.numel() != n_ranks * chunk_numel for t in slot_contrib):
            raise ValueError("slot_contrib: numel must be n_ranks*chunk_numel")
        if any(t.numel() != chunk_numel for t in slot_f32):
            raise ValueError("slot_f32: numel must be chunk_numel")
        self._keep = (host_shard, tuple(slot_contrib), tuple(slot_f32))
        self.n_ranks, self.shard_numel, self.chunk_numel = n_ranks, shard_numel, chunk_numel
        self.n_chunks = -(-shard_numel // chunk_numel)
        h = C.c_void_p()
        check(load().zero_offload_create(n_ranks, shard_numel, chunk_numel, host_shard.data_ptr(),
                                         _ptrs(cp), _ptrs(fp), C.byref(h)), "zero_offload_create")
        self._h = h

    def chunk_len(self, c: int) -> int:
        return min(self.chunk_numel, self.shard_numel - c * self.chunk_numel)

    def reduce(self, chunk: int, micro_batch: int, rank_weights, stream=None) -> None:
        w = np.ascontiguousarray(np.asarray(rank_weights, dtype=np.float32))
        if w.size != self.n_ranks:
            raise ValueError("one weight per rank")
        check(load().zero_offload_stream(self._h, _lib.ZERO_OFFLOAD_REDUCE, chunk, micro_batch,
                                         w.ctypes.data_as(_lib.FP), None, None, None, None, None,
                                         _stream(stream)), "zero_offload_stream(REDUCE)")

    def adam(self, chunk: int, master, exp_avg, exp_avg_sq, bf16_out, hp, stream=None) -> None:
        ptrs = [_dev(master, "master", (torch.float32,)), _dev(exp_avg, "exp_avg", (torch.float32,)),
                _dev(exp_avg_sq, "exp_avg_sq", (torch.float32,)), _dev(bf16_out, "bf16_out", _BF16_LIKE)]
        if any(t.numel() != self.shard_numel for t in (master, exp_avg, exp_avg_sq, bf16_out)):
            raise ValueError("state tensors must cover the whole shard")
        h = hparams(hp)
        check(load().zero_offload_stream(self._h, _lib.ZERO_OFFLOAD_ADAM, chunk, 0, None, *ptrs,
                                         C.byref(h), _stream(stream)), "zero_offload_stream(ADAM)")

    def reduce_adam(self, chunk: int, micro_batch: int, rank_weights, master, exp_avg, exp_avg_sq, bf16_out, hp,
                    stream=None) -> None:
        """The last micro-batch of `chunk`: reduce, add to the host accumulation
        and update in one pass (no copy back to the host)."""
        w = np.ascontiguousarray(np.asarray(rank_weights, dtype=np.float32))
        if w.size != self.n_ranks:
            raise ValueError("one weight per rank")
        ptrs = [_dev(master, "master", (torch.float32,)), _dev(exp_avg, "exp_avg", (torch.float32,)),
                _dev(exp_avg_sq, "exp_avg_sq", (torch.float32,)), _dev(bf16_out, "bf16_out", _BF16_LIKE)]
        if any(t.numel() != self.shard_numel for t in (master, exp_avg, exp_avg_sq, bf16_out)):
            raise ValueError("state tensors must cover the whole shard")
        h = hparams(hp)
        check(load().zero_offload_stream(self._h, _lib.ZERO_OFFLOAD_REDUCE_ADAM, chunk, micro_batch,
                                         w.ctypes.data_as(_lib.FP), *ptrs, C.byref(h), _stream(stream)),
              "zero_offload_stream(REDUCE_ADAM)")

    def sync(self) -> None:
        check(load().zero_offload_sync(self._h), "zero_offload_sync")

    def close(self) -> None:
        if getattr(self, "_h", None):
            st = load().zero_offload_destroy(self._h)
            self._h = None
            check(st, "zero_offload_destroy")

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def zero_offload_create(n_ranks, shard_numel, chunk_numel, host_shard, slot_contrib, slot_f32) -> ZeroOffload:
    return ZeroOffload(n_ranks, shard_numel, chunk_numel, host_shard, slot_contrib, slot_f32)


def zero_offload_stream(h: ZeroOffload, op: int, chunk: int, micro_batch: int = 0, rank_weights=None,
                        master=None, exp_avg=None, exp_avg_sq=None, bf16_out=None, hp=None, stream=None):
    if op == _lib.ZERO_OFFLOAD_REDUCE:
        return h.reduce(chunk, micro_batch, rank_weights, stream)
    if op == _lib.ZERO_OFFLOAD_REDUCE_ADAM:
        return h.reduce_adam(chunk, micro_batch, rank_weights, master, exp_avg, exp_avg_sq, bf16_out, hp, stream)
    return h.adam(chunk, master, exp_avg, exp_avg_sq, bf16_out, hp, stream)


def zero_offload_sync(h: ZeroOffload) -> None:
    h.sync()


def zero_offload_destroy(h: ZeroOffload) -> None:
    h.close()
