"""ZeRO sharded update for MI355X: reduce-scatter, fused mixed-precision Adam
owner update, all-gather, and a two-slot host-offloaded gradient shard.

The work runs in libzero.so (HIP kernels for gfx950 behind a C ABI, declared
in include/zero.h); this package is its Python binding and the step drivers
that sequence its calls.
"""
from ._lib import ZERO_OFFLOAD_ADAM, ZERO_OFFLOAD_REDUCE, ZERO_OFFLOAD_REDUCE_ADAM, ZeroError, load  # noqa: F401
from .api import (  # noqa: F401
    ADAM_SCALARS_FLOATS,
    ZeroOffload,
    adam_scalars_tensor,
    zero_adam_scalars_compute,
    zero_adam_scalars_fetch,
    zero_adam_shard_step,
    zero_adam_shard_step_dev,
    zero_adam_shard_step_scaled,
    zero_all_gather_layer,
    zero_grad_norm_sq,
    zero_grad_norm_sq_no_alloc,
    zero_last_path_vectorized,
    zero_offload_create,
    zero_offload_destroy,
    zero_offload_stream,
    zero_offload_sync,
    zero_rank_weights,
    zero_reduce_scatter,
    zero_reduce_scatter_adam,
    zero_reduce_scatter_adam_dev,
    zero_reduce_scatter_f32,
    zero_shard_layout,
)
