"""The workspace-free gradient norm, zero_grad_norm_sq_no_alloc, against the
workspace form zero_grad_norm_sq, both through the C ABI: three calls in a
row on the library's one per-GPU partial-sum array, the second smaller than
the first (fewer shards, fewer partial sums, the element-wise path), so that
a partial sum left over from an earlier call would show.  The norm and the
clip coefficient must be the same bits as the workspace form's, and the
norm within the FP64 summation bound of the oracle's."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from gpu_helpers import f32_to_dev

pytestmark = pytest.mark.gpu

import zero_sharded_optimizer_reduce_amd as z  # noqa: E402
from zero_sharded_optimizer_reduce_amd import _lib  # noqa: E402

NORM_RTOL = 1e-12


def _both(shards, max_norm):
    n = len(shards)
    # the workspace form, its workspace poisoned so that an unwritten partial sum would show
    ws = torch.full((n * _lib.ZERO_NORM_BLOCKS,), float("nan"), dtype=torch.float64, device="cuda")
    out = [torch.full((1,), float("nan"), dtype=torch.float64, device="cuda") for _ in range(2)]
    coef = [torch.full((1,), float("nan"), dtype=torch.float32, device="cuda") for _ in range(2)]
    z.zero_grad_norm_sq(shards, ws, out[0], max_norm=max_norm, clip_coef_out=coef[0])
    z.zero_grad_norm_sq_no_alloc(shards, out[1], max_norm=max_norm, clip_coef_out=coef[1])
    torch.cuda.synchronize()
    nsq = [o.cpu().numpy() for o in out]
    c = [x.cpu().numpy() for x in coef]
    return nsq, c


@pytest.mark.parametrize("cases", [
    # (n_shards, shard_numel, sigma, max_norm): large, then smaller, then large again
    [(4, 3 * (1 << 20) + 12, 1e-3, 1.0), (2, 1001, 5e-2, 1.0), (3, 1 << 18, 1.0, 0.5)],
])
def test_no_alloc_norm_equals_workspace_form_on_consecutive_calls(cases):
    for i, (n, numel, sigma, max_norm) in enumerate(cases):
        print(f"no-alloc norm call {i}: n_shards={n} shard_numel={numel} sigma={sigma}", flush=True)
        host = [S.normal_f32(S.rng(700 + 10 * i + k), numel, sigma) for k in range(n)]
        shards = [f32_to_dev(h) for h in host]
        (a, b), (ca, cb) = _both(shards, max_norm)
        assert a.view(np.uint64)[0] == b.view(np.uint64)[0], (i, a[0], b[0])
        assert ca.view(np.uint32)[0] == cb.view(np.uint32)[0], (i, ca[0], cb[0])
        ref = oracle.grad_norm_sq(host)
        assert abs(float(b[0]) - ref) <= NORM_RTOL * ref, (i, float(b[0]), ref)
        assert np.float32(cb[0]) == oracle.clip_coefficient(ref, max_norm), (i, cb[0])


def test_no_alloc_norm_without_clip_output_and_empty_shards():
    host = [S.normal_f32(S.rng(801 + k), 4096, 1e-2) for k in range(2)]
    out = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    z.zero_grad_norm_sq_no_alloc([f32_to_dev(h) for h in host], out)
    empty = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    z.zero_grad_norm_sq_no_alloc([torch.empty(0, device="cuda")], empty)
    torch.cuda.synchronize()
    ref = oracle.grad_norm_sq(host)
    assert abs(out.item() - ref) <= NORM_RTOL * ref
    assert empty.item() == 0.0


def test_no_alloc_norm_rejects_bad_arguments_without_launching():
    out = torch.full((1,), 7.0, dtype=torch.float64, device="cuda")
    x = torch.ones(1024, device="cuda")
    with pytest.raises(z.ZeroError, match="ZERO_ERR_ARG"):
        z.zero_grad_norm_sq_no_alloc([x] * (_lib.ZERO_MAX_RANKS + 1), out)
    with pytest.raises(z.ZeroError, match="ZERO_ERR_ARG"):
        z.zero_grad_norm_sq_no_alloc([x], out, max_norm=0.0,
                                     clip_coef_out=torch.empty(1, device="cuda"))
    torch.cuda.synchronize()
    assert out.item() == 7.0
