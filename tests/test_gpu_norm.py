"""GPU parity of the optional global gradient norm and clipping:
zero_grad_norm_sq against the oracle's float64 sum of squares (relative
tolerance: the summation orders differ), bitwise repeatability, and, on
gradients whose sums of squares are exact in FP64, the norm and the clip
coefficient bit-identical to the oracle's and the clipped update
(zero_adam_shard_step_scaled) against the oracle's Adam on the gradient scaled
by the oracle's own coefficient."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from gpu_helpers import assert_state_close, bf16_to_host, f32_to_dev, f32_to_host

pytestmark = pytest.mark.gpu

import zero_sharded_optimizer_reduce_amd as z  # noqa: E402  (a broken package must fail, not skip)

NORM_RTOL = 1e-12      # FP64 sums of up to 2^28 exact squares: error << 1e-12 relative


def _ws(n_shards):
    return torch.empty(n_shards * 1024, dtype=torch.float64, device="cuda")


@pytest.mark.parametrize("n_shards", [1, 3, 4, 16])
@pytest.mark.parametrize("numel", [0, 1, 3, 4, 1000, 4096 * 257 + 5, (1 << 22) + 4])
def test_norm_matches_oracle_and_repeats(n_shards, numel):
    rng = np.random.default_rng(numel + n_shards)
    host = [S.normal_f32(rng, numel, 1e-3) for _ in range(n_shards)]
    dev = [f32_to_dev(x) for x in host]
    out = torch.empty(1, dtype=torch.float64, device="cuda")
    z.zero_grad_norm_sq(dev, _ws(n_shards), out)
    got = float(out.item())
    ref = oracle.grad_norm_sq(host)
    assert abs(got - ref) <= NORM_RTOL * ref, (got, ref)
    for _ in range(2):
        again = torch.empty(1, dtype=torch.float64, device="cuda")
        z.zero_grad_norm_sq(dev, _ws(n_shards), again)
        assert again.view(torch.int64).item() == out.view(torch.int64).item()


def test_norm_element_path_and_special_values():
    rng = np.random.default_rng(5)
    x = S.normal_f32(rng, 10001, 1.0)
    x[17] = 3e38                      # square overflows float32 but not float64
    x[18] = 1e-42                     # subnormal
    dev = f32_to_dev(np.concatenate([[0.0], x]).astype(np.float32))[1:]   # 4-byte, not 16-byte aligned
    out = torch.empty(1, dtype=torch.float64, device="cuda")
    z.zero_grad_norm_sq([dev], _ws(1), out)
    assert z.zero_last_path_vectorized() == 0
    ref = oracle.grad_norm_sq([x])
    assert abs(out.item() - ref) <= NORM_RTOL * ref
    x[20] = np.nan
    z.zero_grad_norm_sq([f32_to_dev(x)], _ws(1), out)
    assert np.isnan(out.item())


@pytest.mark.parametrize("max_norm", [1e-3, 0.05, 10.0])
def test_clipped_update(max_norm):
    # gradients on a grid (integers below 2^8 times 2^-18): every square and
    # every partial sum of squares is exact in FP64, so the norm is the same
    # in any summation order and both sides derive the same clip coefficient
    # from their own norm
    rng = np.random.default_rng(31)
    n_shards, S_ = 4, 8192 + 4
    g = [(rng.integers(-255, 256, S_).astype(np.float64) * 2.0 ** -18).astype(np.float32) for _ in range(n_shards)]
    p, m, v = S.host_state(32, S_, 0.02, 1e-4, 1e-6)
    out = torch.empty(1, dtype=torch.float64, device="cuda")
    coef = torch.empty(1, dtype=torch.float32, device="cuda")
    gd = [f32_to_dev(x) for x in g]
    z.zero_grad_norm_sq(gd, _ws(n_shards), out, max_norm=max_norm, clip_coef_out=coef)
    ref_nsq = oracle.grad_norm_sq(g)
    assert out.item() == ref_nsq                # exact sums: bit-identical norms
    c_ref = oracle.clip_coefficient(ref_nsq, max_norm)
    assert np.float32(coef.item()) == c_ref
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1, step=50)
    sc = oracle.adam_scalars(1e-3, 0.9, 0.999, 1e-8, 0.1, 50)
    for k in range(n_shards):
        P, M, V = f32_to_dev(p), f32_to_dev(m), f32_to_dev(v)
        B = torch.empty(S_, dtype=torch.bfloat16, device="cuda")
        z.zero_adam_shard_step_scaled(P, M, V, B, gd[k], coef, hp)
        ref = oracle.adam_step(p, m, v, oracle.scale_grad(g[k], c_ref), sc)
        assert_state_close(f32_to_host(P), f32_to_host(M), f32_to_host(V), bf16_to_host(B), ref, f"shard {k}")


def test_norm_validation():
    x = [torch.zeros(16, device="cuda")]
    out = torch.empty(1, dtype=torch.float64, device="cuda")
    with pytest.raises(z.ZeroError):           # workspace too small
        z.zero_grad_norm_sq(x, torch.empty(10, dtype=torch.float64, device="cuda"), out)
    with pytest.raises(z.ZeroError):           # clip requested without a positive max_norm
        z.zero_grad_norm_sq(x, _ws(1), out, max_norm=0.0, clip_coef_out=torch.empty(1, device="cuda"))


def test_scaled_update_rejects_a_scale_inside_its_outputs():
    n = 1024
    p, m, v, g = (torch.zeros(n, device="cuda") for _ in range(4))
    b = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, step=1)
    with pytest.raises(z.ZeroError, match="ZERO_ERR_ARG"):
        z.zero_adam_shard_step_scaled(p, m, v, b, g, p[5:6], hp)      # the scale is a master element
    with pytest.raises(z.ZeroError, match="ZERO_ERR_ARG"):
        z.zero_adam_shard_step_scaled(p, m, v, b, g, v[-1:], hp)
    torch.cuda.synchronize()
    assert torch.count_nonzero(p) == 0 and torch.count_nonzero(m) == 0   # nothing was launched
    z.zero_adam_shard_step_scaled(p, m, v, b, g, g[:1], hp)             # inside the read-only gradient: fine
    torch.cuda.synchronize()
