"""Every kernel writes its outputs and nothing else.  Each output is a view
inside a larger buffer whose other elements hold a sentinel bit pattern; after
the call the sentinels must be intact and the outputs must match the oracle.
The sizes put the last tile of each launch at every position relative to the
workgroup sizes (64 and 128 lanes, 4 elements per lane): 1, 63, 64, 65, 127,
128, 129 and 1000 vectors per owner.  A 16-byte aligned margin keeps the
vector kernels in use; a 4-byte margin sends the same calls down the
element-wise path."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from gpu_helpers import (assert_grad_exact, assert_state_close, bf16_to_dev, bf16_to_host, f32_to_dev,
                         f32_to_host)

pytestmark = pytest.mark.gpu

import zero_sharded_optimizer_reduce_amd as z  # noqa: E402  (a broken package must fail, not skip)

SENTINEL = {torch.float32: 0x7FBADBAD, torch.bfloat16: 0x7FBD, torch.uint8: 0xA5}   # NaN payloads / a byte
INT_VIEW = {torch.float32: torch.int32, torch.bfloat16: torch.int16, torch.uint8: torch.uint8}
VECS = [1, 63, 64, 65, 127, 128, 129, 1000]


class Guarded:
    """A view of n elements at element offset `margin` of a buffer with
    `margin` sentinel elements on each side."""

    def __init__(self, n, dtype, margin, init=None):
        self.n, self.dtype, self.margin = n, dtype, margin
        self.whole = torch.empty(n + 2 * margin, dtype=dtype, device="cuda")
        self.whole.view(INT_VIEW[dtype]).fill_(SENTINEL[dtype])   # each fits its signed view
        self.view = self.whole[margin:margin + n]
        if init is not None:
            self.view.copy_(init)

    def assert_margins(self, what):
        bits = self.whole.view(INT_VIEW[self.dtype]).cpu().numpy()
        expect = np.array(SENTINEL[self.dtype]).astype(bits.dtype)
        left, right = bits[:self.margin], bits[self.margin + self.n:]
        for side, part in (("before", left), ("after", right)):
            bad = np.nonzero(part != expect)[0]
            assert bad.size == 0, f"{what}: {bad.size} sentinels overwritten {side} the output (first at {bad[0]})"


def _margin(aligned, dtype):
    # 16 bytes (vector path) or 4 bytes (not 16-byte aligned: element path)
    return 16 // torch.tensor([], dtype=dtype).element_size() if aligned else \
        max(1, 4 // torch.tensor([], dtype=dtype).element_size())


def _hp(wd):
    return dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=wd, step=4)


@pytest.mark.parametrize("vecs", VECS)
@pytest.mark.parametrize("aligned", [True, False])
@pytest.mark.parametrize("accumulate", [False, True])
def test_reduce_scatter_writes_only_its_shards(vecs, aligned, accumulate):
    n_ranks = n_shards = 4
    per = 4 * vecs
    numel = per * n_shards
    print(f"reduce bounds per_shard={per} aligned={aligned} accumulate={accumulate}", flush=True)
    grads = S.host_rank_grads(3100 + vecs, n_ranks, numel, scales=np.linspace(0.5, 2, n_ranks))
    w = oracle.weights_from_counts([4096, 3072, 4096, 2048])
    rng = np.random.default_rng(vecs)
    init = [S.normal_f32(rng, per, 1e-3) for _ in range(n_shards)]
    m = _margin(aligned, torch.float32)
    outs = [Guarded(per, torch.float32, m, f32_to_dev(init[k]) if accumulate else None) for k in range(n_shards)]
    z.zero_reduce_scatter([bf16_to_dev(g) for g in grads], w, [o.view for o in outs], accumulate=accumulate)
    assert z.zero_last_path_vectorized() == int(aligned)
    torch.cuda.synchronize()
    for k, o in enumerate(outs):
        o.assert_margins(f"shard {k}")
        red = oracle.reduce_owner_shard(grads, w, n_shards, k)
        assert_grad_exact(f32_to_host(o.view), init[k] + red if accumulate else red, f"shard {k}")


@pytest.mark.parametrize("vecs", [1, 63, 65, 1000])
@pytest.mark.parametrize("aligned", [True, False])
@pytest.mark.parametrize("accumulate", [False, True])
def test_reduce_scatter_f32_writes_only_its_shards(vecs, aligned, accumulate):
    n_ranks = n_shards = 4
    per = 4 * vecs
    rng = np.random.default_rng(3200 + vecs)
    grads = [S.normal_f32(rng, per * n_shards, 1e-3) for _ in range(n_ranks)]
    w = oracle.weights_from_counts([4096, 3072, 4096, 2048])
    init = [S.normal_f32(rng, per, 1e-3) for _ in range(n_shards)]
    m = _margin(aligned, torch.float32)
    outs = [Guarded(per, torch.float32, m, f32_to_dev(init[k]) if accumulate else None) for k in range(n_shards)]
    print(f"reduce f32 bounds per_shard={per} aligned={aligned} accumulate={accumulate}", flush=True)
    z.zero_reduce_scatter_f32([f32_to_dev(g) for g in grads], w, [o.view for o in outs], accumulate=accumulate)
    assert z.zero_last_path_vectorized() == int(aligned)
    torch.cuda.synchronize()
    for k, o in enumerate(outs):
        o.assert_margins(f"shard {k}")
        red = oracle.reduce_owner_shard(grads, w, n_shards, k)
        assert_grad_exact(f32_to_host(o.view), init[k] + red if accumulate else red, f"shard {k}")


@pytest.mark.parametrize("n", [4 * v for v in VECS] + [4 * 65 + 3, 4 * 1000 + 1])
@pytest.mark.parametrize("aligned", [True, False])
@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_update_writes_only_its_state(n, aligned, wd):
    rng = np.random.default_rng(3300 + n)
    p0, m0, v0, g = (S.normal_f32(rng, n, 0.02), S.normal_f32(rng, n, 1e-4),
                     np.abs(S.normal_f32(rng, n, 1e-6)), S.normal_f32(rng, n, 1e-3))
    mf, mb = _margin(aligned, torch.float32), _margin(aligned, torch.bfloat16)
    P, M, V = (Guarded(n, torch.float32, mf, f32_to_dev(x)) for x in (p0, m0, v0))
    B = Guarded(n, torch.bfloat16, mb)
    hp = _hp(wd)
    print(f"update bounds n={n} aligned={aligned} wd={wd}", flush=True)
    z.zero_adam_shard_step(P.view, M.view, V.view, B.view, f32_to_dev(g), hp)
    assert z.zero_last_path_vectorized() == int(aligned)
    torch.cuda.synchronize()
    for name, t in (("master", P), ("exp_avg", M), ("exp_avg_sq", V), ("bf16", B)):
        t.assert_margins(name)
    sc = oracle.adam_scalars(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], hp["step"])
    ref = oracle.adam_step(p0, m0, v0, g, sc)
    assert_state_close(f32_to_host(P.view), f32_to_host(M.view), f32_to_host(V.view), bf16_to_host(B.view), ref,
                       f"n={n}")


@pytest.mark.parametrize("vecs", VECS)
@pytest.mark.parametrize("with_grad", [False, True])
@pytest.mark.parametrize("with_acc", [False, True])
@pytest.mark.parametrize("aligned", [True, False])
def test_fused_writes_only_its_outputs(vecs, with_grad, with_acc, aligned):
    n = 4
    per = 4 * vecs
    grads = S.host_rank_grads(3400 + vecs, n, n * per, scales=np.linspace(0.5, 2, n))
    w = oracle.weights_from_counts([4096, 3072, 4096, 2048])
    rng = np.random.default_rng(3500 + vecs)
    st = [(S.normal_f32(rng, per, 0.02), S.normal_f32(rng, per, 1e-4), np.abs(S.normal_f32(rng, per, 1e-6)))
          for _ in range(n)]
    acc = [S.normal_f32(rng, per, 1e-3) for _ in range(n)]
    mf, mb = _margin(aligned, torch.float32), _margin(aligned, torch.bfloat16)
    P = [Guarded(per, torch.float32, mf, f32_to_dev(s[0])) for s in st]
    M = [Guarded(per, torch.float32, mf, f32_to_dev(s[1])) for s in st]
    V = [Guarded(per, torch.float32, mf, f32_to_dev(s[2])) for s in st]
    B = [Guarded(per, torch.bfloat16, mb) for _ in range(n)]
    G = [Guarded(per, torch.float32, mf) for _ in range(n)] if with_grad else None
    hp = _hp(0.1)
    print(f"fused bounds per_shard={per} grad_out={with_grad} grad_acc={with_acc} aligned={aligned}", flush=True)
    z.zero_reduce_scatter_adam([bf16_to_dev(g) for g in grads], w, [t.view for t in P], [t.view for t in M],
                               [t.view for t in V], [t.view for t in B], hp,
                               grad_out=[t.view for t in G] if with_grad else None,
                               grad_acc=[f32_to_dev(a) for a in acc] if with_acc else None)
    assert z.zero_last_path_vectorized() == int(aligned)
    torch.cuda.synchronize()
    sc = oracle.adam_scalars(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], hp["step"])
    for k in range(n):
        for name, t in (("master", P[k]), ("exp_avg", M[k]), ("exp_avg_sq", V[k]), ("bf16", B[k])) + \
                ((("grad", G[k]),) if with_grad else ()):
            t.assert_margins(f"{name}[{k}]")
        red = oracle.reduce_owner_shard(grads, w, n, k)
        if with_acc:
            red = (acc[k] + red).astype(np.float32)
        if with_grad:
            assert_grad_exact(f32_to_host(G[k].view), red, f"grad[{k}]")
        ref = oracle.adam_step(*st[k], red, sc)
        assert_state_close(f32_to_host(P[k].view), f32_to_host(M[k].view), f32_to_host(V[k].view),
                           bf16_to_host(B[k].view), ref, f"owner {k}")


@pytest.mark.parametrize("shard_bytes,aligned", [(16, True), (63 * 16, True), (64 * 16, True), (65 * 16, True),
                                                 (1000 * 16, True), (65 * 16 + 4, True), (1001, True),
                                                 (65 * 16, False)])
def test_all_gather_writes_only_the_view(shard_bytes, aligned):
    n_shards = 4
    rng = np.random.default_rng(shard_bytes)
    shards = [torch.from_numpy(rng.integers(0, 256, shard_bytes, dtype=np.uint8)).cuda() for _ in range(n_shards)]
    view = Guarded(n_shards * shard_bytes, torch.uint8, 16 if aligned else 4)
    print(f"all-gather bounds shard_bytes={shard_bytes} aligned={aligned}", flush=True)
    z.zero_all_gather_layer(shards, view.view)
    torch.cuda.synchronize()
    view.assert_margins("view")
    exp = np.concatenate([s.cpu().numpy() for s in shards])
    assert np.array_equal(view.view.cpu().numpy(), exp)
