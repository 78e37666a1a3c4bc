"""The five synthetic workloads: sizes, hyper-parameters and input recipes.

Shapes follow the pages' 7B/8B teaching ledgers (essay, section 从持久状态开始
记账; blog, section 每个参数 16 字节): a 7B-class transformer layer and an
8B Llama-like model.  No dataset is involved; every value is drawn from a
seeded generator.
"""
from __future__ import annotations

from dataclasses import dataclass, field

N_RANKS = 4
SHARD_ALIGN = 256
BUCKET = 1 << 26           # 64M-parameter buckets and offload chunks


def layer_7b_tensors():
    """One 7B-class transformer layer, d=4096, ffn=11008, no bias."""
    d, f = 4096, 11008
    return [("q", d * d), ("k", d * d), ("v", d * d), ("o", d * d),
            ("gate", d * f), ("up", d * f), ("down", f * d)]


def llama8b_units():
    """Units of the 8B Llama-like model in forward order: embedding, 32 layers
    (d=4096, ffn=14336, GQA kv_dim=1024), lm_head (vocab 128256).  Only the
    listed matrices; norms are not modelled."""
    d, f, kv, vocab = 4096, 14336, 1024, 128256
    layer = [("q", d * d), ("k", d * kv), ("v", d * kv), ("o", d * d),
             ("gate", d * f), ("up", d * f), ("down", f * d)]
    units = [("embedding", [("embedding", vocab * d)])]
    units += [(f"layer{i}", layer) for i in range(32)]
    units += [("lm_head", [("lm_head", vocab * d)])]
    return units


def unit_numels(tensors) -> list:
    return [n for _, n in tensors]


@dataclass
class Workload:
    name: str
    description: str
    psi: int                      # real parameters updated per step
    n_ranks: int = N_RANKS
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    grad_sigma: float = 1e-3
    master_sigma: float = 0.02
    m_sigma: float = 0.0
    v_sigma: float = 0.0
    step0: int = 1                # Adam step count t of the first update
    seed: int = 0
    extra: dict = field(default_factory=dict)

    def hparams(self, step: int):
        return dict(lr=self.lr, beta1=self.beta1, beta2=self.beta2, eps=self.eps,
                    weight_decay=self.weight_decay, step=step)


TINY = Workload(
    name="tiny_flat_1m",
    description="flat tensor of 1,048,576 params, N=4 mean-weighted ranks, Adam t=1",
    psi=1 << 20, seed=0)

LAYER_7B = Workload(
    name="layer7b_weighted_adamw",
    description=("7B-class layer d=4096 ffn=11008 (202,375,168 params), N=4 ranks "
                 "weighted by token counts 4096/3072/4096/2048, AdamW wd=0.1"),
    psi=sum(unit_numels(layer_7b_tensors())), weight_decay=0.1, seed=1,
    extra={"token_counts": [4096, 3072, 4096, 2048], "rank_scale": (0.5, 2.0), "steps": 3})

OWNER_8B = Workload(
    name="owner_share_8b_buckets",
    description=("one owner's ZeRO-2/3 share of an 8B model: 2.0e9 params in 64M buckets, "
                 "4 bf16 rank contributions, mid-run state t=1000, Adam wd=0.1"),
    psi=2_000_000_000, weight_decay=0.1, m_sigma=1e-4, v_sigma=1e-6, step0=1000, seed=2,
    extra={"bucket": BUCKET})

CHAIN_8B = Workload(
    name="zero3_chain_llama8b",
    description=("ZeRO-3 per-layer gather/scatter chain on an 8B Llama-like model "
                 "(34 units, 8,029,995,008 params), N=4"),
    psi=sum(sum(unit_numels(t)) for _, t in llama8b_units()), seed=3,
    extra={"units": llama8b_units()})

OFFLOAD_8B = Workload(
    name="offload_owner_8b_two_slots",
    description=("host-offloaded 2.0e9-param FP32 gradient shard, two device slots of "
                 "64M params x 4 bf16 contributions, 4 micro-batches"),
    psi=2_000_000_000, seed=4,
    extra={"chunk": BUCKET, "micro_batches": 4})

WORKLOADS = {w.name: w for w in (TINY, LAYER_7B, OWNER_8B, CHAIN_8B, OFFLOAD_8B)}
WORKLOAD_ORDER = [TINY, LAYER_7B, OWNER_8B, CHAIN_8B, OFFLOAD_8B]
