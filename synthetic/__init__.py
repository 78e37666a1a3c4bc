"""Seeded synthetic inputs, shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the method: it only draws random numbers
(numpy's PCG64 on the host, torch's Philox generator on the device) and rounds
them to bfloat16 with torch's own conversion.  Both the oracle and the HIP path
receive the arrays it returns; neither side generates its own.
"""
from __future__ import annotations

import numpy as np

from .workloads import WORKLOADS, Workload, unit_numels  # noqa: F401


def _torch():
    import torch
    return torch


# ---------------------------------------------------------------- host (numpy)
def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def normal_f32(gen: np.random.Generator, n: int, sigma: float, scale: float = 1.0) -> np.ndarray:
    """float32 samples of N(0, sigma) (sigma is the standard deviation) times scale."""
    return (gen.standard_normal(n) * (sigma * scale)).astype(np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns of float32 values, rounded by torch's conversion."""
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_normal(gen: np.random.Generator, n: int, sigma: float, scale: float = 1.0) -> np.ndarray:
    return to_bf16_bits(normal_f32(gen, n, sigma, scale))


def host_rank_grads(seed: int, n_ranks: int, numel: int, sigma: float = 1e-3,
                    scales=None) -> list:
    g = rng(seed)
    scales = [1.0] * n_ranks if scales is None else list(scales)
    return [bf16_normal(g, numel, sigma, scales[r]) for r in range(n_ranks)]


def host_state(seed: int, numel: int, master_sigma: float = 0.02,
               m_sigma: float = 0.0, v_sigma: float = 0.0):
    """(master, m, v) float32: master ~ N(0, master_sigma); m ~ N(0, m_sigma);
    v ~ |N(0, v_sigma)|; a sigma of 0 gives zeros."""
    g = rng(seed)
    p = normal_f32(g, numel, master_sigma)
    m = normal_f32(g, numel, m_sigma) if m_sigma else np.zeros(numel, np.float32)
    v = np.abs(normal_f32(g, numel, v_sigma)) if v_sigma else np.zeros(numel, np.float32)
    return p, m, v


def rank_scales(seed: int, n_ranks: int, lo: float = 0.5, hi: float = 2.0) -> list:
    """One U(lo, hi) scale per rank, drawn once per run."""
    g = rng(seed + 7919)
    return [float(s) for s in g.uniform(lo, hi, n_ranks)]


# ------------------------------------------------------------- device (torch)
class DeviceGen:
    """Seeded device-side generator; sub-streams are keyed by integers so that
    any region can be regenerated on its own (for sampled parity checks)."""

    def __init__(self, seed: int, device="cuda"):
        torch = _torch()
        self.seed = int(seed)
        self.device = torch.device(device)
        self.gen = torch.Generator(device=self.device)

    def _reseed(self, *keys):
        h = self.seed
        for k in keys:
            h = (h * 1000003 + int(k) + 1) & 0x7FFFFFFFFFFFFFFF
        self.gen.manual_seed(h)

    def normal_(self, out, sigma: float, *keys, scale: float = 1.0):
        """Fill a float32 tensor with N(0, sigma)*scale."""
        self._reseed(*keys)
        out.normal_(0.0, sigma * scale, generator=self.gen)
        return out

    def bf16_normal_(self, out_bf16, sigma: float, *keys, scale: float = 1.0, tmp=None):
        """Fill a bfloat16 tensor with torch's RNE rounding of N(0, sigma)*scale,
        drawn in float32 (tmp: optional float32 scratch of the same size)."""
        torch = _torch()
        self._reseed(*keys)
        if tmp is None:
            tmp = torch.empty(out_bf16.shape, dtype=torch.float32, device=out_bf16.device)
        tmp.normal_(0.0, sigma * scale, generator=self.gen)
        out_bf16.copy_(tmp)
        return out_bf16

    def abs_normal_(self, out, sigma: float, *keys):
        self.normal_(out, sigma, *keys)
        return out.abs_()
