"""Seeded device-side inputs for the large workloads, written into buffers the
caller owns.  Random draws and torch's BF16 conversion only: nothing here
computes any step of the method.  Every region is keyed so that a test can
regenerate exactly the values of the region it checks."""
from __future__ import annotations

import torch

from . import DeviceGen
from .workloads import BUCKET

# key spaces
K_MASTER, K_M, K_V, K_CONTRIB, K_GRAD = 1, 2, 3, 10, 20


def pieces(n: int, piece: int = BUCKET):
    return [(lo, min(lo + piece, n)) for lo in range(0, n, piece)]


def fill_normal_pieces(gen: DeviceGen, out: torch.Tensor, sigma: float, key: int, absolute=False):
    """out (float32) <- N(0, sigma), drawn piece by piece with keys (key, piece)."""
    for i, (lo, hi) in enumerate(pieces(out.numel())):
        gen.normal_(out[lo:hi], sigma, key, i)
        if absolute:
            out[lo:hi].abs_()


def fill_bf16_pieces(gen: DeviceGen, out: torch.Tensor, sigma: float, key: int, tmp: torch.Tensor,
                     scale: float = 1.0):
    """out (bfloat16) <- bf16(N(0, sigma)*scale), piece by piece (tmp: float32 >= one piece)."""
    for i, (lo, hi) in enumerate(pieces(out.numel())):
        gen.bf16_normal_(out[lo:hi], sigma, key, i, scale=scale, tmp=tmp[: hi - lo])


def owner_share_region(gen: DeviceGen, wl, what: str, lo: int, hi: int, device="cuda"):
    """Regenerate [lo, hi) of one owner-share input ('master', 'm', 'v' or
    'contrib<r>') exactly as fill_owner_share drew it; lo, hi within one piece."""
    b = lo // BUCKET
    assert (hi - 1) // BUCKET == b
    base = b * BUCKET
    n = min(BUCKET, wl.psi - base)
    if what.startswith("contrib"):
        r = int(what[7:])
        buf = torch.empty(n, dtype=torch.bfloat16, device=device)
        gen.bf16_normal_(buf, wl.grad_sigma, K_CONTRIB + r, b)
    else:
        key, sigma = {"master": (K_MASTER, wl.master_sigma), "m": (K_M, wl.m_sigma),
                      "v": (K_V, wl.v_sigma)}[what]
        buf = torch.empty(n, dtype=torch.float32, device=device)
        gen.normal_(buf, sigma, key, b)
        if what == "v":
            buf.abs_()
    return buf[lo - base: hi - base]


def fill_owner_share(gen: DeviceGen, wl, master, m, v, contribs, tmp):
    fill_normal_pieces(gen, master, wl.master_sigma, K_MASTER)
    fill_normal_pieces(gen, m, wl.m_sigma, K_M)
    fill_normal_pieces(gen, v, wl.v_sigma, K_V, absolute=True)
    for r, c in enumerate(contribs):
        fill_bf16_pieces(gen, c, wl.grad_sigma, K_CONTRIB + r, tmp)


def chain_unit_grads(gen: DeviceGen, wl, u: int, grads, n: int, tmp):
    """The N BF16 gradient contributions of chain unit u, first n elements of
    each buffer, keyed (unit, rank)."""
    for r, g in enumerate(grads):
        gen.bf16_normal_(g[:n], wl.grad_sigma, K_GRAD + u, r, tmp=tmp[:n])


def offload_contrib(gen: DeviceGen, wl, mb: int, c: int, views, tmp):
    """Chunk c's N contributions for micro-batch mb, keyed (micro-batch, chunk, rank)."""
    for r, vw in enumerate(views):
        gen.bf16_normal_(vw, wl.grad_sigma, K_CONTRIB + mb, c * 64 + r, tmp=tmp[: vw.numel()])
