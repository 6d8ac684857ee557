"""Seeded synthetic Q/K/V generators for the VC-Attention workloads.

This module holds only random-number recipes; it contains none of the
method's arithmetic, and both the CPU oracle's tests and the HIP path's tests
draw their inputs from it.  Every tensor is produced in fp32 with torch's
generator on the requested device, then rounded to bf16, in the layout
[B, S, H, D] (token-major, heads interleaved, head dim contiguous).

Workloads (the shapes of the video-DiT settings on the pages; the pages use
captured post-RoPE activations of real models, which these stand in for):

  tiny      B=1 H=2  S=1024  D=64   Q,K,V ~ N(0,1); 1% of value tokens per
                                    head get 4 random channels scaled x20
  plain     B=1 H=24 S=16384 D=128  Q,K ~ N(0,1), K += per-(h,c) bias drawn
                                    with variance 2; V ~ Student-t(3)
  longcat   B=1 H=32 S=32760 D=128  grid 21x30x52
  wan       B=1 H=40 S=75600 D=128  grid 21x45x80
  minimax   B=1 H=48 S=84672 D=128  grid 21x48x84

Video-shaped workloads (token = (t*Hl + y)*Wl + x, raster order):
  Q, K: per (head, channel) a 3-D Gaussian random field -- white noise
        blurred by a separable Gaussian of sigma 2 voxels and standardised --
        plus N(0,1) noise;
  V:    per head, 64 Voronoi regions around random seed voxels (spatially
        contiguous); each region's centre ~ N(0, 3^2 I); token = centre +
        N(0, 0.5^2 I); 0.5% of tokens per head get +10 * Student-t(3) noise
        on 8 random channels.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    S: int
    D: int
    grid: tuple | None  # (T, Hl, Wl) for video-shaped workloads
    vsmooth: bool
    clusters: int
    iters: int
    index: int

    @property
    def nblk(self) -> int:
        return (self.S + 127) // 128

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def seed(self) -> int:
        return 1000 + self.index

    def flops(self) -> float:
        """Algorithmic attention FLOPs: QK^T and PV, 2 flops per MAC."""
        return 4.0 * self.B * self.H * self.S * self.S * self.D


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 1024, 64, None, True, 8, 3, 0),
    "plain": Workload("plain", 1, 24, 16384, 128, None, False, 0, 0, 1),
    "longcat": Workload("longcat", 1, 32, 32760, 128, (21, 30, 52), True, 64, 4, 2),
    "wan": Workload("wan", 1, 40, 75600, 128, (21, 45, 80), True, 64, 4, 3),
    "minimax": Workload("minimax", 1, 48, 84672, 128, (21, 48, 84), True, 64, 4, 4),
}


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _student_t3(shape, g, device):
    z = torch.randn(shape, generator=g, device=device)
    c = torch.randn((3,) + tuple(shape), generator=g, device=device).square().sum(0) / 3.0
    return z / c.sqrt()


def _blur_axis(x: torch.Tensor, axis: int, sigma: float) -> torch.Tensor:
    """Separable Gaussian blur along one spatial axis of x [F, T, Hl, Wl]
    (reflect padding), written as a weighted sum of shifted slices."""
    r = int(math.ceil(3 * sigma))
    t = torch.arange(-r, r + 1, dtype=torch.float64)
    w = torch.exp(-0.5 * (t / sigma) ** 2)
    w = (w / w.sum()).tolist()
    n = x.shape[axis]
    idx = torch.arange(-r, n + r)
    idx = idx.abs()  # reflect at 0
    idx = torch.where(idx > n - 1, 2 * (n - 1) - idx, idx).clamp(0, n - 1)  # reflect at n-1
    xp = x.index_select(axis, idx.to(x.device))
    out = torch.zeros_like(x)
    for i, wi in enumerate(w):
        out += wi * xp.narrow(axis, i, n)
    return out


def _grf(F: int, grid, g, device, sigma=2.0, chunk=512):
    """F standardised Gaussian random fields on the grid -> [F, S]."""
    T, Hl, Wl = grid
    out = torch.empty((F, T * Hl * Wl), device=device)
    for f0 in range(0, F, chunk):
        f1 = min(F, f0 + chunk)
        x = torch.randn((f1 - f0, T, Hl, Wl), generator=g, device=device)
        for ax in (1, 2, 3):
            x = _blur_axis(x, ax, sigma)
        x = x.reshape(f1 - f0, -1)
        x = (x - x.mean(dim=1, keepdim=True)) / x.std(dim=1, keepdim=True)
        out[f0:f1] = x
    return out


def _video_qk(w: Workload, g, device):
    H, D, S = w.H, w.D, w.S
    field = _grf(H * D, w.grid, g, device)  # [H*D, S]
    x = field.view(H, D, S).permute(2, 0, 1)  # [S, H, D]
    x = x + torch.randn((S, H, D), generator=g, device=device)
    return x.unsqueeze(0)


def _voronoi_labels(grid, nreg: int, g, device):
    T, Hl, Wl = grid
    S = T * Hl * Wl
    tt, yy, xx = torch.meshgrid(torch.arange(T, device=device), torch.arange(Hl, device=device),
                                torch.arange(Wl, device=device), indexing="ij")
    coords = torch.stack([tt.reshape(-1), yy.reshape(-1), xx.reshape(-1)], 1).float()  # [S,3]
    seeds = torch.randperm(S, generator=g, device=device)[:nreg]
    sc = coords[seeds]
    d2 = ((coords[:, None, :] - sc[None, :, :]) ** 2).sum(-1)  # [S, nreg]
    return d2.argmin(dim=1)


def _video_v(w: Workload, g, device, nreg=64):
    H, D, S = w.H, w.D, w.S
    v = torch.empty((S, H, D), device=device)
    nout = int(round(0.005 * S))
    for h in range(H):
        lab = _voronoi_labels(w.grid, nreg, g, device)
        centre = 3.0 * torch.randn((nreg, D), generator=g, device=device)
        vh = centre[lab] + 0.5 * torch.randn((S, D), generator=g, device=device)
        tok = torch.randperm(S, generator=g, device=device)[:nout]
        ch = torch.argsort(torch.rand((nout, D), generator=g, device=device), dim=1)[:, :8]
        noise = 10.0 * _student_t3((nout, 8), g, device)
        rows = vh[tok]
        rows.scatter_add_(1, ch, noise)
        vh[tok] = rows
        v[:, h, :] = vh
    return v.unsqueeze(0)


def make_qkv(name: str, device="cpu", seed: int | None = None, S: int | None = None, H: int | None = None):
    """Q, K, V (bf16, [B,S,H,D]) for a named workload.

    S or H may be overridden for smaller tests of the same recipe (video
    workloads keep their grid and then take the first S tokens of it)."""
    w = WORKLOADS[name]
    if H is not None:
        w = Workload(w.name, w.B, H, w.S, w.D, w.grid, w.vsmooth, w.clusters, w.iters, w.index)
    base = w.seed if seed is None else seed
    gq, gk, gv = (_gen(device, base * 16 + i) for i in (1, 2, 3))
    B, S0, Hh, D = w.B, w.S, w.H, w.D
    if w.grid is None:
        q = torch.randn((B, S0, Hh, D), generator=gq, device=device)
        k = torch.randn((B, S0, Hh, D), generator=gk, device=device)
        if name == "plain":
            k = k + math.sqrt(2.0) * torch.randn((1, 1, Hh, D), generator=gk, device=device)
            v = _student_t3((B, S0, Hh, D), gv, device)
        else:
            v = torch.randn((B, S0, Hh, D), generator=gv, device=device)
            nout = int(0.01 * S0)
            for b in range(B):
                for h in range(Hh):
                    tok = torch.randperm(S0, generator=gv, device=device)[:nout]
                    for t in tok.tolist():
                        ch = torch.randperm(D, generator=gv, device=device)[:4]
                        v[b, t, h, ch] *= 20.0
    else:
        q = _video_qk(w, gq, device)
        k = _video_qk(w, gk, device)
        v = _video_v(w, gv, device)
    if S is not None and S < S0:
        q, k, v = q[:, :S], k[:, :S], v[:, :S]
    return (q.to(torch.bfloat16).contiguous(), k.to(torch.bfloat16).contiguous(),
            v.to(torch.bfloat16).contiguous())


def random_qkv(B, S, H, D, seed, device="cpu", v_kind="normal"):
    """Generic N(0,1) inputs for edge-case tests (ragged S, D=64, ...)."""
    g = _gen(device, seed)
    q = torch.randn((B, S, H, D), generator=g, device=device)
    k = torch.randn((B, S, H, D), generator=g, device=device)
    if v_kind == "t3":
        v = _student_t3((B, S, H, D), g, device)
    else:
        v = torch.randn((B, S, H, D), generator=g, device=device)
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def bf16_bits(x: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (on the host)."""
    return x.detach().contiguous().cpu().view(torch.int16).numpy().view("uint16")


def keys_rising_by_tile(k: torch.Tensor, step: float) -> torch.Tensor:
    """bf16 keys [B,S,H,D] with the keys of 128-token tile t scaled by
    1 + step t, so that in key order each tile's scores reach well past the
    previous tile's: the running maximum keeps rising."""
    t = torch.arange(k.shape[1], device=k.device) // 128
    return (k.float() * (1 + step * t).float()[None, :, None, None]).to(torch.bfloat16)
