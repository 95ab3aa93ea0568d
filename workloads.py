"""Seeded synthetic inputs for the FP8 attention workloads.

This module only draws random tensors with the shapes and value structure of the video-DiT
workloads (it holds none of the method's arithmetic). The same bf16 bytes feed both the CPU
oracle and the HIP library. Shapes follow the pages: Wan2.1 480p latent 21x30x52 and the
Wan2.1-14B 720p latent 21x45x80 (FPSAttention write-up, section 1), D = 128 heads.

Recipe (fixed; every config draws FP32 ``randn`` [1, N, H, 128] for Q, then K, then V from
``torch.Generator('cpu').manual_seed(seed)``, applies its modification, then rounds to bf16):

* ``dense512``   B=1, H=2,  N=512,   seed 1, N(0,1).
* ``sink4096``   B=1, H=8,  N=4096,  seed 20 + Delta. Channels 0..126 are N(0,1)*sqrt(128/127),
  so non-sink logits q.k/sqrt(128) are ~N(0,1); channel 127 is a bias channel: Q = 4 for every
  query, K = 0 except the 4 sink keys 0..3 where K = Delta*sqrt(128)/4, which offsets the sink
  logits by Delta (up to bf16 rounding, seen identically by both sides). V N(0,1).
* ``wan13b``     B=1, H=12, N=32760 (21x30x52), seed 3. For each head and each of Q, K, V
  independently, 4 distinct random channels are multiplied by 8 (channel outliers).
* ``wan14b``     B=1, H=40, N=75600 (21x45x80), seed 4, N(0,1). The sparse variant lays the
  same tensors out in (6,8,8) tiles on the grid padded to 24x48x80 (N' = 92160).
* ``vsmooth``    B=1, H=24, N=49152, seed 5. Q, K N(0,1). V N(0,1) with 5% of the tokens per
  head (2458) multiplied by 20 on 8 distinct random channels each (token outliers).
* ``wan14b_local`` B=1, H=40, N=75600 (21x45x80), seed 6, kind ``video_local`` (below).

Kind ``video_local`` (test and bench inputs for Sol routing; needs ``grid``): attention that
falls off with the distance of the tokens on the (T, Hg, W) latent grid, as in video DiTs. Q, K
and V are first drawn N(0,1) as above; then, drawing in this order from the same generator,
F = randn [3, 128] / sigma (sigma = 1.5 grid steps) and b = 2 pi rand [128] give the random
Fourier features phi(x) = sqrt(2 / 128) cos(x F + b) of each token's grid position x (raster
order t, h, w), and Q = 16 phi + 0.5 Q, K = 16 phi + 0.5 K (so q . k / sqrt(128) peaks near
22 * exp(-|x - y|^2 / (2 sigma^2)) for nearby tokens); V stays N(0,1).

Kind ``channel_offset`` (test inputs for sequence-mean smoothing): Q, K, V N(0,1), then K and V
each get a per-(head, channel) offset drawn after V as 4 * randn [H, 128] (K's first), the
shared token bias that the TeleFuser MiniMax-H3 section removes before quantising.
"""
from __future__ import annotations

import math

import numpy as np
import torch

D = 128

CONFIGS = {
    "dense512": dict(B=1, H=2, N=512, seed=1),
    "sink4096": dict(B=1, H=8, N=4096, seed=20),
    "wan13b": dict(B=1, H=12, N=32760, seed=3, grid=(21, 30, 52)),
    "wan14b": dict(B=1, H=40, N=75600, seed=4, grid=(21, 45, 80)),
    "vsmooth": dict(B=1, H=24, N=49152, seed=5),
    "wan14b_local": dict(B=1, H=40, N=75600, seed=6, grid=(21, 45, 80)),
}


def _bits(x: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 numpy array of its bits (a copy)."""
    return x.contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def make_qkv(B, N, H, seed, kind="normal", delta=None, head_dim=D, sink_keys=4,
             outlier_tokens_frac=0.05, n_outlier_channels=4, grid=None):
    """Returns bf16 torch tensors (q, k, v), each [B, N, H, head_dim], on the CPU."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    shape = (B, N, H, head_dim)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    if kind == "normal":
        pass
    elif kind == "sink":
        a = 4.0
        s = math.sqrt(head_dim / (head_dim - 1.0))
        q[..., : head_dim - 1] *= s
        k[..., : head_dim - 1] *= s
        q[..., head_dim - 1] = a
        k[..., head_dim - 1] = 0.0
        k[:, :sink_keys, :, head_dim - 1] = float(delta) * math.sqrt(head_dim) / a
    elif kind == "channel_outliers":
        for t in (q, k, v):
            ch = torch.rand((H, head_dim), generator=g).argsort(dim=-1)[:, :n_outlier_channels]
            for h in range(H):
                t[:, :, h, ch[h]] *= 8.0
    elif kind == "token_outliers":
        n_out = int(round(outlier_tokens_frac * N))
        for h in range(H):
            toks = torch.randperm(N, generator=g)[:n_out]
            ch = torch.rand((n_out, head_dim), generator=g).argsort(dim=-1)[:, :8]
            sub = v[0, toks, h, :]
            sub.scatter_(1, ch, sub.gather(1, ch) * 20.0)
            v[0, toks, h, :] = sub
    elif kind == "video_local":
        T, Hg, W = grid
        assert T * Hg * W == N
        sigma = 1.5
        Fm = torch.randn((3, head_dim), generator=g, dtype=torch.float64) / sigma
        bph = 2.0 * math.pi * torch.rand((head_dim,), generator=g, dtype=torch.float64)
        t, h, w = torch.meshgrid(torch.arange(T), torch.arange(Hg), torch.arange(W), indexing="ij")
        x = torch.stack([t.reshape(-1), h.reshape(-1), w.reshape(-1)], dim=1).to(torch.float64)
        phi = (math.sqrt(2.0 / head_dim) * torch.cos(x @ Fm + bph)).to(torch.float32)   # [N, D]
        q = 16.0 * phi[None, :, None, :] + 0.5 * q
        k = 16.0 * phi[None, :, None, :] + 0.5 * k
    elif kind == "channel_offset":
        for t in (k, v):
            t += 4.0 * torch.randn((H, head_dim), generator=g, dtype=torch.float32)
    else:
        raise ValueError(kind)
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def workload(name, delta=None, heads=None, tokens=None):
    """Inputs of a named workload as bf16 torch CPU tensors. ``heads`` / ``tokens`` shrink a
    workload for quick checks while keeping its value structure."""
    c = dict(CONFIGS[name])
    B, H, N, seed = c["B"], c["H"], c["N"], c["seed"]
    if heads is not None:
        H = int(heads)
    if tokens is not None:
        N = int(tokens)
    kind = {"dense512": "normal", "sink4096": "sink", "wan13b": "channel_outliers",
            "wan14b": "normal", "vsmooth": "token_outliers", "wan14b_local": "video_local"}[name]
    if name == "sink4096":
        seed = 20 + int(delta)
    return make_qkv(B, N, H, seed, kind=kind, delta=delta, grid=c.get("grid"))


def bits(x: torch.Tensor) -> np.ndarray:
    return _bits(x)


def sample_rows(N: int, n_random: int, seed: int, block: int = 64) -> np.ndarray:
    """Query rows for sampled parity at full size: rows 0 and N-1, every row of the last
    (possibly partial) 64-row block, and seeded random rows; sorted, unique, int32."""
    rng = np.random.default_rng(seed)
    tail0 = ((N - 1) // block) * block
    rows = np.concatenate([[0, N - 1], np.arange(tail0, N), rng.integers(0, N, n_random)])
    return np.unique(rows).astype(np.int32)
