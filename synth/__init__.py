"""Seeded synthetic inputs shaped like the video-DiT attention layers the pages measure.

This module draws random numbers and positional features and nothing else: it holds no step of
the attention method (no pooling, scoring, selection or attention). Both the CPU oracle tests
and the HIP path take their inputs from here, so the two sides see identical bf16 tensors.

Workload shapes follow the pages:
  * 480p Wan2.1 layers: 32,760 tokens = 21 latent frames of 30x52 tokens (CalibAtt page,
    thelatestinai.com/papers/2603.05503, Fig. 2 and Fig. 4 captions, Table S4 caption:
    batch 1, 40 heads, head dim 128).
  * 720p Wan2.1-14B layers: 75,600 tokens = 21 frames of 45x80 (same page, Fig. S9 caption).
  * HunyuanVideo 720p 5 s: 33 frames of 45x80 tokens, block 128 (RECAP,
    paperpeel.com/paper/2610.26244, §4.1 names the model; the frame grid is a reading).

Recipe (all choices not fixed by the pages are readings, listed with the design notes):
  * token n -> (t, y, x) in raster order, t slowest, x fastest;
  * phi(n) in R^64 = [phi_t (20), phi_y (22), phi_x (22)]; an axis with coordinate c and F
    frequencies gives interleaved [sqrt2*sin(c*w_f), sqrt2*cos(c*w_f)], w_f = 100^(-f/F);
  * Q = N(0,1) + w*phi and K = N(0,1) + w*phi on dims [0, 64), pure noise on [64, D);
    V = N(0,1) (+ w*phi on [0,64) for the tiny case); all drawn in fp32, rounded RNE to bf16;
  * residual R = 0.05 * N(0,1), bf16;
  * one CPU torch.Generator per (tensor, batch, head): seed = 1000*tensor_id + 100*b + h,
    tensor ids Q=1, K=2, V=3, R=4, drift E_Q=5, E_K=6, E_V=7; per-head thresholds and
    residual scales use seed 9.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "r": 4, "eq": 5, "ek": 6, "ev": 7}
PHI_DIM = 64
FREQ_BASE = 100.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    head_dim: int
    grid: tuple  # (frames, rows, cols) of latent tokens
    block: int
    top_p: object  # float, or ("uniform", lo, hi)
    pos_weight: float
    v_positional: bool
    residual: bool
    res_scale: object  # None, float, or "uniform"
    refresh_then_sparse: int = 0  # >0: one dense refresh then this many drifted sparse calls

    @property
    def seq(self) -> int:
        t, y, x = self.grid
        return t * y * x

    @property
    def num_blocks(self) -> int:
        return -(-self.seq // self.block)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 64, (4, 32, 32), 64, 0.9, 2.0, True, True, 0.5),
    "wan13b_480p": Workload("wan13b_480p", 1, 12, 128, (21, 30, 52), 64, 0.9, 2.0, False,
                            False, None),
    "wan14b_480p": Workload("wan14b_480p", 1, 40, 128, (21, 30, 52), 64,
                            ("uniform", 0.8, 0.97), 2.0, False, True, "uniform"),
    "wan14b_720p": Workload("wan14b_720p", 1, 40, 128, (21, 45, 80), 64, 0.95, 2.0, False,
                            False, 1.0, refresh_then_sparse=3),
    "hunyuan_720p": Workload("hunyuan_720p", 1, 24, 128, (33, 45, 80), 128, 0.97, 3.0, False,
                             True, 0.5),
}


def workload(name: str, **overrides) -> Workload:
    return dataclasses.replace(WORKLOADS[name], **overrides)


def _axis_features(coord: np.ndarray, nfreq: int) -> np.ndarray:
    f = np.arange(nfreq, dtype=np.float64)
    omega = FREQ_BASE ** (-f / nfreq)
    ang = coord[:, None].astype(np.float64) * omega[None, :]
    out = np.empty((coord.shape[0], 2 * nfreq), dtype=np.float64)
    out[:, 0::2] = math.sqrt(2.0) * np.sin(ang)
    out[:, 1::2] = math.sqrt(2.0) * np.cos(ang)
    return out


def positional_features(grid) -> torch.Tensor:
    """phi(n) for every token of a (frames, rows, cols) grid: float32 [N, 64], unit RMS."""
    t_n, y_n, x_n = grid
    n = np.arange(t_n * y_n * x_n)
    t = n // (y_n * x_n)
    y = (n // x_n) % y_n
    x = n % x_n
    phi = np.concatenate([_axis_features(t, 10), _axis_features(y, 11), _axis_features(x, 11)],
                         axis=1)
    assert phi.shape[1] == PHI_DIM
    return torch.from_numpy(phi.astype(np.float32))


def _gen(tensor: str, b: int, h: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(1000 * TENSOR_IDS[tensor] + 100 * b + h)
    return g


def _noise_plus_features(tensor, cfg: Workload, n, weight, phi, seq_override=None):
    """One bf16 [B, H, N, D] tensor, generated head by head (bounded host memory)."""
    B, H, D = cfg.batch, cfg.heads, cfg.head_dim
    out = torch.empty((B, H, n, D), dtype=torch.bfloat16)
    fd = min(PHI_DIM, D)
    for b in range(B):
        for h in range(H):
            x = torch.randn((n, D), generator=_gen(tensor, b, h), dtype=torch.float32)
            if weight != 0.0:
                x[:, :fd] += weight * phi[:n, :fd]
            out[b, h] = x.to(torch.bfloat16)
    return out


def make_qkv(cfg: Workload, seq: Optional[int] = None):
    """Q, K, V as CPU bf16 tensors [B, H, N, D]; `seq` truncates the raster (ragged tests)."""
    n = cfg.seq if seq is None else seq
    phi = positional_features(cfg.grid) if n <= cfg.seq else None
    if phi is None:  # longer than the grid: extend the frame axis
        frames = -(-n // (cfg.grid[1] * cfg.grid[2]))
        phi = positional_features((frames, cfg.grid[1], cfg.grid[2]))
    q = _noise_plus_features("q", cfg, n, cfg.pos_weight, phi)
    k = _noise_plus_features("k", cfg, n, cfg.pos_weight, phi)
    v = _noise_plus_features("v", cfg, n, cfg.pos_weight if cfg.v_positional else 0.0, phi)
    return q, k, v


def make_residual(cfg: Workload, seq: Optional[int] = None) -> torch.Tensor:
    """Cached residual R = 0.05 * N(0,1), bf16 [B, H, N, D]."""
    n = cfg.seq if seq is None else seq
    B, H, D = cfg.batch, cfg.heads, cfg.head_dim
    out = torch.empty((B, H, n, D), dtype=torch.bfloat16)
    for b in range(B):
        for h in range(H):
            x = torch.randn((n, D), generator=_gen("r", b, h), dtype=torch.float32)
            out[b, h] = (0.05 * x).to(torch.bfloat16)
    return out


def drifted(x: torch.Tensor, tensor: str, step: int) -> torch.Tensor:
    """X_s = bf16(X_0 + 0.05 * s * E), E ~ N(0,1) drawn once per tensor and head."""
    B, H, n, D = x.shape
    out = torch.empty_like(x)
    for b in range(B):
        for h in range(H):
            e = torch.randn((n, D), generator=_gen("e" + tensor, b, h), dtype=torch.float32)
            out[b, h] = (x[b, h].float() + (0.05 * step) * e).to(torch.bfloat16)
    return out


def head_params(cfg: Workload):
    """Per-head top-p thresholds and residual scales, float64 numpy arrays of length H."""
    g = torch.Generator(device="cpu")
    g.manual_seed(9)
    u_p = torch.rand(cfg.heads, generator=g, dtype=torch.float64).numpy()
    u_c = torch.rand(cfg.heads, generator=g, dtype=torch.float64).numpy()
    if isinstance(cfg.top_p, tuple):
        _, lo, hi = cfg.top_p
        p = lo + (hi - lo) * u_p
    else:
        p = np.full(cfg.heads, float(cfg.top_p))
    if cfg.res_scale is None:
        c = np.zeros(cfg.heads)
    elif cfg.res_scale == "uniform":
        c = u_c.copy()
    else:
        c = np.full(cfg.heads, float(cfg.res_scale))
    # thresholds and scales cross the boundary as fp32; keep the exact fp32 values on both sides
    return p.astype(np.float32).astype(np.float64), c.astype(np.float32).astype(np.float64)


def random_bf16(shape, seed: int, scale: float = 1.0) -> torch.Tensor:
    """Plain N(0, scale^2) bf16 tensor for edge-case tests (seeded)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return (scale * torch.randn(shape, generator=g, dtype=torch.float32)).to(torch.bfloat16)


def to_f64(x: torch.Tensor) -> np.ndarray:
    """Exact upcast of a bf16/fp32 CPU tensor to a float64 numpy array."""
    return x.detach().to("cpu").float().numpy().astype(np.float64)


def drift_series(x: torch.Tensor, tensor: str, nsteps: int):
    """[drifted(x, tensor, s) for s = 1..nsteps], drawing each head's E once."""
    B, H, n, D = x.shape
    outs = [torch.empty_like(x) for _ in range(nsteps)]
    for b in range(B):
        for h in range(H):
            e = torch.randn((n, D), generator=_gen("e" + tensor, b, h), dtype=torch.float32)
            base = x[b, h].float()
            for s in range(1, nsteps + 1):
                outs[s - 1][b, h] = (base + (0.05 * s) * e).to(torch.bfloat16)
    return outs
