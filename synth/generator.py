"""Seeded loop-correlated K/V caches, queries, sinks and pre-transform data.

The cache stands in for a looped transformer's per-step keys and values (LoopVQ
review, arXiv 2611.05304, "terms" section and section 1.2): each step's key is
an AR(1) continuation of the previous step's key, with the inter-step
correlation the review reports (Fig. 2a/2b: adjacent-step |r| about 0.85 on
average, rising from 0.69 to 0.94 across the four Ouro steps; 0.16 between
different channels of one 16-channel chunk).

Recipe, per (layer, kv-head, K or V):
  scale s ~ lognormal(0, 0.5) per channel, shared by batch, tokens and steps;
  x_1 ~ N(0, S), x_t = rho_t * x_{t-1} + sqrt(1 - rho_t^2) * eps_t, eps_t ~ N(0, S);
  S = I, or equicorrelation `chunk_corr` inside each chunk of c consecutive
  channels; the stored value is bf16(s * x_t) (round to nearest even).

Every stream has its own seed: 0x5EED0000 + 1000*cfg + 16*layer + role.
"""
from dataclasses import dataclass
import math
import torch

from .configs import LoopConfig

ROLE = {"scale_k": 0, "scale_v": 1, "calib_k": 2, "calib_v": 3, "ctx_k": 4,
        "ctx_v": 5, "sinks": 6, "queries": 7, "kmeans": 8, "w": 9, "perm": 10,
        "toy_x": 11, "toy_w": 12, "toy_y": 13}


@dataclass(frozen=True)
class SeedPlan:
    cfg: int

    def seed(self, layer: int, role: str) -> int:
        return 0x5EED0000 + 1000 * self.cfg + 16 * layer + ROLE[role]

    def gen(self, layer: int, role: str, device) -> torch.Generator:
        g = torch.Generator(device=device)
        g.manual_seed(self.seed(layer, role))
        return g


def _channel_scale(cfg: LoopConfig, layer: int, kind: str, device) -> torch.Tensor:
    g = SeedPlan(cfg.index).gen(layer, "scale_" + kind, device)
    z = torch.randn((cfg.H_kv, cfg.D), generator=g, device=device, dtype=torch.float32)
    return torch.exp(0.5 * z)


def _noise(shape, cfg: LoopConfig, g: torch.Generator, device) -> torch.Tensor:
    """N(0, S) draws over the last axis (D channels)."""
    e = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    a = cfg.chunk_corr
    if a > 0.0:
        lead = shape[:-1]
        shared = torch.randn(tuple(lead) + (cfg.D // cfg.c, 1), generator=g,
                             device=device, dtype=torch.float32)
        e = e.view(tuple(lead) + (cfg.D // cfg.c, cfg.c))
        e = math.sqrt(1.0 - a) * e + math.sqrt(a) * shared
        e = e.reshape(shape)
    return e


def _ar_steps(cfg: LoopConfig, rho, lead_shape, g, device, out: torch.Tensor, scale):
    """Fill out[..., t, :, :] (t = loop step) with the AR(1) recursion, scaled, in bf16.

    out has shape lead_shape[:2] + (T,) + lead_shape[2:] + (D,).
    """
    shape = tuple(lead_shape) + (cfg.D,)
    x = _noise(shape, cfg, g, device)
    sc = scale.view((1, cfg.H_kv) + (1,) * (len(shape) - 3) + (cfg.D,))
    out[:, :, 0] = (x * sc).to(torch.bfloat16)
    for t in range(1, cfg.T):
        r = rho[t - 1]
        x.mul_(r).add_(_noise(shape, cfg, g, device), alpha=math.sqrt(1.0 - r * r))
        out[:, :, t] = (x * sc).to(torch.bfloat16)
    return out


def gen_kv_layer(cfg: LoopConfig, layer: int, kind: str, device="cpu", N=None, B=None) -> torch.Tensor:
    """Context keys (kind='k') or values ('v'), pre-RoPE, bf16 [B][H_kv][T][N][D]."""
    N = cfg.N if N is None else N
    B = cfg.B if B is None else B
    g = SeedPlan(cfg.index).gen(layer, "ctx_" + kind, device)
    out = torch.empty((B, cfg.H_kv, cfg.T, N, cfg.D), dtype=torch.bfloat16, device=device)
    rho = cfg.rho_k if kind == "k" else cfg.rho_v
    return _ar_steps(cfg, rho, (B, cfg.H_kv, N), g, device, out,
                     _channel_scale(cfg, layer, kind, device))


def gen_sinks(cfg: LoopConfig, layer: int, device="cpu", B=None):
    """bf16 sink keys and values, pre-RoPE, [B][H_kv][T][n_s][D] each (positions 0..n_s-1)."""
    B = cfg.B if B is None else B
    g = SeedPlan(cfg.index).gen(layer, "sinks", device)
    res = []
    for kind in ("k", "v"):
        out = torch.empty((B, cfg.H_kv, cfg.T, cfg.n_s, cfg.D), dtype=torch.bfloat16, device=device)
        rho = cfg.rho_k if kind == "k" else cfg.rho_v
        _ar_steps(cfg, rho, (B, cfg.H_kv, cfg.n_s), g, device, out,
                  _channel_scale(cfg, layer, kind, device))
        res.append(out)
    return res[0], res[1]


def gen_queries(cfg: LoopConfig, layer: int, device="cpu", B=None, steps=None) -> torch.Tensor:
    """bf16 N(0,1) queries, already rotated for the current position: [B][H_q][steps][D]."""
    B = cfg.B if B is None else B
    steps = cfg.T if steps is None else steps
    g = SeedPlan(cfg.index).gen(layer, "queries", device)
    q = torch.randn((B, cfg.H_q, steps, cfg.D), generator=g, device=device, dtype=torch.float32)
    return q.to(torch.bfloat16)


def gen_tasq_params(cfg: LoopConfig, layer: int, device="cpu"):
    """Per-channel weights w ~ lognormal(0, 0.3) (fp32 [H_kv][D]) and a seeded
    uniform channel permutation per head (int16 [H_kv][D], z[d'] = x[perm[d']])."""
    gw = SeedPlan(cfg.index).gen(layer, "w", device)
    w = torch.exp(0.3 * torch.randn((cfg.H_kv, cfg.D), generator=gw, device=device,
                                    dtype=torch.float32))
    gp = SeedPlan(cfg.index).gen(layer, "perm", device)
    perm = torch.stack([torch.randperm(cfg.D, generator=gp, device=device)
                        for _ in range(cfg.H_kv)]).to(torch.int16)
    return w, perm


def gen_calibration_kv(cfg: LoopConfig, layer: int, kind: str, device="cpu") -> torch.Tensor:
    """Calibration cache (own stream): bf16 [H_kv][T][n_tok][D], enough tokens
    for cfg.n_calib joint vectors per codebook."""
    n_tok = max(1, cfg.n_calib // cfg.chunks)
    g = SeedPlan(cfg.index).gen(layer, "calib_" + kind, device)
    out = torch.empty((1, cfg.H_kv, cfg.T, n_tok, cfg.D), dtype=torch.bfloat16, device=device)
    rho = cfg.rho_k if kind == "k" else cfg.rho_v
    _ar_steps(cfg, rho, (1, cfg.H_kv, n_tok), g, device, out,
              _channel_scale(cfg, layer, kind, device))
    return out[0]
