"""Seeded weights and inputs of a toy looped attention stack, the synthetic
stand-in for a looped model when the codebooks are fine-tuned against the
model's own outputs (LoopVQ review, arXiv 2611.05304, section 3.2: the
weights stay frozen, only the codebook entries move).

Only random draws live here: embeddings x for the N positions after the
sinks, and the frozen projections W_q, W_o (d x d) and W_u (d x vocab) with
d = H_q * D.  Recipe: x ~ N(0, 1); W_q ~ N(0, 1/d); W_o ~ N(0, 0.25/d);
W_u ~ N(0, 4/d), all fp32.  The cache the stack attends to is the ordinary
synthetic loop-correlated K/V cache of the same workload.
"""
import torch

from .configs import LoopConfig
from .generator import SeedPlan


def gen_targets(cfg: LoopConfig, layer: int = 0, device="cpu", vocab: int = 256, B=None, N=None):
    """Next-token targets int64 [B][N], uniform over the vocabulary (no data
    exists; they stand in for a calibration set's tokens)."""
    B = cfg.B if B is None else B
    N = cfg.N if N is None else N
    g = SeedPlan(cfg.index).gen(layer, "toy_y", "cpu")
    return torch.randint(0, vocab, (B, N), generator=g, dtype=torch.int64).to(device)


def gen_toy_stack(cfg: LoopConfig, layer: int = 0, device="cpu", vocab: int = 256, B=None):
    """dict(x [B][N][d], Wq [d][d], Wo [d][d], Wu [d][vocab]) in fp32 on `device`."""
    B = cfg.B if B is None else B
    d = cfg.H_q * cfg.D
    plan = SeedPlan(cfg.index)
    gx = plan.gen(layer, "toy_x", "cpu")
    gw = plan.gen(layer, "toy_w", "cpu")
    x = torch.randn((B, cfg.N, d), generator=gx, dtype=torch.float32)
    wq = torch.randn((d, d), generator=gw, dtype=torch.float32) * d ** -0.5
    wo = torch.randn((d, d), generator=gw, dtype=torch.float32) * (0.5 * d ** -0.5)
    wu = torch.randn((d, vocab), generator=gw, dtype=torch.float32) * (2.0 * d ** -0.5)
    return {k: t.to(device) for k, t in dict(x=x, Wq=wq, Wo=wo, Wu=wu).items()}
