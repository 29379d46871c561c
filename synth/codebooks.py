"""Calibration stand-in: seeded plain k-means codebooks.

The review (arXiv 2611.05304, section 3.1) initialises codebooks with
Fisher-weighted k-means over calibration joint vectors and then fine-tunes
them; both need model gradients, which this workload does not have.  This
module trains *unweighted* k-means (k-means++ seeding, Lloyd iterations,
empty clusters re-seeded at the worst-fit point) on calibration vectors drawn
from their own seeded stream, then rounds the centroids to bf16.  The result
is an input shared by both the oracle and the HIP path; nothing compares
against it.

Calibration joint vectors are laid out as the review's section 3.1 describes
the code of one block: coordinate i*T_c + m holds channel q*c + i of step m.
For the pre-transform workload, calibration keys are first normalised the way
the review's appendix B describes (weight, per-token scale, permutation), in
fp32; that only shapes the codebook, it is not a step either side is checked on.
"""
import torch

from .configs import LoopConfig
from .generator import SeedPlan, gen_calibration_kv, gen_tasq_params


def _calib_joint(cfg: LoopConfig, x: torch.Tensor) -> torch.Tensor:
    """x [H][T][n][D] -> [H][n_blk][n*chunks][G] (float32)."""
    H, T, n, D = x.shape
    xb = x.float().view(H, cfg.n_blk, cfg.T_c, n, cfg.chunks, cfg.c)
    # -> [H][blk][n][chunk][i][m]
    z = xb.permute(0, 1, 3, 4, 5, 2).contiguous()
    return z.view(H, cfg.n_blk, n * cfg.chunks, cfg.G)


def _calib_tasq(cfg: LoopConfig, layer: int, xk: torch.Tensor) -> torch.Tensor:
    w, perm = gen_tasq_params(cfg, layer, xk.device)
    xf = xk.float()                                      # [H][T][n][D]
    sigma = xf.pow(2).mean(dim=(0, 3), keepdim=True).sqrt().clamp_min(1e-30)
    y = xf * w[:, None, None, :] / sigma
    idx = perm.long()[:, None, None, :].expand_as(y)
    return torch.gather(y, 3, idx)


def _kmeans(X: torch.Tensor, K: int, iters: int, g: torch.Generator) -> torch.Tensor:
    """Batched k-means. X [nb][n][G] -> centroids [nb][K][G] (same dtype)."""
    nb, n, G = X.shape
    dev = X.device
    ar = torch.arange(nb, device=dev)
    first = torch.randint(n, (nb,), generator=g, device=dev)
    C = torch.empty((nb, K, G), dtype=X.dtype, device=dev)
    C[:, 0] = X[ar, first]
    d2 = (X - C[:, :1]).pow(2).sum(-1)
    for k in range(1, K):
        p = d2.clamp_min(0) + 1e-30
        pick = torch.multinomial(p / p.sum(-1, keepdim=True), 1, generator=g).squeeze(1)
        C[:, k] = X[ar, pick]
        d2 = torch.minimum(d2, (X - C[:, k:k + 1]).pow(2).sum(-1))
    prev = None
    xx = X.pow(2).sum(-1, keepdim=True)
    for _ in range(iters):
        dist = xx - 2.0 * X @ C.transpose(1, 2) + C.pow(2).sum(-1)[:, None, :]
        a = dist.argmin(-1)                                           # [nb][n]
        if prev is not None and torch.equal(a, prev):
            break
        prev = a
        sums = torch.zeros_like(C).scatter_add_(1, a[..., None].expand(-1, -1, G), X)
        cnt = torch.zeros((nb, K), dtype=X.dtype, device=dev).scatter_add_(
            1, a, torch.ones_like(a, dtype=X.dtype))
        newC = sums / cnt.clamp_min(1)[..., None]
        empty = cnt == 0
        if bool(empty.any()):
            fit = dist.gather(-1, a[..., None]).squeeze(-1)           # [nb][n]
            for bi in torch.nonzero(empty.any(-1)).flatten().tolist():
                ks = torch.nonzero(empty[bi]).flatten()
                worst = torch.topk(fit[bi], len(ks)).indices
                newC[bi, ks] = X[bi, worst]
        C = newC
    return C


def train_codebooks(cfg: LoopConfig, layer: int, device="cpu", dtype=torch.float64):
    """bf16 codebooks for one layer: (k_cb, v_cb), each [H_kv][n_blk][K][G]."""
    out = []
    for kind in ("k", "v"):
        x = gen_calibration_kv(cfg, layer, kind, device)
        if kind == "k" and cfg.tasq:
            z = _calib_joint(cfg, _calib_tasq(cfg, layer, x))
        else:
            z = _calib_joint(cfg, x)
        nb = cfg.H_kv * cfg.n_blk
        X = z.reshape(nb, -1, cfg.G).to(dtype)
        g = SeedPlan(cfg.index).gen(layer, "kmeans", device)
        C = _kmeans(X, cfg.K, cfg.kmeans_iters, g)
        out.append(C.view(cfg.H_kv, cfg.n_blk, cfg.K, cfg.G).to(torch.bfloat16).contiguous())
    return out[0], out[1]
