"""GPU parity of the importance-weighted k-means update (LoopVQ review,
eq. 3): fp64 sums against the oracle's from the same assignment, and the new
bf16 codebook bit-exact against the oracle's rounding (either neighbour where
the quotient sits within 1e-9 of a bf16 rounding midpoint)."""
import numpy as np
import pytest
import torch

import oracle as ref
from tests.helpers import build_inputs, np64, small_cfg
from tests.test_gpu_parity import _geom, _lib, _say

pytestmark = pytest.mark.gpu


def _near_midpoint(x):
    m, _ = np.frexp(x)
    f = np.abs(m) * 256.0
    return np.abs(f - np.floor(f) - 0.5) < 1e-9 * f


@pytest.mark.parametrize("G,T,H,B,N,tasq", [(16, 8, 2, 2, 333, False), (32, 4, 2, 2, 200, False),
                                           (16, 4, 2, 2, 300, True)])
def test_weighted_update(G, T, H, B, N, tasq):
    s = _lib()
    _say("k-means update G=%d T=%d H=%d B=%d N=%d tasq=%s" % (G, T, H, B, N, tasq))
    cfg = small_cfg(1, G=G, T_c=4, T=T, H_kv=H, H_q=H, B=B, N=N, n_s=4, tasq=tasq,
                    rho_k=(0.85,) * (T - 1), rho_v=(0.9,) * (T - 1), n_calib=1024, kmeans_iters=8)
    inp = build_inputs(cfg, 0, "cuda", kmeans=False)
    g = _geom(s, cfg)
    shp = (B, H, cfg.n_blk, N, cfg.chunks)
    idx = torch.zeros(shp, dtype=torch.uint8, device="cuda")
    pt = sigma = None
    if tasq:
        sigma = torch.zeros((B, N, T), dtype=torch.float16, device="cuda")
        pt = s.pretransform(inp["w"], inp["perm"], sigma)
    s.encode(g, inp["k"], inp["k_cb"], idx, pt=pt)
    rng = np.random.default_rng(500 + G + T + int(tasq))
    om = rng.lognormal(0.0, 1.0, size=shp).astype(np.float32)
    om[0, 0, 0, :5] = 0.0                                   # zero weights are legal
    weight = torch.from_numpy(om).cuda()
    K = cfg.K
    sums = torch.zeros((H, cfg.n_blk, K, G), dtype=torch.float64, device="cuda")
    wsum = torch.zeros((H, cfg.n_blk, K), dtype=torch.float64, device="cuda")
    # two calls over the two halves of the batch accumulate like one
    s.kmeans_accumulate(g, inp["k"][:1], idx[:1], sums, wsum, weight=weight[:1], pt=pt)
    s.kmeans_accumulate(g, inp["k"][1:], idx[1:], sums, wsum, weight=weight[1:],
                        pt=None if pt is None else s.pretransform(inp["w"], inp["perm"], sigma[1:]))
    cb_new = inp["k_cb"].clone()
    s.kmeans_finalize(g, sums, wsum, cb_new)
    torch.cuda.synchronize()

    k_all = np64(inp["k"])
    idx_np = idx.cpu().numpy().astype(np.int64)
    sig = None if sigma is None else sigma.double().cpu().numpy()
    worst = 0.0
    for h in range(H):
        for beta in range(cfg.n_blk):
            zs, ws, asg = [], [], []
            for b in range(B):
                x = k_all[b, h]
                if tasq:
                    w = inp["w"][h].double().cpu().numpy()
                    perm = inp["perm"][h].long().cpu().numpy()
                    x = np.stack([ref.tasq_forward(x[t], w, perm, sig[b][:, t]) for t in range(T)])
                zs.append(ref.joint_vectors(x, cfg.T_c, G)[beta].reshape(-1, G))
                ws.append(om[b, h, beta].reshape(-1))
                asg.append(idx_np[b, h, beta].reshape(-1))
            cb = np64(inp["k_cb"][h, beta])
            _, s_ref, w_ref = ref.weighted_kmeans_sums(np.concatenate(zs), np.concatenate(ws), cb,
                                                       assign=np.concatenate(asg))
            s_gpu = sums[h, beta].cpu().numpy()
            w_gpu = wsum[h, beta].cpu().numpy()
            scale = max(np.abs(s_ref).max(), 1e-300)
            err = max(np.abs(s_gpu - s_ref).max() / scale, np.abs(w_gpu - w_ref).max() / w_ref.max())
            worst = max(worst, err)
            assert err < 1e-12, (h, beta, err)
            q = np.where(w_ref[:, None] > 0, s_ref / np.where(w_ref > 0, w_ref, 1.0)[:, None], cb)
            want = np.where(w_ref[:, None] > 0, ref.bf16_round(q), cb)
            got = np64(cb_new[h, beta])
            diff = got != want
            if diff.any():
                assert np.all(_near_midpoint(q[diff])), "codebook differs away from a rounding midpoint"
    _say("  sums worst rel err %.3g" % worst)
