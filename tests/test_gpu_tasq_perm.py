"""GPU parity of the pre-transform permutation statistics (LoopVQ review,
section 3.3): the fp64 mean and covariance of the block-stacked scaled keys
against the oracle, the permutation grouped from the GPU covariance against
the oracle's, and encode + decode with that permutation against the oracle."""
import numpy as np
import pytest
import torch

import oracle as ref
from tests.helpers import build_inputs, small_cfg
from tests.test_gpu_parity import _check_encode_slice, _check_rows, _decode, _encode_all, _geom, _lib, _say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("G,T,H,B,N", [(16, 8, 2, 2, 300), (32, 4, 1, 3, 257)])
def test_covariance_and_permutation(G, T, H, B, N):
    s = _lib()
    _say("pre-transform covariance G=%d T=%d H=%d B=%d N=%d" % (G, T, H, B, N))
    cfg = small_cfg(1, G=G, T_c=4, T=T, H_kv=H, H_q=H, B=B, N=N, n_s=4, tasq=True,
                    rho_k=(0.85,) * (T - 1), rho_v=(0.9,) * (T - 1), n_calib=1024, kmeans_iters=8)
    inp = build_inputs(cfg, 0, "cuda")
    g = _geom(s, cfg)
    sigma = torch.zeros((B, N, T), dtype=torch.float16, device="cuda")
    mean, cov = s.tasq_covariance(g, inp["k"], inp["w"], sigma)
    torch.cuda.synchronize()
    c = cfg.c
    D = cfg.D
    k_all = inp["k"].double().cpu().numpy()                        # [B, H, T, N, D]
    sig = sigma.double().cpu().numpy()                              # [B, N, T]
    # sigma: the oracle's fp16 rounding of the per-(token, step) RMS
    for b in range(B):
        sref = ref.tasq_sigma(k_all[b])
        sbar = ref.fp16_round(sref)
        mism = sig[b] != sbar
        if mism.any():
            lo, hi = ref.fp16_round(sref * (1 - 1e-6)), ref.fp16_round(sref * (1 + 1e-6))
            assert np.all((lo != hi)[mism])
    perms = np.zeros((H, D), dtype=np.int64)
    worst = 0.0
    for h in range(H):
        w = inp["w"][h].double().cpu().numpy()
        for beta in range(cfg.n_blk):
            steps = slice(beta * 4, beta * 4 + 4)
            # tokens in (batch entry, token) order
            k_blk = np.concatenate([k_all[b, h, steps] for b in range(B)], axis=1)     # [T_c, B*N, D]
            s_blk = np.concatenate([sig[b][:, steps] for b in range(B)], axis=0)      # [B*N, T_c]
            y = ref.tasq_scaled_keys(k_blk, w, s_blk)
            mu_ref, cov_ref = ref.stacked_covariance(y)
            mu_g = mean[h, beta].cpu().numpy()
            cov_g = cov[h, beta].cpu().numpy()
            scale = np.abs(cov_ref).max()
            err = max(np.abs(cov_g - cov_ref).max() / scale,
                      np.abs(mu_g - mu_ref).max() / max(np.abs(mu_ref).max(), 1e-300))
            worst = max(worst, err)
            assert err < 1e-11, (h, beta, err)
            p_ref = ref.pair_grouped_permutation(cov_ref, 4, D, c)
            p_gpu = s.tasq_pair_permutation(cov[h, beta].cpu(), 4, D, c).numpy().astype(np.int64)
            assert p_gpu.tolist() == p_ref.tolist(), (h, beta)
            if beta == 0:
                perms[h] = p_gpu
    _say("  covariance worst rel err %.3g" % worst)

    # encode + decode with the derived permutation (one per kv-head, from block 0)
    inp["perm"] = torch.from_numpy(perms.astype(np.int16)).cuda()
    kidx, vidx, sigma2, pt = _encode_all(s, cfg, inp)
    out, lse = _decode(s, cfg, inp, kidx, vidx, pt)
    torch.cuda.synchronize()
    fails = 0
    for b in range(B):
        for h in range(H):
            rk, rv = _check_encode_slice(cfg, inp, kidx, vidx, sigma2, b, h, slice(None))
            fails += rk[2] + rv[2]
    assert fails == 0
    rows = [(b, hq, t) for b in range(B) for hq in range(H) for t in range(T)]
    w2 = _check_rows(cfg, inp, kidx, vidx, sigma2, out, lse, rows)
    _say("  decode with the derived permutation: worst rel err %.3g" % w2)
