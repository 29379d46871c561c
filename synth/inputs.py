"""One layer's complete input set (caches, sinks, queries, codebooks, and the
key pre-transform's parameters when the workload uses it)."""
import torch

from .configs import LoopConfig
from .generator import gen_kv_layer, gen_queries, gen_sinks, gen_tasq_params
from .codebooks import train_codebooks


def random_codebooks(cfg: LoopConfig, seed: int, device, scale: float = 1.0):
    """bf16 N(0, scale^2) codebooks [H_kv][n_blk][K][G] for K and V (tests of
    the encode/decode machinery that do not need trained codebooks)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    shp = (cfg.H_kv, cfg.n_blk, cfg.K, cfg.G)
    kc = (torch.randn(shp, generator=g) * scale).to(torch.bfloat16)
    vc = (torch.randn(shp, generator=g) * scale).to(torch.bfloat16)
    return kc.to(device), vc.to(device)


def build_inputs(cfg: LoopConfig, layer: int = 0, device="cuda", kmeans: bool = True, cb_seed: int = 1):
    """All inputs of one layer on `device`, as a dict: k, v, sink_k, sink_v,
    q, k_cb, v_cb (+ w, perm for pre-transformed keys)."""
    k = gen_kv_layer(cfg, layer, "k", device)
    v = gen_kv_layer(cfg, layer, "v", device)
    sk, sv = gen_sinks(cfg, layer, device)
    q = gen_queries(cfg, layer, device)
    if kmeans:
        kc, vc = train_codebooks(cfg, layer, device, dtype=torch.float32 if device != "cpu" else torch.float64)
    else:
        kc, vc = random_codebooks(cfg, cb_seed, device)
    d = dict(k=k, v=v, sink_k=sk, sink_v=sv, q=q, k_cb=kc, v_cb=vc)
    if cfg.tasq:
        w, perm = gen_tasq_params(cfg, layer, device)
        d.update(w=w, perm=perm)
    return d
