#!/usr/bin/env python
"""LoopVQ hot-path benchmark on one MI355X.

One step = the whole hot path over one batch of synthetic, HBM-resident input:
encode the layer's K cache, encode its V cache (loop-axis VQ, nearest
codeword), then one fused decode-attention call that serves every loop step
of every block.  The default workload is the 0.5-bit looped-model slice
(B=32, 16 kv-heads / 16 q-heads, D=128, T=T_c=4, G=16, K=256, 8192 context
tokens + 4 bf16 sinks).

Prints one JSON line.  `value` is whole-step throughput in context tokens per
second per loop block (B * N * n_blk / step time); per-kernel rates, the
roofline of the dominant kernel (and of the decode kernel) and the CPU
oracle's rate on a bounded sample are attached.

`--config 5` instead runs the 24-layer workload as one flow (prefill encode of
every layer, then 256 decode calls over all layers with an 8-token page
encoded per layer every 8 calls) and prints its own JSON line.

`--finetune` times the codebook fine-tuning workload (causal attention over
the compressed cache and its backward into the codebooks, plus whole Adam
iterations on the toy looped stack) and prints its own JSON line.
"""
import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "decode-attn context tokens/s per loop block + % HBM peak; encode codes/s"
UNIT = "context tokens/s per loop block"


# Sources whose change invalidates a kernel's committed HBM-traffic figure.
# The figure is taken on the default workload (one q-head per kv-head, so the
# decode call runs decode_half.hip's kernel and decode.hip's merge); the plan
# in loopvq_api.cpp decides that, so it is part of the key too.
KERNEL_SOURCES = {
    "encode": ("encode.hip", "common.h", "kernels.h", "loopvq_api.cpp", "calib.hip"),
    "decode": ("decode.hip", "decode_fast.hip", "decode_half.hip", "common.h", "kernels.h", "loopvq_api.cpp",
               "calib.hip"),
}


def kernel_source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "sub_bit_loop_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current sources of that kernel and on this workload; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    e = d.get("kernels", {}).get(kernel)
    if not e or e.get("workload") != workload or e.get("source_hash") != kernel_source_hash(kernel):
        return None
    return e.get("bytes_per_launch")


# ----------------------------------------------------------------------------- CPU oracle leg

def _oracle_head(args):
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle as ref
    kx, vx, kc, vc, sk, sv, qs, T_c, theta = args
    with threadpool_limits(1):
        t0 = time.perf_counter()
        ki, _ = ref.encode(kx, kc, T_c)
        vi, _ = ref.encode(vx, vc, T_c)
        for t in range(qs.shape[0]):
            ref.decode_attn_row(qs[t], t, ki, vi, kc, vc, sk, sv, T_c, theta)
        return time.perf_counter() - t0, ki.size + vi.size


def cpu_baseline(cfg, inp, n_tok, n_b):
    """Oracle on batch entries 0..n_b-1, every kv-head, the first n_tok context
    tokens: K and V encode plus decode of every loop step over those tokens."""
    from concurrent.futures import ProcessPoolExecutor
    import multiprocessing as mp
    import torch
    f = lambda t: t.float().cpu().double().numpy()
    jobs = []
    for b in range(n_b):
        for h in range(cfg.H_kv):
            hq = h * (cfg.H_q // cfg.H_kv)
            jobs.append((f(inp["k"][b, h, :, :n_tok]), f(inp["v"][b, h, :, :n_tok]), f(inp["k_cb"][h]),
                         f(inp["v_cb"][h]), f(inp["sink_k"][b, h]), f(inp["sink_v"][b, h]),
                         f(inp["q"][b, hq]), cfg.T_c, cfg.theta))
    cores = len(os.sched_getaffinity(0))
    workers = max(1, min(cores, len(jobs), 15))      # with the parent, at most 16 processes
    t0 = time.perf_counter()
    with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn")) as ex:
        res = list(ex.map(_oracle_head, jobs))
    wall = time.perf_counter() - t0
    codes = sum(r[1] for r in res)
    # One q-head per kv-head is decoded; with GQA the other heads of a group
    # are not re-run (the default workload has none).
    tokens_blocks = n_b * n_tok * cfg.n_blk
    return {
        "value": tokens_blocks / wall,
        "unit": UNIT,
        "cores": workers,
        "kind": "oracle",
        "sample": "batch entries 0..%d, all %d kv-heads, first %d context tokens: fp64 NumPy encode of K and V "
                  "(%d codes) + decode attention of every loop step over those tokens and the %d sinks; "
                  "one process per (batch entry, kv-head), %d at a time, 1 BLAS thread each; wall %.1f s"
                  % (n_b - 1, cfg.H_kv, n_tok, codes, cfg.n_s, workers, wall),
        "encode_codes_per_s": codes / wall,
    }


# ----------------------------------------------------------------------------- HBM stream rates

def hbm_stream(torch, nbytes=1 << 30):
    """Time a plain 16-byte-per-lane streaming read and device copy of nbytes
    (libloopvq_calib.so).  Returns GB/s of bytes read, and of bytes read +
    written for the copy.  Their counter readings also calibrate FETCH_SIZE
    and WRITE_SIZE for kernels with the same access width."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "sub_bit_loop_amd", "libloopvq_calib.so"))
    lib.loopvq_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]
    lib.loopvq_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
    lib.loopvq_calib_read_sink_words.argtypes = [ctypes.c_uint64]
    lib.loopvq_calib_read_sink_words.restype = ctypes.c_uint64
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    sink = torch.empty(int(lib.loopvq_calib_read_sink_words(nbytes)), dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream

    def timed(fn, reps):
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def rd():
        if lib.loopvq_calib_read(src.data_ptr(), nbytes, sink.data_ptr(), st) != 0:
            raise RuntimeError("calib read launch failed")

    def cp():
        if lib.loopvq_calib_copy(src.data_ptr(), dst.data_ptr(), nbytes, st) != 0:
            raise RuntimeError("calib copy launch failed")
    r_ms = timed(rd, 10)
    c_ms = timed(cp, 5)
    del src, dst, sink
    return {"read_GBps": nbytes / r_ms / 1e6, "copy_GBps": 2 * nbytes / c_ms / 1e6, "bytes": nbytes,
            "note": "calib_read_kernel / calib_copy_kernel, 16 B per lane, grid-stride"}


# ----------------------------------------------------------------------------- workload 5 flow

def workload5(args, torch, lv, cfg):
    """The 24-layer workload as one flow: prefill-encode every layer (inputs
    generated untimed, one layer at a time), then `decode_steps` decode calls
    over all layers, each serving every loop step, with one 8-token page per
    layer encoded after every `page` calls (the page conversion of the
    review's section 3.4 step 2).  Prints one JSON line."""
    from synth import build_inputs
    B, H, L = cfg.B, cfg.H_kv, cfg.layers
    g = lv.geom(cfg.D, cfg.T, cfg.T_c, cfg.G, cfg.K, cfg.H_kv, cfg.H_q, cfg.theta)
    n_pages = cfg.decode_steps // cfg.page
    N_cap = cfg.N + cfg.page * n_pages
    rope = lv.rope_table(cfg.n_s + N_cap, cfg.D, cfg.theta)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    layers, enc_ms, gen_s = [], 0.0, 0.0
    for layer in range(L):
        t = time.time()
        inp = build_inputs(cfg, layer, "cuda")
        torch.cuda.synchronize()
        gen_s += time.time() - t
        shp = (B, H, cfg.n_blk, N_cap, cfg.chunks)
        lay = dict(q=inp["q"], k_cb=inp["k_cb"], v_cb=inp["v_cb"], sk=inp["sink_k"], sv=inp["sink_v"],
                   w=inp["w"], perm=inp["perm"],
                   kidx=torch.zeros(shp, dtype=torch.uint8, device="cuda"),
                   vidx=torch.zeros(shp, dtype=torch.uint8, device="cuda"),
                   sigma=torch.zeros((B, N_cap, cfg.T), dtype=torch.float16, device="cuda"))
        lay["pt"] = lv.pretransform(lay["w"], lay["perm"], lay["sigma"])
        e0, e1 = ev(), ev()
        e0.record()
        lv.encode(g, inp["k"], lay["k_cb"], lay["kidx"], pt=lay["pt"])
        lv.encode(g, inp["v"], lay["v_cb"], lay["vidx"])
        e1.record()
        torch.cuda.synchronize()
        enc_ms += e0.elapsed_time(e1)
        # the page source: the layer's last 8 tokens (their content does not change the timing)
        lay["page_k"] = inp["k"][:, :, :, -cfg.page:].clone()
        lay["page_v"] = inp["v"][:, :, :, -cfg.page:].clone()
        del inp
        torch.cuda.empty_cache()
        layers.append(lay)
        print("layer %d encoded (%.1f ms); generation so far %.0f s" % (layer, e0.elapsed_time(e1), gen_s),
              file=sys.stderr, flush=True)

    ws = torch.empty(max(4, lv.decode_workspace_bytes(g, B, N_cap, 0, cfg.T)), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, cfg.H_q, cfg.T, cfg.D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, cfg.H_q, cfg.T), dtype=torch.float32, device="cuda")

    def decode_all(N):
        for lay in layers:
            lv.decode_attn(g, lay["q"], lay["kidx"], lay["vidx"], lay["k_cb"], lay["v_cb"], lay["sk"], lay["sv"],
                           rope, N=N, pt=lay["pt"], out=out, lse=lse, workspace=ws)

    decode_all(cfg.N)                       # warm-up
    torch.cuda.synchronize()
    N, tok_blocks = cfg.N, 0
    dec_ev, page_ev = [], []
    t0, t1 = ev(), ev()
    t0.record()
    for call in range(cfg.decode_steps):
        a, b = ev(), ev()
        a.record()
        decode_all(N)
        b.record()
        dec_ev.append((a, b))
        tok_blocks += B * N * cfg.n_blk * L
        if (call + 1) % cfg.page == 0:
            a, b = ev(), ev()
            a.record()
            for lay in layers:
                lv.encode(g, lay["page_k"], lay["k_cb"], lay["kidx"], tok0=N, pt=lay["pt"])
                lv.encode(g, lay["page_v"], lay["v_cb"], lay["vidx"], tok0=N)
            b.record()
            page_ev.append((a, b))
            N += cfg.page
        if (call + 1) % 64 == 0:
            torch.cuda.synchronize()
            print("decode call %d done" % (call + 1), file=sys.stderr, flush=True)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    dec_ms = sum(a.elapsed_time(b) for a, b in dec_ev)
    page_ms = sum(a.elapsed_time(b) for a, b in page_ev)
    idx_bytes = sum(B * H * cfg.n_blk * (cfg.N + cfg.page * (c // cfg.page)) * 2 * cfg.chunks * L
                    for c in range(cfg.decode_steps))
    codes_prefill = 2 * B * H * cfg.n_blk * cfg.N * cfg.chunks * L
    workload = ("config 5 (%s): %d layers x B=%d, %d kv-heads / %d q-heads, D=%d, T=T_c=%d, G=%d, K=%d, "
                "keys pre-transformed; prefill %d tokens + %d sinks, then %d decode calls with an %d-token "
                "page encoded every %d calls" % (cfg.name, L, B, H, cfg.H_q, cfg.D, cfg.T, cfg.G, cfg.K, cfg.N,
                                                 cfg.n_s, cfg.decode_steps, cfg.page, cfg.page))
    dec_gbs = idx_bytes / (dec_ms * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": tok_blocks / (dec_ms * 1e-3),
        "unit": UNIT,
        "n_gpus": 1,
        "steps": cfg.decode_steps,
        "warmup": 1,
        "ms_per_step": total_ms / cfg.decode_steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "global_batch": B, "seq_len": cfg.N + cfg.n_s,
                   "step": "one decode call over all %d layers (every loop step) plus, every %d calls, a page "
                           "encode per layer" % (L, cfg.page)},
        "prefill_encode": {"ms_per_layer": enc_ms / L, "codes_per_s": codes_prefill / (enc_ms * 1e-3),
                           "note": "K (pre-transform, sigma) + V of one layer, %d codes" % (codes_prefill // L)},
        "decode": {"ms_per_call_per_layer": dec_ms / (cfg.decode_steps * L), "index_GBps": dec_gbs,
                   "hbm_frac_index_bytes": dec_gbs / HBM_PEAK_GBS},
        "page_encode": {"events": len(page_ev), "ms_per_event_all_layers": page_ms / max(1, len(page_ev)),
                        "ms_per_layer": page_ms / max(1, len(page_ev) * L)},
        "timed_flow_s": total_ms / 1e3,
        "input_generation_s": gen_s,
    }
    print(json.dumps(res), flush=True)


# ----------------------------------------------------------------------------- fine-tuning workload

FP32_MATRIX_PEAK_TFLOPS = 157.3    # published dense fp32 matrix-core rate


def _oracle_vjp_sample(args):
    import torch as _t
    from threadpoolctl import threadpool_limits
    import oracle as ref
    q, ki, vi, kc, vc, sk, sv, T_c, dout, theta = args
    with threadpool_limits(1):
        _t.set_num_threads(1)
        t0 = time.perf_counter()
        ref.attention_vjp(q, ki, vi, kc, vc, sk, sv, T_c, dout, 0, theta)
        return time.perf_counter() - t0


def finetune_flow(args, torch, lv):
    """Loop-aware codebook fine-tuning (review section 3.2): one calibration
    sequence per iteration, the toy looped stack over the compressed cache of
    the 0.5-bit slice's geometry.  Times the compressed-attention forward and
    backward calls and whole iterations (re-encode, stack forward, KL,
    backward, Adam).  Prints one JSON line."""
    from synth import build_inputs, config_by_index, gen_toy_stack
    from dataclasses import replace
    from sub_bit_loop_amd import finetune as ft
    N, vocab = args.ft_tokens, 4096
    cfg = replace(config_by_index(2), B=1, N=N)
    inp = build_inputs(cfg, 0, "cuda")
    g = lv.geom(cfg.D, cfg.T, cfg.T_c, cfg.G, cfg.K, cfg.H_kv, cfg.H_q, cfg.theta)
    shp = (1, cfg.H_kv, cfg.n_blk, N, cfg.chunks)
    kidx = torch.empty(shp, dtype=torch.uint8, device="cuda")
    vidx = torch.empty(shp, dtype=torch.uint8, device="cuda")
    lv.encode(g, inp["k"], inp["k_cb"], kidx)
    lv.encode(g, inp["v"], inp["v_cb"], vidx)
    rope = lv.rope_table_f32(cfg.n_s + N, cfg.D, cfg.theta)
    gq = torch.Generator(device="cuda").manual_seed(5)
    q = torch.randn((1, cfg.H_q, cfg.T, N, cfg.D), generator=gq, device="cuda")
    dout = torch.randn((1, cfg.H_q, cfg.T, N, cfg.D), generator=gq, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((1, cfg.H_q, cfg.T, N), device="cuda")
    dq = torch.empty_like(q)
    dk = torch.empty(inp["k_cb"].shape, device="cuda")
    dv = torch.empty_like(dk)
    ws = torch.empty(cfg.H_q * cfg.T * N * 4, dtype=torch.uint8, device="cuda")
    sk, sv = inp["sink_k"], inp["sink_v"]

    def fwd():
        lv.prefill_attn(g, q, kidx, vidx, inp["k_cb"], inp["v_cb"], sk, sv, rope, out=out, lse=lse)

    def bwd():
        lv.prefill_attn_backward(g, q, kidx, vidx, inp["k_cb"], inp["v_cb"], sk, sv, rope, out, lse, dout,
                                 d_q=dq, d_k_cb=dk, d_v_cb=dv, workspace=ws)

    def timed(fn, reps):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    fwd_ms = timed(fwd, args.steps)
    bwd_ms = timed(bwd, args.steps)
    pairs = cfg.H_q * cfg.T * (N * (N + 1) // 2 + N * cfg.n_s)      # (query, key) pairs of one call
    D = cfg.D
    fwd_tf = pairs * 4 * D / (fwd_ms * 1e-3) / 1e12
    bwd_tf = pairs * 8 * D / (bwd_ms * 1e-3) / 1e12

    if bwd_ms >= fwd_ms:
        dom_name, dom_tf, dom_ms, dom_flop = ("loopvq_prefill_attn_backward (prefill_bwd_kv_mfma_kernel V and K "
                                              "passes + prefill_bwd_q_mfma_kernel + delta)", bwd_tf, bwd_ms,
                                              pairs * 8 * D)
    else:
        dom_name, dom_tf, dom_ms, dom_flop = ("loopvq_prefill_attn (prefill_fwd_mfma_kernel)", fwd_tf, fwd_ms,
                                              pairs * 4 * D)

    toy = gen_toy_stack(cfg, 0, "cuda", vocab=vocab, B=1)
    stack = ft.ToyLoopedStack(toy["Wq"], toy["Wo"], toy["Wu"], cfg.H_q, cfg.D, cfg.T, cfg.n_s, rope)
    iters = max(2, args.steps // 2)
    ft.finetune_codebooks(stack, g, toy["x"], inp["k"], inp["v"], sk, sv, inp["k_cb"], inp["v_cb"], iters=1)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    _, _, Js = ft.finetune_codebooks(stack, g, toy["x"], inp["k"], inp["v"], sk, sv, inp["k_cb"], inp["v_cb"],
                                     iters=iters)
    b.record()
    torch.cuda.synchronize()
    it_ms = a.elapsed_time(b) / iters

    cpu = None
    if not args.no_cpu_baseline:
        # oracle forward + backward (fp64 autograd) of every q-head and loop
        # step over the first n tokens, one process per q-head
        from concurrent.futures import ProcessPoolExecutor
        import multiprocessing as mp
        n = min(N, args.ft_cpu_tokens)
        f64 = lambda t: t.detach().cpu().double()
        jobs = [(f64(q[:, h:h + 1, :, :n]), kidx[:, h:h + 1, :, :n].long().cpu(),
                 vidx[:, h:h + 1, :, :n].long().cpu(), f64(inp["k_cb"][h:h + 1]), f64(inp["v_cb"][h:h + 1]),
                 f64(sk[:, h:h + 1]), f64(sv[:, h:h + 1]), cfg.T_c, f64(dout[:, h:h + 1, :, :n]), cfg.theta)
                for h in range(cfg.H_q)]
        # each worker imports torch, which opens the GPU device: stay well inside
        # the per-GPU process limit
        workers = max(1, min(len(os.sched_getaffinity(0)), len(jobs), 8))
        t0 = time.perf_counter()
        with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn")) as ex:
            list(ex.map(_oracle_vjp_sample, jobs))
        wall = time.perf_counter() - t0
        sp = cfg.H_q * cfg.T * (n * (n + 1) // 2 + n * cfg.n_s)
        cpu = {"value": sp / wall, "unit": "attention (query, key) pairs/s, forward + backward", "cores": workers,
               "kind": "oracle",
               "sample": "all %d q-heads and %d loop steps, first %d tokens + %d sinks: fp64 torch causal attention "
                         "over the rebuilt cache and its autograd backward (%d pairs); one process per q-head, %d "
                         "at a time, 1 thread each; wall %.1f s" % (cfg.H_q, cfg.T, n, cfg.n_s, sp, workers, wall)}
    workload = ("codebook fine-tuning (section 3.2): one calibration sequence per iteration, %d kv-heads / %d "
                "q-heads, D=%d, T=T_c=%d, G=%d, K=%d, %d tokens + %d sinks; toy looped stack d=%d, vocab %d"
                % (cfg.H_kv, cfg.H_q, cfg.D, cfg.T, cfg.G, cfg.K, N, cfg.n_s, cfg.H_q * cfg.D, vocab))
    res = {
        "metric": "codebook fine-tuning: compressed-attention forward + backward (query, key) pairs/s",
        "value": pairs / ((fwd_ms + bwd_ms) * 1e-3),
        "unit": "attention (query, key) pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": fwd_ms + bwd_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": workload, "global_batch": 1, "seq_len": N + cfg.n_s,
                   "step": "loopvq_prefill_attn + loopvq_prefill_attn_backward over every loop step"},
        "forward": {"ms_per_call": fwd_ms, "tflops": fwd_tf, "flop_per_pair": 4 * D},
        "backward": {"ms_per_call": bwd_ms, "tflops": bwd_tf, "flop_per_pair": 8 * D,
                     "executed_flop_per_pair": 16 * D,
                     "note": "S = QK^T is recomputed in each of the three backward kernels and dP in two"},
        "roofline": {"kernel": dom_name, "bound": "mfma", "achieved": dom_tf, "peak": FP32_MATRIX_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": dom_tf / FP32_MATRIX_PEAK_TFLOPS, "traffic": None,
                     "algorithmic_flop_per_launch": dom_flop, "avg_launch_ms": dom_ms, "dtype": "f32"},
        "iteration": {"ms": it_ms, "objective": Js,
                      "note": "re-encode K and V, toy stack forward over the rebuilt cache (4 compressed-attention "
                              "calls), KL against the precise run, backward, Adam (lr 1e-3)"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


# ----------------------------------------------------------------------------- GPU leg

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2,
                    help="workload index: 1-4 single layer, 5 the 24-layer prefill + decode flow")
    ap.add_argument("--tc", type=int, default=None,
                    help="steps per block T_c override for workloads 1-4 (1: per-step codebooks, as for the "
                         "layers outside the loop)")
    ap.add_argument("--cpu-tokens", type=int, default=8192, help="context tokens in the oracle sample")
    ap.add_argument("--cpu-batch", type=int, default=2, help="batch entries in the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--finetune", action="store_true",
                    help="time the codebook fine-tuning workload (compressed-attention forward + backward)")
    ap.add_argument("--ft-tokens", type=int, default=2048, help="tokens of the fine-tuning sequence")
    ap.add_argument("--ft-cpu-tokens", type=int, default=1536, help="tokens in the fine-tuning oracle sample")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the LoopVQ path has no multi-GPU step in this build "
              "(decode shards over batch x kv-heads with no communication); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import sub_bit_loop_amd as lv
    from synth import config_by_index
    from synth import build_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    lv.lib()
    torch.cuda.set_device(0)
    if args.finetune:
        finetune_flow(args, torch, lv)
        return
    cfg = config_by_index(args.config)
    if args.tc is not None:
        if cfg.layers != 1 or args.tc < 1 or cfg.T % args.tc or cfg.G % args.tc:
            print("--tc needs a single-layer workload and T_c dividing T and G", file=sys.stderr)
            sys.exit(2)
        cfg = dataclasses.replace(cfg, T_c=args.tc)
    if cfg.layers != 1:
        workload5(args, torch, lv, cfg)
        return
    t_gen = time.time()
    inp = build_inputs(cfg, 0, "cuda")
    torch.cuda.synchronize()
    t_gen = time.time() - t_gen
    g = lv.geom(cfg.D, cfg.T, cfg.T_c, cfg.G, cfg.K, cfg.H_kv, cfg.H_q, cfg.theta)
    shp = (cfg.B, cfg.H_kv, cfg.n_blk, cfg.N, cfg.chunks)
    kidx = torch.empty(shp, dtype=torch.uint8, device="cuda")
    vidx = torch.empty(shp, dtype=torch.uint8, device="cuda")
    rope = lv.rope_table(cfg.n_s + cfg.N, cfg.D, cfg.theta)
    out = torch.empty((cfg.B, cfg.H_q, cfg.T, cfg.D), dtype=torch.float32, device="cuda")
    lse = torch.empty((cfg.B, cfg.H_q, cfg.T), dtype=torch.float32, device="cuda")
    ws = torch.empty(lv.decode_workspace_bytes(g, cfg.B, cfg.N, 0, cfg.T), dtype=torch.uint8, device="cuda")

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        lv.encode(g, inp["k"], inp["k_cb"], kidx)
        if ev is not None:
            ev[1].record()
        lv.encode(g, inp["v"], inp["v_cb"], vidx)
        if ev is not None:
            ev[2].record()
        lv.decode_attn(g, inp["q"], kidx, vidx, inp["k_cb"], inp["v_cb"], inp["sink_k"], inp["sink_v"], rope,
                       out=out, lse=lse, workspace=ws)
        if ev is not None:
            ev[3].record()

    stream = hbm_stream(torch)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        step(evs[i])
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_step = total_ms / args.steps
    enc_ms = sum(e[0].elapsed_time(e[1]) + e[1].elapsed_time(e[2]) for e in evs) / (2 * args.steps)
    dec_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps

    # Per-step usage (the review's kernel serves one loop step per call and
    # re-reads the index rows every step): T calls with n_steps = 1.
    ps_ms = None
    if cfg.T > 1:
        qs = [inp["q"][:, :, t:t + 1].contiguous() for t in range(cfg.T)]
        outs = torch.empty((cfg.B, cfg.H_q, 1, cfg.D), dtype=torch.float32, device="cuda")
        lses = torch.empty((cfg.B, cfg.H_q, 1), dtype=torch.float32, device="cuda")
        ws1 = torch.empty(max(4, lv.decode_workspace_bytes(g, cfg.B, cfg.N, 0, 1)), dtype=torch.uint8,
                          device="cuda")

        def per_step():
            for t in range(cfg.T):
                lv.decode_attn(g, qs[t], kidx, vidx, inp["k_cb"], inp["v_cb"], inp["sink_k"], inp["sink_v"],
                               rope, step0=t, out=outs, lse=lses, workspace=ws1)
        per_step()
        torch.cuda.synchronize()
        p0 = torch.cuda.Event(enable_timing=True)
        p1 = torch.cuda.Event(enable_timing=True)
        reps = max(1, min(args.steps, 10))
        p0.record()
        for _ in range(reps):
            per_step()
        p1.record()
        torch.cuda.synchronize()
        ps_ms = p0.elapsed_time(p1) / reps

    units = cfg.B * cfg.H_kv * cfg.N * cfg.n_blk                  # decode units per call
    codes_per_call = cfg.B * cfg.H_kv * cfg.n_blk * cfg.N * cfg.chunks
    idx_bytes = 2 * cfg.chunks                                     # K + V index bytes per unit
    dec_bytes = units * idx_bytes
    enc_bytes = codes_per_call * (2 * cfg.G + 1)                   # bf16 joint vector in, 1 byte out
    dec_gbs = dec_bytes / (dec_ms * 1e-3) / 1e9
    enc_gbs = enc_bytes / (enc_ms * 1e-3) / 1e9
    workload = ("config %d (%s): B=%d, %d kv-heads / %d q-heads, D=%d, T=%d, T_c=%d, G=%d, K=%d, N=%d + %d sinks"
                % (cfg.index, cfg.name, cfg.B, cfg.H_kv, cfg.H_q, cfg.D, cfg.T, cfg.T_c, cfg.G, cfg.K, cfg.N, cfg.n_s))
    roof_dec = {"kernel": "loopvq decode_attn call (decode_kernel + merge_kernel)", "bound": "hbm",
                "achieved": dec_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dec_gbs / HBM_PEAK_GBS,
                "traffic": load_traffic("decode", workload),
                "algorithmic_bytes_per_launch": dec_bytes, "avg_launch_ms": dec_ms,
                "frac_of_measured_read": dec_gbs / stream["read_GBps"]}
    roof_enc = {"kernel": "loopvq encode call (encode_kernel)", "bound": "hbm",
                "achieved": enc_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": enc_gbs / HBM_PEAK_GBS,
                "traffic": load_traffic("encode", workload),
                "algorithmic_bytes_per_launch": enc_bytes, "avg_launch_ms": enc_ms,
                "frac_of_measured_read": enc_gbs / stream["read_GBps"],
                "mfma_tflops": 2.0 * cfg.K * cfg.G * codes_per_call / (enc_ms * 1e-3) / 1e12,
                "mfma_frac_of_bf16_peak": 2.0 * cfg.K * cfg.G * codes_per_call / (enc_ms * 1e-3) / 2.5e15}
    dominant = roof_enc if 2 * enc_ms >= dec_ms else roof_dec
    res = {
        "metric": METRIC,
        "value": cfg.B * cfg.N * cfg.n_blk / (ms_step * 1e-3),
        "unit": UNIT,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "global_batch": cfg.B, "seq_len": cfg.N + cfg.n_s,
                   "step": "encode K + encode V + decode attention of all %d loop steps" % cfg.T},
        "decode": {"ms_per_call": dec_ms, "context_tokens_per_s_per_block": cfg.B * cfg.N * cfg.n_blk / (dec_ms * 1e-3),
                   "units_per_s": units / (dec_ms * 1e-3), "index_GBps": dec_gbs,
                   "hbm_frac_index_bytes": dec_gbs / HBM_PEAK_GBS},
        "encode": {"ms_per_call": enc_ms, "codes_per_s": codes_per_call / (enc_ms * 1e-3), "GBps": enc_gbs},
        "decode_per_step": None if ps_ms is None else {
            "ms_all_steps": ps_ms, "calls": cfg.T, "vs_fused": ps_ms / dec_ms,
            "note": "one call per loop step (n_steps = 1), each re-reading the index rows"},
        "roofline": dominant,
        "roofline_decode": roof_dec,
        "hbm_stream": stream,
        "input_generation_s": t_gen,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, inp, min(args.cpu_tokens, cfg.N), max(1, min(args.cpu_batch, cfg.B)))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
