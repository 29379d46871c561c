#!/usr/bin/env python
"""LoopVQ hot-path benchmark on one MI355X.

Default (`python bench.py`): the 24-layer workload with the keys' channel
pre-transform, as one flow on synthetic HBM-resident inputs:
  * prefill encode of every layer (65,536 tokens x batch 8; keys: per-token
    sigma, weights and permutation, then the loop-axis VQ; values: plain),
    timed per layer, inputs generated untimed;
  * then the timed steps: one step is one decode-attention call over all 24
    layers (each call serves all four loop steps of every kv-head), and after
    every 8th step an 8-token page per layer is encoded and appended (the page
    conversion of the review's section 3.4 step 2), 256 steps by default.
`value` is context tokens per second per loop block over the timed steps
(B * N * n_blk * layers per step, N growing with the pages).  Attached: the
median per-layer decode call with its HBM roofline on index bytes, the
prefill encode with its roofline, HBM stream rates, the CPU oracle on a
bounded sample of the same workload (timed on this host, and compared with the
GPU's results on that sample), and the 0.5-bit single-layer workload (batch
32, 8192 tokens) as a sub-object.

`--config N` (1-4) instead times one single-layer workload (encode K, encode V,
one fused decode call) and prints its own line; `--finetune` times the codebook
fine-tuning workload; `--write-traffic` turns two rocprofv3 counter runs
(FETCH_SIZE, WRITE_SIZE) of one workload into its entries of
profiles/traffic.json.
"""
import argparse
import dataclasses
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
# Packed-fp16 vector peak: 256 CUs x 2.4 GHz x one wave64 instruction per CU
# per clock x 64 lanes x 2 FMA (4 flop) = 157.3 TFLOP/s (the fp32 vector figure
# counts the same packed issue).
F16_VALU_PEAK_TFLOPS = 157.3
METRIC = "decode-attn context tokens/s per loop block + % HBM peak; encode codes/s"
UNIT = "context tokens/s per loop block"
OUT_TOL = 2e-3                      # max-abs error per output row, relative to the row's L2 norm

# Sources whose change invalidates a kernel's committed HBM-traffic figure
# (the host plan in loopvq_api.cpp picks the kernel, the calibration kernels
# give the counter scale factors).
KERNEL_SOURCES = {
    "decode_tasq": ("decode_tasq.hip", "decode.hip", "common.h", "kernels.h", "loopvq_api.cpp", "calib.hip"),
    "decode_half": ("decode_half.hip", "decode.hip", "common.h", "kernels.h", "loopvq_api.cpp", "calib.hip"),
    "encode": ("encode.hip", "common.h", "kernels.h", "loopvq_api.cpp", "calib.hip"),
}
# Which committed traffic entry belongs to which (workload, kernel) of the bench line.
TRAFFIC_ENTRIES = {
    (5, "decode"): ("decode_tasq", "decode_tasq@5"),
    (5, "encode"): ("encode", "encode_prefill_layer@5"),
    (2, "decode"): ("decode_half", "decode_half@2"),
    (2, "encode"): ("encode", "encode@2"),
}


def kernel_source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "sub_bit_loop_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(cfg_index, what):
    """HBM bytes per launch from profiles/traffic.json, if that entry was
    taken on the current sources of its kernel; else None."""
    kern, key = TRAFFIC_ENTRIES[(cfg_index, what)]
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    e = d.get("kernels", {}).get(key)
    if not e or e.get("source_hash") != kernel_source_hash(kern):
        return None
    return e.get("bytes_per_launch")


def host_cpu():
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return cores, model


def valu_roofline(units, T_c, D, gqa, ms, kernel):
    """The decode's arithmetic against the packed-fp16 vector peak (the unit
    the decode kernels are bound by at GQA 1): per (token, step, channel) of a
    unit, the key rotation (2 multiplies + 1 add, shared by the q-heads of a
    GQA group), the score product and the P.V product (2 flop each per
    q-head)."""
    flop = units * T_c * D * (3 + 4 * gqa)
    tf = flop / (ms * 1e-3) / 1e12
    return {"kernel": kernel, "bound": "alu", "achieved": tf, "peak": F16_VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": tf / F16_VALU_PEAK_TFLOPS, "algorithmic_flop_per_launch": flop,
            "algorithmic": "T_c * D * (3 + 4 * gqa) flop per (token, kv-head, block) unit: key rotation 3, "
                           "score 2 and P.V 2 per q-head, per step and channel",
            "note": "secondary view; the metric's roofline is the HBM one"}


def _median_ms(pairs):
    return statistics.median(a.elapsed_time(b) for a, b in pairs)


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
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return _median_ms(ev)

    def rd():
        if lib.loopvq_calib_read(src.data_ptr(), nbytes, sink.data_ptr(), st) != 0:
            raise RuntimeError("calib read launch failed")

    def cp():
        if lib.loopvq_calib_copy(src.data_ptr(), dst.data_ptr(), nbytes, st) != 0:
            raise RuntimeError("calib copy launch failed")
    r_ms = timed(rd, 10)
    c_ms = timed(cp, 6)
    del src, dst, sink
    return {"read_GBps": nbytes / r_ms / 1e6, "copy_GBps": 2 * nbytes / c_ms / 1e6, "bytes": nbytes,
            "note": "calib_read_kernel / calib_copy_kernel, 16 B per lane, grid-stride; median of 10 / 6 launches"}


def onchip_ceilings(torch):
    """Time the on-chip ceiling kernels of libloopvq_calib.so (LDS reads in
    the decode kernels' access patterns, vector and matrix arithmetic).
    Rates per CU per clock assume the 2.4 GHz peak engine clock."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "sub_bit_loop_amd", "libloopvq_calib.so"))
    lib.loopvq_calib_onchip.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p]
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    clk = 2.4e9
    st = torch.cuda.current_stream().cuda_stream
    out = {"clock_assumed_GHz": clk / 1e9, "compute_units": n_cu}

    def run(kind, mode, blocks, iters):
        sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")

        def go():
            if lib.loopvq_calib_onchip(kind, mode, blocks, iters, sink.data_ptr(), st) != 0:
                raise RuntimeError("calib on-chip launch failed")
        go()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
        for a, b in ev:
            a.record()
            go()
            b.record()
        torch.cuda.synchronize()
        return _median_ms(ev) * 1e-3

    lds = {0: ("ds_read_b128, conflict-free (lane l reads slot l)", 16),
           1: ("ds_read_b128, random 16-byte slots", 16),
           2: ("ds_read_b128, random 48-byte codeword rows, half per wave (c = 4 decode layout)", 16),
           3: ("ds_read_b64, random 8-byte slots", 8),
           4: ("ds_read_b64_tr_b16, random 8-byte slots", 8),
           5: ("ds_read_b128, lane pairs read the two halves of a random 32-byte codeword (pre-transform "
               "decode layout)", 16),
           6: ("ds_read_b128, lane pairs read the two halves of a random codeword at a 48-byte stride", 16),
           7: ("ds_bpermute_b32 from random source lanes", 4)}
    blocks = 4 * n_cu
    for mode, (name, width) in lds.items():
        iters = 4096
        t = run(0, mode, blocks, iters)
        out["lds_mode%d" % mode] = {"pattern": name,
                                    "B_per_clk_per_CU": blocks * 256 * iters * 16 * width / t / n_cu / clk}
    valu = {0: ("v_pk_fma_f16", 4), 1: ("v_dot2_f32_f16", 4), 2: ("v_fma_f32", 2), 3: ("v_min3_f32", None),
            4: ("v_med3_f32", None), 5: ("v_perm_b32", None), 6: ("v_mov_b32_dpp (row shuffle)", None),
            7: ("v_exp_f32", None), 8: ("v_add_f32", 1)}
    blocks = 8 * n_cu
    for mode, (name, flop) in valu.items():
        iters = 8192 if mode < 3 else 4096
        t = run(1, mode, blocks, iters)
        ops = blocks * 256 * iters * 16
        e = {"instruction": name, "lane_ops_per_clk_per_CU": ops / t / n_cu / clk,
             # wave instructions issued per SIMD, at the assumed clock
             "clk_per_wave_instruction_per_SIMD": t * clk / (ops / 64 / (n_cu * 4))}
        if flop:
            e["TFLOPs"] = ops * flop / t / 1e12
        out["valu_mode%d" % mode] = e
    mfma = {0: ("v_mfma_f32_16x16x32_bf16", 16384), 1: ("v_mfma_f32_32x32x16_bf16", 32768),
            2: ("v_mfma_f32_32x32x8_bf16", 16384)}
    for mode, (name, flop) in mfma.items():
        iters = 8192
        t = run(2, mode, blocks, iters)
        per_simd = blocks * 4 * iters * 4 / (n_cu * 4)   # wave instructions issued per SIMD
        out["mfma_mode%d" % mode] = {"instruction": name,
                                     "TFLOPs": blocks * 4 * iters * 4 * flop / t / 1e12,
                                     "clk_per_instruction_per_SIMD": t * clk / per_simd}
    return out


# ----------------------------------------------------------------------------- CPU oracle workers
# These run in spawned processes that import only NumPy and the oracle.

def _f64_from_bf16_bits(bits):
    import numpy as np
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _oracle_encode_job(args):
    """Oracle encode of one token range: sigma over every head, then the
    pre-transformed keys and the plain values of the sampled heads."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle as ref
    kbits, vbits, kcb, vcb, w, perm, heads, T_c = args
    with threadpool_limits(1):
        t0 = time.perf_counter()
        k = _f64_from_bf16_bits(kbits)                   # [H, T, n, D]
        sbar = ref.fp16_round(ref.tasq_sigma(k))          # [n, T]
        res = []
        for i, h in enumerate(heads):
            ki, kt = ref.encode_tasq(k[h], kcb[i], T_c, w[i], perm[i], sbar)
            vi, vt = ref.encode(_f64_from_bf16_bits(vbits[i]), vcb[i], T_c)
            res.append((ki.astype(np.uint8), kt, vi.astype(np.uint8), vt))
        return time.perf_counter() - t0, sbar, res


def _oracle_decode_job(args):
    """Oracle decode attention of one (batch entry, q-head, loop step) row."""
    from threadpoolctl import threadpool_limits
    import oracle as ref
    q, t, ki, vi, kcb, vcb, sk, sv, T_c, theta, w, perm, sig = args
    with threadpool_limits(1):
        t0 = time.perf_counter()
        o, l = ref.decode_attn_row(q, t, ki, vi, kcb, vcb, sk, sv, T_c, theta, tasq=(w, perm, sig))
        return time.perf_counter() - t0, o, l


def _pool(workers):
    from concurrent.futures import ProcessPoolExecutor
    import multiprocessing as mp
    return ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"))


# ----------------------------------------------------------------------------- 24-layer workload

def workload5(args, torch, lv, cfg):
    """The 24-layer flow.  Returns the JSON line's dict."""
    import numpy as np
    from synth import build_inputs
    B, H, L, Hq = cfg.B, cfg.H_kv, cfg.layers, cfg.H_q
    steps = cfg.decode_steps if args.steps is None else args.steps
    warmup = 3 if args.warmup is None else args.warmup
    g = lv.geom(cfg.D, cfg.T, cfg.T_c, cfg.G, cfg.K, cfg.H_kv, cfg.H_q, cfg.theta)
    n_pages = steps // cfg.page
    N_cap = cfg.N + cfg.page * n_pages
    rope = lv.rope_table(cfg.n_s + N_cap + cfg.page, cfg.D, cfg.theta)
    stream = hbm_stream(torch)
    ceilings = onchip_ceilings(torch)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # CPU-sample inputs kept on the host: layer 0, batch entry 0 (keys of every
    # head for sigma, values of the sampled heads)
    heads = (0, 1)
    n_enc = min(cfg.N, args.cpu_tokens)
    keep = {}
    layers, enc_k, enc_v, enc_k1, enc_v1, gen_s = [], [], [], [], [], 0.0
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
        # The layer's prefill encode runs twice with the same inputs (the
        # second writes the same indices and sigma): the first launch after the
        # input generation runs 10-14% slower than any later one, so the kernel
        # time is the second call's; the first call's is reported beside it.
        for rep in range(2):
            e0, e1, e2 = ev(), ev(), ev()
            e0.record()
            lv.encode(g, inp["k"], lay["k_cb"], lay["kidx"], pt=lay["pt"])
            e1.record()
            lv.encode(g, inp["v"], lay["v_cb"], lay["vidx"])
            e2.record()
            torch.cuda.synchronize()
            (enc_k1 if rep == 0 else enc_k).append(e0.elapsed_time(e1))
            (enc_v1 if rep == 0 else enc_v).append(e1.elapsed_time(e2))
        # the page source: the layer's last 8 tokens (their content does not change the timing)
        lay["page_k"] = inp["k"][:, :, :, -cfg.page:].clone()
        lay["page_v"] = inp["v"][:, :, :, -cfg.page:].clone()
        if layer == 0 and not args.no_cpu_baseline:
            keep["k"] = inp["k"][0, :, :, :n_enc].view(torch.int16).cpu().numpy().view(np.uint16)
            keep["v"] = inp["v"][0, list(heads), :, :n_enc].view(torch.int16).cpu().numpy().view(np.uint16)
            keep["page_k"] = lay["page_k"][0].view(torch.int16).cpu().numpy().view(np.uint16)
            keep["page_v"] = lay["page_v"][0, list(heads)].view(torch.int16).cpu().numpy().view(np.uint16)
        del inp
        torch.cuda.empty_cache()
        layers.append(lay)
        print("layer %d encoded (K %.2f ms, V %.2f ms; first call %.2f, %.2f); generation so far %.0f s"
              % (layer, enc_k[-1], enc_v[-1], enc_k1[-1], enc_v1[-1], gen_s), file=sys.stderr, flush=True)

    ws = torch.empty(max(4, lv.decode_workspace_bytes(g, B, N_cap, 0, cfg.T)), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, cfg.T, cfg.D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, cfg.T), dtype=torch.float32, device="cuda")

    def decode_layer(lay, N, o=out, ls=lse):
        lv.decode_attn(g, lay["q"], lay["kidx"], lay["vidx"], lay["k_cb"], lay["v_cb"], lay["sk"], lay["sv"],
                       rope, N=N, pt=lay["pt"], out=o, lse=ls, workspace=ws)

    for _ in range(warmup):
        for lay in layers:
            decode_layer(lay, cfg.N)
    torch.cuda.synchronize()

    # timed steps: one decode call over every layer (+ a page encode every 8 steps)
    N, tok_blocks = cfg.N, 0
    lay_ev, page_ev = [], []
    t0, t1 = ev(), ev()
    torch.cuda.synchronize()
    t0.record()
    for call in range(steps):
        for lay in layers:
            a, b = ev(), ev()
            a.record()
            decode_layer(lay, N)
            b.record()
            lay_ev.append((a, b, N))
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
            print("decode step %d done" % (call + 1), file=sys.stderr, flush=True)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)

    # Per-step usage on layer 0 at the final context (outside the timed flow):
    # T calls with n_steps = 1, each re-reading the index rows; median of 20.
    lay0 = layers[0]
    qs = [lay0["q"][:, :, t:t + 1].contiguous() for t in range(cfg.T)]
    outs = torch.empty((B, Hq, 1, cfg.D), dtype=torch.float32, device="cuda")
    lses = torch.empty((B, Hq, 1), dtype=torch.float32, device="cuda")

    def per_step():
        for t in range(cfg.T):
            lv.decode_attn(g, qs[t], lay0["kidx"], lay0["vidx"], lay0["k_cb"], lay0["v_cb"], lay0["sk"], lay0["sv"],
                           rope, N=N, pt=lay0["pt"], step0=t, out=outs, lse=lses, workspace=ws)
    per_step()
    fev = [(ev(), ev()) for _ in range(20)]
    pev = [(ev(), ev()) for _ in range(20)]
    for (a, b), (c, d) in zip(fev, pev):
        a.record()
        decode_layer(lay0, N)
        b.record()
        c.record()
        per_step()
        d.record()
    torch.cuda.synchronize()
    fused_ms = _median_ms(fev)
    ps_ms = _median_ms(pev)

    # per-layer decode calls: median over every (step, layer) call
    lay_ms = [a.elapsed_time(b) for a, b, _ in lay_ev]
    dec_med = statistics.median(lay_ms)
    dec_mean = statistics.fmean(lay_ms)
    units_mean = statistics.fmean(B * H * n * cfg.n_blk for _, _, n in lay_ev)
    idx_bytes_mean = units_mean * 2 * cfg.chunks                    # K + V index bytes per call
    dec_gbs = idx_bytes_mean / (dec_med * 1e-3) / 1e9
    page_ms = [a.elapsed_time(b) for a, b in page_ev]

    # prefill encode of one layer: sigma + keys, then values (median over the layers)
    codes_layer = cfg.codes_per_layer()
    x_bytes = cfg.B * cfg.H_kv * cfg.T * cfg.N * cfg.D * 2            # one of K or V, bf16
    sig_bytes = cfg.B * cfg.N * cfg.T * 2
    enc_bytes = 3 * x_bytes + codes_layer + sig_bytes                 # K read twice (sigma, encode), V once
    enc_layer = [a + b for a, b in zip(enc_k, enc_v)]
    enc_med = statistics.median(enc_layer)
    enc_gbs = enc_bytes / (enc_med * 1e-3) / 1e9
    enc_tf = 2.0 * cfg.K * cfg.G * codes_layer / (enc_med * 1e-3) / 1e12

    workload = ("config 5 (%s): %d layers x B=%d, %d kv-heads / %d q-heads, D=%d, T=T_c=%d, G=%d, K=%d, keys "
                "pre-transformed; prefill %d tokens + %d sinks, then %d decode steps with an %d-token page per "
                "layer encoded every %d steps" % (cfg.name, L, B, H, Hq, cfg.D, cfg.T, cfg.G, cfg.K, cfg.N,
                                                  cfg.n_s, steps, cfg.page, cfg.page))
    roof_dec = {"kernel": "decode_tasq_kernel<4> (+ merge_kernel), one layer per launch", "bound": "hbm",
                "achieved": dec_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dec_gbs / HBM_PEAK_GBS,
                "traffic": load_traffic(5, "decode"),
                "algorithmic_bytes_per_launch": idx_bytes_mean,
                "algorithmic": "64 index bytes (K + V) per (batch, kv-head, token, block) unit; %.4g units per "
                               "launch on average over the steps" % units_mean,
                "launch_ms_median": dec_med, "launch_ms_mean": dec_mean, "launches": len(lay_ms),
                "frac_of_measured_read": dec_gbs / stream["read_GBps"]}
    roof_enc = {"kernel": "prefill encode of one layer: sigma_kernel + encode_kernel<16,4,true> (keys) + "
                          "encode_kernel<16,4,false> (values)", "bound": "hbm",
                "achieved": enc_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": enc_gbs / HBM_PEAK_GBS,
                "traffic": load_traffic(5, "encode"),
                "algorithmic_bytes_per_launch": enc_bytes,
                "algorithmic": "33 B per code (32 B of bf16 joint vector + 1 index byte), the keys read once more "
                               "for sigma, 2 B of sigma per (token, step)",
                "launch_ms_median": enc_med, "keys_ms_median": statistics.median(enc_k),
                "values_ms_median": statistics.median(enc_v),
                "timing": "second call of each layer's prefill encode (same inputs); median over the layers",
                "first_call_ms_median": statistics.median([a + b for a, b in zip(enc_k1, enc_v1)]),
                "codes_per_s": codes_layer / (enc_med * 1e-3),
                "mfma_tflops": enc_tf, "mfma_frac_of_bf16_peak": enc_tf / BF16_MFMA_PEAK_TFLOPS}
    res = {
        "metric": METRIC,
        "value": tok_blocks / (total_ms * 1e-3),
        "unit": UNIT,
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": total_ms / steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "global_batch": B, "seq_len": cfg.N + cfg.n_s,
                   "step": "one decode-attention call per layer over all %d layers (all 4 loop steps), plus a "
                           "page encode per layer after every %d steps" % (L, cfg.page)},
        "roofline": roof_dec,
        "roofline_decode_valu": valu_roofline(units_mean, cfg.T_c, cfg.D, Hq // H, dec_med,
                                              "decode_tasq_kernel<4> (+ merge_kernel), one layer per launch"),
        "roofline_encode": roof_enc,
        "decode": {"ms_per_layer_call_median": dec_med,
                   "context_tokens_per_s_per_block": B * units_mean / (B * H) / (dec_med * 1e-3),
                   "units_per_s": units_mean / (dec_med * 1e-3), "index_GBps": dec_gbs,
                   "hbm_frac_index_bytes": dec_gbs / HBM_PEAK_GBS},
        "prefill_encode": {"ms_per_layer_median": enc_med, "codes_per_s": codes_layer / (enc_med * 1e-3),
                           "codes_per_layer": codes_layer,
                           "keys_with_sigma_ms_median": statistics.median(enc_k),
                           "values_ms_median": statistics.median(enc_v),
                           "first_call_ms_per_layer_median": statistics.median([a + b for a, b in zip(enc_k1, enc_v1)]),
                           "note": "the second of two identical calls per layer; the first launch after the input "
                                   "generation is reported as first_call"},
        "page_encode": {"events": len(page_ev),
                        "ms_per_event_all_layers_median": statistics.median(page_ms) if page_ms else None},
        "decode_per_step": {"ms_all_steps_median": ps_ms, "calls": cfg.T, "fused_ms_median_same_context": fused_ms,
                            "vs_fused": ps_ms / fused_ms,
                            "note": "layer 0 at the final context: one call per loop step (n_steps = 1, the "
                                    "one-step kernel variant), each re-reading the index rows"},
        "hbm_stream": stream,
        "onchip_ceilings": ceilings,
        "timed_s": total_ms / 1e3,
        "input_generation_s": gen_s,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline5(args, torch, lv, cfg, layers, keep, heads, n_enc, steps, rope, ws)
    return res


def cpu_baseline5(args, torch, lv, cfg, layers, keep, heads, n_enc, steps, rope, ws):
    """The oracle on a bounded sample of the 24-layer workload, timed on this
    host, and compared with the GPU on the same sample:
      encode: layer 0, batch entry 0, kv-heads 0 and 1, the first n_enc tokens
              (sigma over every head) plus one 8-token page;
      decode: batch entry 0, q-heads 0 and 1, every loop step, at layers 0, 11,
              23 and decode steps 0, steps/2, steps-1 (the context each had)."""
    import numpy as np
    cores, model = host_cpu()
    workers = max(1, min(cores, 16))
    f64 = lambda t: t.float().cpu().double().numpy()
    lay0 = layers[0]
    kcb = [f64(lay0["k_cb"][h]) for h in heads]
    vcb = [f64(lay0["v_cb"][h]) for h in heads]
    w = [lay0["w"][h].double().cpu().numpy() for h in heads]
    perm = [lay0["perm"][h].long().cpu().numpy() for h in heads]
    chunk = 256
    jobs = [(keep["k"][:, :, j:j + chunk], keep["v"][:, :, j:j + chunk], kcb, vcb, w, perm, heads, cfg.T_c)
            for j in range(0, n_enc, chunk)]
    with_page = steps >= cfg.page                                  # a page was encoded at tok0 = N
    if with_page:
        jobs.append((keep["page_k"], keep["page_v"], kcb, vcb, w, perm, heads, cfg.T_c))
    t0 = time.perf_counter()
    with _pool(workers) as ex:
        enc_res = list(ex.map(_oracle_encode_job, jobs))
    enc_wall = time.perf_counter() - t0
    codes = 2 * len(heads) * (n_enc + (cfg.page if with_page else 0)) * cfg.chunks * cfg.n_blk

    # compare with the GPU's sigma and indices on that sample
    sig_gpu = lay0["sigma"][0].double().cpu().numpy()
    kid = lay0["kidx"][0].cpu().numpy()
    vid = lay0["vidx"][0].cpu().numpy()
    n_fail = n_tie = n_sig = 0
    for ji, (_, sbar, res) in enumerate(enc_res):
        if ji < len(jobs) - int(with_page):
            tok = slice(ji * chunk, min(n_enc, ji * chunk + chunk))
        else:
            tok = slice(cfg.N, cfg.N + cfg.page)                    # the first page event's tokens
        ok_tok = np.all(sig_gpu[tok] == sbar, axis=1)                # sigma at an fp16 midpoint: skip the token
        n_sig += int((~ok_tok).sum())
        for i, h in enumerate(heads):
            ki, kt, vi, vt = res[i]
            for gi, oi, tie, sel in ((kid[h][:, tok], ki, kt, ok_tok), (vid[h][:, tok], vi, vt, None)):
                diff = gi != oi
                uniq = tie == 1
                if sel is not None:
                    diff &= sel[None, :, None]
                n_fail += int((diff & uniq).sum())
                n_tie += int((diff & ~uniq).sum())

    # decode rows
    L = cfg.layers
    lsel = sorted({0, L // 2 - 1 if L > 2 else 0, L - 1})
    ssel = sorted({0, steps // 2, max(0, steps - 1)})
    rows, want = [], []
    o_buf = torch.empty((cfg.B, cfg.H_q, cfg.T, cfg.D), dtype=torch.float32, device="cuda")
    l_buf = torch.empty((cfg.B, cfg.H_q, cfg.T), dtype=torch.float32, device="cuda")
    g = lv.geom(cfg.D, cfg.T, cfg.T_c, cfg.G, cfg.K, cfg.H_kv, cfg.H_q, cfg.theta)
    gqa = cfg.H_q // cfg.H_kv
    for li in lsel:
        lay = layers[li]
        for s in ssel:
            Ns = cfg.N + cfg.page * (s // cfg.page)
            lv.decode_attn(g, lay["q"], lay["kidx"], lay["vidx"], lay["k_cb"], lay["v_cb"], lay["sk"], lay["sv"],
                           rope, N=Ns, pt=lay["pt"], out=o_buf, lse=l_buf, workspace=ws)
            torch.cuda.synchronize()
            for hq in heads:
                h = hq // gqa
                ki = lay["kidx"][0, h, :, :Ns].cpu().numpy()
                vi = lay["vidx"][0, h, :, :Ns].cpu().numpy()
                sig = lay["sigma"][0, :Ns].double().cpu().numpy()
                sk, sv = f64(lay["sk"][0, h]), f64(lay["sv"][0, h])
                for t in range(cfg.T):
                    rows.append((f64(lay["q"][0, hq, t]), t, ki, vi, f64(lay["k_cb"][h]), f64(lay["v_cb"][h]), sk, sv,
                                 cfg.T_c, cfg.theta, lay["w"][h].double().cpu().numpy(),
                                 lay["perm"][h].long().cpu().numpy(), sig))
                    want.append((o_buf[0, hq, t].double().cpu().numpy(), float(l_buf[0, hq, t]), Ns, li, s))
    t0 = time.perf_counter()
    with _pool(workers) as ex:
        dec_res = list(ex.map(_oracle_decode_job, rows))
    dec_wall = time.perf_counter() - t0
    worst, worst_lse = 0.0, 0.0
    for (_, o_ref, l_ref), (o_gpu, l_gpu, _, _, _) in zip(dec_res, want):
        worst = max(worst, float(np.max(np.abs(o_gpu - o_ref)) / max(np.linalg.norm(o_ref), 1e-30)))
        worst_lse = max(worst_lse, abs(l_gpu - l_ref))
    # a row (one batch entry, one q-head, one loop step) over Ns tokens is
    # 1/(H_q * T) of that batch entry's Ns * n_blk context tokens per loop block
    tok_blocks = sum(Ns * cfg.n_blk / (cfg.H_q * cfg.T) for _, _, Ns, _, _ in want)
    ok = n_fail == 0 and worst <= OUT_TOL
    if not ok:
        print("PARITY FAILURE on the bench sample: %d index failures, worst row error %.3g" % (n_fail, worst),
              file=sys.stderr, flush=True)
    return {
        "value": tok_blocks / dec_wall,
        "unit": UNIT,
        "cores": workers,
        "kind": "oracle",
        "sample": "decode: batch entry 0, q-heads 0-1, all %d loop steps at layers %s and decode steps %s (%d rows "
                  "over the context each step had, 65.5k tokens + %d sinks); encode: layer 0, batch entry 0, "
                  "kv-heads 0-1, first %d tokens + one %d-token page, K (sigma over all %d heads, pre-transform) "
                  "and V (%d codes). fp64 NumPy, one process per job, %d processes, 1 BLAS thread each; decode "
                  "wall %.1f s, encode wall %.1f s"
                  % (cfg.T, lsel, ssel, len(rows), cfg.n_s, n_enc, cfg.page, cfg.H_kv, codes, workers, dec_wall,
                     enc_wall),
        "encode_codes_per_s": codes / enc_wall,
        "decode_units_per_s": sum(Ns * cfg.n_blk / cfg.H_q / cfg.T * cfg.H_kv for _, _, Ns, _, _ in want) / dec_wall,
        "host_cpus_available": cores,
        "cpu_model": model,
        "parity_on_sample": {"ok": ok, "index_failures": n_fail, "index_tie_set_choices": n_tie,
                             "tokens_sigma_at_fp16_midpoint": n_sig,
                             "decode_rows": len(rows), "worst_row_rel_err": worst, "tolerance": OUT_TOL,
                             "worst_abs_lse_diff": worst_lse},
    }


# ----------------------------------------------------------------------------- single-layer workloads

def _oracle_head(args):
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle as ref
    kx, vx, kc, vc, sk, sv, qs, T_c, theta = args
    with threadpool_limits(1):
        t0 = time.perf_counter()
        ki, kt, vi, vt = [], [], [], []
        for j in range(0, kx.shape[1], 256):
            a, b = ref.encode(kx[:, j:j + 256], kc, T_c)
            c, d = ref.encode(vx[:, j:j + 256], vc, T_c)
            ki.append(a)
            vi.append(c)
        ki = np.concatenate(ki, axis=1)
        vi = np.concatenate(vi, axis=1)
        for t in range(qs.shape[0]):
            ref.decode_attn_row(qs[t], t, ki, vi, kc, vc, sk, sv, T_c, theta)
        return time.perf_counter() - t0, ki.size + vi.size


def cpu_baseline_single(cfg, inp, n_tok, n_b):
    """Oracle on batch entries 0..n_b-1, every kv-head, the first n_tok context
    tokens: K and V encode plus decode of every loop step over those tokens."""
    f = lambda t: t.float().cpu().double().numpy()
    jobs = []
    for b in range(n_b):
        for h in range(cfg.H_kv):
            hq = h * (cfg.H_q // cfg.H_kv)
            jobs.append((f(inp["k"][b, h, :, :n_tok]), f(inp["v"][b, h, :, :n_tok]), f(inp["k_cb"][h]),
                         f(inp["v_cb"][h]), f(inp["sink_k"][b, h]), f(inp["sink_v"][b, h]),
                         f(inp["q"][b, hq]), cfg.T_c, cfg.theta))
    cores, model = host_cpu()
    workers = max(1, min(cores, len(jobs), 16))
    t0 = time.perf_counter()
    with _pool(workers) as ex:
        res = list(ex.map(_oracle_head, jobs))
    wall = time.perf_counter() - t0
    codes = sum(r[1] for r in res)
    # One q-head per kv-head is decoded; with GQA the other heads of a group
    # are not re-run.
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
        "host_cpus_available": cores,
        "cpu_model": model,
    }


def single_layer(args, torch, lv, cfg, steps, warmup, with_cpu, stream=None):
    """One layer: encode K, encode V, one fused decode call of every loop step.
    Returns the JSON line's dict."""
    from synth import build_inputs
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
    ws = torch.empty(max(4, lv.decode_workspace_bytes(g, cfg.B, cfg.N, 0, cfg.T)), dtype=torch.uint8,
                     device="cuda")

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

    if stream is None:
        stream = hbm_stream(torch)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        step(evs[i])
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_step = total_ms / steps
    enc_ms = statistics.median([e[0].elapsed_time(e[1]) for e in evs] + [e[1].elapsed_time(e[2]) for e in evs])
    dec_ms = statistics.median(e[2].elapsed_time(e[3]) for e in evs)

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
        reps = max(1, min(steps, 20))
        pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in pev:
            a.record()
            per_step()
            b.record()
        torch.cuda.synchronize()
        ps_ms = _median_ms(pev)

    # A bf16 recent window of 64 tokens per (batch, kv-head, step) in the same
    # softmax (the tokens not yet converted into a page), against the call
    # without it; the two alternate, median of 20 each.
    n_r = 64
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0x5EED0000 + 1000 * cfg.index + 99)
    rk = torch.randn((cfg.B, cfg.H_kv, cfg.T, n_r, cfg.D), generator=gen, device="cuda").to(torch.bfloat16)
    rv = torch.randn((cfg.B, cfg.H_kv, cfg.T, n_r, cfg.D), generator=gen, device="cuda").to(torch.bfloat16)
    rope_r = lv.rope_table(cfg.n_s + cfg.N + n_r, cfg.D, cfg.theta)

    def dec(recent):
        lv.decode_attn(g, inp["q"], kidx, vidx, inp["k_cb"], inp["v_cb"], inp["sink_k"], inp["sink_v"], rope_r,
                       out=out, lse=lse, workspace=ws, recent_k=rk if recent else None,
                       recent_v=rv if recent else None)
    dec(True)
    rev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(20)]
    for e in rev:
        e[0].record()
        dec(False)
        e[1].record()
        dec(True)
        e[2].record()
    torch.cuda.synchronize()
    plain_ms = statistics.median(e[0].elapsed_time(e[1]) for e in rev)
    rec_ms = statistics.median(e[1].elapsed_time(e[2]) for e in rev)
    del rk, rv

    units = cfg.B * cfg.H_kv * cfg.N * cfg.n_blk                  # decode units per call
    codes_per_call = cfg.B * cfg.H_kv * cfg.n_blk * cfg.N * cfg.chunks
    dec_bytes = units * 2 * cfg.chunks                             # K + V index bytes per unit
    enc_bytes = codes_per_call * (2 * cfg.G + 1)                   # bf16 joint vector in, 1 byte out
    dec_gbs = dec_bytes / (dec_ms * 1e-3) / 1e9
    enc_gbs = enc_bytes / (enc_ms * 1e-3) / 1e9
    workload = ("config %d (%s): B=%d, %d kv-heads / %d q-heads, D=%d, T=%d, T_c=%d, G=%d, K=%d, N=%d + %d sinks"
                % (cfg.index, cfg.name, cfg.B, cfg.H_kv, cfg.H_q, cfg.D, cfg.T, cfg.T_c, cfg.G, cfg.K, cfg.N, cfg.n_s))
    has_traffic = cfg.index == 2 and cfg.T_c == 4
    roof_dec = {"kernel": "loopvq decode_attn call (decode kernel; + merge_kernel when the context is split)", "bound": "hbm",
                "achieved": dec_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dec_gbs / HBM_PEAK_GBS,
                "traffic": load_traffic(2, "decode") if has_traffic else None,
                "algorithmic_bytes_per_launch": dec_bytes, "launch_ms_median": dec_ms,
                "frac_of_measured_read": dec_gbs / stream["read_GBps"]}
    roof_enc = {"kernel": "loopvq encode call (encode_kernel)", "bound": "hbm",
                "achieved": enc_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": enc_gbs / HBM_PEAK_GBS,
                "traffic": load_traffic(2, "encode") if has_traffic else None,
                "algorithmic_bytes_per_launch": enc_bytes, "launch_ms_median": enc_ms,
                "frac_of_measured_read": enc_gbs / stream["read_GBps"],
                "mfma_tflops": 2.0 * cfg.K * cfg.G * codes_per_call / (enc_ms * 1e-3) / 1e12,
                "mfma_frac_of_bf16_peak": 2.0 * cfg.K * cfg.G * codes_per_call / (enc_ms * 1e-3) / 1e12
                / BF16_MFMA_PEAK_TFLOPS}
    dominant = roof_enc if 2 * enc_ms >= dec_ms else roof_dec
    res = {
        "metric": METRIC,
        "value": cfg.B * cfg.N * cfg.n_blk / (ms_step * 1e-3),
        "unit": UNIT,
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "global_batch": cfg.B, "seq_len": cfg.N + cfg.n_s,
                   "step": "encode K + encode V + decode attention of all %d loop steps" % cfg.T},
        "decode": {"ms_per_call_median": dec_ms,
                   "context_tokens_per_s_per_block": cfg.B * cfg.N * cfg.n_blk / (dec_ms * 1e-3),
                   "units_per_s": units / (dec_ms * 1e-3), "index_GBps": dec_gbs,
                   "hbm_frac_index_bytes": dec_gbs / HBM_PEAK_GBS},
        "encode": {"ms_per_call_median": enc_ms, "codes_per_s": codes_per_call / (enc_ms * 1e-3), "GBps": enc_gbs},
        "decode_per_step": None if ps_ms is None else {
            "ms_all_steps_median": ps_ms, "calls": cfg.T, "vs_fused": ps_ms / dec_ms,
            "note": "one call per loop step (n_steps = 1), each re-reading the index rows"},
        "decode_recent_window": {"n_r": n_r, "ms_median": rec_ms, "ms_without_median": plain_ms,
                                 "vs_without": rec_ms / plain_ms,
                                 "note": "the fused call with 64 bf16 recent tokens per (batch, kv-head, step) "
                                         "in the same softmax, alternating with the call without them"},
        "roofline": dominant,
        "roofline_decode": roof_dec,
        "roofline_decode_valu": valu_roofline(units, cfg.T_c, cfg.D, cfg.H_q // cfg.H_kv, dec_ms,
                                              roof_dec["kernel"]),
        "roofline_encode": roof_enc,
        "hbm_stream": stream,
        "input_generation_s": t_gen,
    }
    if with_cpu:
        res["cpu_baseline"] = cpu_baseline_single(cfg, inp, min(args.cpu_tokens, cfg.N),
                                                  max(1, min(args.cpu_batch, cfg.B)))
    del inp, kidx, vidx
    torch.cuda.empty_cache()
    return res


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
    backward, Adam).  Returns the JSON line's dict."""
    from synth import build_inputs, config_by_index, gen_targets, gen_toy_stack
    from dataclasses import replace
    from sub_bit_loop_amd import finetune as ft
    steps = 20 if args.steps is None else args.steps
    warmup = 3 if args.warmup is None else args.warmup
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
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return _median_ms(ev)

    fwd_ms = timed(fwd, steps)
    bwd_ms = timed(bwd, steps)
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
    # importance weights of the k-means (eq. 3): stack over the precise cache,
    # next-token loss backward into every cached key and value, weights
    targets = gen_targets(cfg, 0, "cuda", vocab=vocab, B=1)
    ft.fisher_importance(stack, g, toy["x"], inp["k"], inp["v"], sk, sv, targets)
    torch.cuda.synchronize()
    fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
    for a_, b_ in fev:
        a_.record()
        ft.fisher_importance(stack, g, toy["x"], inp["k"], inp["v"], sk, sv, targets)
        b_.record()
    torch.cuda.synchronize()
    fisher_ms = _median_ms(fev)
    iters = max(2, steps // 2)
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
        n = min(N, args.ft_cpu_tokens)
        f64 = lambda t: t.detach().cpu().double()
        jobs = [(f64(q[:, h:h + 1, :, :n]), kidx[:, h:h + 1, :, :n].long().cpu(),
                 vidx[:, h:h + 1, :, :n].long().cpu(), f64(inp["k_cb"][h:h + 1]), f64(inp["v_cb"][h:h + 1]),
                 f64(sk[:, h:h + 1]), f64(sv[:, h:h + 1]), cfg.T_c, f64(dout[:, h:h + 1, :, :n]), cfg.theta)
                for h in range(cfg.H_q)]
        # each worker imports torch, which opens the GPU device: stay well inside
        # the per-GPU process limit
        cores, model = host_cpu()
        workers = max(1, min(cores, len(jobs), 8))
        t0 = time.perf_counter()
        with _pool(workers) as ex:
            list(ex.map(_oracle_vjp_sample, jobs))
        wall = time.perf_counter() - t0
        sp = cfg.H_q * cfg.T * (n * (n + 1) // 2 + n * cfg.n_s)
        cpu = {"value": sp / wall, "unit": "attention (query, key) pairs/s, forward + backward", "cores": workers,
               "kind": "oracle", "host_cpus_available": cores, "cpu_model": model,
               "sample": "all %d q-heads and %d loop steps, first %d tokens + %d sinks: fp64 torch causal attention "
                         "over the rebuilt cache and its autograd backward (%d pairs); one process per q-head, %d "
                         "at a time, 1 thread each; wall %.1f s" % (cfg.H_q, cfg.T, n, cfg.n_s, sp, workers, wall)}
    workload = ("codebook fine-tuning (section 3.2): one calibration sequence per iteration, %d kv-heads / %d "
                "q-heads, D=%d, T=T_c=%d, G=%d, K=%d, %d tokens + %d sinks; toy looped stack d=%d, vocab %d"
                % (cfg.H_kv, cfg.H_q, cfg.D, cfg.T, cfg.G, cfg.K, N, cfg.n_s, cfg.H_q * cfg.D, vocab))
    return {
        "metric": "codebook fine-tuning: compressed-attention forward + backward (query, key) pairs/s",
        "value": pairs / ((fwd_ms + bwd_ms) * 1e-3),
        "unit": "attention (query, key) pairs/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": fwd_ms + bwd_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": workload, "global_batch": 1, "seq_len": N + cfg.n_s,
                   "step": "loopvq_prefill_attn + loopvq_prefill_attn_backward over every loop step"},
        "forward": {"ms_per_call_median": fwd_ms, "tflops": fwd_tf, "flop_per_pair": 4 * D},
        "backward": {"ms_per_call_median": bwd_ms, "tflops": bwd_tf, "flop_per_pair": 8 * D,
                     "executed_flop_per_pair": 16 * D,
                     "note": "S = QK^T is recomputed in each of the three backward kernels and dP in two"},
        "roofline": {"kernel": dom_name, "bound": "mfma", "achieved": dom_tf, "peak": FP32_MATRIX_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": dom_tf / FP32_MATRIX_PEAK_TFLOPS, "traffic": None,
                     "algorithmic_flop_per_launch": dom_flop, "launch_ms_median": dom_ms, "dtype": "f32"},
        "fisher_weights": {"ms_per_pass_median": fisher_ms,
                           "note": "importance weights of every joint vector (eq. 3): toy stack over the precise "
                                   "cache (4 loopvq_precise_attn calls), next-token loss, backward "
                                   "(loopvq_precise_attn_backward per step), loopvq_fisher_weights"},
        "iteration": {"ms": it_ms, "objective": Js,
                      "note": "re-encode K and V, toy stack forward over the rebuilt cache (4 compressed-attention "
                              "calls), KL against the precise run, backward, Adam (lr 1e-3)"},
        "cpu_baseline": cpu,
    }


# ----------------------------------------------------------------------------- counter summary

def _counter_rows(d):
    import csv
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        raise SystemExit("no counter_collection.csv under %s" % d)
    return rows


def _per_dispatch(rows, counter):
    """{dispatch id: (kernel name, grid size, value)} summed over the counter's instances."""
    out = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        k = r.get("Dispatch_Id") or r.get("Correlation_Id")
        name = r["Kernel_Name"].split("(")[0]
        grid = r.get("Grid_Size") or r.get("Grid_Size_X") or ""
        prev = out.get(k, (name, grid, 0.0))
        out[k] = (name, grid, prev[2] + float(r["Counter_Value"]))
    return out


def write_traffic(cfg_index, fetch_dir, write_dir, command):
    """Add workload cfg_index's entries to profiles/traffic.json from a
    FETCH_SIZE run and a WRITE_SIZE run of this script on that workload alone
    (`--no-config2` for the 24-layer flow): KiB per dispatch, scaled by what
    the same counter reads for the calibration read and copy of 1 GiB, per
    launch of each bench-line kernel."""
    fetch = _per_dispatch(_counter_rows(fetch_dir), "FETCH_SIZE")
    write = _per_dispatch(_counter_rows(write_dir), "WRITE_SIZE")

    def avg(tab, pred):
        v = [x for (n, gsz, x) in tab.values() if pred(n, gsz)]
        return (sum(v) / len(v), len(v)) if v else (None, 0)

    cf, _ = avg(fetch, lambda n, gsz: "calib_read" in n)
    cw, _ = avg(write, lambda n, gsz: "calib_copy" in n)
    ff, wf = 1048576.0 / cf, 1048576.0 / cw

    def big(tab, name):
        """Dispatches of `name` with the largest grid (prefill launches, not page encodes)."""
        grids = [int(gsz or 0) for (n, gsz, _) in tab.values() if name in n]
        top = max(grids) if grids else -1
        return lambda n, gsz: name in n and int(gsz or 0) == top

    def has(name):
        return lambda n, gsz: name in n

    def after(tab, first, name):
        """Dispatches of `name` launched right after a dispatch of `first`
        (the merge of one decode call)."""
        ids = {int(k) + 1 for k, (n, _, _) in tab.items() if first in n}
        keep = {k for k, (n, _, _) in tab.items() if name in n and int(k) in ids}
        return keep

    entries = {}

    def avg_ids(tab, ids):
        v = [tab[k][2] for k in ids]
        return (sum(v) / len(v), len(v)) if v else (None, 0)

    def entry(key, kern, label, parts):
        f_kib = w_kib = 0.0
        counts = []
        for fp, wp in parts:
            fa, nf = avg_ids(fetch, fp) if isinstance(fp, set) else avg(fetch, fp)
            wa, nw = avg_ids(write, wp) if isinstance(wp, set) else avg(write, wp)
            if fa is None or wa is None:
                raise SystemExit("no dispatches for %s" % label)
            f_kib += fa
            w_kib += wa
            counts.append([nf, nw])
        entries[key] = {"kernel": label, "source_hash": kernel_source_hash(kern), "fetch_KiB": f_kib,
                        "write_KiB": w_kib, "dispatches_averaged": counts,
                        "bytes_per_launch": (f_kib * ff + w_kib * wf) * 1024}

    if cfg_index == 5:
        entry("decode_tasq@5", "decode_tasq", "decode_tasq_kernel<4> + merge_kernel (one layer)",
              [(has("decode_tasq"), has("decode_tasq")),
               (after(fetch, "decode_tasq", "merge_kernel"), after(write, "decode_tasq", "merge_kernel"))])
        entry("encode_prefill_layer@5", "encode", "sigma_kernel + encode_kernel<16,4,true> + "
              "encode_kernel<16,4,false> (one layer's prefill)",
              [(big(fetch, name), big(write, name)) for name in
               ("sigma_kernel", "encode_kernel<16, 4, true>", "encode_kernel<16, 4, false>")])
    elif cfg_index == 2:
        # the step loop's calls (each right after the value encode), not the
        # recent-window calls timed afterwards
        def step_calls(tab):
            dec = after(tab, "encode_kernel", "decode_half")
            merge = {k for k, (n, _, _) in tab.items() if "merge_kernel" in n and int(k) - 1 in {int(j) for j in dec}}
            return dec, merge
        (fd, fm), (wd, wm) = step_calls(fetch), step_calls(write)
        # with one context split (the full workload) the kernel writes the
        # output itself and no merge kernel follows it
        if fm and wm:
            entry("decode_half@2", "decode_half", "decode_half_kernel + merge_kernel (the step loop's calls)",
                  [(fd, wd), (fm, wm)])
        else:
            entry("decode_half@2", "decode_half", "decode_half_kernel (the step loop's calls; one context split, "
                  "no merge launch)", [(fd, wd)])
        entry("encode@2", "encode", "encode_kernel<16, 4, false>",
              [(big(fetch, "encode_kernel<16, 4, false>"), big(write, "encode_kernel<16, 4, false>"))])
    else:
        raise SystemExit("traffic entries are kept for workloads 2 and 5")
    p = os.path.join(ROOT, "profiles", "traffic.json")
    d = {"kernels": {}}
    if os.path.exists(p):
        with open(p) as fh:
            d = json.load(fh)
    for k in ("command", "fetch_factor", "write_factor"):
        d.pop(k, None)
    if not isinstance(d.get("calibration"), dict):
        d["calibration"] = {}
    known = {key for _, key in TRAFFIC_ENTRIES.values()}
    d["kernels"] = {k: v for k, v in d.get("kernels", {}).items() if k in known}
    d.setdefault("kernels", {}).update(entries)
    d.setdefault("commands", {})["workload %d" % cfg_index] = command
    d.setdefault("calibration", {})["workload %d run" % cfg_index] = (
        "calib_read_kernel reads 1 GiB (16 B per lane): FETCH_SIZE %.1f KiB per dispatch -> fetch factor %.4f; "
        "calib_copy_kernel writes 1 GiB: WRITE_SIZE %.1f KiB -> write factor %.4f" % (cf, ff, cw, wf))
    with open(p, "w") as fh:
        json.dump(d, fh, indent=1)
    print(json.dumps(d, indent=1))


# ----------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: the workload's 256 decode steps; 20 for single-layer workloads)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed warm-up steps (default 3)")
    ap.add_argument("--config", type=int, default=5,
                    help="workload: 5 the 24-layer prefill + decode flow (default), 1-4 single layer")
    ap.add_argument("--tc", type=int, default=None,
                    help="steps per block T_c override for workloads 1-4 (1: per-step codebooks, as for the "
                         "layers outside the loop)")
    ap.add_argument("--cpu-tokens", type=int, default=None,
                    help="context tokens in the oracle encode sample (default: 65536 for workload 5, 8192 else)")
    ap.add_argument("--cpu-batch", type=int, default=2, help="batch entries in the single-layer oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-config2", action="store_true", help="skip the single-layer sub-object of the default line")
    ap.add_argument("--finetune", action="store_true",
                    help="time the codebook fine-tuning workload (compressed-attention forward + backward)")
    ap.add_argument("--ft-tokens", type=int, default=2048, help="tokens of the fine-tuning sequence")
    ap.add_argument("--ft-cpu-tokens", type=int, default=1536, help="tokens in the fine-tuning oracle sample")
    ap.add_argument("--write-traffic", nargs=4, metavar=("CONFIG", "FETCH_DIR", "WRITE_DIR", "COMMAND"),
                    help="add workload CONFIG's entries to profiles/traffic.json from the output folders of a "
                         "rocprofv3 --pmc FETCH_SIZE run and a --pmc WRITE_SIZE run, recording COMMAND")
    args = ap.parse_args()
    if args.write_traffic:
        c, fd, wd, cmd = args.write_traffic
        write_traffic(int(c), fd, wd, cmd)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the LoopVQ path has no multi-GPU step in this build "
              "(decode shards over batch x kv-heads with no communication); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import sub_bit_loop_amd as lv
    from synth import config_by_index

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    lv.lib()
    torch.cuda.set_device(0)
    if args.finetune:
        print(json.dumps(finetune_flow(args, torch, lv)), flush=True)
        return
    cfg = config_by_index(args.config)
    if args.tc is not None:
        if cfg.layers != 1 or args.tc < 1 or cfg.T % args.tc or cfg.G % args.tc:
            print("--tc needs a single-layer workload and T_c dividing T and G", file=sys.stderr)
            sys.exit(2)
        cfg = dataclasses.replace(cfg, T_c=args.tc)
    if cfg.layers == 1:
        if args.cpu_tokens is None:
            args.cpu_tokens = 8192
        res = single_layer(args, torch, lv, cfg, 20 if args.steps is None else args.steps,
                           3 if args.warmup is None else args.warmup, not args.no_cpu_baseline)
        print(json.dumps(res), flush=True)
        return
    if args.cpu_tokens is None:
        args.cpu_tokens = cfg.N
    sub = None
    if not args.no_config2:
        # the 0.5-bit single-layer workload first (its inputs are freed before the flow)
        print("single-layer workload 2", file=sys.stderr, flush=True)
        r2 = single_layer(args, torch, lv, config_by_index(2), 20, 3, False)
        sub = {k: r2[k] for k in ("config", "ms_per_step", "value", "decode", "encode", "decode_per_step",
                                  "decode_recent_window",
                                  "roofline_decode", "roofline_decode_valu", "roofline_encode")}
    res = workload5(args, torch, lv, cfg)
    res["config2"] = sub
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
