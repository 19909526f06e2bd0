"""Benchmark of the TurboQuant KV-cache hot path on one MI355X.

One step = the whole hot path over one batch of the workload: encode the
layer's K and V caches (rotation, norm, codebook, packing[, QJL]) and run
fused decode attention of every query head over the packed cache.

Metric: packed-KV decode-attention GB/s (algorithmic packed bytes read per
second; `value`), with encode throughput in Mtok/s beside it.  Inputs are
resident in HBM before timing.  The packed cache and the encode inputs are
rotated over distinct copies (>= 1 GiB each) so the 256 MB Infinity Cache
cannot serve a step from the previous one: step i encodes into copy i and
decodes copy i + R/2, written R/2 steps earlier.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def spread(ms):
    """Median and (p10, p90) of a list of per-step times."""
    v = sorted(ms)
    return v[len(v) // 2], (v[len(v) // 10], v[(9 * len(v)) // 10])
PROFILES = os.path.join(ROOT, "profiles")


def packed_bytes_per_token_head(w, code_bytes_k, code_bytes_v, sign_bytes_k):
    nb = 2 * (w.d // w.norm_group if w.norm_group else 1)   # fp16 norms per vector
    kb = code_bytes_k + nb + (sign_bytes_k + 2 if w.k_qjl else 0)
    return kb + code_bytes_v + nb


def traffic_from_profiles(kernel, workload):
    """HBM bytes per launch measured by rocprofv3 counters, if recorded for the
    current kernel sources (profiles/traffic.json); otherwise None."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except Exception:
        return None
    ent = rec.get(f"{workload}:{kernel}")
    from kv_cache_quantization_05_amd.rocpd_summary import kernel_source_hash

    if not ent or ent.get("source_hash") != kernel_source_hash(kernel):
        return None
    return ent.get("bytes_per_launch")


def _cpu_threads():
    """(threads the oracle's numpy uses, the BLAS pool size): numpy's
    matrix products run on the BLAS pool, everything else on one thread."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] + [1])
    except Exception:
        blas = 1
    return blas, blas


DTYPE = "f16 mfma, f32 acc"   # decode: fp16 matrix-core products, fp32 accumulation


def cpu_baseline(w, budget_s=12.0):
    """The float64 oracle on the host cores, on a bounded slice of the same
    workload: one batch element, one KV head (its Hq/Hkv query heads) and the
    first T_s positions, encode + decode.  Scaled per packed byte / token."""
    import numpy as np
    import torch

    from kv_cache_quantization_05_amd import workloads as wl
    from oracle import decode as odec
    from oracle import encode as oenc

    cores, blas = _cpu_threads()
    G = w.Hq // w.Hkv
    kc = oenc.Config(**wl.context_kwargs(w, "k"))
    vc = oenc.Config(**wl.context_kwargs(w, "v"))
    oenc.get_tables(kc)
    oenc.get_tables(vc)
    Ts = 512
    small = wl.scaled(w, B=1, T=min(w.T, 65536))
    K, V = wl.kv_pair(small, "cpu")
    q = wl.queries(w, "cpu")[0, :G].double().numpy()
    while True:
        k = K[0, 0, :Ts].float().double().numpy()
        v = V[0, 0, :Ts].float().double().numpy()
        t0 = time.perf_counter()
        kp = oenc.encode(k, kc)
        vp = oenc.encode(v, vc)
        t1 = time.perf_counter()
        kpl = {x: kp[x][None, None] for x in ("codes", "norms", "signs", "rnorms") if x in kp}
        vpl = {x: vp[x][None, None] for x in ("codes", "norms")}
        odec.attend_decode(q[None], kpl, vpl, kc, vc, [Ts])
        t2 = time.perf_counter()
        if t2 - t0 > budget_s / 4 or Ts * 2 > small.T:
            break
        Ts *= 2
    enc_s, dec_s = t1 - t0, t2 - t1
    bpt = packed_bytes_per_token_head(w, kc.code_bytes, vc.code_bytes, kc.sign_bytes)
    dec_gbs = Ts * bpt / dec_s / 1e9
    # a token = one position across all KV heads, K and V: Hkv x (K + V) vectors
    enc_mtoks = Ts / (enc_s * w.Hkv) / 1e6
    return {"value": round(dec_gbs, 6), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"batch 0, KV head 0 ({G} query heads), first {Ts} positions; "
                      f"encode {enc_s:.2f} s, decode {dec_s:.2f} s; float64 numpy",
            "host_cpus": os.cpu_count(), "blas_threads": int(blas),
            "encode_mtok_s": round(enc_mtoks, 6)}


def cpu_baseline_prefill(w, budget_s=12.0):
    """The float64 oracle on the host cores for the prefill workload, on a
    bounded slice: batch 0, KV head 0 (its Hq/Hkv query heads), a prompt of
    the first T_s positions (T_s doubled up to about a quarter of the budget):
    encode, then causal prefill of all T_s positions.  In the line's unit:
    the slice's packed bytes over its prefill time (the prefill work grows as
    T_s^2, so the figure is that of the slice, stated with it)."""
    from kv_cache_quantization_05_amd import workloads as wl
    from oracle import decode as odec
    from oracle import encode as oenc

    cores, blas = _cpu_threads()
    G = w.Hq // w.Hkv
    kc = oenc.Config(**wl.context_kwargs(w, "k"))
    vc = oenc.Config(**wl.context_kwargs(w, "v"))
    oenc.get_tables(kc)
    oenc.get_tables(vc)
    K, V = wl.kv_pair(w, "cpu")
    Q = wl.queries(w, "cpu")   # [B, Hq, Tq, d]
    Ts = 256
    while True:
        k = K[0, 0, :Ts].float().double().numpy()
        v = V[0, 0, :Ts].float().double().numpy()
        q = Q[0, :G, :Ts].double().numpy()
        t0 = time.perf_counter()
        kp = oenc.encode(k, kc)
        vp = oenc.encode(v, vc)
        t1 = time.perf_counter()
        kpl = {x: kp[x][None, None] for x in ("codes", "norms", "signs", "rnorms") if x in kp}
        vpl = {x: vp[x][None, None] for x in ("codes", "norms")}
        odec.attend_prefill(q[None], kpl, vpl, kc, vc, [Ts])
        t2 = time.perf_counter()
        if t2 - t0 > budget_s / 4 or Ts * 2 > w.extra["Tq"]:
            break
        Ts *= 2
    enc_s, pf_s = t1 - t0, t2 - t1
    bpt = packed_bytes_per_token_head(w, kc.code_bytes, vc.code_bytes, kc.sign_bytes)
    pairs = Ts * (Ts + 1) // 2
    return {"value": round(Ts * bpt / pf_s / 1e9, 6), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"batch 0, KV head 0 ({G} query heads), a {Ts}-position prompt; encode {enc_s:.2f} s, "
                      f"causal prefill {pf_s:.2f} s; float64 numpy",
            "tflop_s": round(G * pairs * 4 * w.d / pf_s / 1e12, 8),
            "host_cpus": os.cpu_count(), "blas_threads": int(blas)}


def bench_search(args, w):
    """Search workload: encode the database (turbo4 + QJL, d = 256), then the
    fused top-k scorer for all queries.  value = packed database bytes
    scanned per second by one tq_scores call; the scorer's roofline is its
    arithmetic (2d + 2m flops per query-key pair) on fp16 matrix cores."""
    import torch

    from kv_cache_quantization_05_amd import binding as tq
    from kv_cache_quantization_05_amd import workloads as wl

    dev = "cuda"
    kctx = tq.Context(seed=w.seed, head_dim=w.d, bits=w.k_bits, qjl=w.k_qjl)
    X, Q = wl.search_set(w, dev)
    k_top = w.extra["top_k"]
    n, nq = X.shape[0], Q.shape[0]
    planes = kctx.new_planes((n,))
    bpv = kctx.code_bytes + 2 + (kctx.sign_bytes + 2 if w.k_qjl else 0)
    packed = n * bpv
    ws = torch.empty(max(tq.scores_workspace_bytes(kctx, nq, n, k_top), 1), dtype=torch.uint8, device=dev)
    out = torch.empty((nq, k_top), dtype=torch.float32, device=dev)
    idx = torch.empty((nq, k_top), dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        tq.encode(kctx, X, planes)
        if ev:
            ev[1].record(stream)
        tq.scores(kctx, Q, planes, top_k=k_top, scale=1.0, out=out, out_idx=idx, workspace=ws)
        if ev:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    enc_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / len(evs)
    sc_list = [e[1].elapsed_time(e[2]) for e in evs]
    sc_ms = sum(sc_list) / len(sc_list)
    sc_med, sc_pp = spread(sc_list)
    flops = float(nq) * n * (2 * w.d + (2 * kctx.sign_bytes * 8 if w.k_qjl else 0))
    tflops = flops / (sc_ms * 1e-3) / 1e12
    enc_bytes = X.numel() * X.element_size() + packed
    line = {
        "metric": "packed-KV decode-attention GB/s (% of HBM peak) + encode Mtok/s, 1 GPU",
        "value": round(packed / (sc_ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": DTYPE, "data": "synthetic",
        "config": {"workload": w.name, "n": n, "n_queries": nq, "head_dim": w.d, "bits": w.k_bits,
                   "qjl": w.k_qjl, "top_k": k_top, "packed_bytes": int(packed)},
        "scores_ms": round(sc_ms, 4),
        "scores_ms_median": round(sc_med, 4),
        "scores_ms_p10_p90": [round(sc_pp[0], 4), round(sc_pp[1], 4)],
        "encode_us": round(enc_ms * 1e3, 2),
        "encode_mtok_s": round(n / (enc_ms * 1e-3) / 1e6, 2),
        # the scorer is an fp16 matrix-core contraction (algorithmic flops:
        # 2d + 2m per query-key pair) against the dense fp16 MFMA peak
        "roofline": {"kernel": "scores", "bound": "mfma", "achieved": round(tflops, 3), "peak": 2500.0,
                     "unit": "TFLOP/s", "frac": round(tflops / 2500.0, 4),
                     "traffic": traffic_from_profiles("scores", w.name),
                     "flops_per_launch": flops, "avg_ms": round(sc_ms, 5)},
        "roofline_encode": {"kernel": "encode", "bound": "hbm",
                            "achieved": round(enc_bytes / (enc_ms * 1e-3) / 1e9, 2), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(enc_bytes / (enc_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                            "traffic": traffic_from_profiles("encode", w.name), "algorithmic_bytes": int(enc_bytes),
                            "avg_ms": round(enc_ms, 5)},
    }
    line["recall_at_10"] = search_recall(X, Q, idx, k_top)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_search(w, bpv)
    print(json.dumps(line), flush=True)


def search_recall(X, Q, idx, k, n_sample=32):
    """Recall@k of the GPU's top-k (from the packed codes) against the exact
    float64 inner-product top-k of the unquantised vectors, on a fixed
    sample of queries (a quality figure beside the throughput)."""
    import torch

    sel = torch.arange(0, Q.shape[0], Q.shape[0] // n_sample)[:n_sample]
    exact = Q[sel.to(Q.device)].cpu().double() @ X.cpu().double().T
    top = torch.topk(exact, k, dim=1).indices
    got = idx[sel.to(idx.device)].cpu()
    hits = [len(set(got[r].tolist()) & set(top[r].tolist())) for r in range(len(sel))]
    return round(sum(hits) / (k * len(sel)), 4)


def cpu_baseline_search(w, bpv, budget_s=12.0):
    """The float64 oracle on the host cores for the search workload: encode
    of N_s database vectors, then every query's scores against them (plain
    dequantise-then-dot) and its top-k, N_s doubled up to about a quarter of
    the budget.  value = packed bytes of the N_s keys per second of scoring
    all queries, the unit of the GPU line."""
    import numpy as np

    from kv_cache_quantization_05_amd import workloads as wl
    from oracle import decode as odec
    from oracle import encode as oenc

    cores, blas = _cpu_threads()
    cfg = oenc.Config(seed=w.seed, head_dim=w.d, bits=w.k_bits, qjl=w.k_qjl)
    oenc.get_tables(cfg)
    Ns = 1024
    X, Q = wl.search_set(w, "cpu", n=65536)
    Qn = Q.double().numpy()
    while True:
        x = X[:Ns].double().numpy()
        t0 = time.perf_counter()
        p = oenc.encode(x, cfg)
        t1 = time.perf_counter()
        pl = {k: p[k] for k in ("codes", "norms", "signs", "rnorms") if k in p}
        odec.top_k(odec.scores(Qn, pl, cfg), w.extra["top_k"])
        t2 = time.perf_counter()
        if t2 - t0 > budget_s / 4 or Ns * 2 > X.shape[0]:
            break
        Ns *= 2
    enc_s, sc_s = t1 - t0, t2 - t1
    return {"value": round(Ns * bpv / sc_s / 1e9, 6), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {Ns} database vectors, all {Q.shape[0]} queries: encode {enc_s:.2f} s, "
                      f"scores + top-{w.extra['top_k']} {sc_s:.2f} s; float64 numpy",
            "host_cpus": os.cpu_count(), "blas_threads": int(blas),
            "encode_mtok_s": round(Ns / enc_s / 1e6, 6)}


def bench_prefill(args, w):
    """Prefill workload: encode the prompt's K and V into the cache (one
    tq_encode each), then causal prefill attention of every prompt position
    over it (tq_attend_prefill).  value = packed cache bytes per second of
    the attention call; its roofline is the matrix-core contraction:
    algorithmic flops 4 d per (query head, visible key) pair against the
    dense fp16 MFMA peak."""
    import torch

    from kv_cache_quantization_05_amd import binding as tq
    from kv_cache_quantization_05_amd import workloads as wl

    dev = "cuda"
    Tq = w.extra["Tq"]
    kctx = tq.Context(**wl.context_kwargs(w, "k"))
    vctx = tq.Context(**wl.context_kwargs(w, "v"))
    K, V = wl.kv_pair(w, dev)
    q = wl.queries(w, dev)
    lens = torch.full((w.B,), w.T, dtype=torch.int32, device=dev)
    kp, vp = kctx.new_planes((w.B, w.Hkv, w.T)), vctx.new_planes((w.B, w.Hkv, w.T))
    out = torch.empty((w.B, w.Hq, Tq, w.d), dtype=torch.float32, device=dev)
    ws = torch.empty(max(tq.prefill_workspace_bytes(kctx, vctx, w.B, w.Hq, Tq), 1), dtype=torch.uint8, device=dev)
    bpt = packed_bytes_per_token_head(w, kctx.code_bytes, vctx.code_bytes, kctx.sign_bytes)
    packed = w.B * w.Hkv * w.T * bpt
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        tq.encode(kctx, K, kp)
        tq.encode(vctx, V, vp)
        if ev:
            ev[1].record(stream)
        tq.attend_prefill(kctx, vctx, q, kp, vp, lens, t_max=w.T, out=out, workspace=ws)
        if ev:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    enc_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / len(evs)
    pf_list = [e[1].elapsed_time(e[2]) for e in evs]
    pf_ms = sum(pf_list) / len(pf_list)
    pf_med, pf_pp = spread(pf_list)
    pairs = sum(min(i + 1 + (w.T - Tq), w.T) for i in range(Tq))   # visible keys over the block
    flops = float(w.B) * w.Hq * pairs * 4 * w.d
    tflops = flops / (pf_ms * 1e-3) / 1e12
    enc_bytes = (K.numel() + V.numel()) * K.element_size() + packed
    line = {
        "metric": "packed-KV decode-attention GB/s (% of HBM peak) + encode Mtok/s, 1 GPU",
        "value": round(packed / (pf_ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": DTYPE, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "Tq": Tq, "Hkv": w.Hkv, "Hq": w.Hq, "head_dim": w.d,
                   "k_bits": w.k_bits, "v_bits": w.v_bits, "k_qjl": w.k_qjl, "input": w.in_dtype,
                   "packed_bytes": int(packed)},
        "prefill_us": round(pf_ms * 1e3, 2),
        "prefill_us_median": round(pf_med * 1e3, 2),
        "prefill_us_p10_p90": [round(pf_pp[0] * 1e3, 2), round(pf_pp[1] * 1e3, 2)],
        "encode_us": round(enc_ms * 1e3, 2),
        "encode_mtok_s": round(w.B * w.T / (enc_ms * 1e-3) / 1e6, 2),
        "roofline": {"kernel": "attend_prefill", "bound": "mfma", "achieved": round(tflops, 3), "peak": 2500.0,
                     "unit": "TFLOP/s", "frac": round(tflops / 2500.0, 4),
                     "traffic": traffic_from_profiles("attend_prefill", w.name),
                     "flops_per_launch": flops, "avg_ms": round(pf_ms, 5)},
        "roofline_encode": {"kernel": "encode", "bound": "hbm",
                            "achieved": round(enc_bytes / (enc_ms * 1e-3) / 1e9, 2), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(enc_bytes / (enc_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                            "traffic": traffic_from_profiles("encode", w.name), "algorithmic_bytes": int(enc_bytes / 2),
                            "avg_ms": round(enc_ms / 2, 5)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_prefill(w)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama_b4_t128k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--min-rotation-bytes", type=float, default=1.1 * 2**30)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one 1 GiB device copy (a known-size reference for memory counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the single-GPU "
              f"path is the whole scope of this library.", file=sys.stderr)
        sys.exit(2)

    import torch

    from kv_cache_quantization_05_amd import binding as tq
    from kv_cache_quantization_05_amd import workloads as wl

    if args.calibrate_copy:
        src = torch.ones(2**28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w = wl.WORKLOADS[args.workload]
    if w.name == "search_1m":
        return bench_search(args, w)
    if "Tq" in w.extra:
        return bench_prefill(args, w)
    dev = "cuda"
    torch.cuda.set_device(0)
    kctx = tq.Context(**wl.context_kwargs(w, "k"))
    vctx = tq.Context(**wl.context_kwargs(w, "v"))
    K, V = wl.kv_pair(w, dev)
    q = wl.queries(w, dev)
    lens = torch.full((w.B,), w.T, dtype=torch.int32, device=dev)
    in_bytes = (K.numel() + V.numel()) * K.element_size()
    bpt = packed_bytes_per_token_head(w, kctx.code_bytes, vctx.code_bytes, kctx.sign_bytes)
    packed = w.B * w.Hkv * w.T * bpt
    R_in = max(1, math.ceil(args.min_rotation_bytes / in_bytes))
    R_pk = max(2, math.ceil(args.min_rotation_bytes / packed))
    inputs = [(K, V)] + [(K.clone(), V.clone()) for _ in range(R_in - 1)]
    caches = [(kctx.new_planes((w.B, w.Hkv, w.T)), vctx.new_planes((w.B, w.Hkv, w.T))) for _ in range(R_pk)]
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.attend_workspace_bytes(kctx, vctx, w.B, w.Hq, w.Hkv, w.T), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    for i in range(R_pk):  # every copy holds a valid encoding before timing
        tq.encode(kctx, inputs[i % R_in][0], caches[i][0])
        tq.encode(vctx, inputs[i % R_in][1], caches[i][1])
    torch.cuda.synchronize()

    def step(i, ev=None):
        kin, vin = inputs[i % R_in]
        kp, vp = caches[i % R_pk]
        if ev:
            ev[0].record(stream)
        tq.encode(kctx, kin, kp)
        tq.encode(vctx, vin, vp)
        if ev:
            ev[1].record(stream)
        kd, vd = caches[(i + R_pk // 2) % R_pk]
        tq.attend_decode(kctx, vctx, q, kd, vd, lens, t_max=w.T, out=out, workspace=ws)
        if ev:
            ev[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    enc_ms = sorted(e[0].elapsed_time(e[1]) for e in evs)
    dec_ms = sorted(e[1].elapsed_time(e[2]) for e in evs)
    enc_avg = sum(enc_ms) / len(enc_ms)
    dec_avg = sum(dec_ms) / len(dec_ms)
    dec_gbs = packed / (dec_avg * 1e-3) / 1e9
    enc_bytes = in_bytes + packed
    enc_gbs = enc_bytes / (enc_avg * 1e-3) / 1e9
    tokens = w.B * w.T
    enc_mtoks = tokens / (enc_avg * 1e-3) / 1e6

    def roof(kernel, gbs, alg_bytes, ms):
        return {"kernel": kernel, "bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic_from_profiles(kernel, w.name),
                "algorithmic_bytes": int(alg_bytes), "avg_ms": round(ms, 5)}

    # per launch: one tq_attend_decode call; one tq_encode call (the K and V
    # launches of a step averaged, as rocprofv3 averages their dispatches)
    r_dec = roof("attend_decode", dec_gbs, packed, dec_avg)
    r_enc = roof("encode", enc_gbs, enc_bytes / 2, enc_avg / 2)
    line = {
        "metric": "packed-KV decode-attention GB/s (% of HBM peak) + encode Mtok/s, 1 GPU",
        "value": round(dec_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "Hkv": w.Hkv, "Hq": w.Hq, "head_dim": w.d,
                   "k_bits": w.k_bits, "v_bits": w.v_bits, "k_qjl": w.k_qjl, "input": w.in_dtype,
                   "rotation": w.rotation, "norm_group": w.norm_group, "norm_correction": w.norm_correction,
                   "packed_bytes": int(packed), "rotation_copies": [R_in, R_pk]},
        "hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4),
        "decode_us": round(dec_avg * 1e3, 2),
        "decode_us_median": round(spread(dec_ms)[0] * 1e3, 2),
        "decode_us_p10_p90": [round(spread(dec_ms)[1][0] * 1e3, 2), round(spread(dec_ms)[1][1] * 1e3, 2)],
        "encode_us": round(enc_avg * 1e3, 2),
        "encode_mtok_s": round(enc_mtoks, 2),
        "roofline": r_dec,
        "roofline_decode": r_dec,
        "roofline_encode": r_enc,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
