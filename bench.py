"""Benchmark of the OSCAR INT2-KV decode hot path on one MI355X.

One step = one pass of the whole path over the batch through
oscar_decode_step: append one token per sequence (evicting the oldest recent
token into the INT2 history: rotate, clip, quantize, pack) and decode
attention for one query per sequence (INT2 split-KV + BF16 window +
online-softmax merge + de-rotation).  The default workload is the largest
one that fits a GPU: the serving step of 64 sequences of 4K-64K tokens
(32 query / 8 kv heads, d 128).  Steps rotate over several layer pools so
the read set exceeds the 256 MB Infinity Cache.  Prints one JSON line.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0


def algorithmic_decode_bytes(w, lengths):
    """Bytes the decode must read per step: packed codes + fp16 scale/zero of
    every history token, bf16 sink/recent tokens, bf16 queries."""
    d, G, Hkv, Hq = w.head_dim, w.group_size, w.num_kv_heads, w.num_q_heads
    total = 0
    for L in lengths:
        n_hist = max(0, L - 320)
        total += n_hist * Hkv * 2 * (d // 4 + 4 * (d // G))
        total += min(L, 320) * Hkv * d * 2 * 2
    total += len(lengths) * Hq * d * 2
    return total


def traffic_record(kernel_src, workload, kernel="decode_main"):
    """HBM bytes per launch measured with rocprofv3 counters, if the record in
    profiles/ was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    with open(kernel_src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    rec = {}
    with open(path) as f:
        for ln in f:
            if "=" in ln and not ln.startswith("#"):
                k, v = ln.split("=", 1)
                rec[k.strip()] = v.strip()
    if rec.get("kernel_source_sha256_16") != sha:
        return None
    return float(rec["hbm_bytes_per_launch"])


def _cpu_pair(task):
    """One (sequence, kv head) pair of the oracle's step, in a worker process
    (one thread): encode the pair's prompt history (setup, untimed), then the
    step itself, timed: encode the evicted K and V token and attend all g
    query heads over the decoded pool (dequantize and de-rotate the history,
    fp64 softmax attention)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    import synth

    name, b, kv, L, lloyd = task
    w = synth.WORKLOADS[name]
    with threadpool_limits(limits=1):
        import torch
        torch.set_num_threads(1)
        RK, RV, cK, cV = _cpu_tables(name)
        g, d, G = w.gqa, w.head_dim, w.group_size
        if lloyd:  # the Lloyd-Max variant: the oracle's own codebooks
            LK, LV = _cpu_codebooks(name)
            enc = lambda x, R, c, Lc: oracle.encode_lut(x, R, c, G, Lc)
            dec = lambda pk, s16, z16, R, Lc: oracle.decode_history_lut(pk, s16, z16, G, Lc, R)
        else:
            LK = LV = [None] * w.num_kv_heads
            enc = lambda x, R, c, Lc: oracle.encode(x, R, c, G)
            dec = lambda pk, s16, z16, R, Lc: oracle.decode_history(pk, s16, z16, G, R)
        q = synth.bf16_bits(synth.queries(w, 0))
        k = synth.bf16_bits(synth.kv_tokens(w, 0, b, 0, L + 1, heads=[kv]))[:, 0]
        v = synth.bf16_bits(synth.kv_tokens(w, 1, b, 0, L + 1, heads=[kv]))[:, 0]
        n_hist = max(0, L + 1 - 320)
        hk = enc(k[64:64 + n_hist - 1], RK[kv], cK[kv], LK[kv]) if n_hist > 1 else None
        hv = enc(v[64:64 + n_hist - 1], RV[kv], cV[kv], LV[kv]) if n_hist > 1 else None
        t0 = time.perf_counter()
        ek = enc(k[64 + n_hist - 1:64 + n_hist], RK[kv], cK[kv], LK[kv])
        ev = enc(v[64 + n_hist - 1:64 + n_hist], RV[kv], cV[kv], LV[kv])
        cat = (lambda a, e: e if a is None else tuple(np.concatenate([x, y]) for x, y in zip(a, e)))
        pk, sk, zk = cat(hk, ek)
        pv, sv, zv = cat(hv, ev)
        K = oracle.bf16_bits_to_f64(k)
        V = oracle.bf16_bits_to_f64(v)
        K[64:64 + n_hist] = dec(pk, sk, zk, RK[kv], LK[kv])
        V[64:64 + n_hist] = dec(pv, sv, zv, RV[kv], LV[kv])
        qf = oracle.bf16_bits_to_f64(q[b])
        for h in range(kv * g, (kv + 1) * g):
            oracle.attention(qf[h], K, V, 1 / math.sqrt(d))
        return time.perf_counter() - t0


_tables_cache = {}


def _cpu_tables(name):
    """The oracle's own rotation and clip tables (built once per worker)."""
    if name not in _tables_cache:
        import numpy as np

        import oracle
        import synth
        w = synth.WORKLOADS[name]
        RK = oracle.rotation(synth.random_orthogonal_u(w, 0))
        RV = oracle.rotation(synth.random_orthogonal_u(w, 1))
        cal = [synth.bf16_bits(synth.calibration_tokens(w, k, 4096)) for k in (0, 1)]
        cK = np.stack([oracle.clip_thresholds(cal[0][h], RK[h]) for h in range(w.num_kv_heads)])
        cV = np.stack([oracle.clip_thresholds(cal[1][h], RV[h]) for h in range(w.num_kv_heads)])
        _tables_cache[name] = (RK, RV, cK, cV)
    return _tables_cache[name]


_codebook_cache = {}


def _cpu_codebooks(name):
    """The oracle's Lloyd-Max codebooks (built once per worker)."""
    if name not in _codebook_cache:
        import numpy as np

        import oracle
        import synth
        w = synth.WORKLOADS[name]
        RK, RV, cK, cV = _cpu_tables(name)
        out = []
        for kind, (R, c) in enumerate(((RK, cK), (RV, cV))):
            cal = synth.bf16_bits(synth.calibration_tokens(w, kind, 4096))
            out.append(np.stack([oracle.lloyd_max_codebook(oracle.normalized_values(cal[h], R[h], c[h], w.group_size))
                                 for h in range(w.num_kv_heads)]))
        _codebook_cache[name] = tuple(out)
    return _codebook_cache[name]


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, lengths, budget_s, max_workers=16, lloyd=False):
    """The CPU oracle on a bounded sample of one step, on the host's cores:
    (sequence, kv head) pairs in worker processes (one thread each), spread
    over the batch, until about budget_s seconds of timed step work are done.
    Each worker processes pairs independently, so the host's step time is the
    mean timed seconds per pair x pairs / workers.  Runs before anything
    touches the GPU; the workers are fresh interpreters that never do."""
    import multiprocessing as mp

    import numpy as np

    cores = max(1, min(len(os.sched_getaffinity(0)), max_workers))
    rng = np.random.default_rng(7)
    pairs = [(int(i) // w.num_kv_heads, int(i) % w.num_kv_heads) for i in rng.permutation(w.batch * w.num_kv_heads)]
    tasks = [(w.name, b, kv, int(lengths[b]), lloyd) for b, kv in pairs]
    done, timed = 0, 0.0
    t0 = time.perf_counter()
    with mp.get_context("spawn").Pool(cores) as pool:
        for t in pool.imap_unordered(_cpu_pair, tasks):
            timed += t
            done += 1
            if timed >= budget_s and done >= cores:
                pool.terminate()
                break
    wall = time.perf_counter() - t0
    if done == 0:
        return None
    t_step = timed / done * (w.batch * w.num_kv_heads) / cores
    sample_len = sorted({int(lengths[b]) for b, _ in pairs[:done]})
    return {"value": w.batch / t_step, "unit": "tokens/s per layer", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {w.batch * w.num_kv_heads} (sequence, kv head) pairs of one step "
                      f"(lengths {sample_len[0]}..{sample_len[-1]}), {timed:.1f} s of timed oracle work on "
                      f"{cores} worker processes of one thread each ({wall:.1f} s wall with setup); "
                      f"step time = mean per pair x {w.batch * w.num_kv_heads} pairs / {cores}",
            "host": {"nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "cpu_model": _cpu_model()}}


MFMA_F16_PEAK_TFLOPS = 2500.0


def _cpu_prefill(name, L, n_q, n_sample):
    """The oracle's prefill attention of the g query heads of kv head 0 for
    the last n_sample of the chunk's n_q queries over that kv head's pool (its
    history encoded first, untimed); returns the timed seconds."""
    import oracle
    import synth
    w = synth.WORKLOADS[name]
    g = w.num_q_heads // w.num_kv_heads
    RK, RV, cK, cV = _cpu_tables(name)
    k = synth.bf16_bits(synth.kv_tokens(w, 0, 0, 0, L, heads=[0]))
    v = synth.bf16_bits(synth.kv_tokens(w, 1, 0, 0, L, heads=[0]))
    st = oracle.build_sequence(k, v, RK[:1], RV[:1], cK[:1], cV[:1], w.group_size)
    q = synth.bf16_bits(synth.queries(w, 0, batch=n_q))[n_q - n_sample:, :g]
    t0 = time.perf_counter()
    oracle.prefill_attention(st, q, 1 / math.sqrt(w.head_dim))
    return time.perf_counter() - t0


def prefill_main(args):
    """Prefill-attention measurement: the last n_q positions of one prompt of
    L tokens (the final chunk of a chunked prefill, its K/V already in the
    pool) attend causally over the three-segment pool.  Algorithmic flops:
    4 Hq d per (query, visible token) (QK^T and PV)."""
    import numpy as np
    import torch

    import bit_kv_cache_segment_amd as ok
    import harness
    import synth

    w = synth.WORKLOADS[args.workload]
    L, n_q = args.prefill_len, args.prefill_chunk
    cpu = None
    if args.cpu_seconds > 0:
        n_s = min(1024, n_q)
        g = w.num_q_heads // w.num_kv_heads
        secs = _cpu_prefill(w.name, L, n_q, n_s)
        from threadpoolctl import threadpool_info
        blas = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        cpu = {"value": n_q / (secs * (n_q / n_s) * (w.num_q_heads / g)), "unit": "tokens/s per layer",
               "cores": max(blas) if blas else 1, "kind": "oracle",
               "sample": f"oracle prefill attention of the {g} query heads of 1 of {w.num_kv_heads} kv heads for "
                         f"the last {n_s} of {n_q} queries ({secs:.1f} s, history encoding untimed), scaled to "
                         f"the chunk"}
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    RK, RV, cK, cV = harness.tables(w)
    cfg = harness.config_for(w, [L])
    pools = []
    for layer in range(args.layers):
        p = ok.Pool(cfg, RK, RV, cK, cV, max_batch=1)
        harness.prefill_all(p, w, [L])
        pools.append(p)
    q = synth.queries(w, 0, device="cuda", batch=n_q).view(torch.uint16).contiguous()
    out = torch.empty((n_q, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    wsb = ok.oscar_prefill_workspace_bytes(cfg, n_q)
    ws = torch.empty(max(wsb, 4) // 4, dtype=torch.float32, device=dev)
    for s in range(args.warmup):
        pools[s % args.layers].prefill_attn(0, q, out, workspace=ws)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for s in range(args.steps):
        pools[s % args.layers].prefill_attn(0, q, out, workspace=ws)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    visible = sum(L - n_q + i + 1 for i in range(n_q))
    flops = 4.0 * w.num_q_heads * w.head_dim * visible
    tflops = flops / (ms * 1e-3) / 1e12
    res = {
        "metric": "prefill attention tokens/s per layer (chunk over the three-segment pool)",
        "value": n_q / (ms * 1e-3), "unit": "tokens/s per layer", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int2 codes + fp16 scale/zero history, bf16 windows, fp16 (hi + lo) / bf16 MFMA, fp32 accumulate",
        "data": "synthetic (seeded; K/V ~ N(0,1) with 4 outlier channels x20)",
        "config": {"workload": f"{w.name} prefill chunk", "prompt_len": L, "chunk": n_q, "q_heads": w.num_q_heads,
                   "kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "group_size": w.group_size,
                   "layer_pools": args.layers, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / MFMA_F16_PEAK_TFLOPS, "traffic": None,
                     "algorithmic_flops": flops},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


FP32_VECTOR_PEAK_TFLOPS = 157.3


def _cpu_calibration(name, n, heads):
    """The oracle's covariances (Q^T Q and V^T S^T S V) of `heads` query heads
    of a calibration sequence of n tokens, timed (inputs generated first)."""
    import numpy as np

    import oracle
    import synth

    w = synth.WORKLOADS[name]
    g = w.num_q_heads // w.num_kv_heads
    q, k, v = synth.calibration_activations(w, n)
    kvh = -(-heads // g)
    qb = synth.bf16_bits(q[:, :heads].contiguous())
    kb, vb = (synth.bf16_bits(x[:, :kvh].contiguous()) for x in (k, v))
    t0 = time.perf_counter()
    oracle.query_covariance(qb, kvh)
    oracle.value_covariance(qb, kb, vb, 1 / np.sqrt(w.head_dim))
    return time.perf_counter() - t0


def calibrate_main(args):
    """Offline calibration statistics of one layer on the GPU: for one
    calibration sequence of n tokens, the causal attention S V of every
    query head (calib_attn_kernel) and the Gram matrices Q^T Q and
    (S V)^T (S V) per kv head on matrix cores (gram_kernel), i.e. one
    oscar_calib_covariance call.  The attention kernel, which dominates,
    is timed alone (oscar_calib_attention) for the roofline: 4 d flops per
    (query head, visible key) against the fp32 vector peak."""
    import numpy as np
    import torch

    import bit_kv_cache_segment_amd as ok
    import synth

    w = synth.WORKLOADS[args.workload]
    n = args.calib_tokens
    cpu = None
    if args.cpu_seconds > 0:
        # bounded sample: the oracle on 8 query heads (2 kv heads), scaled to all
        heads = min(8, w.num_q_heads)
        secs = _cpu_calibration(w.name, n, heads)
        from threadpoolctl import threadpool_info
        blas = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        cpu = {"value": n / (secs * w.num_q_heads / heads), "unit": "tokens/s per layer",
               "cores": max(blas) if blas else 1, "kind": "oracle",
               "sample": f"oracle covariances of {heads} of {w.num_q_heads} query heads at n = {n}, "
                         f"{secs:.1f} s, scaled to all heads"}
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    q, k, v = (x.to(dev).view(torch.uint16).contiguous() for x in synth.calibration_activations(w, n))
    Hkv, d = w.num_kv_heads, w.head_dim
    scale = 1.0 / np.sqrt(d)
    ck = torch.zeros((Hkv, d, d), dtype=torch.float32, device=dev)
    cv = torch.zeros_like(ck)
    ws = torch.empty(ok.oscar_calib_workspace_bytes(n, w.num_q_heads, d), dtype=torch.uint8, device=dev)
    o = torch.empty((n, w.num_q_heads, d), dtype=torch.float32, device=dev)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms_step = timed(lambda: ok.oscar_calib_covariance(q, k, v, scale, ck, cv, ws))
    ms_attn = timed(lambda: ok.oscar_calib_attention(q, k, v, scale, o))
    flops = 4.0 * w.num_q_heads * d * (n * (n + 1) / 2)
    tflops = flops / (ms_attn * 1e-3) / 1e12
    res = {
        "metric": "calibration tokens/s per layer (query and score-weighted value covariances)",
        "value": n / (ms_step * 1e-3), "unit": "tokens/s per layer", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 inputs, fp32 attention and Gram accumulation",
        "data": "synthetic (seeded; queries with a planted covariance, K/V with 4 outlier channels x20)",
        "config": {"workload": f"{w.name} calibration sequence", "tokens": n, "q_heads": w.num_q_heads,
                   "kv_heads": Hkv, "head_dim": d, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "alu", "achieved": tflops, "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / FP32_VECTOR_PEAK_TFLOPS, "traffic": None,
                     "kernel": "calib_attn_kernel", "algorithmic_flops": flops, "ms_per_launch": ms_attn},
        "cpu_baseline": cpu,
        "detail": {"ms_attention": ms_attn, "ms_gram_both": ms_step - ms_attn},
    }
    print(json.dumps(res), flush=True)


def compare_bf16_main(args):
    """Decode at long context, batch 1: the same tokens in an INT2-history
    pool and in a BF16-history pool (OSCAR_POOL_BF16_HISTORY), decode
    attention (oscar_decode_attn) and the serving step (oscar_decode_step)
    timed on each; pools rotate so the read set exceeds the 256 MB cache."""
    import numpy as np
    import torch

    import bit_kv_cache_segment_amd as ok
    import harness
    import synth

    w = synth.WORKLOADS[args.workload]
    lengths0 = [int(x) for x in synth.lengths(w)]
    # the oracle's INT2 decode step on the same workload, before the GPU is touched
    cpu = cpu_baseline(w, lengths0, args.cpu_seconds) if args.cpu_seconds > 0 else None
    if cpu:
        cpu["unit"] = "tokens/s per layer (INT2 history decode step; the metric is a ratio)"
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    ids = list(range(w.batch))
    total = args.warmup + args.steps
    per = -(-total // args.layers)
    RK, RV, cK, cV = harness.tables(w)
    qs = [synth.queries(w, s, device="cuda").view(torch.uint16).contiguous() for s in range(total)]
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    res = {}
    for name, flags in (("int2", 0), ("bf16", ok.POOL_BF16_HISTORY)):
        cfg = harness.config_for(w, lengths0, extra_tokens=per, flags=flags)
        pools = []
        for layer in range(args.layers):
            p = ok.Pool(cfg, RK, RV, cK, cV, max_batch=w.batch)
            harness.prefill_all(p, w, lengths0)
            pools.append(p)
        toks = [harness.step_tokens(w, [L + a for L in lengths0]) for a in range(per)]
        torch.cuda.synchronize()
        timing = {}
        for kind in ("decode", "step"):
            def run(s):
                p = pools[s % args.layers]
                if kind == "decode":
                    p.decode(ids, qs[s], out)
                else:
                    a = s // args.layers
                    p.step(ids, toks[a][0], toks[a][1], qs[s], out)
            for s in range(args.warmup):
                run(s)
            torch.cuda.synchronize()
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record()
            for s in range(args.warmup, total):
                run(s)
            ev1.record()
            torch.cuda.synchronize()
            timing[kind] = ev0.elapsed_time(ev1) / args.steps * 1e3  # us
        res[name] = timing
        res[name]["pool_bytes_per_layer"] = ok.oscar_pool_bytes(cfg)
        del pools
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    line = {
        "metric": "decode latency at long context, batch 1: INT2 history vs BF16 history (same pool, same tokens)",
        "value": res["bf16"]["decode"] / res["int2"]["decode"], "unit": "x (BF16 time / INT2 time, decode attention)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
        "data": "synthetic (seeded; K/V ~ N(0,1) with 4 outlier channels x20)",
        "config": {"workload": w.name, "batch": w.batch, "context": lengths0[0], "q_heads": w.num_q_heads,
                   "kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "group_size": w.group_size,
                   "layer_pools": args.layers},
        "int2_us": {"decode": res["int2"]["decode"], "step": res["int2"]["step"]},
        "bf16_us": {"decode": res["bf16"]["decode"], "step": res["bf16"]["step"]},
        "step_speedup": res["bf16"]["step"] / res["int2"]["step"],
        "pool_bytes_per_layer": {"int2": res["int2"]["pool_bytes_per_layer"],
                                 "bf16": res["bf16"]["pool_bytes_per_layer"]},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="fused_64x_4k_64k",
                    help="the largest workload by default: 64 sequences of 4K-64K tokens, 32/8 heads")
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="seconds of timed oracle work for the CPU baseline (0 skips it)")
    ap.add_argument("--no-kernel-timing", action="store_true",
                    help="time the steps without per-kernel events (roofline fields become null)")
    ap.add_argument("--separate-calls", action="store_true",
                    help="append and decode as two calls (three launches) instead of one fused step")
    ap.add_argument("--time-every", type=int, default=4,
                    help="events around one decode_main launch in this many, per layer pool "
                         "(each timed launch adds a few microseconds to its step)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run a plain device copy of this size first (counter calibration)")
    ap.add_argument("--mode", choices=["decode", "prefill", "compare_bf16", "calibrate"], default="decode",
                    help="decode: the serving step (headline); prefill: a prefill chunk's attention; "
                         "compare_bf16: INT2 vs BF16 history at long context, batch 1; "
                         "calibrate: offline covariances of one layer")
    ap.add_argument("--calib-tokens", type=int, default=4096, help="calibrate mode: calibration sequence length")
    ap.add_argument("--codebook", choices=["affine", "lloyd_max"], default="affine",
                    help="decode mode: the history levels (lloyd_max: the Lloyd-Max codebook variant)")
    ap.add_argument("--prefill-len", type=int, default=32768, help="prefill mode: prompt length")
    ap.add_argument("--prefill-chunk", type=int, default=2048, help="prefill mode: queries of the last chunk")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the decode path runs on a single device and has no "
              "multi-GPU mode; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.mode == "compare_bf16":
        if args.workload == "fused_64x_4k_64k":
            args.workload = "qwen3_8b_100k_b1"
        compare_bf16_main(args)
        return
    if args.mode == "calibrate":
        if args.workload == "fused_64x_4k_64k":
            args.workload = "qwen3_8b_32k"
        calibrate_main(args)
        return
    if args.mode == "prefill":
        if args.workload == "fused_64x_4k_64k":
            args.workload = "qwen3_8b_32k"
        prefill_main(args)
        return

    import numpy as np

    import synth

    w = synth.WORKLOADS[args.workload]
    lengths0 = [int(x) for x in synth.lengths(w)]
    lloyd = args.codebook == "lloyd_max"
    # the CPU baseline first, before this process touches the GPU
    cpu = cpu_baseline(w, lengths0, args.cpu_seconds, lloyd=lloyd) if args.cpu_seconds > 0 else None

    import torch

    import bit_kv_cache_segment_amd as ok
    import harness

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    total_steps = args.warmup + args.steps
    appends_per_layer = -(-total_steps // args.layers)
    RK, RV, cK, cV = harness.tables(w)
    cfg = harness.config_for(w, lengths0, extra_tokens=appends_per_layer, flags=ok.POOL_LLOYD_MAX if lloyd else 0)
    codebooks = harness.codebooks(w, RK, RV, cK, cV) if lloyd else None
    pools = []
    for layer in range(args.layers):
        p = ok.Pool(cfg, RK, RV, cK, cV, max_batch=w.batch)
        if lloyd:
            p.set_codebook(*codebooks)
        harness.prefill_all(p, w, lengths0)
        pools.append(p)
    ids = list(range(w.batch))
    toks = [harness.step_tokens(w, [L + a for L in lengths0]) for a in range(appends_per_layer)]
    qs = [synth.queries(w, s, device="cuda").view(torch.uint16).contiguous() for s in range(total_steps)]
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    if args.copy_probe_mib:
        # a plain device copy of known size: reads and writes copy_probe_mib MiB
        # (its FETCH_SIZE / WRITE_SIZE calibrate the counter units)
        n = args.copy_probe_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    torch.cuda.synchronize()

    def step(s):
        # one serving step of a layer: append the new token, then attend
        # (one fused call unless --separate-calls)
        layer = s % args.layers
        a = s // args.layers
        if args.separate_calls:
            pools[layer].append(ids, toks[a][0], toks[a][1])
            pools[layer].decode(ids, qs[s], out)
        else:
            pools[layer].step(ids, toks[a][0], toks[a][1], qs[s], out)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    if not args.no_kernel_timing:
        for p in pools:
            p.profile_begin(args.steps, every=args.time_every)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for s in range(args.warmup, total_steps):
        step(s)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    if args.no_kernel_timing:
        ms_main = float("nan")
    else:
        profs = [p.profile_end() for p in pools]
        n_main = sum(p.n_decode_main for p in profs)
        ms_main = sum(p.ms_decode_main for p in profs) / max(n_main, 1)

    # algorithmic bytes of each timed decode launch (lengths after its append):
    # the k-th decode of each layer pool in the timed region, k = 0, every, ...
    bytes_main = []
    for s in range(args.warmup, total_steps):
        a = s // args.layers
        k = sum(1 for t in range(args.warmup, s) if t % args.layers == s % args.layers)
        if k % args.time_every == 0:
            bytes_main.append(algorithmic_decode_bytes(w, [L + a + 1 for L in lengths0]))
    bytes_launch = float(np.mean(bytes_main))
    achieved = bytes_launch / (ms_main * 1e-3) / 1e9
    # (the codebook variant is decode_main_kernel's LUT instantiation: its own
    # traffic record)
    kname = "decode_main_lut" if lloyd else "decode_main"
    traffic = traffic_record(os.path.join(ROOT, "bit_kv_cache_segment_amd", "csrc", "kernels_decode.hip"), w.name,
                             kname)
    value = w.batch / (ms_step * 1e-3)
    step_bytes = bytes_launch + w.batch * w.num_q_heads * w.head_dim * 4
    res = {
        "metric": "INT2-KV decode attention tokens/s per layer + achieved HBM GB/s (% peak)",
        "value": value,
        "unit": "tokens/s per layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("int2 codes (Lloyd-Max codebook) + fp16 scale/zero history, bf16 windows, fp32 accumulate"
                  if lloyd else "int2 codes + fp16 scale/zero history, bf16 windows, fp32 accumulate"),
        "data": "synthetic (seeded; K/V ~ N(0,1) with 4 outlier channels x20)",
        "config": {"workload": w.name, "codebook": args.codebook, "batch": w.batch, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "group_size": w.group_size,
                   "context_min": min(lengths0), "context_max": max(lengths0),
                   "context_mean": float(np.mean(lengths0)),
                   "appended_per_pool": appends_per_layer, "layer_pools": args.layers,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": "decode_main_kernel" + ("<LUT>" if lloyd else ""), "bytes_per_launch": bytes_launch,
                     "ms_per_launch": ms_main},
        "cpu_baseline": cpu,
        "detail": {"ms_decode_main": ms_main,
                   "timed_decode_launches": None if args.no_kernel_timing else n_main,
                   "step_call": "oscar_append_evict + oscar_decode_attn" if args.separate_calls
                   else "oscar_decode_step",
                   "time_every": args.time_every,
                   "step_hbm_gbps": step_bytes / (ms_step * 1e-3) / 1e9,
                   "bits_per_element": (sum(max(0, L - 320) * (2 + 32 / w.group_size) + min(L, 320) * 16
                                            for L in lengths0) / sum(lengths0)),
                   "wall_s": wall},
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
