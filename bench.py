"""Benchmark of the OSCAR INT2-KV decode hot path on one MI355X.

One step = one pass of the whole path over the batch: append one token per
sequence (evicting the oldest recent token into the INT2 history: rotate,
clip, quantize, pack) and decode attention for one query per sequence
(INT2 split-KV + BF16 window + online-softmax merge + de-rotation).
Steps rotate over several layer pools so the read set exceeds the 256 MB
Infinity Cache.  Prints one JSON line.
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


def traffic_record(kernel_src, workload):
    """HBM bytes per launch measured with rocprofv3 counters, if the record in
    profiles/ was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"decode_main_{workload}_traffic.txt")
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


def cpu_baseline(w, lengths, budget_s):
    """The CPU oracle on a bounded sample of the same step: for a few
    (sequence, kv head) pairs, encode the evicted K and V token and attend all
    g query heads over the decoded pool (dequantize + de-rotate the history,
    fp64 softmax attention).  Encoding the prompt's history is setup."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    import synth

    RK = oracle.rotation(synth.random_orthogonal_u(w, 0))
    RV = oracle.rotation(synth.random_orthogonal_u(w, 1))
    cal = [synth.bf16_bits(synth.calibration_tokens(w, k, 4096)) for k in (0, 1)]
    cK = np.stack([oracle.clip_thresholds(cal[0][h], RK[h]) for h in range(w.num_kv_heads)])
    cV = np.stack([oracle.clip_thresholds(cal[1][h], RV[h]) for h in range(w.num_kv_heads)])
    q = synth.bf16_bits(synth.queries(w, 0))
    g, d, G = w.gqa, w.head_dim, w.group_size
    timed, pairs = 0.0, 0
    order = [(b, kv) for kv in range(w.num_kv_heads) for b in range(w.batch)]
    with threadpool_limits(limits=1):
        for b, kv in order:
            L = int(lengths[b])
            k = synth.bf16_bits(synth.kv_tokens(w, 0, b, 0, L + 1, heads=[kv]))[:, 0]
            v = synth.bf16_bits(synth.kv_tokens(w, 1, b, 0, L + 1, heads=[kv]))[:, 0]
            n_hist = max(0, L + 1 - 320)
            hk = oracle.encode(k[64:64 + n_hist - 1], RK[kv], cK[kv], G) if n_hist > 1 else None
            hv = oracle.encode(v[64:64 + n_hist - 1], RV[kv], cV[kv], G) if n_hist > 1 else None
            t0 = time.perf_counter()
            # the step: evict one token per K/V, then decode-then-attend
            ek = oracle.encode(k[64 + n_hist - 1:64 + n_hist], RK[kv], cK[kv], G)
            ev = oracle.encode(v[64 + n_hist - 1:64 + n_hist], RV[kv], cV[kv], G)
            pk = np.concatenate([hk[0], ek[0]]); sk = np.concatenate([hk[1], ek[1]]); zk = np.concatenate([hk[2], ek[2]])
            pv = np.concatenate([hv[0], ev[0]]); sv = np.concatenate([hv[1], ev[1]]); zv = np.concatenate([hv[2], ev[2]])
            K = oracle.bf16_bits_to_f64(k)
            V = oracle.bf16_bits_to_f64(v)
            K[64:64 + n_hist] = oracle.decode_history(pk, sk, zk, G, RK[kv])
            V[64:64 + n_hist] = oracle.decode_history(pv, sv, zv, G, RV[kv])
            qf = oracle.bf16_bits_to_f64(q[b])
            for h in range(kv * g, (kv + 1) * g):
                oracle.attention(qf[h], K, V, 1 / math.sqrt(d))
            timed += time.perf_counter() - t0
            pairs += 1
            if timed >= budget_s:
                break
    if pairs == 0:
        return None
    t_step = timed / pairs * w.batch * w.num_kv_heads
    return {"value": w.batch / t_step, "unit": "tokens/s per layer", "cores": 1, "kind": "oracle",
            "sample": f"{pairs} of {w.batch * w.num_kv_heads} (sequence, kv head) pairs of one step "
                      f"({timed:.1f} s, 1 thread), scaled to the whole batch"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_8b_32k")
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="0 skips the CPU baseline")
    ap.add_argument("--no-kernel-timing", action="store_true",
                    help="time the steps without per-kernel events (roofline fields become null)")
    ap.add_argument("--separate-calls", action="store_true",
                    help="append and decode as two calls (three launches) instead of one fused step")
    ap.add_argument("--time-every", type=int, default=4,
                    help="events around one decode_main launch in this many, per layer pool "
                         "(each timed launch adds a few microseconds to its step)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run a plain device copy of this size first (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the decode path runs on a single device and has no "
              "multi-GPU mode; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_kv_cache_segment_amd as ok
    import harness
    import synth

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    lengths0 = [int(x) for x in synth.lengths(w)]
    total_steps = args.warmup + args.steps
    appends_per_layer = -(-total_steps // args.layers)
    RK, RV, cK, cV = harness.tables(w)
    cfg = harness.config_for(w, lengths0, extra_tokens=appends_per_layer)
    pools = []
    for layer in range(args.layers):
        p = ok.Pool(cfg, RK, RV, cK, cV, max_batch=w.batch)
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
    traffic = traffic_record(os.path.join(ROOT, "bit_kv_cache_segment_amd", "csrc", "kernels_decode.hip"),
                             w.name)
    value = w.batch / (ms_step * 1e-3)
    cpu = cpu_baseline(w, lengths0, args.cpu_seconds) if args.cpu_seconds > 0 else None
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
        "dtype": "int2 codes + fp16 scale/zero history, bf16 windows, fp32 accumulate",
        "data": "synthetic (seeded; K/V ~ N(0,1) with 4 outlier channels x20)",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "group_size": w.group_size, "context": lengths0[0],
                   "layer_pools": args.layers, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": "decode_main_kernel", "bytes_per_launch": bytes_launch,
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
