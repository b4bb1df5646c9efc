"""Benchmark of the compressed-KV decode path on one MI355X.

One step = one whole decode run of the workload on synthetic inputs already
resident in HBM: starting from an empty cache, every token appends one K and
one V row to every layer (the window's oldest 64 rows fold into the low-rank
history whenever it holds w + b rows) and then runs decode attention over the
compressed cache of every layer, both through one iskv_append_decode call per
token. For the Llama-3-8B-shaped workload that is 8192 tokens x 32 layers x
8 kv heads, 126 fold rounds per unit stream.

Printed: one JSON line (metric, value = KV rows folded into history per
second over the whole job, roofline of the dominant kernel measured with HIP
events inside the timed region, CPU-oracle baseline).
"""

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "KV rows compressed/sec and decode-attn tokens/sec; % of HBM roofline"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=3)
    p.add_argument("--warmup", type=int, default=1)
    p.add_argument("--workload", default="llama3_8b_gqa_8k")
    p.add_argument("--tokens", type=int, default=0, help="override decode tokens (profiling runs)")
    p.add_argument("--sample-every", type=int, default=1,
                   help="event-time every n-th run of decode launches between two folds")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-units", type=int, default=0, help="oracle sample size (default: one per core, <= 32)")
    p.add_argument("--prefill", action="store_true",
                   help="time the one-shot prompt factorisation of the long-input workload against "
                        "folding the same prompt block by block, print one JSON line and exit")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run one plain 1 GiB device-to-device copy and exit (reference for HBM byte counters)")
    return p.parse_args()


def copy_calibration():
    """One plain copy kernel of known size: 1 GiB read, 1 GiB written. Under
    rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE its counter readings give the
    factor that turns those counters into bytes."""
    import torch

    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.mul(src, 1.0, out=dst)  # an elementwise kernel: 1 GiB in, 1 GiB out
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n}), flush=True)


def decode_bytes(U, g, n, e, kK, kV, coord_b, kv_b, appended=0):
    """Algorithmic HBM bytes of one decode launch over U units: history
    coordinates of K and V, window rows of K and V (e includes an appended
    row, read from the caller's buffer), both bases, queries in, outputs out
    (fp32), and the appended K and V rows written to the window ring."""
    per = (n * (kK + kV) * coord_b + 2 * e * 128 * kv_b + (kK + kV) * 128 * 4
           + g * 128 * kv_b + g * 128 * 4 + appended * 2 * 128 * kv_b)
    return U * per


def fold_bytes(U, n, b, kK, kV, kKp, kVp, coord_b, kv_b):
    """Algorithmic HBM bytes of one fold round (K and V): old coordinates read
    and rewritten, new rows written, the pending block read, bases and singular
    values read and written."""
    tot = 0
    for k, kp in ((kK, kKp), (kV, kVp)):
        tot += n * k * coord_b + (n + b) * kp * coord_b + b * 128 * kv_b + 4 * (128 * k + 128 * kp + k + kp)
    return U * tot


def source_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def cpu_baseline(w, nunits):
    """The fp64 oracle on a bounded sample of the same workload: full-length
    K/V unit streams (8192 rows each, 126 folds) run in parallel threads."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    import synth

    oracle.load()
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    cores = max(1, min(cores, 16))
    if nunits <= 0:
        nunits = min(2 * cores, 32)
    jobs = []
    for i in range(nunits):
        kind = "KV"[i % 2]
        l, h = (i // 2) // w.kv_heads % w.layers, (i // 2) % w.kv_heads
        X = synth.kv_rows(w, kind, 0, l, h, w.total_tokens)
        jobs.append((X, w.rank_k if kind == "K" else w.rank_v))
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=cores) as ex:
        states = list(ex.map(lambda j: oracle.run_unit(j[0], 128, w.block, j[1], w.window), jobs))
    dt = time.perf_counter() - t0
    rows = sum(s.n for s in states)
    return {"value": rows / dt, "unit": "KV rows compressed/s", "cores": cores, "kind": "oracle",
            "sample": "%d full-length unit streams (%s, %d tokens each, %d folds) of the %s workload, "
                      "fp64 C oracle, %d threads, %.1f s wall" % (
                          nunits, "K and V alternating", w.total_tokens, len(states[0].log), w.name,
                          cores, dt)}


def prefill_bench(args):
    """Prompt compression of the long-input workload (65536 prompt rows per
    unit, 32 layers x 8 kv heads, ranks 32 / 48): one iskv_prefill_oneshot
    call against 1024 iskv_prefill_block calls over the same rows, both timed
    with the inputs resident in HBM. Both leave the whole prompt in the
    history (window empty)."""
    import torch

    import synth
    from incremental_rank_svd_amd import iskv

    w = synth.get_config("long_input_64k")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = iskv.load()
    P = w.prefill_blocks * w.block
    K = synth.kv_rows_torch(w, "K", P, dev)  # [B, L, Hk, P, d]
    V = synth.kv_rows_torch(w, "V", P, dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    res = {}
    for mode in ("oneshot", "blocks"):
        cache = iskv.Cache(iskv.config_from_workload(w), device=dev)
        h = cache.h
        blocks = [(K[:, :, :, s:s + w.block].contiguous(), V[:, :, :, s:s + w.block].contiguous())
                  for s in range(0, P, w.block)] if mode == "blocks" else None
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if mode == "oneshot":
            rc = lib.iskv_prefill_oneshot(h, ctypes.c_void_p(K.data_ptr()), ctypes.c_void_p(V.data_ptr()), P, 0,
                                          w.layers, sp)
            if rc:
                raise RuntimeError("prefill_oneshot failed: %d" % rc)
        else:
            for kb, vb in blocks:
                rc = lib.iskv_prefill_block(h, ctypes.c_void_p(kb.data_ptr()), ctypes.c_void_p(vb.data_ptr()), 0,
                                            w.layers, sp)
                if rc:
                    raise RuntimeError("prefill_block failed: %d" % rc)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        if cache.status():
            raise RuntimeError("numeric flags %#x" % cache.status())
        res[mode] = dt
        del blocks, cache
        torch.cuda.empty_cache()
    rows = 2 * w.batch * w.layers * w.kv_heads * P
    print(json.dumps({
        "metric": "prompt KV rows factorised/sec",
        "value": rows / res["oneshot"], "unit": "KV rows/s", "n_gpus": 1,
        "ms": res["oneshot"] * 1e3, "higher_is_better": True,
        "blockwise_ms": res["blocks"] * 1e3, "blockwise_value": rows / res["blocks"],
        "speedup_vs_blockwise": res["blocks"] / res["oneshot"],
        "dtype": "bf16 storage, f32 compute", "data": "synthetic (power-law spectrum KV, seeded), resident in HBM",
        "config": {"workload": w.name, "batch": w.batch, "layers": w.layers, "kv_heads": w.kv_heads,
                   "prompt_rows": P, "rank_k": w.rank_k, "rank_v": w.rank_v},
    }), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.prefill:
        if args.gpus != 1:
            print("bench.py measures one GPU only; run with --gpus 1", file=sys.stderr)
            sys.exit(2)
        prefill_bench(args)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the compressed-cache path has no cross-GPU step "
              "(units are independent); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    from incremental_rank_svd_amd import iskv

    w = synth.get_config(args.workload)
    if args.tokens:
        from dataclasses import replace
        w = replace(w, decode_tokens=args.tokens)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = iskv.load()
    cfg = iskv.config_from_workload(w)
    cache = iskv.Cache(cfg, device=dev)
    T, L, B, Hk, Hq = w.total_tokens, w.layers, w.batch, w.kv_heads, w.q_heads
    U = B * L * Hk
    kvdt = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
    kv_b = 2 if w.kv_dtype == "bf16" else 4
    coord_b = 2 if w.coord_dtype == "bf16" else 4

    # inputs resident in HBM, token-major so every token's rows are contiguous
    K = synth.kv_rows_torch(w, "K", T, dev)            # [B, L, Hk, T, d]
    V = synth.kv_rows_torch(w, "V", T, dev)
    K = K.permute(3, 0, 1, 2, 4).contiguous()           # [T, B, L, Hk, d]
    V = V.permute(3, 0, 1, 2, 4).contiguous()
    gen = torch.Generator(device=dev)
    gen.manual_seed(synth.unit_key(w.cfg_id, 0, "Q", 0, 0, 0) & ((1 << 63) - 1))
    Q = torch.randn((T, B, L, Hq, 128), generator=gen, device=dev).to(kvdt)
    out = torch.empty((B, L, Hq, 128), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    h = cache.h
    kp0, vp0, qp0, op = K.data_ptr(), V.data_ptr(), Q.data_ptr(), ctypes.c_void_p(out.data_ptr())
    kstr = K[0].numel() * K.element_size()
    qstr = Q[0].numel() * Q.element_size()
    scale = ctypes.c_float(128 ** -0.5)
    step_call, decode = lib.iskv_append_decode, lib.iskv_decode_attn
    VP = ctypes.c_void_p
    n_sample = max(1, args.sample_every)

    def run_step(sampled):
        """One pass of the whole path over the T tokens. With `sampled`, the
        runs of consecutive non-folding tokens (the launches between two folds)
        are bracketed by one pair of events each: kernels on the stream run
        back to back, so a run's elapsed time over its launch count is the
        kernel's average duration, without a per-launch event overhead."""
        if lib.iskv_reset(h, sp) != 0:
            raise RuntimeError("reset failed")
        n = e = kK = kV = 0
        b, wnd = w.block, w.window
        ev = []
        seg = None  # [start event, bytes, launches] of the open run
        nseg = 0
        for t in range(T):
            e += 1
            folds = e >= wnd + b  # this token's append folds: the call runs ingest, fold, decode
            if folds:
                p = min(b, 128 - kK)
                kK = min(w.rank_k, kK + p)
                p = min(b, 128 - kV)
                kV = min(w.rank_v, kV + p)
                n += b
                e -= b
            args = (h, VP(kp0 + t * kstr), VP(vp0 + t * kstr), VP(qp0 + t * qstr), op, 0, L, scale, sp)
            if sampled is not None:
                if folds and seg is not None:
                    e1 = torch.cuda.Event(enable_timing=True)
                    e1.record(stream)
                    ev.append((seg[0], e1, seg[1], seg[2]))
                    seg = None
                if not folds:
                    if seg is None and nseg % n_sample == 0:
                        e0 = torch.cuda.Event(enable_timing=True)
                        e0.record(stream)
                        seg = [e0, 0, 0]
                    if seg is not None:
                        seg[1] += decode_bytes(U, w.group, n, e, kK, kV, coord_b, kv_b, appended=1)
                        seg[2] += 1
                if folds:
                    nseg += 1
            rc = step_call(*args)
            if rc:
                raise RuntimeError("append_decode failed: %d" % rc)
        if seg is not None:
            e1 = torch.cuda.Event(enable_timing=True)
            e1.record(stream)
            ev.append((seg[0], e1, seg[1], seg[2]))
        if sampled is not None:
            sampled.extend(ev)
        return n

    for _ in range(args.warmup):
        run_step(None)
    torch.cuda.synchronize()
    flags = cache.status()
    if flags:
        raise RuntimeError("numeric flags %#x" % flags)

    samples = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n_final = 0
    for _ in range(args.steps):
        n_final = run_step(samples)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_s = (t1 - t0) / args.steps
    flags = cache.status()
    if flags:
        raise RuntimeError("numeric flags %#x" % flags)

    dec_ms = [s[0].elapsed_time(s[1]) for s in samples]
    dec_bytes = sum(s[2] for s in samples)
    dec_launches = sum(s[3] for s in samples)
    dec_avg_us = 1e3 * sum(dec_ms) / dec_launches
    achieved = dec_bytes / (sum(dec_ms) * 1e-3) / 1e9
    dec_share = (dec_avg_us * 1e-6 * T) / step_s

    # decode-only rate and fold-round time at the final state (after the timed region)
    n, e, kK, kV = cache.counts(0)
    reps = 50
    evs = []
    for i in range(reps):
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        decode(h, VP(qp0 + (i % T) * qstr), op, 0, L, scale, sp)
        a1.record(stream)
        evs.append((a0, a1))
    torch.cuda.synchronize()
    final_ms = sorted(a.elapsed_time(b) for a, b in evs)[reps // 2]
    final_bytes = decode_bytes(U, w.group, n, e, kK, kV, coord_b, kv_b)

    rows_folded = 2 * U * n_final
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "decode_traffic.json")
    if os.path.exists(tpath):
        try:
            tr = json.load(open(tpath))
            src = os.path.join(ROOT, "incremental_rank_svd_amd", "csrc", "k_decode.hip")
            if tr.get("source_sha256_16") == source_hash(src) and tr.get("workload") == w.name:
                traffic = tr.get("bytes_per_launch")
        except Exception:
            traffic = None

    res = {
        "metric": METRIC,
        "value": rows_folded / step_s,
        "unit": "KV rows compressed/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 storage, f32 compute" if w.kv_dtype == "bf16" else "f32",
        "data": "synthetic (power-law spectrum KV, seeded), resident in HBM",
        "config": {"workload": w.name, "batch": B, "layers": L, "kv_heads": Hk, "q_heads": Hq,
                   "head_dim": 128, "tokens": T, "block": w.block, "rank_k": w.rank_k,
                   "rank_v": w.rank_v, "window": w.window, "step": "full decode run 0->%d tokens" % T},
        "decode_attn_tokens_per_s": B * T / step_s,
        "decode_attn_tokens_per_s_at_final_n": B / (final_ms * 1e-3),
        "decode_at_final_n": {"n": n, "e": e, "k_k": kK, "k_v": kV, "ms": final_ms,
                              "GBps": final_bytes / (final_ms * 1e-3) / 1e9},
        "roofline": {"kernel": "k_decode", "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "avg_launch_us": dec_avg_us, "launches_sampled": dec_launches,
                     "share_of_step": dec_share},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_units)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
