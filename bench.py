"""Benchmark of the compressed-KV path on one MI355X.

Default: the LLaMA-2-13B-shaped MHA workload (batch 16, 40 layers x 40 kv
heads, b = 128, r_K = 64, r_V = 96, window 256, 16384 tokens), the largest
workload that fits one GPU. Its history is injected before the timed region
(each layer's first n0 rows factorised by iskv_prefill_oneshot, then the
window filled to w rows), so that the timed steps are the last fold rounds of
the 16384-token run. One step = the whole hot path over one batch of new
rows: iskv_append_block of b new K and V rows per unit to all 40 layers
(ingest, fold core, coordinate rewrite, commit: one fold round of 51200 unit
streams), then iskv_decode_attn of one query per head over all 40 layers at
the new n. Inputs (rows, queries) are resident in HBM before the timed region.

value = KV rows folded into history per second over the timed steps. Per
kernel (core, rewrite, decode) durations come from HIP events on the launch
stream inside the timed region (the library records caller events around the
fold's kernels, iskv_set_fold_events); `roofline` is the kernel with the
largest share of the step, `roofline_kernels` all three.

--workload llama3_8b_gqa_8k --full-run: the whole Llama-3-8B-shaped decode run
from an empty cache (one iskv_append_decode call per token, 8192 tokens).
--prefill: one-shot prompt factorisation of the long-input workload.

Printed: one JSON line.
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
    p.add_argument("--workload", default="llama2_13b_mha_16k")
    p.add_argument("--full-run", action="store_true",
                   help="time whole decode runs from an empty cache (one append_decode call per token)")
    p.add_argument("--layers", type=int, default=0, help="override the layer count (profiling runs only)")
    p.add_argument("--tokens", type=int, default=0, help="override decode tokens (profiling runs)")
    p.add_argument("--sample-every", type=int, default=1,
                   help="event-time every n-th run of decode launches between two folds")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-int8", action="store_true", help="skip the int8-coordinate variant of the default step")
    p.add_argument("--cpu-units", type=int, default=0, help="oracle sample size (unit streams)")
    p.add_argument("--prefill", action="store_true",
                   help="time the one-shot prompt factorisation of the long-input workload against "
                        "folding the same prompt block by block, print one JSON line and exit")
    p.add_argument("--coords", choices=("f32", "bf16", "i8"), default=None,
                   help="stored coordinate type (default: the workload's); i8 = int8 codes of U with "
                        "one fp32 scale per row")
    p.add_argument("--decode-snapshots", default="",
                   help="comma-separated history lengths: inject each state by one-shot prefill and time "
                        "decode only (all layers) there, one JSON line")
    p.add_argument("--summarize-traffic", nargs=4, metavar=("COPY_FETCH", "COPY_WRITE", "FETCH", "WRITE"),
                   help="write profiles/traffic_<workload>[_i8].json from four rocprofv3 --pmc output "
                        "folders (copy calibration FETCH_SIZE, WRITE_SIZE; bench FETCH_SIZE, WRITE_SIZE)")
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


def decode_bytes(U, g, n, e, kK, kV, coord_b, kv_b, appended=0, scale_b=0):
    """Algorithmic HBM bytes of one decode launch over U units: history
    coordinates of K and V (plus scale_b bytes of row scale per history row
    and kind for int8 storage), window rows of K and V (e includes an appended
    row, read from the caller's buffer), both bases, queries in, outputs out
    (fp32), and the appended K and V rows written to the window ring."""
    per = (n * (kK + kV) * coord_b + 2 * n * scale_b + 2 * e * 128 * kv_b + (kK + kV) * 128 * 4
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
    """Hash of a kernel source together with the headers every kernel includes
    (a change in either changes the compiled kernel)."""
    h = hashlib.sha256(open(path, "rb").read())
    csrc = os.path.dirname(path)
    for inc in ("iskv_internal.hpp", "fold_common.hpp"):
        q = os.path.join(csrc, inc)
        if os.path.basename(path).endswith(".hip") and os.path.exists(q):
            h.update(open(q, "rb").read())
    return h.hexdigest()[:16]


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


# Peak of the fold core's arithmetic: fp64 and (non-packed) fp32 vector FMAs,
# 256 CUs x 4 SIMDs x 16 lanes x 2 flop x 2.4 GHz. The 157.3 TFLOP/s fp32
# figure needs packed fp32 instructions, which this build leaves disabled.
ALU_PEAK_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12


def core_flops(k, b, r, sweeps, d=128):
    """Floating-point operations of one fold core for one unit stream, in the
    order the kernel computes them (an FMA counts as two): projection (Y = F B,
    and when k + b < d the residual E = F - Y B^T in two passes), the residual
    basis (Householder QR of [B | E^T] and P; when k + b >= d the complement
    of B: pivoted Cholesky of I - B^T B if p < k, else a QR of B, and F P),
    the structured QR of Z (b block rows into the triangle), `sweeps`
    one-sided Jacobi sweeps over the c = k + p rows of R (per pair one dot
    product and the rotation of two c-long columns, every pair counted as
    rotated, plus the column norms; a direct pass over the remaining pairs
    counts as a sweep), then B+, the two Gram matrices (one triangle each),
    the basis correction, H_r G and the new rows."""
    p = min(b, d - k)
    c = k + p
    kp = min(r, c)
    cmpl = k + b >= d
    if cmpl:
        f = 2.0 * b * k * d
        if p > 0 and p < k:
            f += d * d * k + sum(2.0 * (d - s) * (d - s) for s in range(p))
        elif p > 0:
            f += sum(4.0 * (d - j) * (k - j) for j in range(k))
            f += sum(4.0 * (d - j) for col in range(p) for j in range(min(k + col + 1, k)))
        f += 2.0 * b * p * d
    else:
        f = 8.0 * b * k * d
        f += sum(4.0 * (d - j) * max(k + b - j, 0) for j in range(c))
        f += sum(4.0 * (d - j) for col in range(p) for j in range(k + col + 1))
    f += sum(4.0 * (b + 1) * (c - j) for j in range(c))
    f += sweeps * (c * (c - 1) / 2.0 * 8.0 * c + 2.0 * c * c)
    f += 2.0 * d * c * kp + kp * (kp + 1) / 2.0 * (2.0 * d + 2.0 * c) + 2.0 * kp * kp * d + 2.0 * c * kp * kp
    f += 2.0 * b * c * kp
    return f


def rewrite_bytes(U, n, k, kp, coord_b, scale_b=0):
    """Algorithmic HBM bytes of one rewrite launch for one stream kind: the n
    stored rows read (k columns) and written (k+ columns), their row scales
    read and written for int8 storage (scale_b bytes each), H_top read."""
    return U * (coord_b * (n * k + n * kp) + 2 * n * scale_b + 4 * k * kp)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cores():
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return max(1, min(cores or 1, 16))  # the GPU machine's CPU share is 16 cores


def cpu_baseline_fold_decode(w, n0, nunits):
    """The fp64 oracle on a bounded sample of the same step: for each sampled
    unit stream, a history of n0 + w rows (the same stage of the run as the
    GPU's timed steps; its factorisation, taken with LAPACK, is setup and not
    timed), then the oracle's fold of b new rows and its decode attention
    (dense attention of one query over the reconstruction of history and
    window). Units run in parallel threads on the host cores."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    import synth

    oracle.load()
    cores = host_cores()
    if nunits <= 0:
        nunits = 4 * cores
    b, d = w.block, 128

    def setup(i):
        kind = "KV"[i % 2]
        l, h = (i // 2) % w.layers, ((i // 2) * 7) % w.kv_heads
        bb = ((i // 2) * 5) % w.batch
        r = w.rank_k if kind == "K" else w.rank_v
        X = synth.kv_rows(w, kind, bb, l, h, n0 + w.window + b)
        u, sv, vt = np.linalg.svd(X[:n0], full_matrices=False)
        st = oracle.UnitState.empty(d, b, r, n0 + w.window + 2 * b)
        sg = np.sign(vt[np.arange(r), np.argmax(np.abs(vt[:r]), axis=1)])
        st.C[:n0, :r] = u[:, :r] * sv[:r] * sg
        st.sigma[:r] = sv[:r]
        st.Bt[:r] = vt[:r] * sg[:, None]
        st.n, st.k = n0, r
        st.window = [x.copy() for x in X[n0:n0 + w.window]]
        q = synth.queries(w, 0, bb, l)[h * w.group:(h + 1) * w.group]
        return st, X[n0 + w.window:], q

    with ThreadPoolExecutor(max_workers=cores) as ex:
        jobs = list(ex.map(setup, range(nunits)))

    def fold(j):
        st, rows, _ = j
        st.append(rows, w.window)
        return st

    def attend(j):
        st, _, q = j
        rec = st.reconstruct()
        return oracle.attend(rec, rec, q, d ** -0.5)  # one stream's reconstruction stands for K and V

    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=cores) as ex:
        states = list(ex.map(fold, jobs))
    t1 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=cores) as ex:
        list(ex.map(attend, jobs))
    t2 = time.perf_counter()
    assert all(s.n == n0 + b for s in states)
    rows_s = nunits * b / (t1 - t0)
    # decode: each sampled stream is one of the 2 U streams a token's attention reads
    U = w.units
    tok_s = w.batch / ((t2 - t1) / nunits * 2 * U / cores)
    return {"value": rows_s, "unit": "KV rows compressed/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "decode_attn_tokens_per_s": tok_s,
            "sample": "%d unit streams of the %s workload (K and V alternating) at n = %d history rows "
                      "plus a %d-row window: one fold of %d rows each (%.1f s wall), then dense attention "
                      "of one query over the reconstruction (%.1f s wall); fp64 C oracle, %d threads; "
                      "decode tokens/s scaled to the workload's %d streams per token" % (
                          nunits, w.name, n0, w.window, b, t1 - t0, t2 - t1, cores, 2 * U)}


def fold_decode_bench(args, w):
    """One fold round plus one decode step per step, at the end of the run;
    with the workload's own bf16 coordinates the same step is then timed
    again with int8 coordinates (the bf16 state freed first) and attached as
    `int8_coordinates`."""
    import torch
    from dataclasses import replace

    res, n_mid = fold_decode_step(args, w)
    if w.coord_dtype == "bf16" and args.coords is None and not args.no_int8:
        torch.cuda.empty_cache()
        r8, _ = fold_decode_step(args, replace(w, coord_dtype="i8"))
        res["int8_coordinates"] = {k: r8[k] for k in ("value", "unit", "ms_per_step", "dtype", "decode_attn_tokens_per_s",
                                                      "kernel_ms", "roofline_kernels", "decode_one_layer")}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_fold_decode(w, n_mid, args.cpu_units)
    print(json.dumps(res), flush=True)


def fold_decode_step(args, w):
    """The measurement of fold_decode_bench for one coordinate type; returns
    (result dict, history rows at the middle of the timed steps)."""
    import numpy as np
    import torch

    import synth
    from incremental_rank_svd_amd import iskv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = iskv.load()
    B, L, Hk, Hq, b, wnd = w.batch, w.layers, w.kv_heads, w.q_heads, w.block, w.window
    U = B * L * Hk
    kv_b = 2 if w.kv_dtype == "bf16" else 4
    coord_b = {"bf16": 2, "f32": 4, "i8": 1}[w.coord_dtype]
    scale_b = 4 if w.coord_dtype == "i8" else 0  # one fp32 scale per stored row
    kvdt = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
    nsteps = args.warmup + args.steps
    n_end = w.final_counts()[0]
    n0 = n_end - nsteps * b
    if n0 < b:
        print("warmup + steps = %d fold rounds do not fit the %s run (at most %d)" % (
            nsteps, w.name, n_end // b - 1), file=sys.stderr)
        sys.exit(2)
    cache = iskv.Cache(iskv.config_from_workload(w), device=dev)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    h = cache.h

    # inputs: prompt rows per layer (factorised, then freed), window rows,
    # and the rows of every step, resident in HBM
    t_setup = time.perf_counter()
    win = {x: torch.empty((B, L, Hk, wnd, 128), dtype=kvdt, device=dev) for x in "KV"}
    steps_rows = {x: torch.empty((nsteps, B, L, Hk, b, 128), dtype=kvdt, device=dev) for x in "KV"}
    for l in range(L):
        rows = {x: synth.kv_rows_device(w, x, n0 + wnd + nsteps * b, dev, layer0=l, nlayers=1) for x in "KV"}
        cache.prefill_oneshot(rows["K"][:, :, :, :n0].contiguous(), rows["V"][:, :, :, :n0].contiguous(),
                              layer0=l)
        for x in "KV":
            win[x][:, l] = rows[x][:, 0, :, n0:n0 + wnd]
            tail = rows[x][:, 0, :, n0 + wnd:].reshape(B, Hk, nsteps, b, 128)
            steps_rows[x][:, :, l] = tail.permute(2, 0, 1, 3, 4)
        del rows
        if l % 8 == 7 or l == L - 1:
            print("setup: %d of %d layers factorised (%.0f s)" % (l + 1, L, time.perf_counter() - t_setup),
                  file=sys.stderr, flush=True)
    for s0 in range(0, wnd, b):
        s1 = min(wnd, s0 + b)
        cache.append_block(win["K"][:, :, :, s0:s1].contiguous(), win["V"][:, :, :, s0:s1].contiguous())
    del win
    gen = torch.Generator(device=dev)
    gen.manual_seed(synth.unit_key(w.cfg_id, 0, "Q", 0, 0, 0) & ((1 << 63) - 1))
    Q = torch.randn((nsteps, B, L, Hq, 128), generator=gen, device=dev).to(kvdt)
    out = torch.empty((B, L, Hq, 128), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    if cache.status():
        raise RuntimeError("numeric flags %#x after the state injection" % cache.status())
    n_start, e_start, kK, kV = cache.counts(0)
    assert (n_start, e_start) == (n0, wnd), (n_start, e_start)
    setup_s = time.perf_counter() - t_setup

    VP = ctypes.c_void_p
    scale = ctypes.c_float(128 ** -0.5)
    kbytes = steps_rows["K"][0].numel() * steps_rows["K"].element_size()
    qbytes = Q[0].numel() * Q.element_size()
    kp0, vp0, qp0 = steps_rows["K"].data_ptr(), steps_rows["V"].data_ptr(), Q.data_ptr()
    op = VP(out.data_ptr())

    def events(k):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(k)]
        for e in evs:
            e.record(stream)  # creates the underlying HIP event
        return evs

    step_evs = [events(6) for _ in range(nsteps)]  # ingest, core, rewrite, fold end, decode start, decode end
    torch.cuda.synchronize()
    sweeps_last = None

    def run(s):
        ev = step_evs[s]
        arr = (VP * 4)(*[VP(e.cuda_event) for e in ev[:4]])
        if lib.iskv_set_fold_events(h, arr):
            raise RuntimeError("set_fold_events failed")
        rc = lib.iskv_append_block(h, VP(kp0 + s * kbytes), VP(vp0 + s * kbytes), b, 0, L, sp)
        if rc:
            raise RuntimeError("append_block failed: %d" % rc)
        ev[4].record(stream)
        rc = lib.iskv_decode_attn(h, VP(qp0 + s * qbytes), op, 0, L, scale, sp)
        if rc:
            raise RuntimeError("decode_attn failed: %d" % rc)
        ev[5].record(stream)

    for s in range(args.warmup):
        run(s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.warmup, nsteps):
        run(s)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    lib.iskv_set_fold_events(h, None)
    step_s = (t1 - t0) / args.steps
    flags = cache.status()
    if flags:
        raise RuntimeError("numeric flags %#x" % flags)
    n_fin, e_fin, kK, kV = cache.counts(0)
    assert (n_fin, e_fin) == (n_end, wnd), (n_fin, e_fin)
    sw = {x: cache.fold_stats(x)[0].double().mean().item() for x in (0, 1)}

    # per-kernel durations (ms) over the timed steps
    ms = {"ingest": [], "core": [], "rewrite": [], "decode": []}
    for s in range(args.warmup, nsteps):
        ev = step_evs[s]
        ms["ingest"].append(ev[0].elapsed_time(ev[1]))
        ms["core"].append(ev[1].elapsed_time(ev[2]))
        ms["rewrite"].append(ev[2].elapsed_time(ev[3]))
        ms["decode"].append(ev[4].elapsed_time(ev[5]))
    avg = {k: float(np.mean(v)) for k, v in ms.items()}
    # algorithmic work per launch, averaged over the timed steps (n grows by b per step)
    core_f = rw_b = dec_b = 0.0
    for s in range(args.warmup, nsteps):
        n = n0 + s * b  # history rows before this step's fold
        core_f += U * (core_flops(kK, b, w.rank_k, sw[0]) + core_flops(kV, b, w.rank_v, sw[1]))
        rw_b += rewrite_bytes(U, n, kK, kK, coord_b, scale_b) + rewrite_bytes(U, n, kV, kV, coord_b, scale_b)
        dec_b += decode_bytes(U, w.group, n + b, wnd, kK, kV, coord_b, kv_b, scale_b=scale_b)
    core_f /= args.steps
    rw_b /= args.steps
    dec_b /= args.steps
    kern = {
        "k_fold": {"bound": "alu", "achieved": core_f / (avg["core"] * 1e-3) / 1e12, "peak": ALU_PEAK_TFLOPS,
                   "unit": "TFLOP/s", "avg_launch_ms": avg["core"], "work_per_launch": core_f,
                   "sweeps": [sw[0], sw[1]]},
        ("k_rewrite_i8" if scale_b else "k_rewrite_mfma"): {
                           "bound": "hbm", "achieved": rw_b / (avg["rewrite"] * 1e-3) / 1e9,
                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "avg_launch_ms": avg["rewrite"],
                           "work_per_launch": rw_b},
        "k_decode_unit": {"bound": "hbm", "achieved": dec_b / (avg["decode"] * 1e-3) / 1e9,
                          "peak": HBM_PEAK_GBS, "unit": "GB/s", "avg_launch_ms": avg["decode"],
                          "work_per_launch": dec_b},
    }
    traffic = measured_traffic(w.name + ("_i8" if scale_b else ""))
    for name, kr in kern.items():
        kr["frac"] = kr["achieved"] / kr["peak"]
        kr["share_of_step"] = kr["avg_launch_ms"] * 1e-3 / step_s
        kr["traffic"] = traffic.get(name)
    dom = max(kern, key=lambda k: kern[k]["share_of_step"])
    rows_folded = 2 * U * b
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
        "dtype": ("int8 U with fp32 row scales, bf16 rows, f32 compute" if scale_b else
                  "bf16 storage, f32 compute" if w.kv_dtype == "bf16" else "f32"),
        "data": "synthetic (power-law spectrum KV, seeded), resident in HBM",
        "config": {"workload": w.name, "batch": B, "layers": L, "kv_heads": Hk, "q_heads": Hq,
                   "head_dim": 128, "tokens": w.total_tokens, "block": b, "rank_k": w.rank_k,
                   "rank_v": w.rank_v, "window": wnd, "coords": w.coord_dtype,
                   "step": "one fold round (b = %d new K and V rows per unit, all layers) + one decode "
                           "query per head over all layers; history n = %d -> %d over the warmup and "
                           "timed steps (the run's last fold rounds), window %d" % (b, n0, n_end, wnd)},
        "decode_attn_tokens_per_s": B / (avg["decode"] * 1e-3),
        "kernel_ms": avg,
        "setup_s": setup_s,
        "roofline": dict(kernel=dom, **{k: v for k, v in kern[dom].items()}),
        "roofline_kernels": kern,
    }
    # decode of one layer per call, as a model's layer loop issues it (after the timed region)
    res["decode_one_layer"] = one_layer_decode(lib, h, Q[-1], out, L, B, Hk, Hq, n_fin, wnd, kK, kV, w.group,
                                               coord_b, kv_b, stream, sp, scale_b=scale_b)
    print("timed (%s coordinates): %d steps, %.1f ms per step" % (w.coord_dtype, args.steps, step_s * 1e3),
          file=sys.stderr, flush=True)
    return res, n0 + (args.warmup + args.steps // 2) * b


def one_layer_decode(lib, h, q, out, L, B, Hk, Hq, n, e, kK, kV, g, coord_b, kv_b, stream, sp, reps=50,
                     scale_b=0):
    """Median latency of iskv_decode_attn over a single layer (layer 0), the
    call a model's per-layer decode loop makes: B * Hk units, history split
    over several workgroups per unit. q, out: [B, L, Hq, 128] (one layer
    slice is passed)."""
    import torch

    VP = ctypes.c_void_p
    q1 = q[:, :1].contiguous()
    o1 = out[:, :1].contiguous()
    scale = ctypes.c_float(128 ** -0.5)
    evs = []
    for _ in range(reps):
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        if lib.iskv_decode_attn(h, VP(q1.data_ptr()), VP(o1.data_ptr()), 0, 1, scale, sp):
            raise RuntimeError("decode_attn (one layer) failed")
        a1.record(stream)
        evs.append((a0, a1))
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) for a, b in evs)[reps // 2] * 1e3
    U1 = B * Hk
    byts = decode_bytes(U1, g, n, e, kK, kV, coord_b, kv_b, scale_b=scale_b)
    return {"units": U1, "n": n, "median_us_with_event_pair": us, "GBps": byts / (us * 1e-6) / 1e9}


def measured_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, per
    kernel, while the kernel's source is unchanged since it was measured."""
    tpath = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    out = {}
    if not os.path.exists(tpath):
        return out
    try:
        tr = json.load(open(tpath))
        for name, ent in tr.get("kernels", {}).items():
            src = os.path.join(ROOT, "incremental_rank_svd_amd", "csrc", ent["source"])
            if ent.get("source_sha256_16") == source_hash(src):
                out[name] = ent.get("bytes_per_launch")
    except Exception:
        return {}
    return out


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
    # the first one-shot call (on its own cache) loads the kernels; the second is timed
    for mode in ("warmup", "oneshot", "blocks"):
        cache = iskv.Cache(iskv.config_from_workload(w), device=dev)
        h = cache.h
        blocks = [(K[:, :, :, s:s + w.block].contiguous(), V[:, :, :, s:s + w.block].contiguous())
                  for s in range(0, P, w.block)] if mode == "blocks" else None
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if mode in ("warmup", "oneshot"):
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


def decode_snapshots(args, w):
    """Decode-only rate at several history lengths n: per n the cache is
    reset, every layer's first n rows are factorised by iskv_prefill_oneshot
    (device-generated rows of the workload's distribution), the window is
    filled to w rows, then the median of 20 all-layer iskv_decode_attn
    launches (HIP events on the launch stream) gives GB/s against the
    algorithmic bytes of the launch."""
    import numpy as np
    import torch

    import synth
    from incremental_rank_svd_amd import iskv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = iskv.load()
    B, L, Hk, Hq, b, wnd = w.batch, w.layers, w.kv_heads, w.q_heads, w.block, w.window
    U = B * L * Hk
    kv_b = 2
    coord_b = {"bf16": 2, "f32": 4, "i8": 1}[w.coord_dtype]
    scale_b = 4 if w.coord_dtype == "i8" else 0
    ns = [int(x) for x in args.decode_snapshots.split(",")]
    cache = iskv.Cache(iskv.config_from_workload(w), device=dev)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    VP = ctypes.c_void_p
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    Q = torch.randn((B, L, Hq, 128), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty((B, L, Hq, 128), dtype=torch.float32, device=dev)
    scale = ctypes.c_float(128 ** -0.5)
    snaps = []
    for n in ns:
        n = min(n, w.max_tokens - wnd) // b * b
        cache.reset()
        for l in range(L):
            rows = {x: synth.kv_rows_device(w, x, n + wnd, dev, layer0=l, nlayers=1) for x in "KV"}
            cache.prefill_oneshot(rows["K"][:, :, :, :n].contiguous(), rows["V"][:, :, :, :n].contiguous(), layer0=l)
            for s0 in range(0, wnd, b):
                s1 = min(wnd, s0 + b)
                cache.append_block(rows["K"][:, :, :, n + s0:n + s1].contiguous(),
                                   rows["V"][:, :, :, n + s0:n + s1].contiguous(), layer0=l)
            del rows
        torch.cuda.synchronize()
        nn, e, kK, kV = cache.counts(0)
        evs = []
        for i in range(22):
            a0 = torch.cuda.Event(enable_timing=True)
            a1 = torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            if lib.iskv_decode_attn(cache.h, VP(Q.data_ptr()), VP(out.data_ptr()), 0, L, scale, sp):
                raise RuntimeError("decode_attn failed")
            a1.record(stream)
            evs.append((a0, a1))
        torch.cuda.synchronize()
        if cache.status():
            raise RuntimeError("numeric flags after the snapshot at n = %d" % n)
        ms = float(np.median([a.elapsed_time(c) for a, c in evs[2:]]))
        byts = decode_bytes(U, w.group, nn, e, kK, kV, coord_b, kv_b, scale_b=scale_b)
        snaps.append({"n": nn, "e": e, "k_k": kK, "k_v": kV, "state_GB": U * nn * (kK + kV) * coord_b / 1e9,
                      "ms": ms, "GBps": byts / (ms * 1e-3) / 1e9, "frac": byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                      "tokens_per_s": B / (ms * 1e-3)})
        print("snapshot n = %d: %.3f ms, %.0f GB/s" % (nn, ms, snaps[-1]["GBps"]), file=sys.stderr, flush=True)
    print(json.dumps({"metric": "decode-attn tokens/sec and % of HBM roofline at fixed history lengths",
                      "workload": w.name, "coords": w.coord_dtype, "units": U, "window": wnd,
                      "kernel": "k_decode_unit", "snapshots": snaps}), flush=True)


def _pmc_rows(folder):
    """(kernel name, counter value) of every dispatch in a rocprofv3 --pmc csv folder."""
    import csv
    import glob

    out = []
    for path in sorted(glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)):
        with open(path) as f:
            for row in csv.DictReader(f):
                out.append((row.get("Kernel_Name", ""), float(row.get("Counter_Value", 0.0))))
    return out


def summarize_traffic(args, w, scale_b):
    """HBM bytes per launch of the fold core, the rewrite and the decode from
    FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled by what the same
    counter reads for the plain 1 GiB copy of --copy-calibration; the bench
    run is --steps 1 --warmup 1 (two fold rounds, two decodes). Written with
    each kernel's source hash: bench.py reports it only while that matches."""
    cf, cw, fe, wr = args.summarize_traffic
    gib_kib = float(1 << 20)
    copy_f = max(v for k, v in _pmc_rows(cf) if "elementwise" in k or "mul" in k.lower())
    copy_w = max(v for k, v in _pmc_rows(cw) if "elementwise" in k or "mul" in k.lower())
    ff, wf = gib_kib / copy_f, gib_kib / copy_w
    groups = {"k_fold": ("k_fold.hip", "iskv::k_fold<"),
              ("k_rewrite_i8" if scale_b else "k_rewrite_mfma"):
                  ("k_rewrite.hip", "iskv::k_rewrite_i8<" if scale_b else "iskv::k_rewrite_mfma<"),
              "k_decode_unit": ("k_decode.hip", "iskv::k_decode_unit<")}
    fetch, write = _pmc_rows(fe), _pmc_rows(wr)
    kern = {}
    for name, (src, prefix) in groups.items():
        key = prefix.split("::")[-1]
        fs = [v for k, v in fetch if key in k]
        ws = [v for k, v in write if key in k]
        if not fs:
            continue
        # the rewrite runs one launch per kind: a fold round is two dispatches
        per = 2 if name.startswith("k_rewrite") else 1
        rounds = len(fs) / per
        fk, wk = sum(fs) / rounds, sum(ws) / rounds
        # decode: the all-layer launches only (the one-layer calls come after the timed steps)
        if name == "k_decode_unit":
            big = sorted(fs)[-2:]
            bigw = sorted(ws)[-2:]
            fk, wk, rounds = sum(big) / 2, sum(bigw) / 2, 2
        kern[name] = {"source": src,
                      "source_sha256_16": source_hash(os.path.join(ROOT, "incremental_rank_svd_amd", "csrc", src)),
                      "launches": int(rounds), "fetch_size_kib_avg": fk, "write_size_kib_avg": wk,
                      "bytes_per_launch": 1024.0 * (fk * ff + wk * wf)}
    out = {"workload": w.name, "coords": w.coord_dtype, "fetch_factor": ff, "write_factor": wf,
           "calibration": "FETCH_SIZE and WRITE_SIZE of one elementwise copy kernel (bench.py --copy-calibration: "
                          "1 GiB in, 1 GiB out) read %.1f and %.1f KiB" % (copy_f, copy_w),
           "kernels": kern}
    path = os.path.join(ROOT, "profiles", "traffic_%s%s.json" % (w.name, "_i8" if scale_b else ""))
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


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

    import synth

    from dataclasses import replace

    w = synth.get_config(args.workload)
    if args.layers:
        w = replace(w, layers=args.layers)
    if args.coords:
        w = replace(w, coord_dtype=args.coords)
    if args.summarize_traffic:
        summarize_traffic(args, w, 4 if w.coord_dtype == "i8" else 0)
        return
    if args.decode_snapshots:
        decode_snapshots(args, w)
        return
    if not args.full_run:
        fold_decode_bench(args, w)
        return
    full_run_bench(args, w)


def full_run_bench(args, w):
    """Whole decode runs from an empty cache, one iskv_append_decode per token."""
    import torch

    import synth
    from incremental_rank_svd_amd import iskv

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
    coord_b = {"bf16": 2, "f32": 4, "i8": 1}[w.coord_dtype]
    scale_b = 4 if w.coord_dtype == "i8" else 0

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
                        seg[1] += decode_bytes(U, w.group, n, e, kK, kV, coord_b, kv_b, appended=1, scale_b=scale_b)
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
    final_bytes = decode_bytes(U, w.group, n, e, kK, kV, coord_b, kv_b, scale_b=scale_b)

    rows_folded = 2 * U * n_final
    # HBM bytes per decode launch from a committed counter summary of this
    # workload's kernels (none is committed for the full run: null)
    traffic = measured_traffic(w.name).get("k_decode_unit")

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
    res["decode_one_layer"] = one_layer_decode(lib, h, Q[-1], out, L, B, Hk, Hq, n, e, kK, kV, w.group,
                                               coord_b, kv_b, stream, sp, scale_b=scale_b)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_units)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
