"""Parity at the workloads' full per-unit sizes, on sampled units.

Every unit of a workload is run on the GPU (device-generated rows of the same
distribution); a few sampled units get host-generated rows instead, and the
fp64 oracle runs exactly those rows one unit at a time. Gates:
  * fp32 coordinates: singular values and reconstruction (1e-4), rank
    sequence identical;
  * bf16 coordinates (the storage the benchmark times): decode attention on
    the stored factors (2e-3), rank sequence identical, no numeric flags; the
    distance of the bf16 history to the fp64 oracle is reported and bounded
    by the bf16 re-rounding random walk, sqrt(folds) * 2^-8;
  * int8 coordinates (codes of U, one scale per row): decode on the stored
    factors (2e-3), rank sequence identical, no numeric flags, every stored
    row on its own int8 grid, and the history within the summed per-fold
    storage bounds (half a step per entry of U, times sigma) of the fp64
    oracle, its error against the true rows within that of the oracle plus
    the same bound.
The long-input and 13B-MHA workloads keep their full per-unit sizes; the
MHA one runs 2 of its 40 layers (units are independent).
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (D, DEC_TOL, check_unit, decode_err, decode_reference_on_gpu_factors, note,
                      oracle_units, unit_state)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def iskv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from incremental_rank_svd_amd import iskv as m
    return m


def _device_rows(w, samples):
    """Device rows [B, L, H, T, D] for K and V; sampled units overwritten with host rows."""
    T = w.total_tokens
    dev = {x: synth.kv_rows_torch(w, x, T, DEV) for x in "KV"}
    host = {}
    tdt = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
    for (b, l, h) in samples:
        for x in "KV":
            X = synth.kv_rows(w, x, b, l, h, T)
            host[(x, b, l, h)] = X
            dev[x][b, l, h] = torch.tensor(X, dtype=torch.float32, device=DEV).to(tdt)
    torch.cuda.synchronize()
    return dev, host


def _run(iskv, w, coord, samples, per_token=False):
    """Whole workload through the C ABI; returns (cache, host rows, fold k-sequence)."""
    cache = iskv.Cache(iskv.config_from_workload(w, coord_dtype=coord), device=DEV)
    dev, host = _device_rows(w, samples)
    b = w.block
    pre = w.prefill_blocks * b
    seq = []
    for s in range(0, pre, b):
        cache.prefill_block(dev["K"][:, :, :, s:s + b].contiguous(), dev["V"][:, :, :, s:s + b].contiguous())
        seq.append(cache.counts(0)[2:])
    step = 1 if per_token else b
    t = pre
    while t < w.total_tokens:
        s = min(step, w.total_tokens - t)
        n0 = cache.counts(0)[0]
        cache.append_block(dev["K"][:, :, :, t:t + s].contiguous(), dev["V"][:, :, :, t:t + s].contiguous())
        if cache.counts(0)[0] != n0:
            seq.append(cache.counts(0)[2:])
        t += s
    del dev
    return cache, host, seq


def _oracle(w, host, samples):
    jobs = []
    for (b, l, h) in samples:
        for x, r in (("K", w.rank_k), ("V", w.rank_v)):
            jobs.append((host[(x, b, l, h)], w.block, r, w.window, w.prefill_blocks * w.block))
    st = oracle_units(jobs)
    return {(x, smp): st[2 * i + j] for i, smp in enumerate(samples) for j, x in enumerate("KV")}


def _check_ranks(seq, ora):
    k_k = [kk for kk, kv in seq]
    k_v = [kv for kk, kv in seq]
    assert k_k == [kp for (_, _, kp, _, _) in ora["K"].log]
    assert k_v == [kp for (_, _, kp, _, _) in ora["V"].log]


def _decode_check(iskv, cache, w, samples, step=0):
    tdt = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
    gen = torch.Generator(device=DEV)
    gen.manual_seed(1234 + step)
    q = torch.randn((w.batch, w.layers, w.q_heads, D), generator=gen, device=DEV).to(tdt)
    hostq = {}
    for (b, l, h) in samples:
        qs = synth.queries(w, step, b, l)
        hostq[(b, l)] = qs
        q[b, l] = torch.tensor(qs, dtype=torch.float32, device=DEV).to(tdt)
    out = cache.decode_attn(q).cpu().double().numpy()
    g = w.group
    errs = []
    for (b, l, h) in samples:
        ref = decode_reference_on_gpu_factors(cache, b, l, h, hostq[(b, l)][h * g:(h + 1) * g], D ** -0.5)
        errs.append(decode_err(out[b, l, h * g:(h + 1) * g], ref))
    assert max(errs) <= DEC_TOL, errs
    return max(errs)


def _fp32_case(iskv, w, samples):
    cache, host, seq = _run(iskv, w, "f32", samples)
    assert cache.status() == 0
    ora = _oracle(w, host, samples)
    worst = [0.0, 0.0, 0.0]
    for smp in samples:
        _check_ranks(seq, {x: ora[(x, smp)] for x in "KV"})
        for which, x in ((0, "K"), (1, "V")):
            e = check_unit(cache, which, *smp, ora[(x, smp)], label=(w.name, smp, x))
            worst = [max(a, b) for a, b in zip(worst, e)]
    derr = _decode_check(iskv, cache, w, samples)
    note("  %s fp32 coords: sigma %.2e/%.2e recon %.2e decode %.2e folds %d" % (
        w.name, worst[0], worst[1], worst[2], derr, len(seq)))


def _bf16_case(iskv, w, samples, per_token=False):
    cache, host, seq = _run(iskv, w, "bf16", samples, per_token=per_token)
    assert cache.status() == 0
    ora = _oracle(w, host, samples)
    folds = len(seq)
    bound = np.sqrt(folds) * 2.0 ** -8
    worst = 0.0
    for smp in samples:
        _check_ranks(seq, {x: ora[(x, smp)] for x in "KV"})
        for which, x in ((0, "K"), (1, "V")):
            rec = cache.reconstruct(which, *smp).cpu().double().numpy()
            ref = ora[(x, smp)].reconstruct()
            rel = float(np.linalg.norm(rec - ref) / np.linalg.norm(ref))
            assert rel <= bound, (smp, x, rel, bound)
            worst = max(worst, rel)
    derrs = [_decode_check(iskv, cache, w, samples, step=s) for s in range(3)]
    note("  %s bf16 coords: recon vs fp64 oracle %.2e (bound %.2e) decode %.2e folds %d" % (
        w.name, worst, bound, max(derrs), folds))


def _i8_state(cache, which, b, l, h):
    C, sig, Bt, W = cache.export_state(which, b, l, h)
    sc = cache.export_scales(which, b, l, h).cpu().double().numpy()
    n, e, kk, kv = cache.counts(l)
    k = kk if which == 0 else kv
    q = C.cpu().numpy().astype(np.int64)
    sg = sig.cpu().double().numpy()
    return q, sc, sg, Bt.cpu().double().numpy(), W.float().cpu().double().numpy(), n, e, k


def _i8_case(iskv, w, samples, per_token=False):
    cache, host, seq = _run(iskv, w, "i8", samples, per_token=per_token)
    assert cache.status() == 0
    ora = _oracle(w, host, samples)
    folds = len(seq)
    worst = 0.0
    recs = {}
    for smp in samples:
        _check_ranks(seq, {x: ora[(x, smp)] for x in "KV"})
        for which, x in ((0, "K"), (1, "V")):
            q, sc, sg, Bt, W, n, e, k = _i8_state(cache, which, *smp)
            assert np.all(np.abs(q) <= 127) and np.all(q[:, k:] == 0)
            m = np.abs(q[:, :k]).max(axis=1)
            assert np.all((m == 127) | ((m == 0) & (sc == 0)))  # each row reaches its own scale
            C = q[:, :k] * sc[:, None] * sg[:k]
            rec = oracle.reconstruct(C, Bt[:k], W, k=k)
            got = cache.reconstruct(which, *smp).cpu().double().numpy()
            assert np.linalg.norm(got - rec) <= 1e-5 * np.linalg.norm(rec)
            recs[(x, smp)] = rec
            # per-fold storage bound: half a step on each entry of U, times sigma
            step = np.linalg.norm(sc[:, None] * 0.5 * sg[:k]) / np.linalg.norm(C)
            bound = folds * step
            ref = ora[(x, smp)].reconstruct()
            Xt = host[(x,) + smp][: n + e]
            rel = float(np.linalg.norm(rec - ref) / np.linalg.norm(ref))
            assert rel <= bound, (smp, x, rel, bound)
            eg = np.linalg.norm(rec - Xt) / np.linalg.norm(Xt)
            eo = np.linalg.norm(ref - Xt) / np.linalg.norm(Xt)
            assert eg <= eo + bound, (smp, x, eg, eo, bound)
            worst = max(worst, rel)
    tdt = torch.bfloat16
    g = w.group
    derr = 0.0
    for step in range(2):
        gen = torch.Generator(device=DEV)
        gen.manual_seed(4321 + step)
        qd = torch.randn((w.batch, w.layers, w.q_heads, D), generator=gen, device=DEV).to(tdt)
        hostq = {}
        for (b, l, h) in samples:
            qs = synth.queries(w, step, b, l)
            hostq[(b, l)] = qs
            qd[b, l] = torch.tensor(qs, dtype=torch.float32, device=DEV).to(tdt)
        out = cache.decode_attn(qd).cpu().double().numpy()
        for (b, l, h) in samples:
            ref = oracle.attend(recs[("K", (b, l, h))], recs[("V", (b, l, h))], hostq[(b, l)][h * g:(h + 1) * g],
                                D ** -0.5)
            derr = max(derr, decode_err(out[b, l, h * g:(h + 1) * g], ref))
    assert derr <= DEC_TOL, derr
    note("  %s int8 coords: history vs fp64 oracle %.2e, decode %.2e, folds %d" % (w.name, worst, derr, folds))


def test_llama3_8b_bench_configuration_bf16(iskv):
    """The benchmark's launch configuration: every token appended to all 32
    layers one at a time, bf16 storage, then decode on sampled units."""
    w = synth.get_config(1)
    note("case: %s bf16, per-token appends" % w.name)
    _bf16_case(iskv, w, [(0, 0, 0), (0, 31, 7), (0, 17, 3)], per_token=True)


def test_llama3_8b_fp32_coordinates(iskv):
    w = synth.get_config(1)
    note("case: %s fp32 coordinates" % w.name)
    _fp32_case(iskv, w, [(0, 0, 0), (0, 31, 7)])


@pytest.mark.parametrize("coord", ["f32", "bf16"])
def test_qwen3_8b_full(iskv, coord):
    w = synth.get_config(2)
    note("case: %s %s" % (w.name, coord))
    samples = [(3, 35, 7), (1, 17, 3)]
    (_fp32_case if coord == "f32" else _bf16_case)(iskv, w, samples)


@pytest.mark.parametrize("coord", ["f32", "bf16"])
def test_long_input_full(iskv, coord):
    w = synth.get_config(3)
    note("case: %s %s" % (w.name, coord))
    samples = [(0, 0, 0), (0, 31, 5)]
    (_fp32_case if coord == "f32" else _bf16_case)(iskv, w, samples)


@pytest.mark.parametrize("coord", ["f32", "bf16"])
def test_llama2_13b_mha_unit_sizes(iskv, coord):
    w = replace(synth.get_config(4), layers=2)
    note("case: %s (2 layers) %s" % (w.name, coord))
    samples = [(15, 1, 39), (4, 0, 11)]
    (_fp32_case if coord == "f32" else _bf16_case)(iskv, w, samples)


def test_int8_coordinates_llama3_8b_per_token(iskv):
    """The 8B-GQA workload with int8 storage, every token appended to all 32
    layers one at a time (the full-run launch configuration)."""
    w = synth.get_config(1)
    note("case: %s int8, per-token appends" % w.name)
    _i8_case(iskv, w, [(0, 0, 0), (0, 31, 7)], per_token=True)


def test_int8_coordinates_llama2_13b_mha_unit_sizes(iskv):
    """The 13B-MHA workload's full per-unit length (16384 tokens, b = 128,
    ranks 64 / 96) with int8 storage, 2 of its 40 layers."""
    w = replace(synth.get_config(4), layers=2)
    note("case: %s (2 layers) int8" % w.name)
    _i8_case(iskv, w, [(15, 1, 39), (4, 0, 11)])
