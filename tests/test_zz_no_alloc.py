"""iskv_decode_attn_static (allocation-free decode attention) against
iskv_decode_attn on the same cache and queries, through the C ABI: two calls
in a row, the second over a smaller input (one layer, fewer units), each
within the decode tolerance (max |d out| / max |out| <= 2e-3); plus the
host-side rejection of a call whose partials exceed the static array."""

from dataclasses import replace

import numpy as np
import pytest
import torch

import synth
from gpu_util import D, DEC_TOL, note, to_dev

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def iskv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from incremental_rank_svd_amd import iskv as m
    return m


def _rows(w, T):
    out = {}
    for x in "KV":
        a = np.zeros((w.batch, w.layers, w.kv_heads, T, D))
        for b in range(w.batch):
            for l in range(w.layers):
                for h in range(w.kv_heads):
                    a[b, l, h] = synth.kv_rows(w, x, b, l, h, T)
        out[x] = a
    return out


def _err(a, b):
    a = a.double().cpu().numpy()
    b = b.double().cpu().numpy()
    return float(np.abs(a - b).max() / np.abs(b).max())


def test_decode_attn_static_matches_decode_attn(iskv):
    w = replace(synth.get_config(1), layers=3, kv_heads=4, q_heads=16, decode_tokens=3000, cfg_id=70)
    T = w.total_tokens
    rows = _rows(w, T)
    cache = iskv.Cache(iskv.config_from_workload(w), device=DEV)
    K = to_dev(rows["K"], torch.bfloat16, DEV)
    V = to_dev(rows["V"], torch.bfloat16, DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(5)
    # below 2048 history rows iskv_decode_attn runs one workgroup per unit,
    # the static variant still goes through its partials and the merge
    for t in range(0, 1472, w.block):
        cache.append_block(K[:, :, :, t:t + w.block].contiguous(), V[:, :, :, t:t + w.block].contiguous())
    assert cache.counts(0)[0] < 2048
    q0 = torch.randn((w.batch, w.layers, w.q_heads, D), generator=gen, device=DEV).to(torch.bfloat16)
    e0 = _err(cache.decode_attn_static(q0), cache.decode_attn(q0))
    assert e0 <= DEC_TOL, e0
    for t in range(1472, T, w.block):
        cache.append_block(K[:, :, :, t:t + w.block].contiguous(), V[:, :, :, t:t + w.block].contiguous())
    n, e, kk, kv = cache.counts(0)
    note("case: static decode, n=%d e=%d (unsplit reference: %.2e)" % (n, e, e0))
    # call 1: all layers
    q = torch.randn((w.batch, w.layers, w.q_heads, D), generator=gen, device=DEV).to(torch.bfloat16)
    ref = cache.decode_attn(q)
    got = cache.decode_attn_static(q)
    e1 = _err(got, ref)
    assert e1 <= DEC_TOL, e1
    # call 2: a smaller input, one layer (fewer units, more history splits each)
    q1 = q[:, 1:2].contiguous()
    ref1 = cache.decode_attn(q1, layer0=1)
    got1 = cache.decode_attn_static(q1, layer0=1)
    e2 = _err(got1, ref1)
    assert e2 <= DEC_TOL, e2
    assert cache.status() == 0
    note("  max rel difference: %.2e (3 layers), %.2e (1 layer)" % (e1, e2))


def test_decode_attn_static_rejects_oversized_and_fp32(iskv):
    # 13B-MHA units at full batch: one partial per unit is already larger
    # than the static array; the call is refused before anything is enqueued
    w = replace(synth.get_config(4), layers=30, decode_tokens=300, cfg_id=71)
    cache = iskv.Cache(iskv.config_from_workload(w), device=DEV)
    K = torch.zeros((w.batch, w.layers, w.kv_heads, 1, D), dtype=torch.bfloat16, device=DEV)
    cache.append_block(K, K)
    q = torch.zeros((w.batch, w.layers, w.q_heads, D), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(iskv.ISKVError) as ei:
        cache.decode_attn_static(q)
    assert ei.value.code == iskv.ISKV_ERR_SCRATCH
    # fp32 coordinates take the scalar decode, which has no static variant
    w2 = replace(synth.get_config(0), decode_tokens=100, cfg_id=72)
    c2 = iskv.Cache(iskv.config_from_workload(w2), device=DEV)
    k1 = torch.zeros((1, 1, 1, 1, D), dtype=torch.float32, device=DEV)
    c2.append_block(k1, k1)
    with pytest.raises(iskv.ISKVError) as ei:
        c2.decode_attn_static(torch.zeros((1, 1, 1, D), dtype=torch.float32, device=DEV))
    assert ei.value.code == iskv.ISKV_ERR_ARG
    assert cache.status() == 0 and c2.status() == 0
