"""The C-ABI library loads and exports every entry point include/iskv.h
declares, and rejects bad configurations on the host (no GPU needed)."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "iskv.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"ISKV_API\s+[\w\s\*]*?\b(iskv_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from incremental_rank_svd_amd import iskv

    if not os.path.exists(iskv.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    return iskv.load()


def test_header_declares_the_boundary():
    names = _declared()
    for required in ("iskv_init", "iskv_append_block", "iskv_decode_attn", "iskv_reconstruct",
                     "iskv_workspace_bytes", "iskv_status", "iskv_destroy"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    from incremental_rank_svd_amd import iskv

    out = subprocess.run(["nm", "-D", "--defined-only", iskv.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(iskv_\w+)", out))
    declared = set(_declared())
    assert declared == exported, (declared ^ exported)
    assert set(iskv.EXPORTED) == declared
    for name in declared:
        assert hasattr(lib, name)


def test_library_has_no_oracle_dependency(lib):
    from incremental_rank_svd_amd import iskv

    out = subprocess.run(["nm", "-D", iskv.LIB_PATH], capture_output=True, text=True).stdout
    assert "ora_" not in out
    deps = subprocess.run(["readelf", "-d", iskv.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in deps
    assert "gfx950" in subprocess.run(["strings", iskv.LIB_PATH], capture_output=True, text=True).stdout


def _cfg(**kw):
    from incremental_rank_svd_amd import iskv

    base = dict(batch=1, layers=2, kv_heads=2, q_heads=8, block=64, rank_k=32, rank_v=32,
                window=128, max_tokens=1024)
    base.update(kw)
    return iskv.make_config(**base)


@pytest.mark.parametrize("bad", [dict(head_dim=64), dict(q_heads=7), dict(block=0), dict(block=129),
                                 dict(rank_k=0), dict(rank_v=129), dict(window=-1),
                                 dict(max_tokens=0), dict(q_heads=2 * 9), dict(batch=0),
                                 dict(coord_dtype="f32", kv_dtype="f32", layers=0),
                                 # int8 coordinates: bf16 rows, ranks in 8-column pieces, offsets < 2^31
                                 dict(coord_dtype="i8", kv_dtype="f32"), dict(coord_dtype="i8", rank_k=28),
                                 dict(coord_dtype="i8", rank_v=100),
                                 dict(coord_dtype="i8", rank_k=128, max_tokens=1 << 24)])
def test_invalid_configs_rejected_on_host(lib, bad):
    from incremental_rank_svd_amd import iskv

    cfg = _cfg(**bad)
    assert lib.iskv_workspace_bytes(ctypes.byref(cfg)) == 0
    h = ctypes.c_void_p()
    rc = lib.iskv_init(ctypes.byref(cfg), ctypes.c_void_p(1 << 20), 1 << 40, None, ctypes.byref(h))
    assert rc == iskv.ISKV_ERR_ARG and not h.value


def test_int8_coordinates_take_a_byte_per_entry_and_a_row_scale(lib):
    # per unit and kind: ncap r codes (16-byte rounded, 256-byte pad) and ncap fp32 scales
    # instead of 2 ncap r bytes of bf16
    base = dict(batch=2, layers=4, kv_heads=8, q_heads=32, rank_k=64, rank_v=96, max_tokens=16384)
    bf = lib.iskv_workspace_bytes(ctypes.byref(_cfg(**base)))
    i8 = lib.iskv_workspace_bytes(ctypes.byref(_cfg(coord_dtype="i8", **base)))
    U, ncap = 2 * 4 * 8, 16384
    saved = U * ncap * (64 + 96) - 2 * U * ncap * 4
    assert abs((bf - i8) - saved) <= 4 * U * 512, (bf, i8, saved)


def test_workspace_checks_before_any_device_work(lib):
    from incremental_rank_svd_amd import iskv

    cfg = _cfg()
    need = lib.iskv_workspace_bytes(ctypes.byref(cfg))
    assert need > 0
    h = ctypes.c_void_p()
    # too small and misaligned workspaces fail before the library touches the pointer
    assert lib.iskv_init(ctypes.byref(cfg), ctypes.c_void_p(1 << 20), need - 1, None,
                         ctypes.byref(h)) == iskv.ISKV_ERR_WORKSPACE
    assert lib.iskv_init(ctypes.byref(cfg), ctypes.c_void_p((1 << 20) + 8), need, None,
                         ctypes.byref(h)) == iskv.ISKV_ERR_WORKSPACE
    assert lib.iskv_init(ctypes.byref(cfg), None, need, None, ctypes.byref(h)) == iskv.ISKV_ERR_WORKSPACE
    assert not h.value


def test_workspace_grows_with_capacity_and_fits_hbm(lib):
    import synth
    from incremental_rank_svd_amd import iskv

    a = lib.iskv_workspace_bytes(ctypes.byref(_cfg(max_tokens=1024)))
    b = lib.iskv_workspace_bytes(ctypes.byref(_cfg(max_tokens=4096)))
    assert b > a
    for w in synth.CONFIGS:
        need = lib.iskv_workspace_bytes(ctypes.byref(iskv.config_from_workload(w)))
        assert 0 < need < 288 * 2 ** 30, (w.name, need)


def test_null_handle_and_strerror(lib):
    from incremental_rank_svd_amd import iskv

    assert lib.iskv_destroy(None) == iskv.ISKV_ERR_ARG
    assert lib.iskv_counts(None, 0, None, None, None, None) == iskv.ISKV_ERR_ARG
    assert lib.iskv_append_block(None, None, None, 1, 0, 1, None) == iskv.ISKV_ERR_ARG
    assert lib.iskv_set_mode(None, iskv.MODE_JOINT) == iskv.ISKV_ERR_ARG
    assert lib.iskv_append_decode(None, None, None, None, None, 0, 1, ctypes.c_float(1.0), None) == iskv.ISKV_ERR_ARG
    assert lib.iskv_decode_attn(None, None, None, 0, 1, ctypes.c_float(1.0), None) == iskv.ISKV_ERR_ARG
    assert lib.iskv_prefill_oneshot(None, None, None, 16, 0, 1, None) == iskv.ISKV_ERR_ARG
    for code in range(0, -8, -1):
        assert lib.iskv_strerror(code) not in (None, b"", b"unknown status")
    assert lib.iskv_strerror(-99) == b"unknown status"
