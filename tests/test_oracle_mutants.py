"""The oracle's pins must reject a plausible mistake anywhere in it.

Each ORA_PLANT_* switch compiles a copy of the oracle with one planted
mistake (a flipped rotation sign, a dropped core block, a transposed operand,
a wrong sort order, ...). The whole pin suite runs against each copy in a
subprocess (a planted mistake may crash it) and must fail.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PLANTS = [
    "ORA_PLANT_ROT_SIGN",
    "ORA_PLANT_NO_SIGMA",
    "ORA_PLANT_DROP_FB",
    "ORA_PLANT_SORT_ASC",
    "ORA_PLANT_H_TRANSPOSE",
    "ORA_PLANT_NO_REWRITE",
    "ORA_PLANT_P_UNNORMALIZED",
    "ORA_PLANT_DISCARD_UNSQUARED",
    "ORA_PLANT_NEWROW_OFFSET",
    "ORA_PLANT_ATTEND_NOSCALE",
    "ORA_PLANT_RECON_WRONG_ROW",
    "ORA_PLANT_STORAGE_NO_SIGMA",
    "ORA_PLANT_NAIVE_SIGN",
    "ORA_PLANT_NAIVE_PERM",
    "ORA_PLANT_PREFILL_REVERSED",
    "ORA_PLANT_PREFILL_JOINT",
    "ORA_PLANT_Q8_TRUNC",
    "ORA_PLANT_Q8_HALFAWAY",
    "ORA_PLANT_Q8_SCALE128",
    "ORA_PLANT_Q8_OLDROWS",
    "ORA_PLANT_Q8_STORE_C",
]


def _run_pins(lib_path):
    env = dict(os.environ, ISKV_ORACLE_LIB=lib_path, OMP_NUM_THREADS="1",
               OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_oracle_pins.py"),
           os.path.join(ROOT, "tests", "test_oracle_i8.py")]
    p = subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    return p.returncode, p.stdout[-2000:]


def test_pins_pass_on_unmodified_build(tmp_path):
    path = oracle.build_variant(str(tmp_path / "clean.so"))
    rc, out = _run_pins(path)
    assert rc == 0, out


def test_every_planted_mistake_is_caught(tmp_path):
    paths = [oracle.build_variant(str(tmp_path / (p + ".so")), [p]) for p in PLANTS]
    with ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        results = list(ex.map(_run_pins, paths))
    missed = [p for p, (rc, _) in zip(PLANTS, results) if rc == 0]
    assert not missed, "pins did not catch: %s" % missed
