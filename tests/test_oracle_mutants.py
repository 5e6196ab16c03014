"""Plausible mistakes planted in a copy of the oracle must each fail a pin.

Each mutant is the oracle's C source with one edit (a dropped term, a wrong
sign or operand, a transposed product, a wrong step index), built with gcc
into a temporary directory.  The checks of ``oracle_checks.py`` run against
it; at least one must fail.  This shows the pins would catch such a mistake
in the real oracle.  Nothing here touches the GPU library.
"""
from __future__ import annotations

import os
import subprocess

import pytest

from oracle.build import SRC
from oracle_checks import ALL_CHECKS

# (name, text in recurrence.c, replacement, occurrence index or None for all)
MUTANTS = [
    ("gdn-correction-sign", "add_outer(dv, dk, S, -b, Sk, kd);", "add_outer(dv, dk, S, b, Sk, kd);", 0),
    ("kda-correction-sign", "add_outer(dv, dk, S, -b, Sk, kd);", "add_outer(dv, dk, S, b, Sk, kd);", 1),
    ("gdn-no-correction", "add_outer(dv, dk, S, -b, Sk, kd);", ";", 0),
    ("gdn-write-transposed", "add_outer(dv, dk, S, b, vd, kd);", "add_outer(dv, dk, S, b, kd, vd);", 0),
    ("kda-no-write", "add_outer(dv, dk, S, b, vd, kd);", ";", 1),
    ("gdn-no-decay", "scale_all(dv, dk, S, alpha);", ";", 0),
    ("gdn-decay-sign", "exp((double)g[row])", "exp(-(double)g[row])", 0),
    ("kda-decay-after-correction",
     "            scale_columns(dv, dk, S, al);         /* S diag(alpha)      */\n"
     "            matvec(dv, dk, S, kd, Sk);\n"
     "            add_outer(dv, dk, S, -b, Sk, kd);\n",
     "            matvec(dv, dk, S, kd, Sk);\n"
     "            add_outer(dv, dk, S, -b, Sk, kd);\n"
     "            scale_columns(dv, dk, S, al);\n", 0),
    ("rwkv-no-decay", "            scale_columns(dv, dk, S, al);\n            add_outer(dv, dk, S, 1.0, vd, kd);",
     "            add_outer(dv, dk, S, 1.0, vd, kd);", 0),
    ("rwkv-write-scaled", "add_outer(dv, dk, S, 1.0, vd, kd);", "add_outer(dv, dk, S, 0.5, vd, kd);", 0),
    ("readout-with-k", "matvec(dv, dk, S, qd, ot);", "matvec(dv, dk, S, kd, ot);", 0),
    ("matvec-transposed", "acc += S[(size_t)i * dk + j] * x[j];", "acc += S[(size_t)j * dv + i] * x[j];", 0),
    ("key-from-previous-step", "kd[j] = (double)k[row * dk + j];",
     "kd[j] = (double)k[(row >= (size_t)n_pairs ? row - n_pairs : row) * dk + j];", 0),
    ("outer-transposed-index", "S[(size_t)i * dk + j] += c * a[i] * b[j];",
     "S[(size_t)i * dk + j] += c * a[j % dv] * b[i % dk];", 0),
    ("late-start-ignored", "if (t < t_first) {", "if (t < 0) {", 0),
    ("gated-no-erase-gate", "ek[j] = (double)gate[j] * kd[j];", "ek[j] = kd[j];", 0),
    ("gated-no-write-gate", "wv[i] = (double)gate[dk + i] * vd[i];", "wv[i] = vd[i];", 0),
    ("gated-write-gate-from-erase", "wv[i] = (double)gate[dk + i] * vd[i];",
     "wv[i] = (double)gate[i % dk] * vd[i];", 0),
    ("gated-erase-along-gated-key", "add_outer(dv, dk, S, -1.0, Sk, kd);",
     "add_outer(dv, dk, S, -1.0, Sk, ek);", 0),
]


def _mutate(src: str, old: str, new: str, which: int) -> str:
    parts = src.split(old)
    assert len(parts) > which + 1, f"mutation anchor not found: {old!r}"
    return old.join(parts[: which + 1]) + new + old.join(parts[which + 1:])


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new,which", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, source, name, old, new, which):
    c_path = os.path.join(tmp_path, f"{name}.c")
    so_path = os.path.join(tmp_path, f"lib{name}.so")
    with open(c_path, "w") as f:
        f.write(_mutate(source, old, new, which))
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", so_path,
                    c_path, "-lm"], check=True)
    failed = []
    for check in ALL_CHECKS:
        try:
            check(lib_path=so_path)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"mutant {name} passed every pin"
