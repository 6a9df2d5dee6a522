"""Each plausible mistake in the oracle's recurrence is caught by a pin.

The test copies kda_oracle.c, plants one mistake by text substitution,
compiles the copy with gcc into a temporary library, and checks that at least
one pin of tests/oracle_pins.py fails on it. The real oracle is never
modified."""

import os
import shutil
import subprocess

import pytest

import oracle_pins as pins
from oracle import build as oracle_build
from oracle import recurrence

MUTANTS = {
    "beta_only_on_v": ("u[j] = beta * (in_val(v, dtype, v_off + j0 + j) - r);",
                       "u[j] = beta * in_val(v, dtype, v_off + j0 + j) - r;"),
    "decay_sign": ("row[j] *= a;", "row[j] *= 1.0 / a;"),
    "no_decay": ("row[j] *= a;", "row[j] *= 1.0;"),
    "retrieve_with_query": ("r += S[(int64_t)i * nc + j] * kv[i];",
                            "r += S[(int64_t)i * nc + j] * qv[i];"),
    "write_sign": ("row[j] += kv[i] * u[j];", "row[j] -= kv[i] * u[j];"),
    "readout_before_write": ("acc += S[(int64_t)i * nc + j] * qv[i];",
                             "acc += (S[(int64_t)i * nc + j] - kv[i] * u[j]) * qv[i];"),
    "readout_transposed": ("acc += S[(int64_t)i * nc + j] * qv[i];",
                           "acc += S[(int64_t)(j % Dk) * nc + (i % nc)] * qv[i];"),
    "write_with_query": ("row[j] += kv[i] * u[j];", "row[j] += qv[i] * u[j];"),
    "decay_after_write_partial": ("exp(gb_val(g, dtype, qk_off + i))", "exp(0.5 * gb_val(g, dtype, qk_off + i))"),
}


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    return tmp_path_factory.mktemp("mutants")


def _build_mutant(workdir, name, old, new):
    src = open(oracle_build.SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    src = src.replace(old, new)
    cpath = os.path.join(workdir, f"{name}.c")
    lpath = os.path.join(workdir, f"lib{name}.so")
    with open(cpath, "w") as f:
        f.write(src)
    subprocess.run(["gcc", "-std=c99", "-O1", "-fPIC", "-shared", "-fopenmp", "-w",
                    "-o", lpath, cpath, "-lm"], check=True)
    return recurrence.load(lpath)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(workdir, name):
    old, new = MUTANTS[name]
    lib = _build_mutant(workdir, name, old, new)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(recurrence, lib=lib)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
