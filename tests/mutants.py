"""Planted-mistake harness for the oracle pins: builds a copy of the oracle
with one text substitution and reports which pins reject it.

A planted mistake can make the oracle read out of bounds, so the pins run
against the copy in a child process; a child that dies counts as a rejection.
"""
import json
import os
import shutil
import subprocess
import sys

import numpy as np

import oracle

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def build_mutant(tmp_path, fname, old, new):
    """Path of a copy of the oracle library with `old` replaced by `new` in
    `fname`."""
    src_dir = os.path.dirname(oracle.__file__)
    for f in ("dilated_oracle.c", "oracle_core.inc"):
        shutil.copy(os.path.join(src_dir, f), tmp_path / f)
    text = (tmp_path / fname).read_text()
    assert text.count(old) >= 1, f"mutation site not found: {old!r}"
    (tmp_path / fname).write_text(text.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", str(lib),
                    str(tmp_path / "dilated_oracle.c"), "-lm"], check=True)
    return str(lib)


def pins_catching(lib, module, suite):
    """Names of the pins in `module`.`suite` that reject the oracle built at
    `lib` (["<crash>"] when the child process dies)."""
    env = dict(os.environ, OMP_NUM_THREADS="2")
    p = subprocess.run([sys.executable, "-m", "tests.mutants", lib, module, suite], cwd=REPO,
                       env=env, capture_output=True, text=True, timeout=600)
    if p.returncode != 0:
        return ["<crash>"]
    return json.loads(p.stdout.strip().splitlines()[-1])


def _run(lib, module, suite):
    import importlib

    mod = importlib.import_module(module)
    orc = oracle.Oracle(lib)
    caught = []
    with np.errstate(all="ignore"):
        for pin in getattr(mod, suite):
            try:
                pin(orc)
            except (AssertionError, ValueError, RuntimeError):
                caught.append(pin.__name__)
    print(json.dumps(caught))


if __name__ == "__main__":
    _run(*sys.argv[1:4])
