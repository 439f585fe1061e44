"""The oracle's pins catch plausible mistakes (CPU only).

Each numbered mistake of gdn_oracle.c's ORACLE_MUTANT switch (readout before the
write, no 1/sqrt(head_dim), the state read transposed, the gate after the
retrieval, the delta's sign flipped, beta dropped) is compiled into a scratch build
of the oracle, and the pins of tests/test_oracle.py are run against that build in a
child process: each mutant must make at least one pin fail.  The normal build
passes them (the rest of the suite).
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

from oracle import build as oracle_build  # noqa: E402

MUTANTS = {1: "readout before write", 2: "no 1/sqrt(d)", 3: "transposed state",
           4: "gate after retrieval", 5: "delta sign flipped", 6: "beta dropped"}
# the closed-form and worked-example pins (the chunked-form comparisons would catch
# some mutants too, but these alone must)
PINS = ("hand_worked or beta_zero or beta_one or orthonormal or single_token or "
        "tiled_key_heads_beta_zero")


def _run_pins(lib):
    env = dict(os.environ, GDN_ORACLE_PATH=lib)
    return subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_oracle.py"),
                           "-q", "-p", "no:cacheprovider", "-k", PINS],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)


def test_unmutated_scratch_build_passes_the_pins(tmp_path):
    """The control: the same scratch build path with no mistake passes."""
    r = _run_pins(oracle_build.build(mutant=0, out=str(tmp_path / "libgdn_oracle_m0.so")))
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-2000:])


@pytest.mark.parametrize("n", sorted(MUTANTS))
def test_each_planted_mistake_fails_a_pin(n, tmp_path):
    r = _run_pins(oracle_build.build(mutant=n, out=str(tmp_path / ("libgdn_oracle_m%d.so" % n))))
    print("mutant %d (%s): %s" % (n, MUTANTS[n], r.stdout.strip().splitlines()[-1]))
    assert r.returncode == 1, (MUTANTS[n], r.stdout[-2000:], r.stderr[-2000:])
