"""The oracle's pins catch plausible mistakes: each mutation in ``oracle_mutations.MUTATIONS`` is
planted in a copy of the oracle (CPU only), the oracle pin tests run against that copy in a
subprocess, and at least one of them must fail.  The unmodified copy must pass, which shows the
failures come from the planted mistakes and not from the harness."""
import os
import subprocess
import sys

import pytest

from oracle_mutations import MUTATIONS, ROOT

PIN_TESTS = ["tests/test_oracle_e4m3.py", "tests/test_oracle_attention.py", "tests/test_oracle_cache_write.py"]


def _run_pins(mutation: str):
    env = dict(os.environ, FP8ATTN_ORACLE_MUTATION=mutation)
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-p", "no:cacheprovider", *PIN_TESTS],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def test_unmutated_copy_passes():
    r = _run_pins("none")
    assert "mutated oracle: none" in r.stdout, r.stdout[:2000]
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    r = _run_pins(name)
    assert f"mutated oracle: {name}" in r.stdout, "the mutated copy was not the one imported"
    assert r.returncode != 0, f"mutation {name} survived every oracle pin:\n{r.stdout[-1500:]}"
