"""The fp64 reference against its pins (CPU only)."""
import pytest

import oracle
from oracle_pins import PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    pin(orc)


def test_rejects_invalid_shapes(orc):
    import numpy as np
    q = np.zeros((4, 2))
    k = np.zeros((3, 2))
    with pytest.raises(ValueError):
        orc.attention(q, k, k, causal=True, scale=1.0)   # causal needs Nq <= Nkv
    with pytest.raises(ValueError):
        orc.attention(q, np.zeros((0, 2)), np.zeros((0, 2)), causal=False, scale=1.0)


def test_oracle_under_sanitizers(tmp_path):
    # the reference's C code under AddressSanitizer and UndefinedBehaviorSanitizer
    # (gcc, host code only): every entry point on small ragged inputs
    import os
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    here = os.path.dirname(os.path.abspath(__file__))
    exe = str(tmp_path / "oracle_sanitize")
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    os.path.join(here, "c", "oracle_sanitize.c"),
                    os.path.join(os.path.dirname(here), "oracle", "attn_oracle.c"), "-lm", "-o", exe], check=True)
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ran clean" in r.stdout
