"""Planted controls for the oracle's pins (CPU only).

Each case copies the oracle into a temporary directory, plants one plausible
mistake in the copy (a swapped nibble half, a dropped -8, the wrong rounding
of q = round(x / d), a round-half-up binary16 encoder, reversed activation
rows, the wrong Q4_0 rounding bias, /128 for /127, a transposed stream of
quantized activations, the parity bar loosened in either of its two terms)
and runs tests/test_oracle_pins.py against the copy in a fresh interpreter:
the pins must fail. A mistake they let through would make
every GPU parity test that trusts the oracle meaningless."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

PLANTED = [
    ("oracle.c", "int lo = blk[2 + j] & 0x0F;", "int lo = blk[2 + j] >> 4;", "nibble halves swapped"),
    ("oracle.c", "out[b * ORC_QK + j] = (float)(lo - 8) * d;", "out[b * ORC_QK + j] = (float)(lo) * d;",
     "Q4_0 bias dropped"),
    ("oracle.c", "q = (int)roundf(xb[j] / d);", "q = (int)rintf(xb[j] / d);",
     "Q8_0 ties to even instead of away from zero"),
    ("oracle.c", "double r = rint(a / ulp);", "double r = floor(a / ulp + 0.5);",
     "binary16 encoder rounds half up"),
    ("oracle.c", "orc_dot_row(a + (size_t)m * K, wrow, K,", "orc_dot_row(a + (size_t)(M-1-m) * K, wrow, K,",
     "activation rows reversed"),
    ("oracle.c", "t = t + 8.5f;", "t = t + 8.0f;", "Q4_0 quantize bias 8 for 8.5"),
    ("oracle.c", "float d = amax / 127.0f;", "float d = amax / 128.0f;", "Q8_0 scale /128"),
    ("__init__.py", "return q8_0_dequant(b).reshape(M, K)", "return q8_0_dequant(b).reshape(K, M).T.copy()",
     "quantized-activation stream transposed"),
    ("__init__.py", "REL_TOL = 1e-5", "REL_TOL = 1e-4", "parity bar loosened to 1e-4 relative"),
    ("__init__.py", "ABS_TOL = 1e-6", "ABS_TOL = 1e-5", "parity bar floor loosened to 1e-5"),
    ("__init__.py", "return REL_TOL * np.asarray(bound, dtype=np.float64) + ABS_TOL",
     "return REL_TOL * np.abs(np.asarray(bound, dtype=np.float64)) * 10 + ABS_TOL",
     "parity bar's relative term ten times too loose"),
]


def _run_pins_on_copy(tmp_path, plant=None):
    """Copy the oracle to tmp_path/oracle, apply plant = (file, old, new) if
    given, and run the pins against the copy; returns the pytest exit code."""
    pkg = tmp_path / "oracle"
    pkg.mkdir()
    for f in ("oracle.c", "__init__.py"):
        shutil.copy(os.path.join(ROOT, "oracle", f), pkg / f)
    if plant is not None:
        fname, old, new = plant
        text = (pkg / fname).read_text()
        assert text.count(old) == 1, "the planted mistake no longer applies: " + old
        (pkg / fname).write_text(text.replace(old, new))
    env = dict(os.environ, PYTHONPATH=os.pathsep.join([str(tmp_path), ROOT]))
    proc = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                           "--rootdir", str(tmp_path), PINS],
                          cwd=str(tmp_path), env=env, capture_output=True, text=True, timeout=600)
    # The copy, not the repository's oracle, was under test (it builds its own library).
    assert (pkg / "liboracle.so").exists()
    return proc.returncode, proc.stdout[-2000:]


def test_an_unplanted_copy_passes(tmp_path):
    # The control: the same harness on an unchanged copy passes every pin.
    rc, out = _run_pins_on_copy(tmp_path)
    assert rc == 0, out


@pytest.mark.parametrize("fname,old,new,what", PLANTED, ids=[p[3] for p in PLANTED])
def test_pins_catch_the_planted_mistake(tmp_path, fname, old, new, what):
    rc, out = _run_pins_on_copy(tmp_path, (fname, old, new))
    assert rc == 1, "%s: pins did not fail (rc %d)\n%s" % (what, rc, out)
