"""The C-ABI tests again, against a build whose host code runs under
AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library's host side -- argument validation with its overlap, overflow
and alignment arithmetic, status strings, workspace sizing and launch
set-up -- is built with both sanitizers (``_build_sanitized``; the gfx950
device code is unchanged) and ``tests/test_abi.py`` runs in a child Python
that loads that build with the sanitizer runtime preloaded. Any report
aborts the child, so the test fails with the report in its output.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    from weight_activation_quantized_amd import _build_sanitized
    return _build_sanitized.build()


def test_abi_under_address_and_ub_sanitizers(sanitized_lib, tmp_path):
    from weight_activation_quantized_amd import _build_sanitized
    env = _build_sanitized.sanitizer_env(sanitized_lib)
    logs = tmp_path / "san"
    env["ASAN_OPTIONS"] += f":log_path={logs}"
    env["UBSAN_OPTIONS"] += f":log_path={logs}"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = "".join(p.read_text() for p in tmp_path.glob("san*"))
    assert r.returncode == 0 and not reports, (
        f"rc={r.returncode}\n{reports}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}")
    assert " passed" in r.stdout
