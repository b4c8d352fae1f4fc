"""The index-checked build (libgdn_debug.so, the same sources built with
-DGDN_DEBUG): every entry point is called in a child process that loads only
that build (GDN_LIBRARY), and every call must leave the status word at GDN_OK
-- no kernel index past the end of its array -- with results at the parity bar
(tests/debug_build_calls.py)."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(os.path.dirname(HERE), "gated_deltanet_recurrence_gdn_amd", "libgdn_debug.so")


def test_debug_build_reports_no_index_errors():
    if not os.path.exists(LIB):
        pytest.skip("libgdn_debug.so is not built (build() makes it beside libgdn.so)")
    env = {**os.environ, "GDN_LIBRARY": LIB}
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "debug_build_calls.py")], env=env,
                       capture_output=True, text=True, timeout=240)
    print(r.stdout[-3000:], r.stderr[-3000:], file=sys.stderr)
    assert r.returncode == 0, r.stderr[-3000:]
    assert "debug build: all calls clean" in r.stdout
