"""The C ABI used from C++ without torch (tests/c_abi_check.cpp, built by the
package build next to the library): hipMalloc'd buffers, host cutoff table,
RoPE -> prefill -> decode on one stream; the decode of the last token must
reproduce the prefill's last row (max-abs 2e-2), and invalid calls must
return their status codes.  Runs as a child process."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_c_abi_standalone():
    exe = os.path.join(HERE, "c_abi_check")
    if not os.path.exists(exe):
        raise RuntimeError("tests/c_abi_check is not built: run `python -m rope_positional_encoding_amd.build`")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c_abi_check OK" in r.stdout
