"""The library's host code under AddressSanitizer (CPU only).

The C++ of the ABI (argument validation, error messages, create's release of
everything on failure, the stack and quantisation entry points) is built for
the host alone with AddressSanitizer, together with a driver that walks every
path the ABI can take without launching a kernel; on a machine without a
usable device that includes a full create that fails at the device lookup.
The run must report every check passed and no sanitizer error.
"""

import os
import shutil
import subprocess

import pytest


def test_abi_host_paths_under_address_sanitizer(tmp_path):
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("no hipcc")
    from moe_ffn_amd.build import build_host_asan
    exe = build_host_asan(str(tmp_path / "asan"))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert r.stdout.startswith("ok "), r.stdout
    assert int(r.stdout.split()[1]) >= 50, r.stdout
    # the sanitizer is really in the build: a planted heap overread is reported
    r = subprocess.run([exe, "--plant"], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
