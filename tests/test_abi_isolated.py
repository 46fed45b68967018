"""Runs tests/test_abi.py in a child process that sees no HIP device.

Those tests hand the library fake device addresses and expect every call to
be rejected by its argument checks. Without a visible device, a call that got
past the checks would fail in the HIP runtime on the host rather than launch
a kernel that dereferences the fake addresses."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_suite_without_a_visible_device():
    env = dict(os.environ, CLSA_ABI_CHILD="1", HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1",
               CUDA_VISIBLE_DEVICES="-1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-2000:]
    assert " passed" in r.stdout and " failed" not in r.stdout and "skipped" not in r.stdout, r.stdout[-2000:]
