"""Every kernel of the library compiles to straight-line device code: no
private (scratch) segment, no dynamic stack and no calls. A helper the
compiler leaves out of line turns into a call whose arguments pass through
scratch memory and whose LDS pointers become generic (flat) ones; the
kernel still gives the same results, only slower, so only the generated
code shows it. The device assembly is compiled here from the library's own
sources with the library's own flags (hipcc cross-compiles for gfx950
without a GPU)."""

import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from token_sparse_attention_clsa_amd import build as b


def _hipcc():
    try:
        return b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")


def _device_asm(src, tmp_path):
    out = tmp_path / (os.path.splitext(src)[0] + ".s")
    cmd = [_hipcc()] + b.compile_flags() + ["--cuda-device-only", "-S", os.path.join(b.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _kernels(asm):
    """(name, descriptor text) of every kernel in the assembly."""
    return re.findall(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", asm, re.S)


def test_no_kernel_uses_scratch_or_calls(tmp_path):
    srcs = [s for s in b.SOURCES if s.endswith(".hip")]
    with ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        asms = dict(zip(srcs, ex.map(lambda s: _device_asm(s, tmp_path), srcs)))
    n = 0
    for src, asm in asms.items():
        assert "s_swappc_b64" not in asm, f"{src}: a device function is called, not inlined"
        for name, desc in _kernels(asm):
            n += 1
            seg = re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", desc)
            dyn = re.search(r"\.amdhsa_uses_dynamic_stack (\d+)", desc)
            assert seg and int(seg.group(1)) == 0, f"{src}: {name} uses scratch"
            assert dyn is None or int(dyn.group(1)) == 0, f"{src}: {name} uses a dynamic stack"
    assert n >= len(srcs)  # every source holds at least one kernel
