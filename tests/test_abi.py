"""The C ABI boundary, on the CPU: libclsa.so loads, exports every entry point
that include/clsa.h declares, and rejects bad arguments before it enqueues
anything (these calls never reach a HIP API, so no GPU is needed).

The rejection tests pass fake device addresses. They run only in a child
process that sees no HIP device (tests/test_abi_isolated.py starts it), so a
call that slipped past validation would fail on the host instead of
launching a kernel on unmapped addresses."""

import ctypes
import os
import re
import subprocess

import pytest

pytestmark = pytest.mark.skipif(os.environ.get("CLSA_ABI_CHILD") != "1",
                                reason="runs in a child process without a visible HIP device "
                                       "(tests/test_abi_isolated.py)")

import token_sparse_attention_clsa_amd as clsa
from token_sparse_attention_clsa_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from token_sparse_attention_clsa_amd import build
        build.build()
    return clsa.load()


def test_every_declared_symbol_is_exported(lib):
    names = clsa.declared_symbols()
    assert len(names) == 16
    for required in ("clsa_index_score", "clsa_topk", "clsa_topk_margin", "clsa_sparse_attn",
                     "clsa_decode_step"):
        assert required in names
    raw = ctypes.CDLL(binding.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_abi_version_matches_header(lib):
    text = open(os.path.join(ROOT, "include", "clsa.h")).read()
    ver = int(re.search(r"#define CLSA_ABI_VERSION (\d+)", text).group(1))
    assert lib.clsa_abi_version() == ver


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, 7):
        assert lib.clsa_status_string(s)
    assert lib.clsa_status_string(0) == b"ok"


def test_workspace_sizes(lib):
    assert clsa.workspace_bytes(binding.OP_TOPK, B=4, T=1, kv_len=131072, k=2048) >= 4 * 131072 * 4
    assert clsa.workspace_bytes(binding.OP_SPARSE_ATTN, B=4, T=1, Hq=32, Hkv=8, D=128, k=2048) > 0
    assert clsa.workspace_bytes(binding.OP_BLOCK_UNION, B=1, T=1, kv_len=133120, block=64) >= 2080 * 4
    assert clsa.workspace_bytes(binding.OP_TOPK, B=0, T=1, kv_len=10, k=1) == 0
    assert clsa.workspace_bytes(binding.OP_SPARSE_ATTN, B=1, T=1, Hq=3, Hkv=2, D=128, k=8) == 0
    assert clsa.workspace_bytes(99, B=1, T=1) == 0


FAKE = 1 << 20  # aligned non-null address; never dereferenced by a rejected call


def test_index_score_rejects(lib):
    rc = lib.clsa_index_score(None, FAKE, 1, FAKE, FAKE, 1, 1, 64, 128, 100, 100, None)
    assert rc == -1 and b"null" in lib.clsa_last_error()
    rc = lib.clsa_index_score(FAKE, FAKE, 1, FAKE, FAKE, 1, 5, 64, 128, 4, 100, None)  # kv_len < T
    assert rc == -1
    rc = lib.clsa_index_score(FAKE, FAKE, 1, FAKE, FAKE, 1, 1, 64, 128, 100, 50, None)  # L_cap < kv_len
    assert rc == -1
    rc = lib.clsa_index_score(FAKE, FAKE, 1, FAKE, FAKE, 1, 1, 8, 128, 100, 100, None)  # H_I=8 on MFMA
    assert rc == -2
    rc = lib.clsa_index_score(FAKE, FAKE, 9, FAKE, FAKE, 1, 1, 64, 128, 100, 100, None)
    assert rc == -1
    rc = lib.clsa_index_score(FAKE + 2, FAKE, 1, FAKE, FAKE, 1, 1, 64, 128, 100, 100, None)
    assert rc == -1 and b"misaligned" in lib.clsa_last_error()


def test_topk_rejects(lib):
    assert lib.clsa_topk(FAKE, 1, 1, 100, 0, FAKE, FAKE, 1 << 20, None) == -1      # k = 0
    assert lib.clsa_topk(None, 1, 1, 100, 5, FAKE, FAKE, 1 << 20, None) == -1
    assert lib.clsa_topk(FAKE, 1, 1, 100, 5, FAKE, None, 0, None) == -3            # no workspace
    assert lib.clsa_topk(FAKE, 1, 1, 100, 5, FAKE, FAKE, 16, None) == -3           # too small
    assert lib.clsa_topk(FAKE, 70000, 1, 100, 5, FAKE, FAKE, 1 << 40, None) == -2    # B*T above grid limit
    assert lib.clsa_topk(FAKE, 1, 1, 5_000_000, 5, FAKE, FAKE, 1 << 40, None) == -2  # kv_len above 4M


def test_sparse_attn_rejects(lib):
    args = dict(q=FAKE, k=FAKE, v=FAKE, dtype=1, idx=FAKE, kk=16, out=FAKE, lse=None, B=1, T=1, Hq=32,
                Hkv=8, D=128, kv_len=100, L_cap=100, scale=0.0, ws=FAKE, wsb=1 << 30)

    def call(**kw):
        a = dict(args, **kw)
        return lib.clsa_sparse_attn(a["q"], a["k"], a["v"], a["dtype"], a["idx"], a["kk"], a["out"], a["lse"],
                                    a["B"], a["T"], a["Hq"], a["Hkv"], a["D"], a["kv_len"], a["L_cap"],
                                    a["scale"], a["ws"], a["wsb"], None)

    assert call(Hq=30) == -1                 # Hq % Hkv
    assert call(kk=0) == -1
    assert call(D=64) == -2                  # only D = 128 is implemented
    assert call(Hq=48, Hkv=4) == -2          # group size 12
    assert call(dtype=2) == -2               # fp8 attention not implemented
    assert call(idx=None) == -1
    assert call(ws=None, wsb=0) == -3
    assert call(scale=float("nan")) == -1
    assert call(out=FAKE + 8) == -1


def _desc(layer_src, fake=FAKE, **kw):
    n = len(layer_src)
    PA = ctypes.c_void_p * n
    d = binding.StepDesc()
    d.n_layers = n
    d.layer_src = (ctypes.c_int32 * n)(*layer_src)
    for f in ("q", "k_cache", "v_cache", "out", "q_idx", "k_idx", "w"):
        setattr(d, f, PA(*([fake] * n)))
    d.idx_out = fake
    d.dtype, d.idx_dtype = 1, 1
    d.B, d.T, d.Hq, d.Hkv, d.D, d.H_I, d.D_I = 2, 1, 32, 8, 128, 64, 128
    d.kv_len, d.L_cap, d.k, d.scale = 1000, 1000, 64, 0.0
    for key, v in kw.items():
        setattr(d, key, v)
    return d


@pytest.mark.parametrize("src", [[1, 1], [0, 2, 2], [0, 0, 1], [0, 1, 0]])
def test_decode_step_rejects_bad_layer_maps(lib, src):
    d = _desc(src)
    assert lib.clsa_decode_step_workspace_bytes(ctypes.byref(d)) == 0
    assert lib.clsa_decode_step(ctypes.byref(d), FAKE, 1 << 40, None) == -1
    assert b"layer" in lib.clsa_last_error()


def test_decode_step_checks_workspace(lib):
    d = _desc([0, 0, 0, 4, 4][:3])
    need = lib.clsa_decode_step_workspace_bytes(ctypes.byref(d))
    assert need > 2 * 1000 * 4  # at least the scores
    assert lib.clsa_decode_step(ctypes.byref(d), FAKE, need - 1, None) == -3
    d2 = _desc([0, 0, 2, 2, 4, 4])
    assert lib.clsa_decode_step_workspace_bytes(ctypes.byref(d2)) == need  # F count does not matter
    d3 = _desc([0, 0], k=0)
    assert lib.clsa_decode_step(ctypes.byref(d3), FAKE, 1 << 40, None) == -1


def test_decode_step_rejects_missing_indexer_inputs(lib):
    d = _desc([0, 1])
    d.q_idx = (ctypes.c_void_p * 2)(FAKE, None)   # layer 1 is F but has no indexer query
    assert lib.clsa_decode_step(ctypes.byref(d), FAKE, 1 << 40, None) == -1


def test_block_calls_reject(lib):
    assert lib.clsa_block_union_build(None, 1, 1, 4, 100, 64, 8, FAKE, FAKE, FAKE, 1 << 20, None) == -1
    assert lib.clsa_block_union_build(FAKE, 1, 1, 4, 100, 0, 8, FAKE, FAKE, FAKE, 1 << 20, None) == -1
    assert lib.clsa_block_union_build(FAKE, 1, 1, 4, 100, 64, 8, FAKE, FAKE, FAKE, 0, None) == -3
    assert lib.clsa_block_paged_attn(FAKE, FAKE, FAKE, 0, FAKE, FAKE, 64, FAKE, None, 1, 1, 32, 8, 128,
                                     100, 100, 0.0, None) == -2   # f32 comparator not built


def test_cache_append_rejects(lib):
    A, Bp, C, Dp = FAKE, FAKE + (1 << 24), FAKE + (1 << 26), FAKE + (1 << 28)
    E, Fp = FAKE + (1 << 30), FAKE + (1 << 31)

    def call(k_new=A, v_new=Bp, kc=C, vc=Dp, dtype=1, ki_new=None, ki=None, idt=1, B=2, T=1, Hkv=8,
             D=128, D_I=128, pos=10, cap=64):
        return lib.clsa_cache_append(k_new, v_new, kc, vc, dtype, ki_new, ki, idt, B, T, Hkv, D, D_I, pos,
                                     cap, None)

    assert call(k_new=None) == -1
    assert call(ki_new=E) == -1 and b"both" in lib.clsa_last_error()     # indexer keys without a cache
    assert call(pos=64) == -1                                             # past L_cap
    assert call(pos=62, T=3) == -1
    assert call(pos=-1) == -1
    assert call(dtype=2) == -1                                            # fp8 K/V caches not supported
    assert call(ki_new=E, ki=Fp, idt=7) == -1
    assert call(k_new=A + 4) == -1 and b"misaligned" in lib.clsa_last_error()
    assert call(k_new=C + 4096) == -1 and b"overlap" in lib.clsa_last_error()  # source inside a cache
    assert call(B=0) == -1


def test_topk_vark_and_head_major_reject(lib):
    assert lib.clsa_topk_vark(FAKE, 1, 1, 100, 5, FAKE + 2, FAKE, FAKE, 1 << 20, None) == -1   # misaligned counts
    assert lib.clsa_topk_vark(FAKE, 1, 1, 100, 0, FAKE, FAKE, FAKE, 1 << 20, None) == -1       # k = 0
    assert lib.clsa_topk_vark(FAKE, 1, 1, 100, 5, FAKE, FAKE, None, 0, None) == -3            # no workspace
    assert lib.clsa_block_paged_attn_hm(FAKE, FAKE, FAKE, 0, FAKE, FAKE, 64, FAKE, None, 1, 1, 32, 8,
                                        128, 100, 100, 0.0, None) == -2   # f32 comparator not built
    assert lib.clsa_block_paged_attn_hm(None, FAKE, FAKE, 1, FAKE, FAKE, 64, FAKE, None, 1, 1, 32, 8,
                                        128, 100, 100, 0.0, None) == -1


def test_step_descriptor_layout_matches_header(lib):
    """The binding's descriptor mirrors clsa_step_desc field for field: a
    misaligned per-query count pointer set through it is seen (and rejected)
    by the library."""
    import ctypes
    from token_sparse_attention_clsa_amd import binding
    n = 1
    P = ctypes.c_void_p
    arr = (P * n)(FAKE)
    src = (ctypes.c_int32 * n)(0)
    d = binding.StepDesc(n, src, arr, arr, arr, arr, ctypes.POINTER(P)(), arr, arr, arr, FAKE, 1, 1,
                         1, 1, 32, 8, 128, 64, 128, 100, 100, 16, 0.0, ctypes.POINTER(P)(), FAKE + 2)
    assert lib.clsa_decode_step(ctypes.byref(d), FAKE, 1 << 30, None) == -1
    assert b"k_per_query" in lib.clsa_last_error()


def test_topk_margin_rejects(lib):
    f = lib.clsa_topk_margin
    assert f(FAKE, 1, 1, 100, 5, None, -1.0, FAKE, None, FAKE, 1 << 20, None) == -1
    assert b"margin" in lib.clsa_last_error()
    assert f(FAKE, 1, 1, 100, 5, None, float("nan"), FAKE, None, FAKE, 1 << 20, None) == -1
    assert f(FAKE, 1, 1, 100, 5, None, 1.0, FAKE, FAKE + 2, FAKE, 1 << 20, None) == -1  # kept misaligned
    assert f(FAKE, 1, 1, 100, 0, None, 1.0, FAKE, None, FAKE, 1 << 20, None) == -1      # k = 0
    assert f(FAKE, 1, 1, 100, 5, None, 1.0, FAKE, None, FAKE, 16, None) == -3           # workspace


def test_decode_step_rejects_negative_skip_margin(lib):
    for bad in (-0.5, float("nan")):
        m = ctypes.c_float(bad)
        d = _desc([0, 0], skip_margin=ctypes.pointer(m))
        assert lib.clsa_decode_step_workspace_bytes(ctypes.byref(d)) == 0
        assert lib.clsa_decode_step(ctypes.byref(d), FAKE, 1 << 40, None) == -1
        assert b"skip_margin" in lib.clsa_last_error()


def test_step_desc_layout_matches_the_header(tmp_path):
    # The binding's ctypes mirror of clsa_step_desc must have the C layout:
    # compile a probe against include/clsa.h and compare every field offset.
    fields = [name for name, _ in binding.StepDesc._fields_]
    src = tmp_path / "probe.c"
    src.write_text(
        "#include <stdio.h>\n#include <stddef.h>\n#include \"clsa.h\"\nint main(void) {\n"
        '  printf("size %zu\\n", sizeof(clsa_step_desc));\n'
        + "".join(f'  printf("{n} %zu\\n", offsetof(clsa_step_desc, {n}));\n' for n in fields)
        + "  return 0;\n}\n")
    exe = tmp_path / "probe"
    subprocess.check_call(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    out = dict(line.split() for line in subprocess.check_output([str(exe)]).decode().splitlines())
    assert int(out["size"]) == ctypes.sizeof(binding.StepDesc)
    for n in fields:
        assert int(out[n]) == getattr(binding.StepDesc, n).offset, n


def test_decode_step_static_rejects(lib):
    # an invalid layer map: the regular step's message, nothing launched
    d = _desc([1, 1])
    assert lib.clsa_decode_step_static(ctypes.byref(d), None) == -1
    assert b"layer" in lib.clsa_last_error()
    # a step whose scratch exceeds the library's array
    big = _desc([0, 0], B=8, kv_len=4_000_000, L_cap=4_000_000)
    need = lib.clsa_decode_step_workspace_bytes(ctypes.byref(big))
    text = open(os.path.join(ROOT, "include", "clsa.h")).read()
    cap = eval(re.search(r"#define CLSA_STATIC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
               .expand(r"\1 << \2"))
    assert need > cap
    assert lib.clsa_decode_step_static(ctypes.byref(big), None) == -3
    assert b"scratch" in lib.clsa_last_error()
