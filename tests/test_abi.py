"""The C-ABI boundary, exercised on the CPU (no GPU needed, nothing launched).

* the built ``libfp8kv.so`` loads and exports every function ``include/fp8kv.h``
  declares, with the ABI version the header states;
* host-side argument checks return the documented negative codes before any
  HIP call is made (fake, aligned, never-dereferenced addresses are used);
* the workspace-size function is deterministic and grows with the problem.
"""

import os
import re

import pytest

import decode_attention_fp8_kv_amd as fk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8kv.h")


def _header_text():
    with open(HEADER) as f:
        return f.read()


def _header_functions():
    text = re.sub(r"/\*.*?\*/", "", _header_text(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def _header_define(name):
    m = re.search(rf"#define\s+{name}\s+\(?(-?\d+)", _header_text())
    return int(m.group(1))


@pytest.fixture(scope="module")
def lib():
    # FP8KV_TEST_LIB: run these checks against another build of the library (the sanitized host build of
    # tests/test_abi_sanitized.py)
    if os.environ.get("FP8KV_TEST_LIB"):
        fk.lib_path = os.environ["FP8KV_TEST_LIB"]
    return fk.load_library()


def test_library_exports_every_declared_function(lib):
    names = _header_functions()
    assert set(names) >= {"kv_quant_append", "paged_decode_attn", "paged_decode_attn_workspace_size",
                          "fp8kv_abi_version", "fp8kv_status_string", "fp8kv_last_hip_error",
                          "paged_decode_attn_path"}
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings(lib):
    assert lib.fp8kv_abi_version() == _header_define("FP8KV_ABI_VERSION")
    for code in range(-8, 1):
        s = lib.fp8kv_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.fp8kv_status_string(-99).decode() == "unknown status"
    assert lib.fp8kv_last_hip_error().decode() == ""


def test_python_constants_match_header():
    assert fk.KV_FP8_E4M3 == _header_define("FP8KV_KV_FP8_E4M3")
    assert fk.KV_BF16 == _header_define("FP8KV_KV_BF16")
    assert fk.ABORT_TAG_MISMATCH == _header_define("FP8KV_ABORT_TAG_MISMATCH")
    assert fk.ABORT_BAD_METADATA == _header_define("FP8KV_ABORT_BAD_METADATA")
    assert fk.AMAX_WORK_FLOATS == _header_define("FP8KV_AMAX_WORK_FLOATS")


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def _decode(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, kv_dtype=0, ks=1.0, vs=1.0, pt=FAKE, max_pages=8, lens=FAKE,
             tags=None, exp=None, out=FAKE, abort=FAKE, ws=FAKE, ws_bytes=1 << 30, batch=2, hq=8, hkv=2,
             d=64, ps=16, num_pages=64, sm=0.125, blocks=0)
    a.update(kw)
    return lib.paged_decode_attn(a["q"], a["k"], a["v"], a["kv_dtype"], a["ks"], a["vs"], a["pt"],
                                 a["max_pages"], a["lens"], a["tags"], a["exp"], a["out"], a["abort"],
                                 a["ws"], a["ws_bytes"], a["batch"], a["hq"], a["hkv"], a["d"], a["ps"],
                                 a["num_pages"], a["sm"], a["blocks"], None)


def test_decode_validation_codes(lib):
    E = {n: _header_define("FP8KV_ERR_" + n) for n in
         ["NULL", "SHAPE", "UNSUPPORTED", "WORKSPACE", "SCALE", "TAGS", "ALIGN"]}
    assert _decode(lib, q=None) == E["NULL"]
    assert _decode(lib, out=None) == E["NULL"]
    assert _decode(lib, ws=None) == E["NULL"]
    assert _decode(lib, batch=0) == E["SHAPE"]
    assert _decode(lib, hq=7, hkv=2) == E["SHAPE"]
    assert _decode(lib, num_pages=0) == E["SHAPE"]
    assert _decode(lib, max_pages=-1) == E["SHAPE"]
    assert _decode(lib, blocks=-1) == E["SHAPE"]
    assert _decode(lib, batch=65535, hkv=65535, hq=65535, max_pages=1 << 20, ps=16) == E["SHAPE"]
    assert _decode(lib, batch=70000) == E["SHAPE"]
    assert _decode(lib, d=96) == E["UNSUPPORTED"]
    assert _decode(lib, ps=24) == E["UNSUPPORTED"]
    assert _decode(lib, ps=8) == E["UNSUPPORTED"]
    assert _decode(lib, ps=512) == E["UNSUPPORTED"]
    assert _decode(lib, hq=34, hkv=1) == E["UNSUPPORTED"]
    assert _decode(lib, kv_dtype=2) == E["UNSUPPORTED"]
    assert _decode(lib, tags=FAKE) == E["TAGS"]
    assert _decode(lib, exp=FAKE) == E["TAGS"]
    assert _decode(lib, ks=0.0) == E["SCALE"]
    assert _decode(lib, vs=float("inf")) == E["SCALE"]
    assert _decode(lib, vs=-1.0) == E["SCALE"]
    assert _decode(lib, sm=float("nan")) == E["SCALE"]
    assert _decode(lib, q=FAKE + 2) == E["ALIGN"]
    assert _decode(lib, out=FAKE + 4) == E["ALIGN"]      # out takes 8-byte stores
    assert _decode(lib, out=FAKE + 2) == E["ALIGN"]
    assert _decode(lib, ws=FAKE + 16) == E["ALIGN"]
    assert _decode(lib, ws_bytes=16) == E["WORKSPACE"]
    assert _decode(lib, max_pages=1 << 28, ps=256) == E["SHAPE"]
    # BF16 ignores the scales, so a zero scale is not an error there: it fails later (workspace)
    assert _decode(lib, kv_dtype=1, ks=0.0, ws_bytes=16) == E["WORKSPACE"]


def _step(lib, **kw):
    a = dict(k=FAKE, v=FAKE, seq=FAKE, pos=FAKE, n_rows=2, q=FAKE, kc=FAKE, vc=FAKE, kv_dtype=0, ks=1.0, vs=1.0,
             pt=FAKE, max_pages=8, lens=FAKE, tags=None, exp=None, out=FAKE, abort=FAKE, ws=FAKE,
             ws_bytes=1 << 30, batch=2, hq=8, hkv=2, d=64, ps=16, num_pages=64, sm=0.125, blocks=0, ev0=None,
             ev1=None)
    a.update(kw)
    return lib.paged_decode_step(a["k"], a["v"], a["seq"], a["pos"], a["n_rows"], a["q"], a["kc"], a["vc"],
                                 a["kv_dtype"], a["ks"], a["vs"], a["pt"], a["max_pages"], a["lens"], a["tags"],
                                 a["exp"], a["out"], a["abort"], a["ws"], a["ws_bytes"], a["batch"], a["hq"],
                                 a["hkv"], a["d"], a["ps"], a["num_pages"], a["sm"], a["blocks"], a["ev0"],
                                 a["ev1"], None)


def test_step_validation_codes(lib):
    # the decode's arguments are checked first, then the append's; nothing is launched on an error
    E = {n: _header_define("FP8KV_ERR_" + n) for n in
         ["NULL", "SHAPE", "UNSUPPORTED", "WORKSPACE", "SCALE", "TAGS", "ALIGN"]}
    assert _step(lib, q=None) == E["NULL"]
    assert _step(lib, tags=FAKE) == E["TAGS"]
    assert _step(lib, ws_bytes=16) == E["WORKSPACE"]
    assert _step(lib, out=FAKE + 4) == E["ALIGN"]
    assert _step(lib, ks=float("nan")) == E["SCALE"]
    assert _step(lib, d=96) == E["UNSUPPORTED"]
    assert _step(lib, k=None) == E["NULL"]                    # rows to append, no rows given
    assert _step(lib, n_rows=-1) == E["SHAPE"]
    assert _step(lib, k=FAKE + 8) == E["ALIGN"]
    assert _step(lib, ws_bytes=16, k=None) == E["WORKSPACE"]  # decode first
    # with no rows the append's pointers are not needed; this one still fails on the workspace
    assert _step(lib, n_rows=0, k=None, v=None, seq=None, pos=None, ws_bytes=16) == E["WORKSPACE"]


def test_noalloc_validation_codes(lib):
    # the no-allocation decode checks every argument before it looks up its scratch; sizes whose
    # workspace exceeds the fixed scratch are FP8KV_ERR_SCRATCH (nothing launched, no device touched)
    E = {n: _header_define("FP8KV_ERR_" + n) for n in ["NULL", "SHAPE", "TAGS", "ALIGN", "SCRATCH"]}
    assert fk.ERR_SCRATCH == E["SCRATCH"]
    m = re.search(r"#define\s+FP8KV_NOALLOC_SCRATCH_BYTES\s+\((\d+)u << (\d+)\)", _header_text())
    assert fk.NOALLOC_SCRATCH_BYTES == int(m.group(1)) << int(m.group(2))

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, kv_dtype=0, ks=1.0, vs=1.0, pt=FAKE, max_pages=8, lens=FAKE, tags=None,
                 exp=None, out=FAKE, abort=FAKE, batch=2, hq=8, hkv=2, d=64, ps=16, num_pages=64, sm=0.125,
                 blocks=65535)
        a.update(kw)
        return lib.paged_decode_attn_noalloc(a["q"], a["k"], a["v"], a["kv_dtype"], a["ks"], a["vs"], a["pt"],
                                             a["max_pages"], a["lens"], a["tags"], a["exp"], a["out"], a["abort"],
                                             a["batch"], a["hq"], a["hkv"], a["d"], a["ps"], a["num_pages"],
                                             a["sm"], a["blocks"], None)
    assert fk.paged_decode_attn_workspace_size(2, 8, 2, 64, 16, 8, 65535) > fk.NOALLOC_SCRATCH_BYTES
    assert call() == E["SCRATCH"]                   # 65535 blocks: far more partial slots than the scratch holds
    assert call(q=None) == E["NULL"]
    assert call(batch=0) == E["SHAPE"]
    assert call(tags=FAKE) == E["TAGS"]
    assert call(out=FAKE + 4) == E["ALIGN"]


def _append(lib, **kw):
    a = dict(k=FAKE, v=FAKE, seq=FAKE, pos=FAKE, pt=FAKE, batch=2, max_pages=8, ks=1.0, vs=1.0,
             kc=FAKE, vc=FAKE, num_pages=64, n_rows=4, hkv=2, d=64, ps=16, kv_dtype=0)
    a.update(kw)
    return lib.kv_quant_append(a["k"], a["v"], a["seq"], a["pos"], a["pt"], a["batch"], a["max_pages"],
                               a["ks"], a["vs"], a["kc"], a["vc"], a["num_pages"], a["n_rows"], a["hkv"],
                               a["d"], a["ps"], a["kv_dtype"], None)


def test_append_validation_codes(lib):
    E = {n: _header_define("FP8KV_ERR_" + n) for n in ["NULL", "SHAPE", "UNSUPPORTED", "SCALE", "ALIGN"]}
    assert _append(lib, n_rows=0, k=None) == 0           # nothing to do, nothing launched
    assert _append(lib, k=None) == E["NULL"]
    assert _append(lib, pt=None) == E["NULL"]
    assert _append(lib, n_rows=-1) == E["SHAPE"]
    assert _append(lib, hkv=0) == E["SHAPE"]
    assert _append(lib, hkv=65536) == E["SHAPE"]
    assert _append(lib, d=32) == E["UNSUPPORTED"]
    assert _append(lib, ps=48) == E["UNSUPPORTED"]
    assert _append(lib, kv_dtype=5) == E["UNSUPPORTED"]
    assert _append(lib, ks=float("nan")) == E["SCALE"]
    assert _append(lib, vs=0.0) == E["SCALE"]
    assert _append(lib, kc=FAKE + 8) == E["ALIGN"]


def test_workspace_size_is_deterministic_and_grows(lib):
    f = fk.paged_decode_attn_workspace_size
    a = f(32, 64, 8, 128, 64, 513)
    assert a > 0 and a % 256 == 0 and a == f(32, 64, 8, 128, 64, 513)
    assert f(64, 64, 8, 128, 64, 513) >= a
    assert f(32, 64, 8, 128, 64, 513, 64) >= f(32, 64, 8, 128, 64, 513, 8)
    assert f(0, 64, 8, 128, 64, 513) == 0
    assert f(2, 7, 2, 64, 16, 17) == 0


def test_path_selection(lib, monkeypatch):
    monkeypatch.delenv("FP8KV_FORCE_PATH", raising=False)
    assert fk.paged_decode_attn_path(64, 8) == 1
    assert fk.paged_decode_attn_path(128, 8) == 1
    assert fk.paged_decode_attn_path(8, 2) == 0
    assert fk.paged_decode_attn_path(8, 8) == 0
    assert fk.paged_decode_attn_path(7, 2) == -1
    monkeypatch.setenv("FP8KV_FORCE_PATH", "mfma")
    assert fk.paged_decode_attn_path(8, 2) == 1
    monkeypatch.setenv("FP8KV_FORCE_PATH", "valu")
    assert fk.paged_decode_attn_path(8, 2) == 0
    assert fk.paged_decode_attn_path(64, 8) == 1      # VALU covers groups up to 4 only


def test_pool_and_checked_append_validation_codes(lib):
    E = {n: _header_define("FP8KV_ERR_" + n) for n in ["NULL", "SHAPE"]}
    assert lib.page_pool_init(None, FAKE, 8, None) == E["NULL"]
    assert lib.page_pool_init(FAKE, FAKE, 0, None) == E["SHAPE"]
    args = [FAKE] * 8
    assert lib.page_alloc(*args, 0, 4, 8, None) == E["SHAPE"]
    assert lib.page_alloc(*args, 2, 4, 0, None) == E["SHAPE"]
    assert lib.page_alloc(None, *args[1:], 2, 4, 8, None) == E["NULL"]
    assert lib.page_alloc(*args[:7], None, 2, 4, 8, None) == E["NULL"]
    args = [FAKE] * 6
    assert lib.page_free(*args, 2, 0, 8, None) == E["SHAPE"]
    assert lib.page_free(*args[:5], None, 2, 4, 8, None) == E["NULL"]
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 1.0, 1.0, FAKE, FAKE, 64, 4, 2, 64, 16, 0]
    assert lib.kv_quant_append_checked(*base, None, FAKE, FAKE, None) == E["NULL"]
    assert lib.kv_quant_append_checked(*base, FAKE, FAKE, None, None) == E["NULL"]
    base[12] = 0  # no rows: nothing to check, nothing launched
    assert lib.kv_quant_append_checked(*base, None, None, None, None) == 0


def test_handoff_validation_codes(lib):
    E = {n: _header_define("FP8KV_ERR_" + n) for n in ["NULL", "SHAPE", "ALIGN"]}
    assert lib.kv_absmax_scale(FAKE, -1, FAKE, FAKE, None) == E["SHAPE"]
    assert lib.kv_absmax_scale(None, 8, FAKE, FAKE, None) == E["NULL"]
    assert lib.kv_absmax_scale(FAKE, 8, None, FAKE, None) == E["NULL"]
    assert lib.kv_absmax_scale(FAKE, 8, FAKE, None, None) == E["NULL"]
    assert lib.kv_absmax_scale(FAKE + 2, 8, FAKE, FAKE, None) == E["ALIGN"]
    assert lib.kv_absmax_scale(FAKE, 8, FAKE + 2, FAKE, None) == E["ALIGN"]
    assert lib.kv_absmax_scale(FAKE, 8, FAKE, FAKE + 2, None) == E["ALIGN"]
    assert lib.kv_absmax_scale_kv(FAKE, FAKE, -1, FAKE, FAKE, None) == E["SHAPE"]
    assert lib.kv_absmax_scale_kv(FAKE, None, 8, FAKE, FAKE, None) == E["NULL"]
    assert lib.kv_absmax_scale_kv(FAKE, FAKE, 8, FAKE, None, None) == E["NULL"]
    assert lib.kv_absmax_scale_kv(FAKE, FAKE + 2, 8, FAKE, FAKE, None) == E["ALIGN"]
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8]
    tail = [FAKE, FAKE, 64, 4, 2, 64, 16, None]
    assert lib.kv_quant_append_dscale(*base, None, FAKE, *tail) == E["NULL"]
    assert lib.kv_quant_append_dscale(*base, FAKE, FAKE + 2, *tail) == E["ALIGN"]


def test_int4_gemv_validation_codes(lib):
    E = {n: _header_define("FP8KV_ERR_" + n) for n in ["NULL", "SHAPE", "ALIGN"]}
    assert fk.INT4_GROUP == _header_define("FP8KV_INT4_GROUP")
    assert fk.INT4_MAX_M == _header_define("FP8KV_INT4_MAX_M")
    ok = [FAKE, FAKE, FAKE, FAKE, 1, 64, 256, None]
    for i, v in ((4, 0), (4, 65), (5, 0), (6, 0), (6, 64), (6, 200)):
        a = list(ok); a[i] = v
        assert lib.int4_gemv(*a) == E["SHAPE"], (i, v)
    for i in range(4):
        a = list(ok); a[i] = None
        assert lib.int4_gemv(*a) == E["NULL"], i
    for i, off in ((0, 8), (1, 4), (2, 1), (3, 1)):
        a = list(ok); a[i] = FAKE + off
        assert lib.int4_gemv(*a) == E["ALIGN"], i


def test_int4_pack_validation_codes(lib):
    E = {n: _header_define("FP8KV_ERR_" + n) for n in ["NULL", "SHAPE", "ALIGN"]}
    ok = [FAKE, FAKE, FAKE, FAKE, 16, 256, None]
    for i, v in ((4, 0), (5, 0), (5, 64), (5, 200)):
        a = list(ok); a[i] = v
        assert lib.int4_pack_weights(*a) == E["SHAPE"], (i, v)
    for i in range(4):
        a = list(ok); a[i] = None
        assert lib.int4_pack_weights(*a) == E["NULL"], i
    for i, off in ((0, 2), (1, 1), (2, 4), (3, 1)):
        a = list(ok); a[i] = FAKE + off
        assert lib.int4_pack_weights(*a) == E["ALIGN"], i


def test_a_c_program_builds_and_runs_against_the_library(tmp_path):
    """The header is plain C and the library links from C: compile
    tests/c_abi_consumer.c with gcc against include/fp8kv.h and libfp8kv.so
    and run it (ABI version, status strings, workspace size, argument errors;
    nothing is launched)."""
    import shutil
    import subprocess

    fk.load_library()
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not installed")
    lib_dir = os.path.dirname(fk.lib_path)
    exe = str(tmp_path / "c_abi_consumer")
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_abi_consumer.c"), "-o", exe, "-L", lib_dir, "-l:libfp8kv.so",
                    f"-Wl,-rpath,{lib_dir}", "-lm"], check=True)
    res = subprocess.run([exe], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    assert "passed" in res.stdout
