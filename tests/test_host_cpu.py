"""CPU-only checks of the host side: the C ABI loads and exports every
declared symbol, host-only entry points follow their closed forms, argument
errors are reported before any launch, and the split partition arithmetic is
exact (compiled with g++ from the same header the kernels use)."""
import ctypes
import os
import re
import subprocess

import pytest

from tests.conftest import ROOT


def _header_functions():
    txt = open(os.path.join(ROOT, "include", "mla.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def m():
    import latent_kv_cache_mla_amd as m
    return m


def test_library_exports_every_declared_symbol(m):
    declared = _header_functions()
    assert len(declared) >= 17
    for name in declared:
        assert hasattr(m.lib, name), f"{name} declared in include/mla.h but not exported"
        assert hasattr(m, name), f"{name} has no binding of the same name"
    out = subprocess.run(["nm", "-D", "--defined-only", m.LIB_PATH], capture_output=True, text=True).stdout
    for name in declared:
        assert re.search(rf"\bT {name}\b", out), name


def test_cache_bytes_per_token_closed_forms(m, golden):
    # 576 numbers per token ([Mishra] Step 4) at 2 bytes each
    assert m.mla_cache_bytes_per_token(512, 64, m.MLA_BF16) == 2 * golden["mla_elements_per_token"]["value"]
    assert m.mla_cache_bytes_per_token(512, 64, m.MLA_FP8_E4M3) == 512 + 128 + 4
    assert m.mla_cache_bytes_per_token(64, 16, m.MLA_FP32) == 4 * 80
    # 57x less than MHA's 32768 16-bit numbers
    mha_bytes = 2 * golden["mha_elements_per_token_128x128"]["value"]
    assert round(mha_bytes / m.mla_cache_bytes_per_token(512, 64, m.MLA_BF16)) == 57
    assert m.mla_cache_bytes_per_token(512, 64, 7) == 0


def test_workspace_size_is_pure_and_monotone(m):
    d = m.decode_desc(32, 1, 128, 512, 64, 64)
    a = m.mla_decode_workspace_size(d)
    assert a == m.mla_decode_workspace_size(d) and a % 256 == 0
    d2 = m.decode_desc(64, 1, 128, 512, 64, 256)
    assert m.mla_decode_workspace_size(d2) >= a
    # partials: at most (G + B) slots of rows x d_c floats plus the plan
    d3 = m.decode_desc(4, 2, 8, 64, 16, 10, "fp32", "fp32", "fp32", num_partitions=3)
    assert m.mla_decode_workspace_size(d3) >= (3 + 4) * 16 * 64 * 4


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, 1), ("q_len", 0, 1), ("n_heads", 0, 1), ("d_c", 12, 2), ("d_c", 2048, 2),
    ("d_rope", 5, 2), ("page_size", 32, 2), ("max_blocks_per_seq", 0, 1), ("cache_dtype", 9, 1),
    ("q_dtype", 2, 1), ("out_dtype", 2, 1), ("num_partitions", -1, 1), ("flags", 2, 1),
    ("flags", -1, 1),
])
def test_bad_descriptors_rejected(m, field, value, status):
    d = m.decode_desc(2, 1, 16, 512, 64, 4)
    setattr(d, field, value)
    assert m.lib.mla_decode_workspace_size(ctypes.byref(d)) == 0
    r = m.lib.mla_decode(ctypes.byref(d), 16, 16, 16, 16, 16, 16, 1.0, 16, None, 256, 1 << 30, None)
    assert r == status, m.mla_last_error()
    assert m.mla_last_error() != ""


def test_fp8_math_flag_is_accepted_for_every_cache(m):
    """MLA_DECODE_FP8_MATH only changes how an fp8 cache on the matrix-core
    shape is multiplied; the workspace layout does not depend on it."""
    for dt in ("bf16", "fp8"):
        a = m.decode_desc(128, 2, 128, 512, 64, 128, dt)
        b = m.decode_desc(128, 2, 128, 512, 64, 128, dt, flags=m.MLA_DECODE_FP8_MATH)
        assert m.mla_decode_workspace_size(a) == m.mla_decode_workspace_size(b) > 0


def test_fp32_queries_need_fp32_cache(m):
    d = m.decode_desc(2, 1, 16, 512, 64, 4, "bf16", "fp32")
    assert m.lib.mla_decode(ctypes.byref(d), 16, 16, 16, 16, 16, 16, 1.0, 16, None, 256, 1 << 30,
                            None) == m.MLA_ERR_UNSUPPORTED


def test_decode_argument_errors_return_before_launch(m):
    d = m.decode_desc(2, 1, 16, 512, 64, 4)
    need = m.mla_decode_workspace_size(d)
    call = lambda **kw: m.lib.mla_decode(  # noqa: E731
        ctypes.byref(d), kw.get("q", 16), kw.get("qr", 16), kw.get("c", 16), kw.get("sc", None),
        16, 16, kw.get("scale", 0.1), kw.get("o", 16), None, kw.get("ws", 256),
        kw.get("wsb", need), None)
    assert call(q=None) == m.MLA_ERR_INVALID_ARGUMENT
    assert call(qr=None) == m.MLA_ERR_INVALID_ARGUMENT
    assert call(scale=float("nan")) == m.MLA_ERR_INVALID_ARGUMENT
    assert call(scale=float("inf")) == m.MLA_ERR_INVALID_ARGUMENT
    assert call(q=17) == m.MLA_ERR_MISALIGNED
    assert call(o=8) == m.MLA_ERR_MISALIGNED
    assert call(ws=128) == m.MLA_ERR_MISALIGNED
    assert call(wsb=need - 1) == m.MLA_ERR_WORKSPACE_TOO_SMALL
    d.cache_dtype = m.MLA_FP8_E4M3
    assert call() == m.MLA_ERR_INVALID_ARGUMENT          # fp8 without scales
    assert "cache_scale" in m.mla_last_error()


def test_other_entry_points_check_arguments(m):
    L = m.lib
    assert L.mla_fold_query(None, 16, 2, 2, 2, 2, 16, None) == m.MLA_ERR_INVALID_ARGUMENT
    assert L.mla_fold_output(16, 16, 0, 2, 2, 2, 16, None) == m.MLA_ERR_INVALID_ARGUMENT
    assert L.mla_output_proj(16, 5, 1, 2, 2, 2, 2, 0, 16, 16, 16, None, 0, None) == m.MLA_ERR_INVALID_ARGUMENT
    assert L.mla_output_proj(16, 0, 1, 2, 2, 2, 2, 1, 16, 16, 16, None, 0, None) == m.MLA_ERR_WORKSPACE_TOO_SMALL
    assert L.mla_cache_write(16, 1, 8, 3, 1e4, 16, 16, 1, 16, None, None) == m.MLA_ERR_INVALID_ARGUMENT
    assert L.mla_cache_write(16, 1, 8, 2, 1e4, 16, 16, 2, 16, None, None) == m.MLA_ERR_INVALID_ARGUMENT
    assert L.mla_absorb_query(16, 1, 4, 16, 16, 2, 8, 2, 1e4, 16, 3, 16, 16, 16, 1 << 20, None) == \
        m.MLA_ERR_INVALID_ARGUMENT
    assert L.mla_absorb_query(16, 1, 4, 16, 16, 2, 8, 2, 1e4, 16, 1, 16, 16, 16, 4, None) == \
        m.MLA_ERR_WORKSPACE_TOO_SMALL
    assert m.mla_output_proj_workspace_size(3, 4, 5, m.MLA_PROJ_TWO_STAGE) == 3 * 4 * 5 * 4
    assert m.mla_cache_append_workspace_size(3, 8, 4) == 3 * 12 * 4
    assert m.mla_absorb_query_workspace_size(3, 2, 8, 4) == 3 * 2 * 12 * 4
    for s in range(7):
        assert m.mla_status_string(s).startswith("MLA_")
    assert m.mla_version() >= 100


def test_partition_arithmetic(tmp_path):
    exe = tmp_path / "test_partition"
    src = os.path.join(ROOT, "tests", "cpp", "test_partition.cpp")
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Werror", src, "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout


def test_partition_arithmetic_under_sanitizers(tmp_path):
    exe = tmp_path / "test_partition_san"
    src = os.path.join(ROOT, "tests", "cpp", "test_partition.cpp")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", src, "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
