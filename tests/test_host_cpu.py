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
    # the intermediates (fp32) plus the split-K partial tiles for few rows
    assert m.mla_output_proj_workspace_size(3, 4, 8, 5, 16, m.MLA_PROJ_TWO_STAGE) >= 3 * 4 * 5 * 4
    assert m.mla_cache_append_workspace_size(3, 16, 8, 4) >= 3 * 12 * 4
    assert m.mla_absorb_query_workspace_size(3, 16, 2, 8, 4) >= 3 * 2 * 12 * 4
    # DeepSeek widths with 32 decode tokens: the merged output projection splits K
    # (5120 outputs over 128 x 512 inputs), so its workspace holds partial tiles
    assert m.mla_output_proj_workspace_size(32, 128, 512, 128, 5120, m.MLA_PROJ_MERGED) >= 2 * 32 * 5120 * 4
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


# ----------------------------------------------------------------------------
# build guards of the matrix-core kernel
# ----------------------------------------------------------------------------

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _have_hipcc():
    return os.path.exists(HIPCC)


@pytest.mark.skipif(not _have_hipcc(), reason="hipcc not installed")
def test_decode_kernels_use_no_scratch(tmp_path):
    """Every instantiation of the matrix-core decode kernel compiles with no
    scratch memory and no vector-register spills (its speed depends on that:
    a scratch reload waits for every memory operation in flight, including
    the cache copies), one wavefront per SIMD, and LDS within 160 KB."""
    src = os.path.join(ROOT, "latent_kv_cache_mla_amd", "csrc", "decode_mfma.hip")
    r = subprocess.run([HIPCC, *DEVICE_FLAGS, "-c", src, "-o", str(tmp_path / "d.o"),
                        "-Rpass-analysis=kernel-resource-usage"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    blocks = re.split(r"remark: Function Name: ", r.stderr)[1:]
    kernels = {}
    for blk in blocks:
        name = blk.split()[0]
        field = lambda k: int(re.search(rf"{k}: (\d+)", blk).group(1))  # noqa: E731
        kernels[name] = {"scratch": field(r"ScratchSize \[bytes/lane\]"),
                         "vspill": field("VGPRs Spill"), "lds": field(r"LDS Size \[bytes/block\]")}
    decode = {k: v for k, v in kernels.items() if "decode_mfma" in k}
    assert len(decode) >= 6, sorted(kernels)
    for name, v in decode.items():
        assert v["scratch"] == 0 and v["vspill"] == 0, (name, v)
        assert v["lds"] <= 160 * 1024, (name, v)


@pytest.mark.skipif(not _have_hipcc(), reason="hipcc not installed")
def test_wait_states_after_inline_matrix_ops_cover_the_hazard(tmp_path):
    """The score MFMAs are inline asm, which the compiler's hazard checker does
    not see into; the last of each chain is followed by 16 wait states
    (s_nop 7, twice) before vector-ALU code reads its result. Ask the compiler
    how many it places itself between the same instruction and a dependent
    vector-ALU read, and check that 16 covers it."""
    src = tmp_path / "probe.hip"
    src.write_text(
        "#include <hip/hip_runtime.h>\n"
        "typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));\n"
        "typedef float f32x16 __attribute__((ext_vector_type(16)));\n"
        "__global__ void probe(float* out, const bf16x8* a, const bf16x8* b) {\n"
        "  const int t = threadIdx.x;\n"
        "  f32x16 c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t], b[t], f32x16{}, 0, 0, 0);\n"
        "  out[t] = c[0] * 3.0f + c[5];\n"
        "}\n")
    asm = tmp_path / "probe.s"
    r = subprocess.run([HIPCC, *DEVICE_FLAGS, "-S", str(src), "-o", str(asm)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = asm.read_text().splitlines()
    i = next(k for k, l in enumerate(lines) if "v_mfma_f32_32x32x16_bf16" in l)
    needed = 0
    for l in lines[i + 1:]:
        m = re.match(r"\s*s_nop\s+(\d+)", l)
        if not m:
            break
        needed += int(m.group(1)) + 1
    assert 0 < needed <= 16, needed
    kernel = open(os.path.join(ROOT, "latent_kv_cache_mla_amd", "csrc", "decode_mfma.hip")).read()
    assert 'v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\\n\\ts_nop 7\\n\\ts_nop 7' in kernel


def test_one_hip_runtime_whatever_the_import_order(tmp_path):
    """Importing the binding before torch must not load a second HIP runtime
    (the binding loads torch's first, and libmla then binds to it)."""
    code = ("import latent_kv_cache_mla_amd, torch\n"
            "paths = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len(paths)); print(sorted(paths))\n")
    r = subprocess.run(["python", "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.splitlines()[0] == "1", r.stdout


def test_noalloc_decode_rejects_calls_above_its_array(m):
    """mla_decode_noalloc refuses, on the host and before any launch, a
    descriptor whose workspace exceeds its fixed device array; the five
    workloads all fit."""
    import ctypes
    big = m.decode_desc(4096, 2, 128, 512, 64, 64, "bf16", "bf16", "bf16")
    assert m.mla_decode_workspace_size(big) > m.mla_decode_noalloc_max_workspace()
    dummy = ctypes.c_void_p(256)   # never dereferenced: the size check comes first
    st = m.lib.mla_decode_noalloc(ctypes.byref(big), dummy, dummy, dummy, None, dummy, dummy,
                                  ctypes.c_float(0.1), dummy, None, None)
    assert st == m.MLA_ERR_WORKSPACE_TOO_SMALL, m.mla_last_error()
    assert "scratch" in m.mla_last_error()
    for B, q, S, dt in ((32, 1, 4096, "bf16"), (4, 1, 32768, "bf16"), (64, 1, 16384, "bf16"),
                        (128, 2, 8192, "fp8")):
        d = m.decode_desc(B, q, 128, 512, 64, (S + 63) // 64, dt, "bf16", "bf16")
        assert m.mla_decode_workspace_size(d) <= m.mla_decode_noalloc_max_workspace()


def test_binding_rejects_short_buffers_before_the_call(m):
    """The marshalling layer compares every buffer the shapes determine with
    what the call reads or writes through it, and raises before the C call:
    a short buffer would otherwise be an out-of-bounds device access. CPU
    tensors suffice: nothing reaches the library."""
    import torch

    f32 = lambda n: torch.zeros(n, dtype=torch.float32)  # noqa: E731
    i32 = lambda n: torch.zeros(n, dtype=torch.int32)  # noqa: E731
    T, n_h, d_c, d_r, d_in, d_h, d = 4, 2, 8, 4, 16, 8, 32
    cases = [
        lambda: m.mla_absorb_query(f32(T * d_in), T, d_in, f32(n_h * d_c * d_in), f32(n_h * d_r * d_in),
                                   n_h, d_c, d_r, 1e4, i32(T), m.MLA_FP32, f32(T * n_h * d_c - 1),
                                   f32(T * n_h * d_r), f32(1)),
        lambda: m.mla_absorb_query(f32(T * d_in - 1), T, d_in, f32(n_h * d_c * d_in), f32(n_h * d_r * d_in),
                                   n_h, d_c, d_r, 1e4, i32(T), m.MLA_FP32, f32(T * n_h * d_c),
                                   f32(T * n_h * d_r), f32(1)),
        lambda: m.mla_output_proj(f32(T * n_h * d_c), m.MLA_FP32, T, n_h, d_c, d_h, d, m.MLA_PROJ_MERGED,
                                  f32(d * n_h * d_c - 1), None, f32(T * d)),
        lambda: m.mla_output_proj(f32(T * n_h * d_c), m.MLA_FP32, T, n_h, d_c, d_h, d, m.MLA_PROJ_TWO_STAGE,
                                  f32(n_h * d_h * d_c), f32(d * n_h * d_h), f32(T * d - 1)),
        lambda: m.mla_cache_append(f32(T * d), T, d, f32(d_c * d), f32(d_r * d - 1), d_c, d_r, 1e4,
                                   i32(T), i32(T), m.MLA_BF16, f32(1), None, f32(1)),
        lambda: m.mla_cache_write(f32(T * (d_c + d_r)), T, d_c, d_r, 1e4, i32(T - 1), i32(T), m.MLA_BF16,
                                  f32(1)),
        lambda: m.mla_fold_query(f32(n_h * d_h * d_in), f32(n_h * d_h * d_c), n_h, d_h, d_c, d_in,
                                 f32(n_h * d_c * d_in - 1)),
        lambda: m.mla_fold_output(f32(d * n_h * d_h - 1), f32(n_h * d_h * d_c), n_h, d_h, d_c, d,
                                  f32(d * n_h * d_c)),
    ]
    for i, call in enumerate(cases):
        with pytest.raises(m.MlaArgumentError):
            call()
