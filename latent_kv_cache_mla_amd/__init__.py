"""Python binding of libmla (include/mla.h): absorbed-MLA decode on MI355X.

Argument marshalling only: every function below forwards to the C entry point
of the same name in the in-tree ``libmla.so`` (built by
``latent_kv_cache_mla_amd.build``). Tensors are ``torch`` tensors on the GPU;
torch supplies device memory and the current HIP stream, nothing else. There
is no fallback: if the library is missing, importing this package raises.
"""
from __future__ import annotations

import ctypes
import os

# torch first: the library then binds to the HIP runtime torch has loaded. A
# library loaded before torch would bring in a second HIP runtime (the
# system's), and kernels launched through it would not see the device that
# torch's allocations live on.
import torch  # noqa: F401,E402

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python -m latent_kv_cache_mla_amd.build)")

lib = ctypes.CDLL(LIB_PATH)

MLA_OK = 0
MLA_ERR_INVALID_ARGUMENT = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_WORKSPACE_TOO_SMALL = 3
MLA_ERR_MISALIGNED = 4
MLA_ERR_HIP = 5
MLA_ERR_BAD_CONTENTS = 6

MLA_FP32, MLA_BF16, MLA_FP8_E4M3 = 0, 1, 2
MLA_PROJ_MERGED, MLA_PROJ_TWO_STAGE = 0, 1
MLA_PAGE_SIZE = 64
MLA_DECODE_FP8_MATH = 1

DTYPE_CODES = {"fp32": MLA_FP32, "bf16": MLA_BF16, "fp8": MLA_FP8_E4M3}


class MlaDecodeDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "q_len", "n_heads", "d_c", "d_rope", "page_size",
        "max_blocks_per_seq", "cache_dtype", "q_dtype", "out_dtype",
        "num_partitions", "plan_ready", "flags")]


class MlaPrefillDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "max_seq_len", "d_model", "n_heads", "d_head", "d_rope", "d_c", "d_cq")] + \
        [("rope_theta", ctypes.c_float)]


class MlaPrefillWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("W_DKVR", "W_DQ", "W_UQR", "W_UKV", "W_O")]


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.mla_last_error().decode()
        super().__init__(f"{where}: {lib.mla_status_string(status).decode()}: {msg}")


_P = ctypes.c_void_p
_I = ctypes.c_int32
_S = ctypes.c_size_t
_DESC = ctypes.POINTER(MlaDecodeDesc)

_SIGS = {
    "mla_decode_workspace_size": (_S, [_DESC]),
    "mla_decode_plan": (_I, [_DESC, _P, _P, _S, _P]),
    "mla_decode": (_I, [_DESC, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P, _S, _P]),
    "mla_decode_partial": (_I, [_DESC, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _S, _P]),
    "mla_decode_noalloc": (_I, [_DESC, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P]),
    "mla_decode_noalloc_max_workspace": (_S, []),
    "mla_decode_combine": (_I, [_DESC, _P, _S, _P, _P, _P]),
    "mla_decode_validate": (_I, [_DESC, _P, _P, ctypes.c_int64, _P]),
    "mla_fold_query": (_I, [_P, _P, _I, _I, _I, _I, _P, _P]),
    "mla_fold_output": (_I, [_P, _P, _I, _I, _I, _I, _P, _P]),
    "mla_output_proj_workspace_size": (_S, [_I, _I, _I, _I, _I, _I]),
    "mla_output_proj": (_I, [_P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _S, _P]),
    "mla_cache_write": (_I, [_P, _I, _I, _I, ctypes.c_float, _P, _P, _I, _P, _P, _P]),
    "mla_cache_append_workspace_size": (_S, [_I, _I, _I, _I]),
    "mla_cache_append": (_I, [_P, _I, _I, _P, _P, _I, _I, ctypes.c_float, _P, _P, _I, _P, _P,
                              _P, _S, _P]),
    "mla_absorb_query_workspace_size": (_S, [_I, _I, _I, _I, _I]),
    "mla_absorb_query": (_I, [_P, _I, _I, _P, _P, _I, _I, _I, ctypes.c_float, _P, _I, _P, _P,
                              _P, _S, _P]),
    "mla_cache_bytes_per_token": (_S, [_I, _I, _I]),
    "mla_gemm_bf16": (_I, [_I, _I, _I, _P, ctypes.c_int64, _P, ctypes.c_int64, _P, ctypes.c_int64,
                           _I, _I, _P, _P]),
    "mla_gemm_bf16_partial_size": (_S, [_I, _I, _I, _I]),
    "mla_prefill_attention": (_I, [ctypes.POINTER(MlaPrefillDesc), ctypes.c_int64, _P, ctypes.c_int64,
                                   _P, ctypes.c_int64, _P, ctypes.c_int64, _P, ctypes.c_int64, _P,
                                   ctypes.c_int64, _P, ctypes.c_float, _P, ctypes.c_int64, _P, _P]),
    "mla_prefill_workspace_size": (_S, [ctypes.POINTER(MlaPrefillDesc), ctypes.c_int64]),
    "mla_prefill": (_I, [ctypes.POINTER(MlaPrefillDesc), _P, ctypes.c_int64, _P, _P,
                         ctypes.POINTER(MlaPrefillWeights), ctypes.c_float, _P, _P, _P, _P, _S, _P]),
    "mla_status_string": (ctypes.c_char_p, [_I]),
    "mla_last_error": (ctypes.c_char_p, []),
    "mla_version": (_I, []),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_SIGS)


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status: int, where: str):
    if status != MLA_OK:
        raise MlaError(status, where)


def _dev(t, name):
    if t is not None and (not t.is_cuda or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    return t


class MlaArgumentError(MlaError):
    """A buffer too small for what the descriptor says the call touches,
    found by the binding before the C call (no device access happened)."""

    def __init__(self, where: str, msg: str):
        self.status = MLA_ERR_INVALID_ARGUMENT
        RuntimeError.__init__(self, f"{where}: MLA_ERR_INVALID_ARGUMENT: {msg}")


_ELEM = {MLA_FP32: 4, MLA_BF16: 2}


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _need(t, nbytes, name, where):
    """`t` must hold at least `nbytes` bytes (a size check only: the library
    reads or writes exactly that many through the pointer)."""
    if t is not None and _nbytes(t) < nbytes:
        raise MlaArgumentError(where, f"{name} holds {_nbytes(t)} bytes, the descriptor needs {nbytes}")


def _check_decode_buffers(desc, where, q_abs=None, q_rope=None, block_table=None, seq_lens=None,
                          o_latent=None, lse_out=None):
    rows = int(desc.batch) * int(desc.q_len) * int(desc.n_heads)
    qe = _ELEM.get(int(desc.q_dtype), 4)
    oe = _ELEM.get(int(desc.out_dtype), 4)
    _need(q_abs, rows * int(desc.d_c) * qe, "q_abs", where)
    _need(q_rope, rows * int(desc.d_rope) * qe, "q_rope", where)
    _need(block_table, int(desc.batch) * int(desc.max_blocks_per_seq) * 4, "block_table", where)
    _need(seq_lens, int(desc.batch) * 4, "seq_lens", where)
    _need(o_latent, rows * int(desc.d_c) * oe, "o_latent", where)
    _need(lse_out, rows * 4, "lse_out", where)


def decode_desc(batch, q_len, n_heads, d_c, d_rope, max_blocks_per_seq, cache_dtype="bf16",
                q_dtype="bf16", out_dtype="bf16", num_partitions=0, plan_ready=0,
                flags=0) -> MlaDecodeDesc:
    code = lambda x: DTYPE_CODES[x] if isinstance(x, str) else int(x)  # noqa: E731
    return MlaDecodeDesc(batch, q_len, n_heads, d_c, d_rope, MLA_PAGE_SIZE, max_blocks_per_seq,
                         code(cache_dtype), code(q_dtype), code(out_dtype), num_partitions,
                         plan_ready, flags)


# ----------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ----------------------------------------------------------------------------

def mla_decode_workspace_size(desc: MlaDecodeDesc) -> int:
    n = lib.mla_decode_workspace_size(ctypes.byref(desc))
    if n == 0:
        raise MlaError(MLA_ERR_INVALID_ARGUMENT, "mla_decode_workspace_size")
    return n


def mla_decode_plan(desc, seq_lens, workspace, stream=None):
    _check_decode_buffers(desc, "mla_decode_plan", seq_lens=seq_lens)
    _check(lib.mla_decode_plan(ctypes.byref(desc), _ptr(_dev(seq_lens, "seq_lens")),
                               _ptr(_dev(workspace, "workspace")), workspace.numel() * workspace.element_size(),
                               _stream(stream)), "mla_decode_plan")


def mla_decode(desc, q_abs, q_rope, cache, cache_scale, block_table, seq_lens, scale,
               o_latent, lse_out, workspace, stream=None):
    for t, n in ((q_abs, "q_abs"), (q_rope, "q_rope"), (cache, "cache"), (cache_scale, "cache_scale"),
                 (block_table, "block_table"), (seq_lens, "seq_lens"), (o_latent, "o_latent"),
                 (lse_out, "lse_out"), (workspace, "workspace")):
        _dev(t, n)
    _check_decode_buffers(desc, "mla_decode", q_abs, q_rope, block_table, seq_lens, o_latent,
                          lse_out)
    _check(lib.mla_decode(ctypes.byref(desc), _ptr(q_abs), _ptr(q_rope), _ptr(cache),
                          _ptr(cache_scale), _ptr(block_table), _ptr(seq_lens), float(scale),
                          _ptr(o_latent), _ptr(lse_out), _ptr(workspace),
                          workspace.numel() * workspace.element_size(), _stream(stream)),
           "mla_decode")


def mla_decode_noalloc(desc, q_abs, q_rope, cache, cache_scale, block_table, seq_lens, scale,
                       o_latent, lse_out, stream=None):
    for t, n in ((q_abs, "q_abs"), (q_rope, "q_rope"), (cache, "cache"), (cache_scale, "cache_scale"),
                 (block_table, "block_table"), (seq_lens, "seq_lens"), (o_latent, "o_latent"),
                 (lse_out, "lse_out")):
        _dev(t, n)
    _check_decode_buffers(desc, "mla_decode_noalloc", q_abs, q_rope, block_table, seq_lens,
                          o_latent, lse_out)
    _check(lib.mla_decode_noalloc(ctypes.byref(desc), _ptr(q_abs), _ptr(q_rope), _ptr(cache),
                                  _ptr(cache_scale), _ptr(block_table), _ptr(seq_lens),
                                  float(scale), _ptr(o_latent), _ptr(lse_out), _stream(stream)),
           "mla_decode_noalloc")


def mla_decode_noalloc_max_workspace():
    return lib.mla_decode_noalloc_max_workspace()


def mla_decode_partial(desc, q_abs, q_rope, cache, cache_scale, block_table, seq_lens, scale,
                       workspace, stream=None):
    for t, n in ((q_abs, "q_abs"), (q_rope, "q_rope"), (cache, "cache"), (cache_scale, "cache_scale"),
                 (block_table, "block_table"), (seq_lens, "seq_lens"), (workspace, "workspace")):
        _dev(t, n)
    _check_decode_buffers(desc, "mla_decode_partial", q_abs, q_rope, block_table, seq_lens)
    _check(lib.mla_decode_partial(ctypes.byref(desc), _ptr(q_abs), _ptr(q_rope), _ptr(cache),
                                  _ptr(cache_scale), _ptr(block_table), _ptr(seq_lens),
                                  float(scale), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)),
           "mla_decode_partial")


def mla_decode_combine(desc, workspace, o_latent, lse_out=None, stream=None):
    _check_decode_buffers(desc, "mla_decode_combine", o_latent=o_latent, lse_out=lse_out)
    _check(lib.mla_decode_combine(ctypes.byref(desc), _ptr(_dev(workspace, "workspace")),
                                  workspace.numel() * workspace.element_size(),
                                  _ptr(_dev(o_latent, "o_latent")), _ptr(_dev(lse_out, "lse_out")),
                                  _stream(stream)), "mla_decode_combine")


def mla_decode_validate(desc, seq_lens, block_table, n_pages, stream=None):
    _check(lib.mla_decode_validate(ctypes.byref(desc), _ptr(seq_lens), _ptr(block_table),
                                   int(n_pages), _stream(stream)), "mla_decode_validate")


def mla_fold_query(W_UQ, W_UK, n_h, d_h, d_c, d_in, W_qabs, stream=None):
    w = "mla_fold_query"
    _need(W_UQ, 4 * n_h * d_h * d_in, "W_UQ", w)
    _need(W_UK, 4 * n_h * d_h * d_c, "W_UK", w)
    _need(W_qabs, 4 * n_h * d_c * d_in, "W_qabs", w)
    _check(lib.mla_fold_query(_ptr(W_UQ), _ptr(W_UK), n_h, d_h, d_c, d_in, _ptr(W_qabs),
                              _stream(stream)), "mla_fold_query")


def mla_fold_output(W_O, W_UV, n_h, d_h, d_c, d, W_ov, stream=None):
    w = "mla_fold_output"
    _need(W_O, 4 * d * n_h * d_h, "W_O", w)
    _need(W_UV, 4 * n_h * d_h * d_c, "W_UV", w)
    _need(W_ov, 4 * d * n_h * d_c, "W_ov", w)
    _check(lib.mla_fold_output(_ptr(W_O), _ptr(W_UV), n_h, d_h, d_c, d, _ptr(W_ov),
                               _stream(stream)), "mla_fold_output")


def mla_output_proj_workspace_size(T, n_h, d_c, d_h, d, mode):
    return lib.mla_output_proj_workspace_size(T, n_h, d_c, d_h, d, mode)


def mla_output_proj(o_latent, o_dtype, T, n_h, d_c, d_h, d, mode, W1, W2, out, workspace=None,
                    stream=None):
    w = "mla_output_proj"
    _need(o_latent, _ELEM.get(int(o_dtype), 4) * T * n_h * d_c, "o_latent", w)
    if int(mode) == MLA_PROJ_TWO_STAGE:
        _need(W1, 4 * n_h * d_h * d_c, "W1 (W_UV)", w)
        _need(W2, 4 * d * n_h * d_h, "W2 (W_O)", w)
    else:
        _need(W1, 4 * d * n_h * d_c, "W1 (W_ov)", w)
    _need(out, 4 * T * d, "out", w)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.mla_output_proj(_ptr(o_latent), o_dtype, T, n_h, d_c, d_h, d, mode, _ptr(W1),
                               _ptr(W2), _ptr(out), _ptr(workspace), nbytes, _stream(stream)),
           "mla_output_proj")


def mla_cache_write(rows, T, d_c, d_rope, theta, positions, slots, cache_dtype, cache,
                    cache_scale=None, stream=None):
    w = "mla_cache_write"
    _need(rows, 4 * T * (d_c + d_rope), "rows", w)
    _need(positions, 4 * T, "positions", w)
    _need(slots, 4 * T, "slots", w)
    _check(lib.mla_cache_write(_ptr(rows), T, d_c, d_rope, float(theta), _ptr(positions),
                               _ptr(slots), cache_dtype, _ptr(cache), _ptr(cache_scale),
                               _stream(stream)), "mla_cache_write")


def mla_cache_append_workspace_size(T, d, d_c, d_rope):
    return lib.mla_cache_append_workspace_size(T, d, d_c, d_rope)


def mla_cache_append(h, T, d, W_DKV, W_KR, d_c, d_rope, theta, positions, slots, cache_dtype,
                     cache, cache_scale, workspace, stream=None):
    w = "mla_cache_append"
    _need(h, 4 * T * d, "h", w)
    _need(W_DKV, 4 * d_c * d, "W_DKV", w)
    _need(W_KR, 4 * d_rope * d, "W_KR", w)
    _need(positions, 4 * T, "positions", w)
    _need(slots, 4 * T, "slots", w)
    _check(lib.mla_cache_append(_ptr(h), T, d, _ptr(W_DKV), _ptr(W_KR), d_c, d_rope,
                                float(theta), _ptr(positions), _ptr(slots), cache_dtype,
                                _ptr(cache), _ptr(cache_scale), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream)),
           "mla_cache_append")


def mla_absorb_query_workspace_size(T, d_in, n_h, d_c, d_rope):
    return lib.mla_absorb_query_workspace_size(T, d_in, n_h, d_c, d_rope)


def mla_absorb_query(x, T, d_in, W_qabs, W_QR, n_h, d_c, d_rope, theta, positions, q_dtype,
                     q_abs, q_rope, workspace, stream=None):
    w = "mla_absorb_query"
    qe = _ELEM.get(int(q_dtype), 4)
    _need(x, 4 * T * d_in, "x", w)
    _need(W_qabs, 4 * n_h * d_c * d_in, "W_qabs", w)
    _need(W_QR, 4 * n_h * d_rope * d_in, "W_QR", w)
    _need(positions, 4 * T, "positions", w)
    _need(q_abs, qe * T * n_h * d_c, "q_abs", w)
    _need(q_rope, qe * T * n_h * d_rope, "q_rope", w)
    _check(lib.mla_absorb_query(_ptr(x), T, d_in, _ptr(W_qabs), _ptr(W_QR), n_h, d_c, d_rope,
                                float(theta), _ptr(positions), q_dtype, _ptr(q_abs),
                                _ptr(q_rope), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream)),
           "mla_absorb_query")


def mla_gemm_bf16(A, B, C, splits=1, partial=None, stream=None):
    """C = A B^T for bf16 A [M, K], B [N, K] (row-major, possibly strided
    rows); C [M, N] fp32 or bf16."""
    for t, n in ((A, "A"), (B, "B"), (C, "C"), (partial, "partial")):
        if t is not None and not t.is_cuda:
            raise ValueError(f"{n} must be a GPU tensor")
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or tuple(C.shape) != (M, N) or A.stride(1) != 1 or B.stride(1) != 1 \
            or C.stride(1) != 1:
        raise ValueError("mla_gemm_bf16: shapes or layouts do not match")
    import torch
    cdt = MLA_BF16 if C.dtype == torch.bfloat16 else MLA_FP32
    _check(lib.mla_gemm_bf16(M, N, K, _ptr(A), A.stride(0), _ptr(B), B.stride(0), _ptr(C), C.stride(0),
                             cdt, splits, _ptr(partial), _stream(stream)), "mla_gemm_bf16")


def mla_gemm_bf16_partial_size(M, N, K, splits):
    return lib.mla_gemm_bf16_partial_size(M, N, K, splits)


def prefill_desc(batch, max_seq_len, d_model, n_heads, d_head, d_rope, d_c, d_cq=0,
                 rope_theta=10000.0) -> MlaPrefillDesc:
    return MlaPrefillDesc(batch, max_seq_len, d_model, n_heads, d_head, d_rope, d_c, d_cq,
                          float(rope_theta))


def mla_prefill_attention(desc, T, q, ldq, q_rope, ldqr, k, ldk, k_rope, ldkr, v, ldv, cu_seqlens,
                          scale, o, ldo, lse=None, stream=None):
    for t, n in ((q, "q"), (q_rope, "q_rope"), (k, "k"), (k_rope, "k_rope"), (v, "v"),
                 (cu_seqlens, "cu_seqlens"), (o, "o"), (lse, "lse")):
        if t is not None and not t.is_cuda:
            raise ValueError(f"{n} must be a GPU tensor")
    _check(lib.mla_prefill_attention(ctypes.byref(desc), int(T), _ptr(q), ldq, _ptr(q_rope), ldqr,
                                     _ptr(k), ldk, _ptr(k_rope), ldkr, _ptr(v), ldv, _ptr(cu_seqlens),
                                     float(scale), _ptr(o), ldo, _ptr(lse), _stream(stream)),
           "mla_prefill_attention")


def mla_prefill_workspace_size(desc, T):
    n = lib.mla_prefill_workspace_size(ctypes.byref(desc), int(T))
    if n == 0:
        raise MlaError(MLA_ERR_INVALID_ARGUMENT, "mla_prefill_workspace_size")
    return n


def mla_prefill(desc, h, cu_seqlens, positions, weights, scale, out, latent, lse, workspace,
                stream=None):
    """weights: dict with W_DKVR, W_DQ (or None), W_UQR, W_UKV, W_O (bf16 GPU tensors)."""
    T = h.shape[0]
    for t, n in ((h, "h"), (cu_seqlens, "cu_seqlens"), (positions, "positions"), (out, "out"),
                 (latent, "latent"), (lse, "lse"), (workspace, "workspace")):
        _dev(t, n)
    for n, t in weights.items():
        _dev(t, n)
    w = MlaPrefillWeights(*[None if weights.get(n) is None else weights[n].data_ptr()
                            for n in ("W_DKVR", "W_DQ", "W_UQR", "W_UKV", "W_O")])
    _need(out, T * int(desc.d_model) * 4, "out", "mla_prefill")
    _need(latent, T * (int(desc.d_c) + int(desc.d_rope)) * 4, "latent", "mla_prefill")
    _need(lse, T * int(desc.n_heads) * 4, "lse", "mla_prefill")
    _need(h, T * int(desc.d_model) * 2, "h", "mla_prefill")
    _check(lib.mla_prefill(ctypes.byref(desc), _ptr(h), T, _ptr(cu_seqlens), _ptr(positions),
                           ctypes.byref(w), float(scale), _ptr(out), _ptr(latent), _ptr(lse),
                           _ptr(workspace), _nbytes(workspace), _stream(stream)), "mla_prefill")


def mla_cache_bytes_per_token(d_c, d_rope, cache_dtype):
    return lib.mla_cache_bytes_per_token(d_c, d_rope, cache_dtype)


def mla_status_string(s):
    return lib.mla_status_string(s).decode()


def mla_last_error():
    return lib.mla_last_error().decode()


def mla_version():
    return lib.mla_version()
