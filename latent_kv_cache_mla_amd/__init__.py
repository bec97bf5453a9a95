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
    "mla_decode_combine": (_I, [_DESC, _P, _S, _P, _P, _P]),
    "mla_decode_validate": (_I, [_DESC, _P, _P, ctypes.c_int64, _P]),
    "mla_fold_query": (_I, [_P, _P, _I, _I, _I, _I, _P, _P]),
    "mla_fold_output": (_I, [_P, _P, _I, _I, _I, _I, _P, _P]),
    "mla_output_proj_workspace_size": (_S, [_I, _I, _I, _I]),
    "mla_output_proj": (_I, [_P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _S, _P]),
    "mla_cache_write": (_I, [_P, _I, _I, _I, ctypes.c_float, _P, _P, _I, _P, _P, _P]),
    "mla_cache_append_workspace_size": (_S, [_I, _I, _I]),
    "mla_cache_append": (_I, [_P, _I, _I, _P, _P, _I, _I, ctypes.c_float, _P, _P, _I, _P, _P,
                              _P, _S, _P]),
    "mla_absorb_query_workspace_size": (_S, [_I, _I, _I, _I]),
    "mla_absorb_query": (_I, [_P, _I, _I, _P, _P, _I, _I, _I, ctypes.c_float, _P, _I, _P, _P,
                              _P, _S, _P]),
    "mla_cache_bytes_per_token": (_S, [_I, _I, _I]),
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
    _check(lib.mla_decode_plan(ctypes.byref(desc), _ptr(_dev(seq_lens, "seq_lens")),
                               _ptr(_dev(workspace, "workspace")), workspace.numel() * workspace.element_size(),
                               _stream(stream)), "mla_decode_plan")


def mla_decode(desc, q_abs, q_rope, cache, cache_scale, block_table, seq_lens, scale,
               o_latent, lse_out, workspace, stream=None):
    for t, n in ((q_abs, "q_abs"), (q_rope, "q_rope"), (cache, "cache"), (cache_scale, "cache_scale"),
                 (block_table, "block_table"), (seq_lens, "seq_lens"), (o_latent, "o_latent"),
                 (lse_out, "lse_out"), (workspace, "workspace")):
        _dev(t, n)
    _check(lib.mla_decode(ctypes.byref(desc), _ptr(q_abs), _ptr(q_rope), _ptr(cache),
                          _ptr(cache_scale), _ptr(block_table), _ptr(seq_lens), float(scale),
                          _ptr(o_latent), _ptr(lse_out), _ptr(workspace),
                          workspace.numel() * workspace.element_size(), _stream(stream)),
           "mla_decode")


def mla_decode_partial(desc, q_abs, q_rope, cache, cache_scale, block_table, seq_lens, scale,
                       workspace, stream=None):
    for t, n in ((q_abs, "q_abs"), (q_rope, "q_rope"), (cache, "cache"), (cache_scale, "cache_scale"),
                 (block_table, "block_table"), (seq_lens, "seq_lens"), (workspace, "workspace")):
        _dev(t, n)
    _check(lib.mla_decode_partial(ctypes.byref(desc), _ptr(q_abs), _ptr(q_rope), _ptr(cache),
                                  _ptr(cache_scale), _ptr(block_table), _ptr(seq_lens),
                                  float(scale), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)),
           "mla_decode_partial")


def mla_decode_combine(desc, workspace, o_latent, lse_out=None, stream=None):
    _check(lib.mla_decode_combine(ctypes.byref(desc), _ptr(_dev(workspace, "workspace")),
                                  workspace.numel() * workspace.element_size(),
                                  _ptr(_dev(o_latent, "o_latent")), _ptr(_dev(lse_out, "lse_out")),
                                  _stream(stream)), "mla_decode_combine")


def mla_decode_validate(desc, seq_lens, block_table, n_pages, stream=None):
    _check(lib.mla_decode_validate(ctypes.byref(desc), _ptr(seq_lens), _ptr(block_table),
                                   int(n_pages), _stream(stream)), "mla_decode_validate")


def mla_fold_query(W_UQ, W_UK, n_h, d_h, d_c, d_in, W_qabs, stream=None):
    _check(lib.mla_fold_query(_ptr(W_UQ), _ptr(W_UK), n_h, d_h, d_c, d_in, _ptr(W_qabs),
                              _stream(stream)), "mla_fold_query")


def mla_fold_output(W_O, W_UV, n_h, d_h, d_c, d, W_ov, stream=None):
    _check(lib.mla_fold_output(_ptr(W_O), _ptr(W_UV), n_h, d_h, d_c, d, _ptr(W_ov),
                               _stream(stream)), "mla_fold_output")


def mla_output_proj_workspace_size(T, n_h, d_h, mode):
    return lib.mla_output_proj_workspace_size(T, n_h, d_h, mode)


def mla_output_proj(o_latent, o_dtype, T, n_h, d_c, d_h, d, mode, W1, W2, out, workspace=None,
                    stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.mla_output_proj(_ptr(o_latent), o_dtype, T, n_h, d_c, d_h, d, mode, _ptr(W1),
                               _ptr(W2), _ptr(out), _ptr(workspace), nbytes, _stream(stream)),
           "mla_output_proj")


def mla_cache_write(rows, T, d_c, d_rope, theta, positions, slots, cache_dtype, cache,
                    cache_scale=None, stream=None):
    _check(lib.mla_cache_write(_ptr(rows), T, d_c, d_rope, float(theta), _ptr(positions),
                               _ptr(slots), cache_dtype, _ptr(cache), _ptr(cache_scale),
                               _stream(stream)), "mla_cache_write")


def mla_cache_append_workspace_size(T, d_c, d_rope):
    return lib.mla_cache_append_workspace_size(T, d_c, d_rope)


def mla_cache_append(h, T, d, W_DKV, W_KR, d_c, d_rope, theta, positions, slots, cache_dtype,
                     cache, cache_scale, workspace, stream=None):
    _check(lib.mla_cache_append(_ptr(h), T, d, _ptr(W_DKV), _ptr(W_KR), d_c, d_rope,
                                float(theta), _ptr(positions), _ptr(slots), cache_dtype,
                                _ptr(cache), _ptr(cache_scale), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream)),
           "mla_cache_append")


def mla_absorb_query_workspace_size(T, n_h, d_c, d_rope):
    return lib.mla_absorb_query_workspace_size(T, n_h, d_c, d_rope)


def mla_absorb_query(x, T, d_in, W_qabs, W_QR, n_h, d_c, d_rope, theta, positions, q_dtype,
                     q_abs, q_rope, workspace, stream=None):
    _check(lib.mla_absorb_query(_ptr(x), T, d_in, _ptr(W_qabs), _ptr(W_QR), n_h, d_c, d_rope,
                                float(theta), _ptr(positions), q_dtype, _ptr(q_abs),
                                _ptr(q_rope), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream)),
           "mla_absorb_query")


def mla_cache_bytes_per_token(d_c, d_rope, cache_dtype):
    return lib.mla_cache_bytes_per_token(d_c, d_rope, cache_dtype)


def mla_status_string(s):
    return lib.mla_status_string(s).decode()


def mla_last_error():
    return lib.mla_last_error().decode()


def mla_version():
    return lib.mla_version()
