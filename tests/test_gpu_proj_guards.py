"""Guard tests of the projection and cache-write entry points (through the C
ABI): every output, the workspace and the cache pool sit between guard regions
of a byte pattern, and the shapes are those at the edges of the kernels' fast
paths (partial 32-k stages, ragged row and output tiles, split-K partials in
the workspace, the vector-ALU fallback). The outputs start as NaN and must be
overwritten completely and agree with the oracle; the cache pool starts as
zeros and only the named slots may change; no guard byte may change.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _rel(g, r):
    return float(np.linalg.norm(np.asarray(g, np.float64) - r) / np.linalg.norm(r))


Guarded = H.Guarded


def _workspace(nbytes):
    return Guarded((max(int(nbytes), 1),), torch.uint8)


@pytest.mark.parametrize("T,nh,dc,dh,d,mode,o_dtype", [
    (5, 6, 134, 0, 130, 0, "fp32"),    # K = 804 in splits, element-wise split sums
    (5, 6, 134, 0, 256, 0, "bf16"),    # split sums 4 outputs per thread
    (33, 2, 44, 0, 260, 0, "bf16"),    # two row blocks, the second of one row; ragged output tile
    (4, 2, 21, 0, 64, 0, "fp32"),      # K not a multiple of 4: the vector-ALU GEMM
    (257, 1, 64, 0, 64, 0, "fp32"),    # more than 256 rows: the vector-ALU GEMM
    (5, 3, 64, 40, 130, 1, "fp32"),    # two-stage: per-head W^UV, then W^O over n_h d_h = 120
    (33, 4, 96, 64, 520, 1, "fp32"),   # two-stage with two row blocks and a ragged output tile
])
def test_output_projection_writes_only_its_output(T, nh, dc, dh, d, mode, o_dtype):
    m = H.lib()
    H.say(f"case guards output_proj T={T} n_h={nh} d_c={dc} d_h={dh} d={d} mode={mode} {o_dtype}")
    rng = np.random.default_rng(60 + T + dc + mode)
    o = (rng.standard_normal((T, nh, dc)) * 0.05).astype(np.float32)
    if o_dtype == "bf16":
        o = wl.bf16_round(o)
        og = torch.from_numpy(o).to(torch.bfloat16).cuda()
    else:
        og = _t(o)
    if mode == 0:
        W = (rng.standard_normal((d, nh * dc)) * 0.02).astype(np.float32)
        ref = oracle.output_projection_merged(o.astype(np.float64), W)
        W1, W2 = _t(W), None
    else:
        W_UV = (rng.standard_normal((nh * dh, dc)) * 0.02).astype(np.float32)
        W_O = (rng.standard_normal((d, nh * dh)) * 0.02).astype(np.float32)
        ref = oracle.output_projection_two_stage(o.astype(np.float64), W_UV, W_O, nh, dh)
        W1, W2 = _t(W_UV), _t(W_O)
    out = Guarded((T, d), torch.float32)
    ws = _workspace(m.mla_output_proj_workspace_size(T, nh, dc, dh, d, mode))
    m.mla_output_proj(og, m.DTYPE_CODES[o_dtype], T, nh, dc, dh, d, mode, W1, W2, out.t, ws.t)
    torch.cuda.synchronize()
    assert out.guards_intact(), "a store landed outside the output"
    assert ws.guards_intact(), "a store landed outside the workspace"
    g = out.t.cpu().numpy()
    assert np.all(np.isfinite(g)), "an output was not written"
    e = _rel(g, ref)
    H.say(f"  rel {e:.2e}")
    assert e < 1e-5


@pytest.mark.parametrize("T,nh,dc,dr,din,q_dtype", [
    (3, 2, 64, 16, 100, "fp32"),
    (40, 4, 128, 32, 260, "fp32"),
    (40, 4, 128, 32, 260, "bf16"),
    (5, 16, 512, 64, 384, "bf16"),
])
def test_absorb_query_writes_only_its_outputs(T, nh, dc, dr, din, q_dtype):
    m = H.lib()
    H.say(f"case guards absorb_query T={T} n_h={nh} d_c={dc} d_R={dr} d_in={din} {q_dtype}")
    rng = np.random.default_rng(70 + T + din)
    W_qabs = (rng.standard_normal((nh, dc, din)) * 0.05).astype(np.float32)
    W_QR = (rng.standard_normal((nh * dr, din)) * 0.05).astype(np.float32)
    x = rng.standard_normal((T, din)).astype(np.float32)
    pos = rng.integers(0, 32768, T).astype(np.int32)
    dt = torch.float32 if q_dtype == "fp32" else torch.bfloat16
    qa = Guarded((T, nh, dc), dt)
    qr = Guarded((T, nh, dr), dt)
    ws = _workspace(m.mla_absorb_query_workspace_size(T, din, nh, dc, dr))
    m.mla_absorb_query(_t(x), T, din, _t(W_qabs), _t(W_QR), nh, dc, dr, 10000.0,
                       torch.from_numpy(pos).cuda(), m.DTYPE_CODES[q_dtype], qa.t, qr.t, ws.t)
    torch.cuda.synchronize()
    for buf, name in ((qa, "q_abs"), (qr, "q_rope"), (ws, "workspace")):
        assert buf.guards_intact(), f"a store landed outside {name}"
    ga, gr = qa.t.float().cpu().numpy(), qr.t.float().cpu().numpy()
    assert np.all(np.isfinite(ga)) and np.all(np.isfinite(gr)), "an output was not written"
    ra, rr = oracle.absorb_query(W_qabs, W_QR, x, pos, 10000.0)
    ea, er = _rel(ga, ra), _rel(gr, rr)
    H.say(f"  q_abs rel {ea:.2e}, q_rope rel {er:.2e}")
    tol = 1e-5 if q_dtype == "fp32" else 4e-3
    assert ea < tol and er < tol


@pytest.mark.parametrize("cache_dtype", ["fp32", "bf16", "fp8"])
def test_cache_append_writes_only_its_slots(cache_dtype):
    """The cache append (projection, RoPE, quantisation, scatter) into a pool
    of four pages whose first and last slots are among those named, with one
    skipped token: only the named slots change."""
    m = H.lib()
    T, d, dc, dr, n_pages = 70, 200, 512, 64, 4
    H.say(f"case guards cache_append {cache_dtype} T={T} d={d}")
    rng = np.random.default_rng(80)
    h = rng.standard_normal((T, d)).astype(np.float32)
    W_DKV = (rng.standard_normal((dc, d)) * 0.02).astype(np.float32)
    W_KR = (rng.standard_normal((dr, d)) * 0.02).astype(np.float32)
    pos = rng.integers(0, 32768, T).astype(np.int32)
    slots = rng.permutation(np.arange(1, n_pages * 64 - 1))[:T].astype(np.int32)
    slots[0], slots[1] = 0, n_pages * 64 - 1                # the pool's first and last slots
    slots[7] = -1                                            # a skipped token
    if cache_dtype == "fp8":
        cache = Guarded((n_pages, 64, dc + 2 * dr), torch.uint8, fill=0)
        sc = Guarded((n_pages, 64), torch.float32, fill=0)
    else:
        dt = torch.float32 if cache_dtype == "fp32" else torch.bfloat16
        cache = Guarded((n_pages, 64, dc + dr), dt, fill=0)
        sc = None
    ws = _workspace(m.mla_cache_append_workspace_size(T, d, dc, dr))
    m.mla_cache_append(_t(h), T, d, _t(W_DKV), _t(W_KR), dc, dr, 10000.0,
                       torch.from_numpy(pos).cuda(), torch.from_numpy(slots).cuda(),
                       m.DTYPE_CODES[cache_dtype], cache.t, None if sc is None else sc.t, ws.t)
    torch.cuda.synchronize()
    for buf, name in ((cache, "the cache pool"), (sc, "the scales"), (ws, "the workspace")):
        assert buf is None or buf.guards_intact(), f"a store landed outside {name}"
    keep = slots >= 0
    flat = cache.t.view(n_pages * 64, -1).cpu()
    raw = flat.view(torch.uint8).numpy() if cache_dtype != "fp8" else flat.numpy()
    others = np.setdiff1d(np.arange(n_pages * 64), slots[keep])
    assert np.all(raw[others] == 0), "a slot that no token names was written"
    if sc is not None:
        assert np.all(sc.t.view(-1).cpu().numpy()[others] == 0), "a scale that no token names was written"
    c_ref, kr_ref = oracle.cache_append(W_DKV, W_KR, h, pos, 10000.0)
    if cache_dtype == "fp8":
        got = flat.numpy()[slots[keep]]
        c = oracle.fp8_cache_dequant(got[:, :dc], sc.t.view(-1).cpu().numpy()[slots[keep]])
        kr = oracle.bf16_bits_to_f64(got[:, dc:].copy().view(np.uint16))
        c_tol = 2.0 ** -4   # e4m3 to nearest: at most 2^-4 of a normal value
    else:
        got = flat.float().numpy()[slots[keep]]
        c, kr = got[:, :dc], got[:, dc:]
        c_tol = 1e-5 if cache_dtype == "fp32" else 2.0 ** -8
    ec, ek = _rel(c, c_ref[keep]), _rel(kr, kr_ref[keep])
    H.say(f"  c rel {ec:.2e}, k^R rel {ek:.2e}")
    assert ec < c_tol and ek < (1e-5 if cache_dtype == "fp32" else 2.0 ** -8)
