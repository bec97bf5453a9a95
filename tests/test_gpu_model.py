"""The steps around the decode kernel, through the C ABI, against the oracle:
offline folds, absorbed query projection, cache append (fp32, bf16, fp8),
output projection (merged and two-stage), and the tiny model end to end
against the unabsorbed definition."""
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


@pytest.mark.parametrize("shape", [(8, 64, 64, 512, 512), (16, 128, 512, 1536, 1024)])
def test_folds(shape):
    m = H.lib()
    nh, dh, dc, din, d = shape
    H.say(f"case folds n_h={nh} d_h={dh} d_c={dc} d_in={din} d={d}")
    rng = np.random.default_rng(21)
    W_UQ = (rng.standard_normal((nh * dh, din)) * 0.02).astype(np.float32)
    W_UK = (rng.standard_normal((nh * dh, dc)) * 0.02).astype(np.float32)
    W_UV = (rng.standard_normal((nh * dh, dc)) * 0.02).astype(np.float32)
    W_O = (rng.standard_normal((d, nh * dh)) * 0.02).astype(np.float32)
    A = torch.empty((nh, dc, din), dtype=torch.float32, device="cuda")
    F = torch.empty((d, nh * dc), dtype=torch.float32, device="cuda")
    m.mla_fold_query(_t(W_UQ), _t(W_UK), nh, dh, dc, din, A)
    m.mla_fold_output(_t(W_O), _t(W_UV), nh, dh, dc, d, F)
    torch.cuda.synchronize()
    ra = oracle.fold_query(W_UQ, W_UK, nh, dh)
    rf = oracle.fold_output(W_O, W_UV, nh, dh)
    ea, ef = _rel(A.cpu().numpy(), ra), _rel(F.cpu().numpy(), rf)
    H.say(f"  fold_query rel {ea:.2e}, fold_output rel {ef:.2e}")
    assert ea < 1e-5 and ef < 1e-5


@pytest.mark.parametrize("q_dtype", ["fp32", "bf16"])
def test_absorb_query(q_dtype):
    m = H.lib()
    nh, dc, dr, din, T = 16, 512, 64, 384, 5
    H.say(f"case absorb_query {q_dtype}")
    rng = np.random.default_rng(22)
    W_qabs = (rng.standard_normal((nh, dc, din)) * 0.05).astype(np.float32)
    W_QR = (rng.standard_normal((nh * dr, din)) * 0.05).astype(np.float32)
    x = rng.standard_normal((T, din)).astype(np.float32)
    pos = np.array([0, 1, 777, 4095, 32767], dtype=np.int32)
    code = m.DTYPE_CODES[q_dtype]
    dt = torch.float32 if q_dtype == "fp32" else torch.bfloat16
    qa = torch.empty((T, nh, dc), dtype=dt, device="cuda")
    qr = torch.empty((T, nh, dr), dtype=dt, device="cuda")
    ws = torch.empty(m.mla_absorb_query_workspace_size(T, din, nh, dc, dr), dtype=torch.uint8, device="cuda")
    m.mla_absorb_query(_t(x), T, din, _t(W_qabs), _t(W_QR), nh, dc, dr, 10000.0,
                       torch.from_numpy(pos).cuda(), code, qa, qr, ws)
    torch.cuda.synchronize()
    ra, rr = oracle.absorb_query(W_qabs, W_QR, x, pos, 10000.0)
    ea, er = _rel(qa.float().cpu().numpy(), ra), _rel(qr.float().cpu().numpy(), rr)
    H.say(f"  q_abs rel {ea:.2e}, q_rope rel {er:.2e}")
    tol = 1e-5 if q_dtype == "fp32" else 4e-3
    assert ea < tol and er < tol


@pytest.mark.parametrize("cache_dtype", ["fp32", "bf16", "fp8"])
def test_cache_write_rows(cache_dtype):
    """Given projected rows: RoPE, quantisation and scatter through the slots."""
    m = H.lib()
    dc, dr, T = 512, 64, 70
    H.say(f"case cache_write {cache_dtype}")
    rng = np.random.default_rng(23)
    rows = (rng.standard_normal((T, dc + dr)) / 24).astype(np.float32)
    rows[3, :dc] = 0.0                                   # a zero latent: scale 1, codes 0
    pos = rng.integers(0, 30000, T).astype(np.int32)
    n_pages = 4
    slots = rng.permutation(n_pages * 64)[:T].astype(np.int32)
    slots[5] = -1                                        # skipped token
    code = m.DTYPE_CODES[cache_dtype]
    if cache_dtype == "fp8":
        cache = torch.zeros((n_pages, 64, dc + 2 * dr), dtype=torch.uint8, device="cuda")
        sc = torch.zeros((n_pages, 64), dtype=torch.float32, device="cuda")
    else:
        dt = torch.float32 if cache_dtype == "fp32" else torch.bfloat16
        cache = torch.zeros((n_pages, 64, dc + dr), dtype=dt, device="cuda")
        sc = None
    m.mla_cache_write(_t(rows), T, dc, dr, 10000.0, torch.from_numpy(pos).cuda(),
                      torch.from_numpy(slots).cuda(), code, cache, sc)
    torch.cuda.synchronize()
    kr_ref = oracle.rope(rows[:, dc:].astype(np.float64), pos, 10000.0)
    flat = cache.view(n_pages * 64, -1).cpu()
    keep = slots >= 0
    if cache_dtype == "fp8":
        codes_ref, s_ref = oracle.fp8_quantize_tokens(rows[:, :dc])
        got = flat.numpy()[slots[keep]]
        assert np.array_equal(got[:, :dc], codes_ref[keep])          # bit-exact codes
        assert np.array_equal(sc.view(-1).cpu().numpy()[slots[keep]], s_ref[keep])
        kr = oracle.bf16_bits_to_f64(got[:, dc:].copy().view(np.uint16))
    else:
        got = flat.float().numpy()[slots[keep]]
        c_tol = 0 if cache_dtype == "fp32" else 2.0 ** -8
        assert np.all(np.abs(got[:, :dc] - rows[keep, :dc]) <= c_tol * np.abs(rows[keep, :dc]))
        kr = got[:, dc:]
    err = np.abs(kr - kr_ref[keep])
    tol = (1e-6 if cache_dtype == "fp32" else 2.0 ** -8) * np.abs(kr_ref[keep]) + 1e-6
    H.say(f"  rope key max err {err.max():.2e}")
    assert np.all(err <= tol)
    # untouched slots stay zero (the skipped token wrote nothing)
    others = np.setdiff1d(np.arange(n_pages * 64), slots[keep])
    assert np.all(flat.float().numpy()[others] == 0)


def _tiny_chain(cfg, cache_dtype, mode):
    """fold -> absorbed queries -> cache append -> decode -> projection, GPU."""
    m = H.lib()
    model = wl.make_tiny_model(cfg)
    nh, dh, dc, dr, d = cfg.n_heads, cfg.d_head, cfg.d_c, cfg.d_rope, cfg.d_model
    S = model.H.shape[0]
    A = torch.empty((nh, dc, d), dtype=torch.float32, device="cuda")
    m.mla_fold_query(_t(model.W_UQ), _t(model.W_UK), nh, dh, dc, d, A)
    q_dt = "fp32" if cache_dtype == "fp32" else "bf16"
    qdt = torch.float32 if q_dt == "fp32" else torch.bfloat16
    qa = torch.empty((1, 1, nh, dc), dtype=qdt, device="cuda")
    qr = torch.empty((1, 1, nh, dr), dtype=qdt, device="cuda")
    ws = torch.empty(m.mla_absorb_query_workspace_size(1, d, nh, dc, dr), dtype=torch.uint8, device="cuda")
    pos_q = torch.tensor([S - 1], dtype=torch.int32, device="cuda")
    m.mla_absorb_query(_t(model.H[S - 1:]), 1, d, A, _t(model.W_QR), nh, dc, dr, cfg.rope_theta,
                       pos_q, m.DTYPE_CODES[q_dt], qa, qr, ws)
    n_pages = wl.pages_for(S)
    if cache_dtype == "fp8":
        cache = torch.zeros((n_pages, 64, dc + 2 * dr), dtype=torch.uint8, device="cuda")
        sc = torch.ones((n_pages, 64), dtype=torch.float32, device="cuda")
    else:
        cache = torch.zeros((n_pages, 64, dc + dr), dtype=qdt, device="cuda")
        sc = None
    pos = torch.arange(S, dtype=torch.int32, device="cuda")
    wa = torch.empty(m.mla_cache_append_workspace_size(S, d, dc, dr), dtype=torch.uint8, device="cuda")
    m.mla_cache_append(_t(model.H), S, d, _t(model.W_DKV), _t(model.W_KR), dc, dr, cfg.rope_theta,
                       pos, pos, m.DTYPE_CODES[cache_dtype], cache, sc, wa)
    desc = m.decode_desc(1, 1, nh, dc, dr, n_pages, cache_dtype, q_dt, "fp32")
    wsd = torch.empty(m.mla_decode_workspace_size(desc), dtype=torch.uint8, device="cuda")
    o = torch.empty((1, 1, nh, dc), dtype=torch.float32, device="cuda")
    bt = torch.arange(n_pages, dtype=torch.int32, device="cuda").view(1, -1)
    sl = torch.tensor([S], dtype=torch.int32, device="cuda")
    m.mla_decode(desc, qa, qr, cache, sc, bt, sl, cfg.softmax_scale, o, None, wsd)
    out = torch.empty((1, d), dtype=torch.float32, device="cuda")
    wp = torch.empty(m.mla_output_proj_workspace_size(1, nh, dc, dh, d, mode), dtype=torch.uint8,
                     device="cuda")
    if mode == m.MLA_PROJ_MERGED:
        F = torch.empty((d, nh * dc), dtype=torch.float32, device="cuda")
        m.mla_fold_output(_t(model.W_O), _t(model.W_UV), nh, dh, dc, d, F)
        m.mla_output_proj(o, m.MLA_FP32, 1, nh, dc, dh, d, mode, F, None, out, wp)
    else:
        m.mla_output_proj(o, m.MLA_FP32, 1, nh, dc, dh, d, mode, _t(model.W_UV), _t(model.W_O), out, wp)
    torch.cuda.synchronize()
    return model, o.cpu().numpy().astype(np.float64), out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("mode", [0, 1])
def test_tiny_model_end_to_end_fp32(mode):
    cfg = wl.CONFIGS["tiny"]
    H.say(f"case tiny end-to-end fp32 mode={mode}")
    model, o, out = _tiny_chain(cfg, "fp32", mode)
    r1 = oracle.mla_unabsorbed(model)
    r2 = oracle.mla_absorbed(model)
    eo, eout = _rel(o[0], r2["o_latent"]), _rel(out, r1["out"])
    H.say(f"  o_latent rel {eo:.2e}, out vs unabsorbed rel {eout:.2e}")
    H.assert_close(out, r1["out"], "fp32", "tiny-out")
    assert eo < 1e-5 and eout < 1e-5


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8"])
def test_tiny_model_end_to_end_quantised_cache(cache_dtype):
    # the tiny model with the DeepSeek head shapes' storage formats: the
    # result must stay within the gate of the corresponding cache dtype
    cfg = wl.scaled(wl.CONFIGS["tiny"], seq_len=200)
    H.say(f"case tiny end-to-end {cache_dtype}")
    model, o, out = _tiny_chain(cfg, cache_dtype, 1)
    r1 = oracle.mla_unabsorbed(model)
    H.assert_close(out, r1["out"], cache_dtype, f"tiny-out-{cache_dtype}")


# ----------------------------------------------------------------------------
# the per-step projections at DeepSeek-V2 widths (32 decode tokens)
# ----------------------------------------------------------------------------

DS = dict(T=32, d=5120, d_in=1536, nh=128, dc=512, dh=128, dr=64)


def test_absorbed_query_projection_at_deepseek_widths():
    """q_abs_i = W_qabs_i x and q^R_i = RoPE(W^QR_i x) for 32 tokens with the
    query latent of 1536 ([LLMsBlog] "Query Key Absorption"): W_qabs holds
    128 x 512 x 1536 fp32 weights (403 MB), streamed once."""
    m = H.lib()
    T, din, nh, dc, dr = DS["T"], DS["d_in"], DS["nh"], DS["dc"], DS["dr"]
    H.say(f"case absorb_query DeepSeek T={T} d_in={din} n_h={nh}")
    rng = np.random.default_rng(31)
    W_qabs = (rng.standard_normal((nh, dc, din), dtype=np.float32) * 0.02)
    W_QR = (rng.standard_normal((nh * dr, din), dtype=np.float32) * 0.02)
    x = rng.standard_normal((T, din), dtype=np.float32)
    pos = rng.integers(0, 32768, T).astype(np.int32)
    qa = torch.empty((T, nh, dc), dtype=torch.float32, device="cuda")
    qr = torch.empty((T, nh, dr), dtype=torch.float32, device="cuda")
    ws = torch.empty(m.mla_absorb_query_workspace_size(T, din, nh, dc, dr), dtype=torch.uint8, device="cuda")
    m.mla_absorb_query(_t(x), T, din, _t(W_qabs), _t(W_QR), nh, dc, dr, 10000.0,
                       torch.from_numpy(pos).cuda(), m.MLA_FP32, qa, qr, ws)
    torch.cuda.synchronize()
    ra, rr = oracle.absorb_query(W_qabs, W_QR, x, pos, 10000.0)
    ea, er = _rel(qa.cpu().numpy(), ra), _rel(qr.cpu().numpy(), rr)
    H.say(f"  q_abs rel {ea:.2e}, q_rope rel {er:.2e}")
    assert ea < 1e-5 and er < 1e-5


@pytest.mark.parametrize("mode", [0, 1])
def test_output_projection_at_deepseek_widths(mode):
    """out = W_ov concat_i(o_i) (merged: 5120 x 65536 fp32 = 1.34 GB of
    weights) or W^O concat_i(W^UV_i o_i) (two-stage) for 32 tokens ([Zhang]
    "Value absorption: weight and sum first, project after")."""
    m = H.lib()
    T, d, nh, dc, dh = DS["T"], DS["d"], DS["nh"], DS["dc"], DS["dh"]
    H.say(f"case output_proj DeepSeek mode={mode} T={T} d={d}")
    rng = np.random.default_rng(32 + mode)
    o = rng.standard_normal((T, nh, dc), dtype=np.float32) * 0.05
    if mode == 0:
        W_ov = rng.standard_normal((d, nh * dc), dtype=np.float32) * 0.02
        ref = oracle.output_projection_merged(o, W_ov)
        W1, W2 = _t(W_ov), None
    else:
        W_UV = rng.standard_normal((nh * dh, dc), dtype=np.float32) * 0.02
        W_O = rng.standard_normal((d, nh * dh), dtype=np.float32) * 0.02
        ref = oracle.output_projection_two_stage(o, W_UV, W_O, nh, dh)
        W1, W2 = _t(W_UV), _t(W_O)
    out = torch.empty((T, d), dtype=torch.float32, device="cuda")
    wp = torch.empty(m.mla_output_proj_workspace_size(T, nh, dc, dh, d, mode), dtype=torch.uint8,
                     device="cuda")
    m.mla_output_proj(_t(o), m.MLA_FP32, T, nh, dc, dh, d, mode, W1, W2, out, wp)
    torch.cuda.synchronize()
    e = _rel(out.cpu().numpy(), ref)
    H.say(f"  rel {e:.2e}")
    assert e < 1e-5


def test_cache_append_at_deepseek_widths():
    """c = W^DKV h and k^R = RoPE(W^KR h) for 32 tokens of d 5120 ([Mishra]
    "Step 1: a low-rank latent"), stored in an fp32 cache."""
    m = H.lib()
    T, d, dc, dr = DS["T"], DS["d"], DS["dc"], DS["dr"]
    H.say(f"case cache_append DeepSeek T={T} d={d}")
    rng = np.random.default_rng(34)
    h = rng.standard_normal((T, d), dtype=np.float32)
    W_DKV = rng.standard_normal((dc, d), dtype=np.float32) * 0.02
    W_KR = rng.standard_normal((dr, d), dtype=np.float32) * 0.02
    pos = rng.integers(0, 32768, T).astype(np.int32)
    slots = np.arange(T, dtype=np.int32)[::-1].copy()       # rows land in reverse order
    cache = torch.zeros((1, 64, dc + dr), dtype=torch.float32, device="cuda")
    ws = torch.empty(m.mla_cache_append_workspace_size(T, d, dc, dr), dtype=torch.uint8, device="cuda")
    m.mla_cache_append(_t(h), T, d, _t(W_DKV), _t(W_KR), dc, dr, 10000.0,
                       torch.from_numpy(pos).cuda(), torch.from_numpy(slots).cuda(), m.MLA_FP32,
                       cache, None, ws)
    torch.cuda.synchronize()
    c, kR = oracle.cache_append(W_DKV, W_KR, h, pos, 10000.0)
    g = cache.cpu().numpy()[0]
    ec, ek = _rel(g[slots, :dc], c), _rel(g[slots, dc:], kR)
    H.say(f"  c rel {ec:.2e}, k^R rel {ek:.2e}")
    assert ec < 1e-5 and ek < 1e-5


@pytest.mark.parametrize("T,nh,dc,d,o_dtype,offset", [
    (5, 3, 20, 130, "fp32", 0),    # K = 60: a partial last 32-k stage; 130 outputs: a ragged tile
    (33, 2, 44, 260, "bf16", 0),   # 33 rows: two row blocks, the second of one row; bf16 rows, 4 at a time
    (7, 3, 20, 128, "bf16", 2),    # activation rows 4-byte aligned only: bf16 loaded element by element
    (5, 6, 134, 130, "fp32", 0),   # K = 804 in 7 splits, the last ending 4 k into a stage; split sums element-wise
    (5, 6, 134, 256, "bf16", 0),   # the same with split sums 4 outputs per thread
    (4, 2, 21, 64, "fp32", 0),     # K = 42, not a multiple of 4: the vector-ALU GEMM
    (257, 1, 64, 64, "fp32", 0),   # more than 256 rows: the vector-ALU GEMM
])
def test_output_projection_edge_shapes(T, nh, dc, d, o_dtype, offset):
    """The merged output projection on shapes at the edges of the skinny
    matrix-core GEMM's fast paths (partial stages, ragged row and output
    tiles, unaligned bf16 activations) and of its fallback, against the oracle.
    bf16 activations are compared with the oracle on the same rounded values."""
    m = H.lib()
    H.say(f"case output_proj edges T={T} n_h={nh} d_c={dc} d={d} {o_dtype} offset={offset}")
    rng = np.random.default_rng(40 + T + dc)
    o = (rng.standard_normal((T, nh, dc)) * 0.05).astype(np.float32)
    W = (rng.standard_normal((d, nh * dc)) * 0.02).astype(np.float32)
    if o_dtype == "bf16":
        o = wl.bf16_round(o)
        flat = torch.zeros(T * nh * dc + offset, dtype=torch.bfloat16, device="cuda")
        flat[offset:] = torch.from_numpy(o.reshape(-1)).to(torch.bfloat16).cuda()
        og = flat[offset:]
    else:
        og = _t(o)
    ref = oracle.output_projection_merged(o.astype(np.float64), W)
    out = torch.empty((T, d), dtype=torch.float32, device="cuda")
    wp = torch.empty(max(m.mla_output_proj_workspace_size(T, nh, dc, 0, d, 0), 256), dtype=torch.uint8,
                     device="cuda")
    m.mla_output_proj(og, m.DTYPE_CODES[o_dtype], T, nh, dc, 0, d, 0, _t(W), None, out, wp)
    torch.cuda.synchronize()
    e = _rel(out.cpu().numpy(), ref)
    H.say(f"  rel {e:.2e}")
    assert np.all(np.isfinite(out.cpu().numpy()))
    assert e < 1e-5


@pytest.mark.parametrize("T,nh,dc,dr,din", [(3, 2, 64, 16, 100), (40, 4, 128, 32, 260)])
def test_absorb_query_edge_shapes(T, nh, dc, dr, din):
    """The absorbed query as one GEMM over W_qabs and W_QR (the second matrix's
    columns start at n_h d_c, a multiple of 128) with a K that ends inside a
    32-k stage and row counts that are not multiples of 32."""
    m = H.lib()
    H.say(f"case absorb_query edges T={T} n_h={nh} d_c={dc} d_R={dr} d_in={din}")
    rng = np.random.default_rng(50 + T)
    W_qabs = (rng.standard_normal((nh, dc, din)) * 0.05).astype(np.float32)
    W_QR = (rng.standard_normal((nh * dr, din)) * 0.05).astype(np.float32)
    x = rng.standard_normal((T, din)).astype(np.float32)
    pos = rng.integers(0, 32768, T).astype(np.int32)
    qa = torch.empty((T, nh, dc), dtype=torch.float32, device="cuda")
    qr = torch.empty((T, nh, dr), dtype=torch.float32, device="cuda")
    ws = torch.empty(m.mla_absorb_query_workspace_size(T, din, nh, dc, dr), dtype=torch.uint8, device="cuda")
    m.mla_absorb_query(_t(x), T, din, _t(W_qabs), _t(W_QR), nh, dc, dr, 10000.0,
                       torch.from_numpy(pos).cuda(), m.MLA_FP32, qa, qr, ws)
    torch.cuda.synchronize()
    ra, rr = oracle.absorb_query(W_qabs, W_QR, x, pos, 10000.0)
    ea, er = _rel(qa.cpu().numpy(), ra), _rel(qr.cpu().numpy(), rr)
    H.say(f"  q_abs rel {ea:.2e}, q_rope rel {er:.2e}")
    assert ea < 1e-5 and er < 1e-5
