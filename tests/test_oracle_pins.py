"""Pins of the CPU oracle against what the pages and mathematics fix.

None of these compare the oracle with itself: each check is a page figure, a
closed form, an identity the pages state between two *different*
computations (unabsorbed vs absorbed), brute force written differently, a
special case with a known answer, or an independent library routine.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import closed_forms as cf
import workloads as wl


# ----------------------------------------------------------------------------
# closed forms vs the pages' printed numbers
# ----------------------------------------------------------------------------

def test_cache_sizes_match_pages(golden):
    g = golden
    assert cf.mha_elements_per_token(128, 128) == g["mha_elements_per_token_128x128"]["value"]
    assert cf.latent_only_elements_per_token(512) == g["latent_only_elements_per_token"]["value"]
    assert cf.mha_elements_per_token(128, 128) // cf.latent_only_elements_per_token(512) == \
        g["latent_only_reduction_factor"]["value"]
    assert cf.mla_elements_per_token(512, 64) == g["mla_elements_per_token"]["value"]
    assert round(cf.mha_elements_per_token(128, 128) / cf.mla_elements_per_token(512, 64)) == \
        g["mla_vs_mha_factor_approx"]["value"]
    assert cf.gqa_elements_per_token(8, 128) == g["gqa8_elements_per_token"]["value"]
    assert cf.mqa_elements_per_token(128) == g["mqa_elements_per_token"]["value"]
    assert round(cf.reduction_pct(576, 32768), 1) == g["reduction_vs_mha_pct"]["value"]
    assert round(cf.reduction_pct(576, 2048), 1) == g["reduction_vs_gqa8_pct"]["value"]
    assert cf.mha_elements_per_token(8, 64) > g["eight_heads_of_64_elements_per_token_more_than"]["value"]


def test_equivalent_gqa_groups(golden):
    e = golden["equivalent_gqa_groups_definition"]
    g = cf.equivalent_gqa_groups(e["d_c"], e["d_R"], e["d_h"])
    # the definition: 2 g d_h equals the MLA per-token cache
    assert 2 * g * e["d_h"] == cf.mla_elements_per_token(e["d_c"], e["d_R"])
    assert g == 2.25


def test_bytes_formula_consistent_with_elements():
    # the 16-bit bytes formula is 2 bytes x the MHA element count x layers x tokens x batch
    for n_l, L, B in [(1, 1, 1), (61, 4096, 3)]:
        assert cf.mha_cache_bytes(n_l, 128, 128, L, B) == 2 * cf.mha_elements_per_token(128, 128) * n_l * L * B


def test_absorption_cost_example(golden):
    e = golden["absorption_example"]
    n, w, dc = e["n_tokens"], e["kv_width"], e["d_c"]
    un = cf.score_macs(n, w, dc, absorbed=False)
    ab = cf.score_macs(n, w, dc, absorbed=True)
    assert un == n * sum(e["unabsorbed_per_token_terms"])
    assert ab == e["absorbed_once"] + n * e["absorbed_per_token"]
    assert abs(un / ab - e["approx_ratio"]) < 1.0          # 99.59
    # the gap grows with context
    assert cf.score_macs(1000, w, dc, False) / cf.score_macs(1000, w, dc, True) > un / ab


def test_merged_output_weights_nearly_four_times(golden):
    d = golden["deepseek_v2_dims"]
    r = cf.output_weights(d["d_model"], d["n_h"], d["d_h"], d["d_c"], True) / \
        cf.output_weights(d["d_model"], d["n_h"], d["d_h"], d["d_c"], False)
    assert 3.5 < r < golden["merged_output_weights_vs_separate"]["value_below"]
    # and the oracle's fold really produces n_h blocks of d x d_c
    rng = np.random.default_rng(0)
    W_O, W_UV = rng.standard_normal((20, 4 * 3)), rng.standard_normal((4 * 3, 5))
    assert oracle.fold_output(W_O, W_UV, 4, 3).shape == (20, 4 * 5)


def test_deepseek_dims(golden):
    d = golden["deepseek_v2_dims"]
    assert d["n_h"] * d["d_h"] == d["kv_width"]
    assert d["n_h"] * d["d_R"] == d["q_rope_width"]


# ----------------------------------------------------------------------------
# absorbed == unabsorbed (the pages' identity, two different computations)
# ----------------------------------------------------------------------------

def _close(a, b, tol=1e-10):
    a, b = np.asarray(a), np.asarray(b)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin)
    err = np.max(np.abs(a[fin] - b[fin])) if fin.any() else 0.0
    assert err <= tol * max(1.0, np.max(np.abs(b[fin])) if fin.any() else 1.0), err


def test_tiny_config_absorbed_equals_unabsorbed():
    model = wl.make_tiny_model()
    o1 = oracle.mla_unabsorbed(model)
    o2 = oracle.mla_absorbed(model)
    _close(o2["scores"], o1["scores"])
    _close(o2["attn"], o1["attn"])
    _close(o2["o_heads"], o1["o_heads"])
    _close(o2["out"], o1["out"])
    _close(o2["lse"], o1["lse"])
    # the tiny config's attention is close to uniform but not uniform
    a = o1["attn"]
    assert a.max() / a.min() > 1.3


@pytest.mark.parametrize("case", range(24))
def test_random_shapes_absorbed_equals_unabsorbed(case):
    rng = np.random.default_rng(100 + case)
    nh = int(rng.integers(1, 6))
    dh = int(rng.integers(1, 5)) * 4
    dc = int(rng.integers(1, 6)) * 4
    dr = int(rng.integers(1, 4)) * 2
    d = int(rng.integers(4, 24))
    S = int(rng.integers(1, 12))
    q_len = int(rng.integers(1, min(S, 3) + 1))
    d_cq = int(rng.integers(0, 2)) * int(rng.integers(3, 9))
    cfg = wl.scaled(wl.CONFIGS["tiny"], n_heads=nh, d_head=dh, d_c=dc, d_rope=dr,
                    d_model=d, seq_len=S, seed=200 + case)
    model = wl.make_tiny_model(cfg, d_cq=d_cq)
    # larger weights so that attention is far from uniform
    for k in ("W_UQ", "W_QR", "W_UK"):
        setattr(model, k, getattr(model, k) * 40.0)
    pos0 = int(rng.integers(0, 1000))
    o1 = oracle.mla_unabsorbed(model, q_len=q_len, pos0=pos0)
    o2 = oracle.mla_absorbed(model, q_len=q_len, pos0=pos0)
    for k in ("scores", "attn", "o_heads", "out", "lse"):
        _close(o2[k], o1[k])


# ----------------------------------------------------------------------------
# softmax / attention: brute force, special cases, library routines
# ----------------------------------------------------------------------------

def _brute_force_one(qa, qr, c, kr, scale, visible):
    """Pure-Python attention for one query row (no numpy in the arithmetic)."""
    logits = []
    for j in range(visible):
        s = sum(qa[k] * c[j][k] for k in range(len(qa))) + sum(qr[k] * kr[j][k] for k in range(len(qr)))
        logits.append(s * scale)
    if not logits:
        return [0.0] * len(c[0]), -math.inf
    mx = max(logits)
    w = [math.exp(x - mx) for x in logits]
    z = sum(w)
    o = [sum(w[j] / z * c[j][k] for j in range(visible)) for k in range(len(c[0]))]
    return o, mx + math.log(z)


@pytest.mark.parametrize("S,q_len", [(1, 1), (2, 1), (3, 1), (4, 1), (2, 2), (4, 2), (3, 3)])
def test_brute_force_latent_attention(S, q_len):
    rng = np.random.default_rng(S * 10 + q_len)
    nh, dc, dr = 3, 5, 2
    qa = rng.standard_normal((q_len, nh, dc)) * 2
    qr = rng.standard_normal((q_len, nh, dr)) * 2
    c = rng.standard_normal((S, dc))
    kr = rng.standard_normal((S, dr))
    scale = 0.37
    r = oracle.latent_attention(qa, qr, c, kr, scale)
    for m in range(q_len):
        for i in range(nh):
            o, lse = _brute_force_one(qa[m, i].tolist(), qr[m, i].tolist(), c.tolist(), kr.tolist(),
                                      scale, S - q_len + m + 1)
            np.testing.assert_allclose(r["o"][m, i], o, rtol=0, atol=1e-13)
            assert abs(r["lse"][m, i] - lse) < 1e-13


def test_softmax_matches_scipy():
    rng = np.random.default_rng(7)
    s = rng.standard_normal((5, 33)) * 10
    np.testing.assert_allclose(oracle.softmax(s), scipy.special.softmax(s, axis=-1), atol=1e-15)
    r = oracle.latent_attention(rng.standard_normal((1, 2, 4)), rng.standard_normal((1, 2, 2)),
                                rng.standard_normal((9, 4)), rng.standard_normal((9, 2)), 0.5)
    np.testing.assert_allclose(r["lse"], scipy.special.logsumexp(r["scores"], axis=-1), atol=1e-13)


def test_single_token_returns_that_latent():
    rng = np.random.default_rng(1)
    c = rng.standard_normal((1, 6))
    r = oracle.latent_attention(rng.standard_normal((1, 4, 6)) * 9, rng.standard_normal((1, 4, 2)),
                                c, rng.standard_normal((1, 2)), 0.3)
    assert np.array_equal(r["o"], np.broadcast_to(c[0], (1, 4, 6)))


def test_zero_query_gives_mean_latent():
    rng = np.random.default_rng(2)
    c = rng.standard_normal((17, 6))
    r = oracle.latent_attention(np.zeros((1, 3, 6)), np.zeros((1, 3, 2)), c,
                                rng.standard_normal((17, 2)), 0.3)
    np.testing.assert_allclose(r["o"][0], np.broadcast_to(c.mean(axis=0), (3, 6)), atol=1e-15)
    np.testing.assert_allclose(r["lse"], math.log(17), atol=1e-14)


def test_planted_spike_selects_its_latent():
    rng = np.random.default_rng(3)
    S, dc = 40, 8
    c = rng.standard_normal((S, dc)) * 0.1
    kr = np.zeros((S, 2))
    kr[13] = [50.0, 0.0]                   # one logit +50 above the others
    q_rope = np.array([[[1.0, 0.0]]])
    r = oracle.latent_attention(np.zeros((1, 1, dc)), q_rope, c, kr, 1.0)
    np.testing.assert_allclose(r["o"][0, 0], c[13], atol=1e-12 * 40 + 1e-20)


def test_empty_sequence():
    r = oracle.latent_attention(np.ones((1, 2, 4)), np.ones((1, 2, 2)),
                                np.zeros((0, 4)), np.zeros((0, 2)), 1.0)
    assert np.array_equal(r["o"], np.zeros((1, 2, 4)))
    assert np.all(np.isneginf(r["lse"]))


def test_causal_pair_equals_truncated_single():
    rng = np.random.default_rng(4)
    S = 11
    qa, qr = rng.standard_normal((2, 3, 5)), rng.standard_normal((2, 3, 2))
    c, kr = rng.standard_normal((S, 5)), rng.standard_normal((S, 2))
    pair = oracle.latent_attention(qa, qr, c, kr, 0.4)
    first = oracle.latent_attention(qa[:1], qr[:1], c[:S - 1], kr[:S - 1], 0.4)
    second = oracle.latent_attention(qa[1:], qr[1:], c, kr, 0.4)
    np.testing.assert_allclose(pair["o"][0], first["o"][0], atol=1e-15)
    np.testing.assert_allclose(pair["o"][1], second["o"][0], atol=1e-15)


# ----------------------------------------------------------------------------
# RoPE
# ----------------------------------------------------------------------------

def test_rope_position_zero_is_identity_and_norm_preserving():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 16))
    assert np.array_equal(oracle.rope(x, np.zeros(7)), x)
    y = oracle.rope(x, rng.integers(0, 10 ** 5, 7))
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def test_rope_equals_complex_rotation():
    # independent formulation: pairs as complex numbers times e^{i pos w_k}
    rng = np.random.default_rng(6)
    d, theta = 16, 10000.0
    x = rng.standard_normal((5, d))
    pos = rng.integers(0, 5000, 5)
    z = x[:, 0::2] + 1j * x[:, 1::2]
    w = np.array([theta ** (-2.0 * k / d) for k in range(d // 2)])
    zr = z * np.exp(1j * pos[:, None] * w[None, :])
    y = oracle.rope(x, pos, theta)
    np.testing.assert_allclose(y[:, 0::2], zr.real, atol=1e-12)
    np.testing.assert_allclose(y[:, 1::2], zr.imag, atol=1e-12)


def test_rope_relative_position_property():
    # (R_t q)^T (R_j k) depends only on j - t: shift every position by D
    model = wl.make_tiny_model(wl.scaled(wl.CONFIGS["tiny"], seq_len=12), seed=9)
    a = oracle.mla_unabsorbed(model, pos0=0)
    b = oracle.mla_unabsorbed(model, pos0=777)
    np.testing.assert_allclose(a["scores"], b["scores"], atol=1e-12)
    np.testing.assert_allclose(a["out"], b["out"], atol=1e-12)


# ----------------------------------------------------------------------------
# folds: definition checked against the unfolded products
# ----------------------------------------------------------------------------

def test_fold_query_is_key_absorption():
    rng = np.random.default_rng(8)
    nh, dh, dc, din = 3, 4, 5, 6
    W_UQ, W_UK = rng.standard_normal((nh * dh, din)), rng.standard_normal((nh * dh, dc))
    A = oracle.fold_query(W_UQ, W_UK, nh, dh)
    assert A.shape == (nh, dc, din)
    h, c = rng.standard_normal(din), rng.standard_normal(dc)
    for i in range(nh):
        lhs = (W_UQ[i * dh:(i + 1) * dh] @ h) @ (W_UK[i * dh:(i + 1) * dh] @ c)
        assert abs((A[i] @ h) @ c - lhs) < 1e-12


def test_output_projection_modes_agree():
    rng = np.random.default_rng(10)
    nh, dh, dc, d, T = 3, 4, 5, 7, 2
    W_O, W_UV = rng.standard_normal((d, nh * dh)), rng.standard_normal((nh * dh, dc))
    o = rng.standard_normal((T, nh, dc))
    a = oracle.output_projection_merged(o, oracle.fold_output(W_O, W_UV, nh, dh))
    b = oracle.output_projection_two_stage(o, W_UV, W_O, nh, dh)
    np.testing.assert_allclose(a, b, atol=1e-12)


# ----------------------------------------------------------------------------
# number formats vs an independent library implementation
# ----------------------------------------------------------------------------

def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x38] == 1.0
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])


def test_e4m3_encode_matches_torch_and_roundtrips():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.1, 3.0, 100.0)]).astype(np.float32)
    x = np.clip(x, -448, 448).astype(np.float32)
    ours = oracle.e4m3_encode_f32(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    # every finite code round-trips, and exact midpoints go to the even code
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_decode(finite).astype(np.float32)
    back = oracle.e4m3_encode_f32(vals)
    assert np.array_equal(oracle.e4m3_decode(back), oracle.e4m3_decode(finite))
    mid = np.float32((1.0 + 1.125) / 2)            # between codes 0x38 and 0x39
    assert oracle.e4m3_encode_f32(np.array([mid]))[0] == 0x38
    assert oracle.e4m3_encode_f32(np.array([1e6], np.float32))[0] == 0x7E


def test_fp8_token_quantizer_amax_lane_hits_448():
    rng = np.random.default_rng(12)
    c = rng.standard_normal((50, 64)) / 24
    codes, s = oracle.fp8_quantize_tokens(c)
    dec = oracle.e4m3_decode(codes)
    assert np.all(np.abs(dec).max(axis=1) == 448.0)
    np.testing.assert_allclose(oracle.fp8_cache_dequant(codes, s), c, rtol=0.07, atol=1e-6)
    z_codes, z_s = oracle.fp8_quantize_tokens(np.zeros((1, 8)))
    assert z_s[0] == 1.0 and np.all(z_codes == 0)


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(13)
    bits = rng.integers(0, 2 ** 16, 5000, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]          # finite only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), ref)


# ----------------------------------------------------------------------------
# the softmax scale: the page fixes the denominator
# ----------------------------------------------------------------------------

def test_score_scale_is_the_pages_denominator(golden):
    """[Zhang] "Value absorption": the summed content and rope score is divided
    by the square root of 128 + 64 for the DeepSeek head; the same rule gives
    64 + 16 for the tiny model's heads. Not sqrt(d_h), not sqrt(576)."""
    g = golden["score_scale_denominator_squared"]
    assert g["d_h"] + g["d_R"] == g["value"]
    assert oracle.score_scale(g["d_h"], g["d_R"]) == 1.0 / math.sqrt(g["value"])
    assert oracle.score_scale(64, 16) == 1.0 / math.sqrt(80)
    for wrong in (1.0 / math.sqrt(g["d_h"]), 1.0 / math.sqrt(512 + g["d_R"])):
        assert oracle.score_scale(g["d_h"], g["d_R"]) != wrong


def _py_matvec(W, x):
    return [sum(W[r][k] * x[k] for k in range(len(x))) for r in range(len(W))]


def _py_rope(x, pos, theta):
    """Rotation of interleaved pairs (2k, 2k+1) by pos * theta^(-2k/d), one
    pair at a time (the oracle's layout reading, written out)."""
    d = len(x)
    out = list(x)
    for k in range(d // 2):
        ang = pos * theta ** (-2.0 * k / d)
        cs, sn = math.cos(ang), math.sin(ang)
        out[2 * k] = x[2 * k] * cs - x[2 * k + 1] * sn
        out[2 * k + 1] = x[2 * k] * sn + x[2 * k + 1] * cs
    return out


def test_unabsorbed_scores_brute_force(golden):
    """O1's scores at the DeepSeek head widths (d_h 128, d_R 64; two heads,
    tiny d_c and d_model) recomputed in plain Python loops from the weights:
    q_i = [W^UQ_i h_t ; RoPE(W^QR_i h_t)], k_{j,i} = [W^UK_i W^DKV h_j ;
    RoPE(W^KR h_j)], score = (q_i . k_{j,i}) / sqrt(192) with 192 the page's
    128 + 64 ([Mishra] "Step 4: decoupled RoPE"; [Zhang] "Value absorption").
    Independent of the absorbed form O2, so a wrong scale shared by O1 and O2
    fails here."""
    g = golden["score_scale_denominator_squared"]
    dh, dr = g["d_h"], g["d_R"]
    cfg = wl.scaled(wl.CONFIGS["tiny"], n_heads=2, d_head=dh, d_rope=dr, d_c=8, d_model=6,
                    seq_len=3)
    model = wl.make_tiny_model(cfg, seed=21)
    r = oracle.mla_unabsorbed(model)
    W = {k: np.asarray(v, np.float64).tolist() for k, v in model.__dict__.items()
         if k.startswith("W_") and v is not None}
    H = np.asarray(model.H, np.float64).tolist()
    S, t = len(H), len(H) - 1
    theta = cfg.rope_theta
    c = [_py_matvec(W["W_DKV"], H[j]) for j in range(S)]
    kR = [_py_rope(_py_matvec(W["W_KR"], H[j]), j, theta) for j in range(S)]
    for i in range(cfg.n_heads):
        qC = _py_matvec(W["W_UQ"][i * dh:(i + 1) * dh], H[t])
        qR = _py_rope(_py_matvec(W["W_QR"][i * dr:(i + 1) * dr], H[t]), t, theta)
        for j in range(S):
            kC = _py_matvec(W["W_UK"][i * dh:(i + 1) * dh], c[j])
            dot = sum(a * b for a, b in zip(qC + qR, kC + kR[j]))
            want = dot / math.sqrt(g["value"])
            assert abs(r["scores"][0, i, j] - want) <= 1e-12 * max(1.0, abs(want)), (i, j)


# ----------------------------------------------------------------------------
# the expanded (prefill) attention of one head
# ----------------------------------------------------------------------------

def test_expanded_attention_is_o1_for_every_position():
    """expanded_attention, fed O1's own per-head query, key and value
    projections at every position, reproduces O1's per-position head outputs
    and log-sum-exps (O1 recomputes each position separately, in its own
    loop)."""
    cfg = wl.scaled(wl.CONFIGS["tiny"], seq_len=40)
    model = wl.make_tiny_model(cfg, seed=5)
    S = cfg.seq_len
    r1 = oracle.mla_unabsorbed(model, q_len=S)
    H = model.H.astype(np.float64)
    c, kR = r1["c"], r1["kR"]
    dh, dr = cfg.d_head, cfg.d_rope
    for i in range(cfg.n_heads):
        qC = H @ np.asarray(model.W_UQ, np.float64)[i * dh:(i + 1) * dh].T
        qR = oracle.rope(H @ np.asarray(model.W_QR, np.float64)[i * dr:(i + 1) * dr].T, np.arange(S))
        kC = c @ np.asarray(model.W_UK, np.float64)[i * dh:(i + 1) * dh].T
        v = c @ np.asarray(model.W_UV, np.float64)[i * dh:(i + 1) * dh].T
        e = oracle.expanded_attention(qC, qR, kC, kR, v, oracle.score_scale(dh, dr))
        assert np.max(np.abs(e["o"] - r1["o_heads"][:, i])) < 1e-12
        assert np.max(np.abs(e["lse"] - r1["lse"][:, i])) < 1e-12


def test_expanded_attention_brute_force():
    """Three positions, written out: position t weighs values 0..t by the
    exponentials of its scaled scores, normalised."""
    rng = np.random.default_rng(3)
    qC, kC = rng.standard_normal((3, 4)), rng.standard_normal((3, 4))
    qR, kR = rng.standard_normal((3, 2)), rng.standard_normal((3, 2))
    v = rng.standard_normal((3, 5))
    sc = 0.7
    r = oracle.expanded_attention(qC, qR, kC, kR, v, sc)
    for t in range(3):
        e = [math.exp(sc * (sum(qC[t] * kC[j]) + sum(qR[t] * kR[j]))) for j in range(t + 1)]
        want = sum(e[j] * v[j] for j in range(t + 1)) / sum(e)
        assert np.max(np.abs(r["o"][t] - want)) < 1e-13
        assert abs(r["lse"][t] - math.log(sum(e))) < 1e-13
    assert np.allclose(r["o"][0], v[0], atol=0, rtol=0)   # position 0 sees only itself
