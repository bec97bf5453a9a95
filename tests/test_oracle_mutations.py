"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch each one: a dropped rope term, a wrong softmax scale, an off-by-one
causal limit, a wrong head index in the fold, a wrong RoPE frequency, and a
wrong scale shared by the unabsorbed and the absorbed forms."""
import math

import numpy as np
import pytest

import oracle
import oracle.reference as ref
import workloads as wl
import tests.test_oracle_pins as pins


def _mutant_latent_attention(kind):
    orig = ref.latent_attention

    def f(q_abs, q_rope, c, kR, scale):
        if kind == "drop_rope":
            q_rope = np.zeros_like(np.asarray(q_rope, dtype=np.float64))
        if kind == "scale":
            scale = 1.0 / math.sqrt(np.shape(q_abs)[-1] + np.shape(q_rope)[-1])
        r = orig(q_abs, q_rope, c, kR, scale)
        if kind == "causal":
            q_len = np.shape(q_abs)[0]
            S = np.shape(c)[0]
            s = scale * (np.einsum("mid,jd->mij", q_abs, c) + np.einsum("mid,jd->mij", q_rope, kR))
            for m in range(q_len):
                s[m, :, S - q_len + m + 2:] = -np.inf     # one position too many
            a = ref.softmax(s)
            r = dict(r, o=np.einsum("mij,jd->mid", a, c), scores=s, attn=a)
        return r
    return f


@pytest.mark.parametrize("kind,check", [
    ("drop_rope", lambda: pins.test_tiny_config_absorbed_equals_unabsorbed()),
    ("scale", lambda: pins.test_brute_force_latent_attention(4, 1)),
    ("causal", lambda: pins.test_causal_pair_equals_truncated_single()),
])
def test_planted_attention_mistakes_are_caught(monkeypatch, kind, check):
    m = _mutant_latent_attention(kind)
    monkeypatch.setattr(ref, "latent_attention", m)
    monkeypatch.setattr(oracle, "latent_attention", m)
    with pytest.raises(AssertionError):
        check()


def test_planted_fold_head_index_is_caught(monkeypatch):
    def bad_fold(W_UQ, W_UK, n_h, d_h):
        W_UQ, W_UK = np.asarray(W_UQ, np.float64), np.asarray(W_UK, np.float64)
        # strided head slices instead of contiguous ones
        return np.stack([W_UK[i::n_h].T @ W_UQ[i::n_h] for i in range(n_h)])
    monkeypatch.setattr(ref, "fold_query", bad_fold)
    # same shape as the true fold, different values: the identity pin must fail
    model = wl.make_tiny_model(wl.scaled(wl.CONFIGS["tiny"], d_model=64, d_c=64, seq_len=16))
    o1 = oracle.mla_unabsorbed(model)
    o2 = ref.mla_absorbed(model)
    assert np.max(np.abs(o1["scores"] - o2["scores"])) > 1e-6


def test_planted_rope_frequency_is_caught(monkeypatch):
    orig = ref.rope

    def bad_rope(x, pos, theta=10000.0):
        return orig(x, pos, theta * 1.01)
    monkeypatch.setattr(ref, "rope", bad_rope)
    monkeypatch.setattr(oracle, "rope", bad_rope)
    with pytest.raises(AssertionError):
        pins.test_rope_equals_complex_rotation()


@pytest.mark.parametrize("wrong", ["d_h", "latent_width"])
def test_planted_common_scale_is_caught(monkeypatch, wrong):
    """The same wrong scale in O1 and O2 (1/sqrt(d_h), as one of the pages
    writes for plain attention, or 1/sqrt(d_c + d_R)): the absorbed/unabsorbed
    identity cannot see it, the page's denominator and the brute-force scores
    must."""
    def bad_scale(d_h, d_rope):
        return 1.0 / math.sqrt(d_h if wrong == "d_h" else 512 + d_rope)
    monkeypatch.setattr(ref, "score_scale", bad_scale)
    monkeypatch.setattr(oracle, "score_scale", bad_scale)
    golden = pins_golden()
    pins.test_tiny_config_absorbed_equals_unabsorbed()   # common mode: still agrees
    with pytest.raises(AssertionError):
        pins.test_score_scale_is_the_pages_denominator(golden)
    with pytest.raises(AssertionError):
        pins.test_unabsorbed_scores_brute_force(golden)


def pins_golden():
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")) as f:
        return json.load(f)
