"""Plain fp64 reference of MLA decode, unabsorbed and absorbed (test infrastructure).

Notation follows the pages: h_t hidden state, c_j = W^DKV h_j the cached
latent (d_c), k^R_j = RoPE(W^KR h_j) the shared rotated key (d_R), per head i
the content query q^C_i = W^UQ_i x_t and rope query q^R_i = RoPE(W^QR_i x_t)
(x_t = h_t, or the query latent c^Q_t = W^DQ h_t when queries are
compressed), content keys k^C_{j,i} = W^UK_i c_j and values v_{j,i} = W^UV_i c_j.

Head i owns rows [i*d_h, (i+1)*d_h) of W^UQ, W^UK, W^UV and the same columns of
W^O; rows [i*d_R, (i+1)*d_R) of W^QR.

Readings where the pages leave a step open:
* softmax scale: 1/sqrt(d_h + d_R) ([Zhang] "Value absorption: weight and
  sum first, project after" divides by the root of content plus position
  width);
* the newest token's latent is cached before its query attends, so the query
  at position t sees j = 0..t; with q_len > 1 queries of one sequence sit at
  the last q_len positions and each sees only positions up to its own;
* RoPE rotates interleaved pairs (2k, 2k+1) by angle pos * theta^(-2k/d_R);
* the rope key is cached already rotated ([Zhang] "Decoupled RoPE").
"""
from __future__ import annotations

import math

import numpy as np


# ----------------------------------------------------------------------------
# building blocks
# ----------------------------------------------------------------------------

def rope(x, pos, theta: float = 10000.0) -> np.ndarray:
    """Rotary position embedding of x[..., d] at positions pos (broadcast
    against x[..., 0]). [Mishra] "Step 3: RoPE breaks it": a rotation whose
    angle depends on the token's position, so that rotated dot products
    depend only on the position difference."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % 2 == 0
    k = np.arange(d // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * k / d)                          # [d/2]
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    cos, sin = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * cos - x1 * sin
    out[..., 1::2] = x0 * sin + x1 * cos
    return out


def softmax(s, axis: int = -1) -> np.ndarray:
    """Standard softmax with max subtraction; rows that are entirely -inf
    give all-zero weights. [Zhang] "Value absorption": softmax over the
    scaled scores gives the attention weights A(i, j)."""
    s = np.asarray(s, dtype=np.float64)
    m = np.max(s, axis=axis, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m)
    z = e.sum(axis=axis, keepdims=True)
    return np.where(z > 0, e / np.where(z > 0, z, 1.0), 0.0)


def _log_sum_exp(s, axis: int = -1) -> np.ndarray:
    s = np.asarray(s, dtype=np.float64)
    m = np.max(s, axis=axis, keepdims=True)
    finite = np.isfinite(m)
    m0 = np.where(finite, m, 0.0)
    z = np.exp(s - m0).sum(axis=axis, keepdims=True)
    out = np.where(finite & (z > 0), m0 + np.log(np.where(z > 0, z, 1.0)), -np.inf)
    return np.squeeze(out, axis=axis)


def _head(W, i, width):
    return W[i * width:(i + 1) * width]


def score_scale(d_h: int, d_rope: int) -> float:
    """The factor applied to a summed content + rope score: one over the
    square root of one head's content width plus its rope width ([Zhang]
    "Value absorption: weight and sum first, project after": 128 + 64 for
    DeepSeek-V2). The latent width d_c does not enter it."""
    return 1.0 / math.sqrt(d_h + d_rope)


# ----------------------------------------------------------------------------
# O1: the unabsorbed definition
# ----------------------------------------------------------------------------

def mla_unabsorbed(model, q_len: int = 1, pos0: int = 0) -> dict:
    """Unabsorbed MLA for the last q_len positions of model.H (O1).

    [Mishra] "Step 1: a low-rank latent" (c_t = W^DKV h_t, k = W^UK c,
    v = W^UV c); [LLMsBlog] "The Positional Problem and Decoupled RoPE"
    (q^R_{t,i} = RoPE(W^QR_i c^Q_t, t), k^R_t = RoPE(W^KR h_t, t), per-head
    query and key are the concatenations [q^C; q^R], [k^C; k^R]); [Zhang]
    "Value absorption" (score / sqrt(d_h + d_R), softmax, o_i = sum_j A v_j);
    [Mishra] "Step 2" (out = W^O applied to the concatenated head outputs).
    Positions are pos0 + 0..S-1.
    """
    cfg = model.cfg
    nh, dh, dc, dr = cfg.n_heads, cfg.d_head, cfg.d_c, cfg.d_rope
    H = model.H.astype(np.float64)
    S = H.shape[0]
    pos = pos0 + np.arange(S)
    W = {k: None if v is None else np.asarray(v, dtype=np.float64)
         for k, v in model.__dict__.items() if k.startswith("W_")}
    scale = score_scale(dh, dr)

    c = H @ W["W_DKV"].T                                     # [S, d_c]
    kR = rope(H @ W["W_KR"].T, pos, cfg.rope_theta)          # [S, d_R]
    scores = np.full((q_len, nh, S), -np.inf)
    attn = np.zeros((q_len, nh, S))
    o_heads = np.zeros((q_len, nh, dh))
    lse = np.zeros((q_len, nh))
    for m in range(q_len):
        t = S - q_len + m
        x = H[t] if W["W_DQ"] is None else W["W_DQ"] @ H[t]
        for i in range(nh):
            qC = _head(W["W_UQ"], i, dh) @ x
            qR = rope(_head(W["W_QR"], i, dr) @ x, pos[t], cfg.rope_theta)
            q = np.concatenate([qC, qR])
            kC = c[:t + 1] @ _head(W["W_UK"], i, dh).T          # [t+1, d_h]
            v = c[:t + 1] @ _head(W["W_UV"], i, dh).T           # [t+1, d_h]
            k = np.concatenate([kC, kR[:t + 1]], axis=1)        # [t+1, d_h+d_R]
            s = (k @ q) * scale
            a = softmax(s)
            scores[m, i, :t + 1] = s
            attn[m, i, :t + 1] = a
            o_heads[m, i] = a @ v
            lse[m, i] = _log_sum_exp(s)
    out = o_heads.reshape(q_len, nh * dh) @ W["W_O"].T          # [q_len, d]
    return dict(c=c, kR=kR, scores=scores, attn=attn, o_heads=o_heads,
                lse=lse, out=out)


def expanded_attention(qC, qR, kC, kR, v, scale: float, causal: bool = True) -> dict:
    """One head of the unabsorbed form over T positions of one sequence:
    s[t, j] = scale * (qC[t] . kC[j] + qR[t] . kR[j]) for j <= t (all j when
    not causal), a = softmax(s), o[t] = sum_j a[t, j] v[j]. [Mishra] "Step 4:
    decoupled RoPE" (the concatenated content and rope parts, whose dot
    products add); [Zhang] "Value absorption: weight and sum first, project
    after" (scaled scores, softmax, weighted sum of the values). qC [T, d_h],
    qR [T, d_R], kC [S, d_h], kR [S, d_R], v [S, d_v]; query t sits at key
    position t. Returns o [T, d_v] and lse [T] (natural log)."""
    qC, qR, kC, kR, v = (np.asarray(x, dtype=np.float64) for x in (qC, qR, kC, kR, v))
    s = scale * (qC @ kC.T + qR @ kR.T)
    if causal:
        T, S = s.shape
        s = np.where(np.arange(S)[None, :] <= np.arange(T)[:, None], s, -np.inf)
    a = softmax(s)
    return dict(o=a @ v, lse=_log_sum_exp(s), scores=s, attn=a)


# ----------------------------------------------------------------------------
# folds (offline absorption)
# ----------------------------------------------------------------------------

def fold_query(W_UQ, W_UK, n_h: int, d_h: int) -> np.ndarray:
    """W_qabs[i] = (W^UK_i)^T W^UQ_i, shape [n_h, d_c, d_in].

    [Mishra] "Step 2: absorb the up-projections", boxed identity: the product
    of the transposed key up-projection and the query projection is formed
    once, offline; [LLMsBlog] "Query Key Absorption"."""
    W_UQ = np.asarray(W_UQ, dtype=np.float64)
    W_UK = np.asarray(W_UK, dtype=np.float64)
    return np.stack([_head(W_UK, i, d_h).T @ _head(W_UQ, i, d_h) for i in range(n_h)])


def fold_output(W_O, W_UV, n_h: int, d_h: int) -> np.ndarray:
    """W_ov = [W^O_i W^UV_i]_i, shape [d, n_h*d_c] (block i is W^O's head-i
    columns times W^UV_i). [Mishra] "Step 2" (out = (W^O W^UV) sum a c);
    [Zhang] "Value absorption" (W^O and W^UV merge ahead of time)."""
    W_O = np.asarray(W_O, dtype=np.float64)
    W_UV = np.asarray(W_UV, dtype=np.float64)
    return np.concatenate(
        [W_O[:, i * d_h:(i + 1) * d_h] @ _head(W_UV, i, d_h) for i in range(n_h)], axis=1)


def output_projection_merged(o_lat, W_ov) -> np.ndarray:
    """out[t] = W_ov concat_i(o_lat[t, i]). o_lat [T, n_h, d_c] -> [T, d].
    [Mishra] "Step 2"; [LLMsBlog] "Value Output Absorption"."""
    o = np.asarray(o_lat, dtype=np.float64)
    return o.reshape(o.shape[0], -1) @ np.asarray(W_ov, dtype=np.float64).T


def output_projection_two_stage(o_lat, W_UV, W_O, n_h: int, d_h: int) -> np.ndarray:
    """out[t] = W^O concat_i(W^UV_i o_lat[t, i]): the factors kept apart
    ([Zhang] "Value absorption", the note on keeping the two projections
    separate and applying them after the weighted sum)."""
    o = np.asarray(o_lat, dtype=np.float64)
    W_UV = np.asarray(W_UV, dtype=np.float64)
    heads = np.stack([o[:, i] @ _head(W_UV, i, d_h).T for i in range(n_h)], axis=1)
    return heads.reshape(o.shape[0], -1) @ np.asarray(W_O, dtype=np.float64).T


# ----------------------------------------------------------------------------
# O3: attention in latent space on given absorbed queries
# ----------------------------------------------------------------------------

def latent_attention(q_abs, q_rope, c, kR, scale: float) -> dict:
    """One sequence: q_abs [q_len, n_h, d_c], q_rope [q_len, n_h, d_R] against
    the cached latent c [S, d_c] and rotated rope key kR [S, d_R].

    s_j = scale * (q_abs . c_j + q_rope . k^R_j)  ([LLMsBlog] "Query Key
    Absorption": logits straight against the cached latent plus the rope
    term; [Mishra] "Step 4: decoupled RoPE"), a = softmax(s) ([Zhang] "Value
    absorption"), o = sum_j a_j c_j ([LLMsBlog] "Value Output Absorption").
    Query m sees positions j <= S - q_len + m. A query that sees no position
    gets o = 0 and lse = -inf. lse is the natural log of sum_j exp(s_j).
    """
    q_abs = np.asarray(q_abs, dtype=np.float64)
    q_rope = np.asarray(q_rope, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    kR = np.asarray(kR, dtype=np.float64)
    q_len, nh, dc = q_abs.shape
    S = c.shape[0]
    if S == 0:
        return dict(o=np.zeros((q_len, nh, dc)), lse=np.full((q_len, nh), -np.inf),
                    scores=np.zeros((q_len, nh, 0)), attn=np.zeros((q_len, nh, 0)))
    s = scale * (q_abs.reshape(-1, dc) @ c.T + q_rope.reshape(q_len * nh, -1) @ kR.T)
    s = s.reshape(q_len, nh, S)
    for m in range(q_len):
        s[m, :, max(S - q_len + m + 1, 0):] = -np.inf
    a = softmax(s)
    o = (a.reshape(q_len * nh, S) @ c).reshape(q_len, nh, dc)
    return dict(o=o, lse=_log_sum_exp(s), scores=s, attn=a)


# ----------------------------------------------------------------------------
# O2: the absorbed CPU form
# ----------------------------------------------------------------------------

def absorb_query(W_qabs, W_QR, x, pos, theta: float = 10000.0) -> tuple[np.ndarray, np.ndarray]:
    """Absorbed queries for inputs x [T, d_in] at positions pos [T]:
    q_abs[t, i] = W_qabs[i] x_t and q_rope[t, i] = RoPE(W^QR_i x_t, pos_t).
    [LLMsBlog] "Query Key Absorption" (the absorbed query is computed once per
    step) and "The Positional Problem and Decoupled RoPE"."""
    W_qabs = np.asarray(W_qabs, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    nh = W_qabs.shape[0]
    q_abs = np.einsum("icd,td->tic", W_qabs, x)
    W_QR = np.asarray(W_QR, dtype=np.float64)
    dr = W_QR.shape[0] // nh
    qr = (x @ W_QR.T).reshape(x.shape[0], nh, dr)
    q_rope = rope(qr, np.asarray(pos)[:, None], theta)
    return q_abs, q_rope


def cache_append(W_DKV, W_KR, h, pos, theta: float = 10000.0) -> tuple[np.ndarray, np.ndarray]:
    """New cache rows for hidden states h [T, d] at positions pos [T]:
    c = W^DKV h ([Mishra] "Step 1"), k^R = RoPE(W^KR h, pos), stored rotated
    ([Zhang] "Decoupled RoPE")."""
    h = np.asarray(h, dtype=np.float64)
    c = h @ np.asarray(W_DKV, dtype=np.float64).T
    kR = rope(h @ np.asarray(W_KR, dtype=np.float64).T, pos, theta)
    return c, kR


def mla_absorbed(model, q_len: int = 1, pos0: int = 0) -> dict:
    """Absorbed MLA on the same inputs as mla_unabsorbed (O2): fold W^UK into
    the query side and W^UV into W^O, attend against the latent, project
    once. [Mishra] "Step 2" and "Step 4"; [LLMsBlog] "Query Key Absorption",
    "Value Output Absorption"."""
    cfg = model.cfg
    nh, dh, dr = cfg.n_heads, cfg.d_head, cfg.d_rope
    H = model.H.astype(np.float64)
    S = H.shape[0]
    pos = pos0 + np.arange(S)
    scale = score_scale(dh, dr)
    W_qabs = fold_query(model.W_UQ, model.W_UK, nh, dh)
    W_ov = fold_output(model.W_O, model.W_UV, nh, dh)
    c, kR = cache_append(model.W_DKV, model.W_KR, H, pos, cfg.rope_theta)
    t = np.arange(S - q_len, S)
    x = H[t] if model.W_DQ is None else H[t] @ np.asarray(model.W_DQ, np.float64).T
    q_abs, q_rope = absorb_query(W_qabs, model.W_QR, x, pos[t], cfg.rope_theta)
    r = latent_attention(q_abs, q_rope, c, kR, scale)
    out = output_projection_merged(r["o"], W_ov)
    W_UV = np.asarray(model.W_UV, dtype=np.float64)
    o_heads = np.stack([r["o"][:, i] @ _head(W_UV, i, dh).T for i in range(nh)], axis=1)
    return dict(c=c, kR=kR, q_abs=q_abs, q_rope=q_rope, W_qabs=W_qabs, W_ov=W_ov,
                scores=r["scores"], attn=r["attn"], o_latent=r["o"], lse=r["lse"],
                o_heads=o_heads, out=out)
