"""Closed-form cache sizes and operation counts (test infrastructure).

Each function is the formula a page states, written out; the tests compare
them with the numbers the pages print (tests/golden/).
"""
from __future__ import annotations


def mha_elements_per_token(n_h: int, d_h: int) -> int:
    """Keys and values of every head: 2 * n_h * d_h per token per layer.
    [Mishra] "Step 1: a low-rank latent"; [Zhang] "Multi-head attention:
    every head caches its own keys and values"."""
    return 2 * n_h * d_h


def gqa_elements_per_token(n_kv: int, d_h: int) -> int:
    """Grouped heads share keys and values: 2 * h_kv * d_h ([Mishra] "The full
    accounting"; [LLMsBlog] "Quantitative Comparison and Serving Economics")."""
    return 2 * n_kv * d_h


def mqa_elements_per_token(d_h: int) -> int:
    """One shared key/value head: 2 * d_h ([Mishra] "The full accounting")."""
    return 2 * d_h


def latent_only_elements_per_token(d_c: int) -> int:
    """Only the joint latent c_t is cached ([Mishra] "Step 1"; [Zhang]
    "Low-rank joint compression: cache one latent vector")."""
    return d_c


def mla_elements_per_token(d_c: int, d_R: int) -> int:
    """Latent plus the shared rotated key: d_c + d_R ([Mishra] "Step 4:
    decoupled RoPE", boxed; [Zhang] "Decoupled RoPE")."""
    return d_c + d_R


def mha_cache_bytes(n_l: int, n_h: int, d_h: int, L: int, B: int, bytes_per: int = 2) -> int:
    """Whole-model KV cache at 16-bit: 2 * 2 * n_l * n_h * d_h * L * B
    ([LLMsBlog] "The Memory Bottleneck in Transformer Attention")."""
    return 2 * bytes_per * n_l * n_h * d_h * L * B


def equivalent_gqa_groups(d_c: int, d_R: int, d_h: int) -> float:
    """g solving 2 g d_h = d_c + d_R: the grouped-query head count with the
    same per-token cache ([Mishra] "Step 4", the cache calculator caption)."""
    return (d_c + d_R) / (2.0 * d_h)


def reduction_pct(ours: int, theirs: int) -> float:
    """Percent less cache than `theirs` ([LLMsBlog] "Quantitative Comparison
    and Serving Economics")."""
    return 100.0 * (1.0 - ours / theirs)


def score_macs(n_tokens: int, kv_width: int, d_c: int, absorbed: bool) -> int:
    """Multiply-accumulates for one query head-set's scores over n cached
    tokens ([Zhang] "Matrix absorption: compression that also saves
    compute"): unabsorbed expands every cached latent (kv_width x d_c) then
    dots with the query (kv_width); absorbed folds once (kv_width x d_c) then
    dots in latent width d_c per token."""
    if absorbed:
        return kv_width * d_c + n_tokens * d_c
    return n_tokens * (kv_width * d_c + kv_width)


def output_weights(d: int, n_h: int, d_h: int, d_c: int, merged: bool) -> int:
    """Parameters of the output side: merged W^O W^UV is n_h blocks of
    d x d_c; separate factors are W^O (d x n_h d_h) plus W^UV (n_h d_h x d_c)
    ([Zhang] "Value absorption", the note on merging)."""
    if merged:
        return n_h * d * d_c
    return d * n_h * d_h + n_h * d_h * d_c
