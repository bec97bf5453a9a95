"""The seeded input generators: storage conversions and layout (CPU)."""
import math

import numpy as np
import torch

import oracle
import workloads as wl


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-8, 8, 100000)).astype(np.float32)
    ours = wl.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_generator_e4m3_encoder_agrees_with_oracle_and_torch():
    rng = np.random.default_rng(1)
    x = np.clip(rng.standard_normal(30000) * 60, -448, 448).astype(np.float32)
    g = wl.encode_e4m3(x)
    assert np.array_equal(g, oracle.e4m3_encode_f32(x))
    assert np.array_equal(g, torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy())


def test_generator_token_quantizer_agrees_with_oracle():
    rng = np.random.default_rng(2)
    c = rng.standard_normal((300, 512)) / 24
    c[5] = 0.0
    gc, gs = wl.quantize_tokens_e4m3(c)
    oc, os_ = oracle.fp8_quantize_tokens(c)
    assert np.array_equal(gc, oc) and np.array_equal(gs, os_)


def test_ragged_lengths_and_pages():
    cfg = wl.scaled(wl.CONFIGS["c4"], batch=5, ragged=(1, 200))
    inp = wl.make_decode_inputs(cfg)
    assert inp.seq_lens.min() >= 1 and inp.seq_lens.max() <= 200
    n_pages = sum(wl.pages_for(int(s)) for s in inp.seq_lens)
    assert sorted(inp.page_perm.tolist()) == list(range(n_pages))
    bt = wl.block_table(inp.seq_lens, inp.page_perm)
    pool, _ = wl.paged_cache(inp)
    # every token row is found through the table where it belongs
    for b in range(cfg.batch):
        for j in range(int(inp.seq_lens[b])):
            assert np.array_equal(pool[bt[b, j // 64], j % 64], inp.lat_bits[b][j])
        assert np.all(bt[b, wl.pages_for(int(inp.seq_lens[b])):] == -1)


def test_fp8_rows_layout():
    cfg = wl.scaled(wl.CONFIGS["c5"], batch=2, seq_len=70)
    inp = wl.make_decode_inputs(cfg)
    pool, spool = wl.paged_cache(inp)
    assert pool.shape == (4, 64, 512 + 128) and pool.dtype == np.uint8
    assert spool.shape == (4, 64)
    bt = wl.block_table(inp.seq_lens, inp.page_perm)
    row = pool[bt[1, 1], 5]           # sequence 1, token 69
    assert np.array_equal(row[:512], inp.lat_codes[1][69])
    assert np.array_equal(row[512:].view(np.uint16), inp.krope_bits[1][69])
    assert spool[bt[1, 1], 5] == inp.lat_scales[1][69]


def test_draws_are_reproducible():
    cfg = wl.scaled(wl.CONFIGS["c2"], batch=2, seq_len=10)
    a, b = wl.make_decode_inputs(cfg), wl.make_decode_inputs(cfg)
    assert np.array_equal(a.q_abs_bits, b.q_abs_bits)
    assert all(np.array_equal(x, y) for x, y in zip(a.lat_bits, b.lat_bits))


# ----------------------------------------------------------------------------
# the configurations against the workload text they were transcribed from
# ----------------------------------------------------------------------------

def _spec():
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "workload_spec.json")
    with open(path) as f:
        return json.load(f)["workloads"]


def _parse(text: str, inherit: dict) -> dict:
    """Numbers of one workload description; fields a description leaves to
    another ("same 128-head bf16 shapes") come from `inherit`."""
    import re

    def num(pat):
        m = re.search(pat, text)
        return int(m.group(1)) if m else None
    f = dict(inherit)
    for key, pat in (("batch", r"[Bb]atch (\d+)"), ("seq_len", r"context (\d+)"),
                     ("n_heads", r"n_h=(\d+)"), ("d_c", r"d_c=(\d+)"), ("d_rope", r"d_R=(\d+)"),
                     ("d_head", r"d_h=(\d+)"), ("d_model", r"d_model=(\d+)"),
                     ("scale_sq", r"1/sqrt\((\d+)\)")):
        v = num(pat)
        if v is not None:
            f[key] = v
    v = num(r"(\d+)-head") or num(r"(\d+) heads")
    if v is not None:
        f["n_heads"] = v
    v = num(r"(\d+) query tokens?")
    if v is not None:
        f["q_len"] = v
    m = re.search(r"uniform in \[(\d+), (\d+)\]", text)
    f["ragged"] = (int(m.group(1)), int(m.group(2))) if m else None
    if f["ragged"] is not None:
        f["seq_len"] = None
    f["permute_pages"] = "permutation" in text
    m = re.search(r"theta=(\d+)", text)
    if m:
        f["rope_theta"] = float(m.group(1))
    first = re.search(r"\b(fp32|fp8|bf16)\b", text).group(1)
    f["cache_dtype"] = first
    if "bf16 output" in text:
        f["out_dtype"] = "bf16"
    return f


def test_configs_match_the_workload_specification():
    """Every field of workloads.CONFIGS that the workload text states: batch,
    context or ragged range, query tokens, heads, d_c, d_R, dtypes, page
    permutation, and the softmax scale 1/sqrt(192) of the 128-head workloads
    (the tiny model's 1/sqrt(64 + 16) by the same rule)."""
    spec = _spec()
    tiny = _parse(spec["tiny"], {"q_len": 1, "out_dtype": "fp32"})
    c2 = _parse(spec["c2"], {"out_dtype": "bf16", "d_head": 128})
    c3 = _parse(spec["c3"], {k: c2[k] for k in ("q_len", "n_heads", "d_c", "d_rope", "out_dtype",
                                                 "scale_sq", "d_head")})
    c4 = _parse(spec["c4"], {k: c2[k] for k in ("q_len", "out_dtype", "scale_sq", "d_head")})
    c5 = _parse(spec["c5"], {k: c2[k] for k in ("scale_sq", "d_head")})
    parsed = {"tiny": tiny, "c2": c2, "c3": c3, "c4": c4, "c5": c5}
    assert (tiny["batch"], tiny["seq_len"], tiny["n_heads"], tiny["d_head"], tiny["d_c"],
            tiny["d_rope"], tiny["d_model"], tiny["rope_theta"]) == (1, 256, 8, 64, 64, 16, 512, 10000.0)
    assert c2["scale_sq"] == 192 and c5["q_len"] == 2 and c4["ragged"] == (512, 16384)
    for name, f in parsed.items():
        cfg = wl.CONFIGS[name]
        for key in ("batch", "seq_len", "q_len", "n_heads", "d_c", "d_rope", "cache_dtype",
                    "out_dtype", "ragged", "permute_pages", "d_head"):
            assert getattr(cfg, key) == f[key], (name, key, getattr(cfg, key), f[key])
        if name == "tiny":
            assert cfg.d_model == f["d_model"] and cfg.rope_theta == f["rope_theta"]
            assert cfg.softmax_scale == 1.0 / math.sqrt(f["d_head"] + f["d_rope"]) == 1.0 / math.sqrt(80)
        else:
            assert cfg.softmax_scale == 1.0 / math.sqrt(f["scale_sq"]) == 1.0 / math.sqrt(192)
