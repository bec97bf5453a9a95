"""The seeded input generators: storage conversions and layout (CPU)."""
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
