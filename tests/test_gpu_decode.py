"""Parity of the HIP decode path (through the C ABI) with the CPU oracle.

Every case prints its name and shape before touching the GPU. Gates: bf16
max-abs 2e-2 / rel-Frobenius 1e-2, fp8 5e-2 / 3e-2, fp32 held to the bf16
gate plus a tight fp32 check.
"""
import math

import numpy as np
import pytest

import workloads as wl
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

C = wl.CONFIGS

# reduced cases: several 64-token tiles, ragged tails, many splits
SMALL = {
    "c2": wl.scaled(C["c2"], batch=3, seq_len=700),
    "c3": wl.scaled(C["c3"], batch=2, seq_len=5000),
    "c4": wl.scaled(C["c4"], batch=6, ragged=(1, 2000)),
    "c5": wl.scaled(C["c5"], batch=4, seq_len=1000),
}


def _kind(cfg):
    return cfg.cache_dtype


def _check(inp, o, lse, label, batches=None):
    ro, rl = H.oracle_decode(inp, batches)
    H.assert_close(o, ro, _kind(inp.cfg), label)
    if lse is not None:
        H.assert_lse_close(lse, rl, 2e-3, label)
    return ro


def test_tiny_fp32_config():
    cfg = C["tiny"]
    H.say(f"case tiny fp32 B={cfg.batch} S={cfg.seq_len} n_h={cfg.n_heads} d_c={cfg.d_c}")
    inp = wl.make_decode_inputs(cfg)
    o, lse = H.run_decode(inp)
    ro = _check(inp, o, lse, "tiny")
    ma, rf = H.errors(o, ro)
    assert rf < 1e-5, rf   # fp32 arithmetic throughout


@pytest.mark.parametrize("name", ["c2", "c3", "c4", "c5"])
def test_reduced_configs(name):
    cfg = SMALL[name]
    H.say(f"case {name}-reduced lens={cfg.seq_len or cfg.ragged} B={cfg.batch} q_len={cfg.q_len}")
    inp = wl.make_decode_inputs(cfg)
    o, lse = H.run_decode(inp)
    _check(inp, o, lse, f"{name}-reduced")


@pytest.mark.parametrize("name", ["c2", "c3", "c4", "c5"])
def test_full_size_configs(name):
    """Full shapes, the launch configuration the benchmark times (automatic
    partitions). The oracle checks every sequence, element by element."""
    cfg = C[name]
    H.say(f"case {name}-full B={cfg.batch} q_len={cfg.q_len} ({cfg.cache_dtype})")
    inp = wl.make_decode_inputs(cfg)
    o, lse = H.run_decode(inp)
    _check(inp, o, lse, f"{name}-full")


@pytest.mark.parametrize("parts", [1, 2, 7, 20, 0, 100])
def test_split_count_invariance(parts):
    """Results do not depend on the number of page ranges. With 2 sequences of
    24 pages: 1, 2 and 7 ranges merge with one wavefront per row, 20 with two
    (more than 8 ranges per sequence), the automatic 48 with four and 100
    (more ranges than pages: some are empty) with eight."""
    cfg = wl.scaled(C["c2"], batch=2, seq_len=1500)
    H.say(f"case split-invariance parts={parts}")
    inp = wl.make_decode_inputs(cfg, q_mult=27.7)
    o, lse = H.run_decode(inp, num_partitions=parts)
    _check(inp, o, lse, f"parts={parts}")


@pytest.mark.parametrize("base", ["c2", "c5"])
def test_fp32_output_on_the_matrix_core_path(base):
    """fp32 output: the matrix-core kernel then keeps fp32 unnormalised partials
    (with their row sums) and the combine writes fp32."""
    cfg = wl.scaled(SMALL[base], out_dtype="fp32")
    H.say(f"case fp32 output on {base}-reduced")
    inp = wl.make_decode_inputs(cfg)
    o, lse = H.run_decode(inp)
    ro, rl = H.oracle_decode(inp)
    H.assert_close(o, ro, _kind(cfg), f"fp32out-{base}")
    H.assert_lse_close(lse, rl, 2e-3, f"fp32out-{base}")


@pytest.mark.parametrize("n_h,q_len,dtype", [(64, 2, "bf16"), (16, 8, "bf16"), (32, 4, "fp8")])
def test_row_groups_spanning_several_query_tokens(n_h, q_len, dtype):
    """Fewer than 128 heads: a 128-row group of the matrix-core kernel holds
    several query tokens, so the causal limit differs between the lanes of a
    wavefront (including chunks that end inside the speculative window)."""
    base = C["c2"] if dtype == "bf16" else C["c5"]
    cfg = wl.scaled(base, batch=3, n_heads=n_h, q_len=q_len, seq_len=None, ragged=(1, 300))
    H.say(f"case n_h={n_h} q_len={q_len} {dtype} rows={n_h * q_len}")
    inp = wl.make_decode_inputs(cfg, seq_lens=[1 + q_len, 97, 250])
    o, lse = H.run_decode(inp)
    ro, rl = H.oracle_decode(inp)
    H.assert_close(o, ro, _kind(cfg), f"rows-n{n_h}-q{q_len}")
    H.assert_lse_close(lse, rl, 2e-3, f"rows-n{n_h}-q{q_len}")


def test_page_permutation_is_bitwise_invariant():
    cfg = wl.scaled(C["c2"], batch=3, seq_len=333)
    H.say("case page-permutation")
    a = wl.make_decode_inputs(cfg, q_mult=27.7)
    b = wl.make_decode_inputs(cfg, q_mult=27.7)
    b.page_perm = np.random.default_rng(9).permutation(len(a.page_perm)).astype(np.int32)
    oa, la = H.run_decode(a)
    ob, lb = H.run_decode(b)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_sequence_length_edges(dtype):
    base = C["c2"] if dtype == "bf16" else wl.scaled(C["c5"], q_len=1)
    lens = [0, 1, 2, 63, 64, 65, 127, 4097]
    cfg = wl.scaled(base, batch=len(lens), seq_len=None, ragged=(0, 1))
    H.say(f"case length-edges {dtype} lens={lens}")
    inp = wl.make_decode_inputs(cfg, seq_lens=lens, q_mult=27.7)
    o, lse = H.run_decode(inp)
    ro = _check(inp, o, lse, f"edges-{dtype}")
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))   # empty sequence


@pytest.mark.parametrize("S", [1, 2, 3, 65])
def test_speculative_pair_short_sequences(S):
    cfg = wl.scaled(C["c5"], batch=2, seq_len=S)
    H.say(f"case q_len=2 S={S}")
    inp = wl.make_decode_inputs(cfg, q_mult=27.7)
    o, lse = H.run_decode(inp)
    _check(inp, o, lse, f"pair-S{S}")
    if S == 1:   # the first query of the pair sees nothing
        assert np.all(o[:, 0] == 0) and np.all(np.isneginf(lse[:, 0]))


def test_bitwise_determinism():
    cfg = wl.scaled(C["c4"], batch=5, ragged=(100, 3000))
    H.say("case determinism")
    inp = wl.make_decode_inputs(cfg, q_mult=27.7)
    dev = H.device_inputs(inp)
    a = H.run_decode(inp, dev=dev)
    b = H.run_decode(inp, dev=dev)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_plan_once_decode_many():
    cfg = wl.scaled(C["c4"], batch=4, ragged=(10, 900))
    H.say("case plan-ready")
    inp = wl.make_decode_inputs(cfg)
    dev = H.device_inputs(inp)
    a = H.run_decode(inp, dev=dev)
    b = H.run_decode(inp, dev=dev, plan_separately=True)
    assert np.array_equal(a[0], b[0])


def test_no_lse_output():
    cfg = SMALL["c2"]
    H.say("case lse=NULL")
    inp = wl.make_decode_inputs(cfg)
    o, _ = H.run_decode(inp, with_lse=False)
    _check(inp, o, None, "no-lse")


# ----------------------------------------------------------------------------
# stress self-checks: sharper attention than the gated workloads
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("base", ["c2", "c5"])
@pytest.mark.parametrize("variant", ["sharp", "rope_only", "content_only", "needle"])
def test_stress(base, variant):
    cfg = wl.scaled(SMALL[base], batch=3)
    H.say(f"case stress {base} {variant}")
    inp = H.stress_inputs(cfg, variant)
    o, lse = H.run_decode(inp)
    _check(inp, o, lse, f"stress-{base}-{variant}")


@pytest.mark.parametrize("name", ["c2", "c3", "c4", "c5"])
@pytest.mark.parametrize("variant", ["sharp", "needle"])
def test_full_size_sharp_attention(name, variant):
    """The full shapes in the launch configuration the benchmark times (8-page
    pieces on c2, 64 ranges per sequence and the four-wavefront merge on c3,
    permuted ragged pages on c4, whole-sequence direct output on c5), with
    attention sharp enough that a kernel that ignored the scores, or a rope
    or causal mistake, fails the gate. Every sequence, element by element."""
    cfg = C[name]
    H.say(f"case {name}-full-{variant} B={cfg.batch} q_len={cfg.q_len} ({cfg.cache_dtype})")
    inp = H.stress_inputs(cfg, variant)
    o, lse = H.run_decode(inp)
    _check(inp, o, lse, f"{name}-full-{variant}")


def test_validate_catches_bad_contents():
    import torch
    m = H.lib()
    cfg = wl.scaled(C["c2"], batch=2, seq_len=130)
    H.say("case validate")
    inp = wl.make_decode_inputs(cfg)
    dev = H.device_inputs(inp)
    desc = m.decode_desc(cfg.batch, 1, cfg.n_heads, cfg.d_c, cfg.d_rope, dev["max_blocks"])
    m.mla_decode_validate(desc, dev["seq_lens"], dev["block_table"], dev["n_pages"])
    bad = dev["block_table"].clone()
    bad[1, 2] = dev["n_pages"]
    with pytest.raises(m.MlaError) as e:
        m.mla_decode_validate(desc, dev["seq_lens"], bad, dev["n_pages"])
    assert e.value.status == m.MLA_ERR_BAD_CONTENTS
    long = torch.tensor([130, 64 * dev["max_blocks"] + 1], dtype=torch.int32, device="cuda")
    with pytest.raises(m.MlaError):
        m.mla_decode_validate(desc, long, dev["block_table"], dev["n_pages"])
    # with two query tokens a non-empty sequence needs at least two cached
    # tokens; an empty one is still accepted
    desc2 = m.decode_desc(cfg.batch, 2, cfg.n_heads, cfg.d_c, cfg.d_rope, dev["max_blocks"])
    m.mla_decode_validate(desc2, dev["seq_lens"], dev["block_table"], dev["n_pages"])
    for lens, ok in (([0, 2], True), ([1, 130], False)):
        t = torch.tensor(lens, dtype=torch.int32, device="cuda")
        if ok:
            m.mla_decode_validate(desc2, t, dev["block_table"], dev["n_pages"])
        else:
            with pytest.raises(m.MlaError) as e:
                m.mla_decode_validate(desc2, t, dev["block_table"], dev["n_pages"])
            assert e.value.status == m.MLA_ERR_BAD_CONTENTS


def test_batch_above_the_in_kernel_prefix_limit():
    """More than 1024 sequences: the matrix-core kernel reads the page prefix
    sums the plan kernel wrote instead of forming them itself."""
    cfg = wl.scaled(C["c4"], batch=1100, ragged=(1, 130))
    H.say(f"case large batch B={cfg.batch} lens={cfg.ragged} (plan kernel path)")
    inp = wl.make_decode_inputs(cfg)
    o, lse = H.run_decode(inp)
    pick = sorted({0, 1, 2, 511, 1023, 1024, 1025, 1098, 1099} | set(range(100, 1100, 97)))
    ro, rl = H.oracle_decode(inp, pick)
    H.assert_close(o[pick], ro, "bf16", "large-batch")
    H.assert_lse_close(lse[pick], rl, 2e-3, "large-batch")


@pytest.mark.parametrize("batch", [1023, 1024])
def test_batch_at_the_in_kernel_prefix_limit(batch):
    """1023 and 1024 sequences: the largest batches whose page prefix sums
    the matrix-core kernel forms itself (at 1024 no thread's sequences reach
    index B, so the total is stored separately)."""
    cfg = wl.scaled(C["c4"], batch=batch, ragged=(1, 130))
    H.say(f"case batch B={cfg.batch} lens={cfg.ragged} (in-kernel prefix sums)")
    inp = wl.make_decode_inputs(cfg)
    o, lse = H.run_decode(inp)
    pick = sorted({0, 1, 2, 255, 256, 511, 767, 1020, batch - 2, batch - 1} | set(range(100, batch, 89)))
    ro, rl = H.oracle_decode(inp, pick)
    H.assert_close(o[pick], ro, "bf16", f"batch{batch}")
    H.assert_lse_close(lse[pick], rl, 2e-3, f"batch{batch}")


@pytest.mark.parametrize("base,factor", [("c2", -1.0), ("c2", 0.0), ("c5", -1.0)])
def test_negative_and_zero_scale(base, factor):
    """The softmax scale enters the formula as given: a negative scale flips
    the scores (the matrix-core kernel negates the queries, exactly), a zero
    scale gives the mean latent."""
    cfg = SMALL[base]
    scale = factor * cfg.softmax_scale
    H.say(f"case scale={scale:+.4g} on {base}-reduced")
    inp = wl.make_decode_inputs(cfg)
    o, lse = H.run_decode(inp, scale=scale)
    ro, rl = H.oracle_decode(inp, scale=scale)
    H.assert_close(o, ro, _kind(cfg), f"scale{factor:+g}-{base}")
    H.assert_lse_close(lse, rl, 2e-3, f"scale{factor:+g}-{base}")


@pytest.mark.parametrize("n_h,q_len,dtype,flags", [
    (16, 1, "bf16", 0), (32, 1, "bf16", 0), (8, 1, "bf16", 0), (48, 2, "bf16", 0),
    (96, 2, "bf16", 0), (16, 2, "fp8", 0), (16, 1, "fp8", 1), (40, 3, "fp8", 1),
])
def test_row_counts_that_pad_the_last_row_group(n_h, q_len, dtype, flags):
    """q_len x n_heads not a multiple of 128 (for example 16 local heads of a
    head-sharded model): the matrix-core kernel pads the last 128-row group;
    its missing rows load the group's first query row and are never stored.
    96 x 2 = 192 rows gives one full group and one with 64 rows."""
    base = C["c2"] if dtype == "bf16" else C["c5"]
    cfg = wl.scaled(base, batch=3, n_heads=n_h, q_len=q_len, seq_len=None, ragged=(1, 300))
    H.say(f"case padded rows n_h={n_h} q_len={q_len} rows={n_h * q_len} {dtype} flags={flags}")
    inp = wl.make_decode_inputs(cfg, seq_lens=[q_len, 97, 700], q_mult=27.7)
    o, lse = H.run_decode(inp, flags=flags)
    ro, rl = H.oracle_decode(inp)
    H.assert_close(o, ro, _kind(cfg), f"pad-n{n_h}-q{q_len}-{dtype}-{flags}")
    tol = 2e-3 if flags == 0 else H.fp8_math_lse_tol(inp)
    H.assert_lse_close(lse, rl, tol, f"pad-n{n_h}-q{q_len}-{dtype}-{flags}")


@pytest.mark.parametrize("dtype,flags", [("bf16", 0), ("fp8", 0), ("fp8", 1)])
def test_pages_beyond_four_gib(dtype, flags):
    """Page ids whose byte offsets exceed 2^32: the sequences' pages sit at
    the top of a pool of a little over 4 GiB (the rest of the pool is never
    read), so every cache address needs 64-bit arithmetic."""
    import torch
    base = C["c2"] if dtype == "bf16" else C["c5"]
    cfg = wl.scaled(base, batch=2, seq_len=300)
    H.say(f"case pages beyond 4 GiB {dtype} flags={flags}")
    inp = wl.make_decode_inputs(cfg)
    dev = H.device_inputs(inp)
    pool = dev["cache"]
    page_bytes = pool[0].numel() * pool.element_size()
    first = (1 << 32) // page_bytes + 7          # first page id used
    big = torch.empty((first + pool.shape[0],) + tuple(pool.shape[1:]), dtype=pool.dtype,
                      device="cuda")
    big[first:] = pool
    assert first * page_bytes > (1 << 32)
    dev["cache"] = big
    if dev["cache_scale"] is not None:
        sbig = torch.empty((first + pool.shape[0], 64), dtype=torch.float32, device="cuda")
        sbig[first:] = dev["cache_scale"]
        dev["cache_scale"] = sbig
    bt = dev["block_table"]
    dev["block_table"] = torch.where(bt >= 0, bt + first, bt)
    dev["n_pages"] = first + pool.shape[0]
    o, lse = H.run_decode(inp, dev=dev, flags=flags)
    ro, rl = H.oracle_decode(inp)
    H.assert_close(o, ro, _kind(cfg), f"4GiB-{dtype}-{flags}")
    tol = 2e-3 if flags == 0 else H.fp8_math_lse_tol(inp)
    H.assert_lse_close(lse, rl, tol, f"4GiB-{dtype}-{flags}")


@pytest.mark.parametrize("dtype,flags", [("bf16", 0), ("fp8", 1)])
def test_graph_capture_replays_match_eager(dtype, flags):
    """mla_decode issues kernels only (no allocation, no memset, no host
    synchronisation), so it can be captured in a HIP graph: the graph is
    replayed with new queries written into the captured buffers, with eager
    work between replays, and every replay matches an eager call bitwise."""
    import torch
    m = H.lib()
    base = C["c2"] if dtype == "bf16" else C["c5"]
    cfg = wl.scaled(base, batch=3, seq_len=900)
    H.say(f"case graph capture {dtype} flags={flags}")
    inp = wl.make_decode_inputs(cfg)
    dev = H.device_inputs(inp)
    desc = m.decode_desc(cfg.batch, cfg.q_len, cfg.n_heads, cfg.d_c, cfg.d_rope, dev["max_blocks"],
                         cfg.cache_dtype, "bf16", cfg.out_dtype, flags=flags)
    ws = torch.empty(m.mla_decode_workspace_size(desc), dtype=torch.uint8, device="cuda")
    qa, qr = dev["q_abs"].clone(), dev["q_rope"].clone()
    shape = (cfg.batch, cfg.q_len, cfg.n_heads, cfg.d_c)
    o_g = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    l_g = torch.empty(shape[:3], dtype=torch.float32, device="cuda")

    def call(q1, q2, o, lse):
        m.mla_decode(desc, q1, q2, dev["cache"], dev["cache_scale"], dev["block_table"],
                     dev["seq_lens"], cfg.softmax_scale, o, lse, ws)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call(qa, qr, o_g, l_g)   # warm-up on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(qa, qr, o_g, l_g)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda").manual_seed(5)
    for rep in range(3):
        qa.copy_((torch.randn(qa.shape, device="cuda", generator=gen) * 0.05).to(qa.dtype))
        qr.copy_((torch.randn(qr.shape, device="cuda", generator=gen) * 0.05).to(qr.dtype))
        o_e = torch.empty_like(o_g)
        l_e = torch.empty_like(l_g)
        call(qa, qr, o_e, l_e)   # eager reference (and eager work between replays)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e) and torch.equal(l_g, l_e), f"replay {rep}"


@pytest.mark.parametrize("seed", range(12))
def test_random_shape_sweep(seed):
    """Seeded random shapes on the matrix-core path: batch, ragged lengths,
    head count (any, so row groups pad), query tokens, cache dtype, fp8 flag,
    split count and output dtype, each against the oracle."""
    rng = np.random.default_rng(1000 + seed)
    dtype = ["bf16", "fp8"][int(rng.integers(0, 2))]
    flags = int(rng.integers(0, 2)) if dtype == "fp8" else 0
    n_h = int(rng.choice([1, 3, 8, 16, 24, 40, 64, 100, 128]))
    q_len = int(rng.integers(1, 5))
    batch = int(rng.integers(1, 5))
    lens = [int(x) for x in rng.integers(q_len, 900, size=batch)]
    parts = int(rng.choice([0, 1, 3, 11]))
    out = ["bf16", "fp32"][int(rng.integers(0, 2))]
    base = C["c2"] if dtype == "bf16" else C["c5"]
    cfg = wl.scaled(base, batch=batch, n_heads=n_h, q_len=q_len, seq_len=None,
                    ragged=(1, 900), out_dtype=out)
    H.say(f"case sweep seed={seed} {dtype} flags={flags} n_h={n_h} q_len={q_len} "
          f"lens={lens} parts={parts} out={out}")
    inp = wl.make_decode_inputs(cfg, seq_lens=lens, q_mult=27.7)
    o, lse = H.run_decode(inp, num_partitions=parts, flags=flags)
    ro, rl = H.oracle_decode(inp)
    H.assert_close(o, ro, _kind(cfg), f"sweep-{seed}")
    tol = 2e-3 if flags == 0 else H.fp8_math_lse_tol(inp)
    H.assert_lse_close(lse, rl, tol, f"sweep-{seed}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_partial_then_combine_matches_the_fused_call(dtype):
    """mla_decode_partial followed by mla_decode_combine (partials for every
    piece) against mla_decode (which writes the sequences that one piece
    covers whole straight from its accumulators): both match the oracle, and
    the sequences cut into several pieces agree bitwise."""
    import torch
    m = H.lib()
    base = C["c2"] if dtype == "bf16" else wl.scaled(C["c5"], q_len=1)
    cfg = wl.scaled(base, batch=4, seq_len=None, ragged=(1, 3000))
    lens = [700, 64, 3000, 0]
    H.say(f"case partial+combine {dtype} lens={lens}")
    inp = wl.make_decode_inputs(cfg, seq_lens=lens, q_mult=27.7)
    dev = H.device_inputs(inp)
    o1, l1 = H.run_decode(inp, dev=dev, num_partitions=5)
    desc = m.decode_desc(cfg.batch, cfg.q_len, cfg.n_heads, cfg.d_c, cfg.d_rope, dev["max_blocks"],
                         cfg.cache_dtype, "bf16", cfg.out_dtype, 5)
    ws = torch.empty(m.mla_decode_workspace_size(desc), dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)
    o2 = torch.full((cfg.batch, cfg.q_len, cfg.n_heads, cfg.d_c), float("nan"),
                    dtype=torch.bfloat16, device="cuda")
    l2 = torch.full((cfg.batch, cfg.q_len, cfg.n_heads), float("nan"), dtype=torch.float32,
                    device="cuda")
    m.mla_decode_partial(desc, dev["q_abs"], dev["q_rope"], dev["cache"], dev["cache_scale"],
                         dev["block_table"], dev["seq_lens"], cfg.softmax_scale, ws)
    m.mla_decode_combine(desc, ws, o2, l2)
    torch.cuda.synchronize()
    o2 = o2.float().cpu().numpy().astype(np.float64)
    l2 = l2.cpu().numpy().astype(np.float64)
    ro, rl = H.oracle_decode(inp)
    for o, l, tag in ((o1, l1, "fused"), (o2, l2, "split")):
        H.assert_close(o, ro, _kind(cfg), f"{tag}-{dtype}")
        H.assert_lse_close(l, rl, 2e-3, f"{tag}-{dtype}")
    # pages 11, 1, 47, 0 in 5 ranges starting at pages 0, 11, 23, 35, 47:
    # sequences 0 and 1 lie inside one range each (written directly by the
    # fused call, without the bf16 partial rounding of the split path),
    # sequence 2 crosses four ranges, sequence 3 is empty
    assert np.array_equal(o1[2], o2[2]) and np.array_equal(l1[2], l2[2])
    for b in (0, 1):
        assert np.max(np.abs(o1[b] - o2[b])) < 1e-3, b
    assert np.all(o1[3] == 0) and np.all(o2[3] == 0) and np.all(np.isneginf(l1[3]))
