"""Parity of the fp8 matrix-core decode (MLA_DECODE_FP8_MATH) with the CPU
oracle, through the C ABI.

With the flag, an e4m3 cache's content scores are taken on the fp8 matrix
cores from the codes as stored, against queries rounded to e4m3 with a
power-of-two scale per 32 lanes; the rope part and the weighted sum stay in
bf16. The oracle is unchanged (fp64 on the dequantised cache and the bf16
queries), so the query rounding counts against the fp8 gate (max-abs 5e-2,
rel-Frobenius 3e-2). Every case prints its name and shape before touching
the GPU.
"""
import numpy as np
import pytest

import workloads as wl
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

C = wl.CONFIGS
F8 = 1   # MLA_DECODE_FP8_MATH
SMALL = wl.scaled(C["c5"], batch=4, seq_len=1000)


def _lse_tol(inp, batches=None, scale=None):
    return H.fp8_math_lse_tol(inp, batches, scale)


def _check(inp, o, lse, label, batches=None, scale=None):
    ro, rl = H.oracle_decode(inp, batches, scale=scale)
    H.assert_close(o, ro, "fp8", label)
    if lse is not None:
        H.assert_lse_close(lse, rl, _lse_tol(inp, batches, scale), label)
    return ro


def test_reduced_speculative_pair():
    H.say(f"case fp8-math c5-reduced B={SMALL.batch} S={SMALL.seq_len} q_len={SMALL.q_len}")
    inp = wl.make_decode_inputs(SMALL)
    o, lse = H.run_decode(inp, flags=F8)
    _check(inp, o, lse, "f8m-c5-reduced")


@pytest.mark.parametrize("variant", ["workload", "sharp", "needle"])
def test_full_size(variant):
    """The full c5 shape in the launch configuration the benchmark times, on
    the workload's own inputs and with sharp or needle attention; every
    sequence, both query tokens, all heads and lanes."""
    cfg = C["c5"]
    H.say(f"case fp8-math c5-full-{variant} B={cfg.batch} q_len={cfg.q_len}")
    inp = wl.make_decode_inputs(cfg) if variant == "workload" else H.stress_inputs(cfg, variant)
    o, lse = H.run_decode(inp, flags=F8)
    _check(inp, o, lse, f"f8m-c5-full-{variant}")


def test_close_to_the_dequantising_path():
    """The two fp8 paths differ only by the query rounding (and the order of
    the sums): their outputs agree well inside the gate."""
    H.say("case fp8-math vs dequantised path")
    inp = wl.make_decode_inputs(SMALL)
    dev = H.device_inputs(inp)
    a, la = H.run_decode(inp, dev=dev, flags=F8)
    b, lb = H.run_decode(inp, dev=dev)
    ma, rf = H.errors(a, b)
    H.say(f"  max-abs {ma:.3e}, rel-F {rf:.3e}, lse max-abs {np.max(np.abs(la - lb)):.3e}")
    assert rf < 1e-2 and np.max(np.abs(la - lb)) < _lse_tol(inp)


@pytest.mark.parametrize("parts", [1, 7, 20, 0])
def test_split_count_invariance(parts):
    cfg = wl.scaled(C["c5"], batch=2, seq_len=1500)
    H.say(f"case fp8-math split parts={parts}")
    inp = wl.make_decode_inputs(cfg, q_mult=27.7)
    o, lse = H.run_decode(inp, num_partitions=parts, flags=F8)
    _check(inp, o, lse, f"f8m-parts={parts}")


def test_sequence_length_edges():
    lens = [0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 4097]
    cfg = wl.scaled(C["c5"], q_len=1, batch=len(lens), seq_len=None, ragged=(0, 1))
    H.say(f"case fp8-math length-edges lens={lens}")
    inp = wl.make_decode_inputs(cfg, seq_lens=lens, q_mult=27.7)
    o, lse = H.run_decode(inp, flags=F8)
    _check(inp, o, lse, "f8m-edges")
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))


@pytest.mark.parametrize("S", [1, 2, 3, 65])
def test_speculative_pair_short_sequences(S):
    cfg = wl.scaled(C["c5"], batch=2, seq_len=S)
    H.say(f"case fp8-math q_len=2 S={S}")
    inp = wl.make_decode_inputs(cfg, q_mult=27.7)
    o, lse = H.run_decode(inp, flags=F8)
    _check(inp, o, lse, f"f8m-pair-S{S}")
    if S == 1:
        assert np.all(o[:, 0] == 0) and np.all(np.isneginf(lse[:, 0]))


@pytest.mark.parametrize("n_h,q_len", [(32, 4), (64, 2)])
def test_row_groups_spanning_several_query_tokens(n_h, q_len):
    cfg = wl.scaled(C["c5"], batch=3, n_heads=n_h, q_len=q_len, seq_len=None, ragged=(1, 300))
    H.say(f"case fp8-math n_h={n_h} q_len={q_len}")
    inp = wl.make_decode_inputs(cfg, seq_lens=[1 + q_len, 97, 250])
    o, lse = H.run_decode(inp, flags=F8)
    _check(inp, o, lse, f"f8m-rows-n{n_h}-q{q_len}")


def test_fp32_output():
    cfg = wl.scaled(SMALL, out_dtype="fp32")
    H.say("case fp8-math fp32 output")
    inp = wl.make_decode_inputs(cfg)
    o, lse = H.run_decode(inp, flags=F8)
    _check(inp, o, lse, "f8m-fp32out")


@pytest.mark.parametrize("factor", [-1.0, 0.0])
def test_negative_and_zero_scale(factor):
    scale = factor * SMALL.softmax_scale
    H.say(f"case fp8-math scale={scale:+.4g}")
    inp = wl.make_decode_inputs(SMALL)
    o, lse = H.run_decode(inp, scale=scale, flags=F8)
    _check(inp, o, lse, f"f8m-scale{factor:+g}", scale=scale)


def test_bitwise_determinism():
    cfg = wl.scaled(C["c5"], batch=5, seq_len=None, ragged=(100, 3000))
    H.say("case fp8-math determinism")
    inp = wl.make_decode_inputs(cfg, q_mult=27.7)
    dev = H.device_inputs(inp)
    a = H.run_decode(inp, dev=dev, flags=F8)
    b = H.run_decode(inp, dev=dev, flags=F8)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_batch_above_the_in_kernel_prefix_limit():
    """More than 256 sequences: in this mode the kernel reads the prefix sums
    the plan kernel wrote (its query staging leaves less LDS for them)."""
    cfg = wl.scaled(C["c5"], q_len=1, batch=300, seq_len=None, ragged=(1, 130))
    H.say(f"case fp8-math B={cfg.batch} (plan kernel path)")
    inp = wl.make_decode_inputs(cfg)
    o, lse = H.run_decode(inp, flags=F8)
    pick = sorted({0, 1, 2, 255, 256, 257, 298, 299} | set(range(10, 300, 37)))
    _check(inp, o[pick], lse[pick], "f8m-B300", pick)


@pytest.mark.parametrize("batch", [255, 256])
def test_batch_at_the_in_kernel_prefix_limit(batch):
    cfg = wl.scaled(C["c5"], q_len=1, batch=batch, seq_len=None, ragged=(1, 130))
    H.say(f"case fp8-math B={batch} (in-kernel prefix sums)")
    inp = wl.make_decode_inputs(cfg)
    o, lse = H.run_decode(inp, flags=F8)
    pick = sorted({0, 1, 127, 128, batch - 2, batch - 1} | set(range(5, batch, 41)))
    _check(inp, o[pick], lse[pick], f"f8m-B{batch}", pick)


@pytest.mark.parametrize("variant", ["rope_only", "needle"])
def test_stress(variant):
    """Attention dominated by the bf16 rope part (which the flag leaves in
    bf16): the same gate as the workload."""
    cfg = wl.scaled(SMALL, batch=3)
    H.say(f"case fp8-math stress {variant}")
    inp = wl.make_decode_inputs(cfg, q_mult=27.7)
    if variant == "rope_only":
        inp.q_abs_bits[...] = 0
    else:
        inp.q_rope_bits[...] = 0
        inp.q_rope_bits[..., 0] = wl.to_bf16_bits(np.array([1.0]))[0]
        rng = np.random.default_rng(77)
        for b in range(cfg.batch):
            j = int(rng.integers(0, inp.seq_lens[b] - cfg.q_len + 1))
            inp.krope_bits[b][j, :] = 0
            inp.krope_bits[b][j, 0] = wl.to_bf16_bits(np.array([20.0 / cfg.softmax_scale]))[0]
    o, lse = H.run_decode(inp, flags=F8)
    _check(inp, o, lse, f"f8m-stress-{variant}")


@pytest.mark.parametrize("variant", ["sharp", "content_only"])
def test_sharp_content_scores_error_report(variant):
    """Much sharper content scores (queries x 600: logits spread over a few
    units): the query rounding to 3 mantissa bits moves each logit by about
    2.6% of its size, so the error grows with the spread of the scores. The
    test reports it and bounds it loosely (rel-Frobenius 0.1): this is what
    the flag trades for speed."""
    cfg = wl.scaled(SMALL, batch=3)
    H.say(f"case fp8-math sharp {variant}")
    inp = wl.make_decode_inputs(cfg, q_mult=600.0)
    if variant == "content_only":
        inp.q_rope_bits[...] = 0
    o, lse = H.run_decode(inp, flags=F8)
    ro, rl = H.oracle_decode(inp)
    ma, rf = H.errors(o, ro)
    H.say(f"  [f8m-{variant}] max-abs {ma:.3e}, rel-F {rf:.3e}, "
          f"lse max-abs {np.max(np.abs(lse - rl)):.3e}")
    assert rf < 0.1
    H.assert_lse_close(lse, rl, _lse_tol(inp), f"f8m-{variant}")


def test_flag_has_no_effect_on_a_bf16_cache():
    """The flag only changes how an fp8 cache is multiplied: with a bf16
    cache the results are bitwise those of the call without it."""
    cfg = wl.scaled(C["c2"], batch=3, seq_len=700)
    H.say("case fp8-math flag on a bf16 cache")
    inp = wl.make_decode_inputs(cfg)
    dev = H.device_inputs(inp)
    a = H.run_decode(inp, dev=dev, flags=F8)
    b = H.run_decode(inp, dev=dev)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("flags", [0, F8])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_restart_on_a_late_larger_logit(dtype, flags):
    """One page range for the whole batch (num_partitions=1: one workgroup
    walks both sequences), and rope needles in late chunks whose logits
    exceed everything before them by far more than the lazy-reference
    threshold (2^8): each sequence's pass raises its reference twice and
    restarts, and the result must still match the oracle."""
    base = C["c2"] if dtype == "bf16" else C["c5"]
    cfg = wl.scaled(base, batch=2, q_len=1, seq_len=700)
    H.say(f"case restart {dtype} flags={flags}")
    inp = wl.make_decode_inputs(cfg)
    inp.q_rope_bits[...] = 0
    inp.q_rope_bits[..., 0] = wl.to_bf16_bits(np.array([1.0]))[0]
    for b in range(cfg.batch):
        kr = inp.krope_bits[b] if dtype == "fp8" else inp.lat_bits[b][:, cfg.d_c:]
        for j, logit in ((300, 12.0), (650, 24.0)):   # chunks 9 and 20 of the pass
            kr[j, :] = 0
            kr[j, 0] = wl.to_bf16_bits(np.array([logit / cfg.softmax_scale]))[0]
    o, lse = H.run_decode(inp, num_partitions=1, flags=flags)
    ro, rl = H.oracle_decode(inp)
    H.assert_close(o, ro, dtype, f"restart-{dtype}-{flags}")
    tol = 2e-3 if flags == 0 or dtype == "bf16" else _lse_tol(inp)
    H.assert_lse_close(lse, rl, tol, f"restart-{dtype}-{flags}")
