"""Parity of the prefill path (the unabsorbed layer over whole prompts) with
the CPU oracle, through the C ABI: the bf16 matrix-core GEMM, the causal
attention over expanded keys and values, and the whole layer against the
unabsorbed definition O1.

Gates (bf16 arithmetic with fp32 accumulation; every intermediate activation
is rounded to bf16 between products, each rounding within 2^-9 of the value):
the layer output and the attention output at relative Frobenius 1e-2 and
max-abs 2e-2 of the reference's largest magnitude; log-sum-exps within 2e-2;
the latent rows (one fp32-accumulated product of bf16 values) and fp32 GEMM
outputs at a bound of 4 K 2^-24 sum_k |a_k b_k| per element.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu
P = wl.PREFILL_CONFIGS


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def b64(bits: np.ndarray) -> np.ndarray:
    return wl.bf16_bits_as_f32(bits).astype(np.float64)


def rel_errors(g, r):
    g, r = np.asarray(g, np.float64), np.asarray(r, np.float64)
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    return float(np.max(np.abs(g - r))), float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))


def assert_bf16_gate(g, r, label):
    ma, rf = rel_errors(g, r)
    scale = float(np.max(np.abs(r)))
    H.say(f"  [{label}] max-abs {ma:.3e} (gate {2e-2 * scale:.3e}), rel-F {rf:.3e} (gate 1e-2)")
    assert rf <= 1e-2 and ma <= 2e-2 * scale, (label, ma, rf)


# ----------------------------------------------------------------------------
# the GEMM
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K,splits,out", [
    (1, 1, 8, 1, "fp32"), (37, 129, 200, 1, "fp32"), (128, 128, 64, 1, "bf16"),
    (300, 257, 1032, 1, "fp32"), (300, 257, 1032, 4, "fp32"), (32, 640, 4096, 8, "bf16"),
    (513, 96, 72, 1, "bf16"),
    # grids of at least 240 tiles of 256 x 256 (x splits), K a multiple of 32
    # and at least 1024 k per split take the large-tile kernel: ragged M and N
    # edges, both output forms, split-K (full rows checked at the tile edges
    # and at random)
    (2000, 7777, 1024, 1, "fp32"), (4096, 3900, 1536, 1, "bf16"), (512, 7680, 4096, 4, "fp32"),
    # the same grids with short k ranges stay on the 128 x 128 tile
    (2000, 7777, 96, 1, "fp32"), (1100, 4100, 512, 3, "bf16")])
def test_gemm_matches_float64(M, N, K, splits, out):
    m = H.lib()
    H.say(f"case gemm M={M} N={N} K={K} splits={splits} out={out}")
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    # A is a column slice of a wider matrix (row stride > K)
    Aw = wl.to_bf16_bits(rng.standard_normal((M, K + 24)))
    Bb = wl.to_bf16_bits(rng.standard_normal((N, K)))
    A = bf16_dev(Aw)[:, 8:8 + K]
    rows = np.arange(M)
    if M * N * K > 4e9:   # the fp64 reference on sampled full rows
        rows = np.array(sorted({0, 1, 31, 32, 127, 128, 255, 256, 511, M - 2, M - 1} |
                               set(rng.integers(0, M, 32).tolist())))
        rows = rows[rows < M]
    Ar = b64(Aw[rows, 8:8 + K])
    ref = Ar @ b64(Bb).T
    bound = 4 * K * 2.0 ** -24 * (np.abs(Ar) @ np.abs(b64(Bb)).T)
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    C = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
    part = None
    if splits > 1:
        part = torch.empty(m.mla_gemm_bf16_partial_size(M, N, K, splits) // 4, device="cuda")
    m.mla_gemm_bf16(A, bf16_dev(Bb), C, splits, part)
    torch.cuda.synchronize()
    Cf = C.float()
    assert bool(torch.isfinite(Cf).all()), "unwritten or non-finite outputs"
    g = Cf[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    if out == "fp32":
        assert np.all(np.abs(g - ref) <= bound + 1e-30)
    else:   # the fp32 result rounded once to bf16
        assert np.all(np.abs(g - ref) <= 2.0 ** -8 * np.abs(ref) + bound + 1e-30)
    if splits > 1:   # the split sum is in a fixed order
        C2 = torch.empty_like(C)
        m.mla_gemm_bf16(A, bf16_dev(Bb), C2, splits, part)
        torch.cuda.synchronize()
        assert torch.equal(C, C2)


# ----------------------------------------------------------------------------
# the attention over expanded keys and values
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dh,dr", [(64, 16), (128, 64), (64, 32), (128, 0)])
def test_attention_matches_the_oracle(dh, dr):
    m = H.lib()
    lens = [1, 32, 33, 167, 300]
    nh = 3
    cu = wl.prefill_cu_seqlens(lens)
    T = int(cu[-1])
    H.say(f"case prefill attention d_h={dh} d_R={dr} lens={lens} heads={nh}")
    rng = np.random.default_rng(dh + dr)
    q = wl.to_bf16_bits(rng.standard_normal((T, nh * dh)) * 0.3)
    qr = wl.to_bf16_bits(rng.standard_normal((T, nh * max(dr, 8))) * 0.3)
    k = wl.to_bf16_bits(rng.standard_normal((T, nh * dh)))
    kr = wl.to_bf16_bits(rng.standard_normal((T, max(dr, 8))))
    v = wl.to_bf16_bits(rng.standard_normal((T, nh * dh)))
    scale = oracle.score_scale(dh, dr)
    d = m.prefill_desc(len(lens), max(lens), 64, nh, dh, dr, 64)
    o = torch.full((T, nh * dh), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((nh, T), float("nan"), device="cuda")
    ldr = nh * max(dr, 8)
    m.mla_prefill_attention(d, T, bf16_dev(q), nh * dh, bf16_dev(qr), ldr, bf16_dev(k), nh * dh,
                            bf16_dev(kr), max(dr, 8), bf16_dev(v), nh * dh,
                            torch.from_numpy(cu).cuda(), scale, o, nh * dh, lse)
    torch.cuda.synchronize()
    g = o.float().cpu().numpy().astype(np.float64)
    gl = lse.cpu().numpy().astype(np.float64)
    ref = np.zeros((T, nh * dh))
    rl = np.zeros((nh, T))
    for b in range(len(lens)):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        for i in range(nh):
            hs = slice(i * dh, (i + 1) * dh)
            rs = slice(i * dr, (i + 1) * dr)
            e = oracle.expanded_attention(b64(q[s0:s1, hs]), b64(qr[s0:s1, rs]), b64(k[s0:s1, hs]),
                                          b64(kr[s0:s1, :dr]), b64(v[s0:s1, hs]), scale)
            ref[s0:s1, hs] = e["o"]
            rl[i, s0:s1] = e["lse"]
    assert_bf16_gate(g, ref, f"attn-{dh}-{dr}")
    err = float(np.max(np.abs(gl - rl)))
    H.say(f"  lse max-abs {err:.3e}")
    assert err <= 2e-2


# ----------------------------------------------------------------------------
# the whole layer against the unabsorbed definition
# ----------------------------------------------------------------------------

def _run_prefill(pcfg, model):
    m = H.lib()
    lay = wl.prefill_gpu_layout(model)
    T = pcfg.T
    d = m.prefill_desc(len(pcfg.seq_lens), max(pcfg.seq_lens), pcfg.d_model, pcfg.n_heads,
                       pcfg.d_head, pcfg.d_rope, pcfg.d_c, pcfg.d_cq, pcfg.rope_theta)
    ws = torch.empty(m.mla_prefill_workspace_size(d, T), dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)
    out = torch.full((T, pcfg.d_model), float("nan"), device="cuda")
    lat = torch.full((T, pcfg.d_c + pcfg.d_rope), float("nan"), device="cuda")
    lse = torch.full((pcfg.n_heads, T), float("nan"), device="cuda")
    w = {k: (None if v is None else bf16_dev(v)) for k, v in lay.items() if k != "h"}
    m.mla_prefill(d, bf16_dev(lay["h"]), torch.from_numpy(wl.prefill_cu_seqlens(pcfg.seq_lens)).cuda(),
                  torch.from_numpy(wl.prefill_positions(pcfg.seq_lens)).cuda(), w,
                  pcfg.softmax_scale, out, lat, lse, ws)
    torch.cuda.synchronize()
    return (out.cpu().numpy().astype(np.float64), lat.cpu().numpy().astype(np.float64),
            lse.cpu().numpy().astype(np.float64))


def _positions_to_check(pcfg):
    picks = []
    cu = wl.prefill_cu_seqlens(pcfg.seq_lens)
    rng = np.random.default_rng(pcfg.seed)
    for b, S in enumerate(pcfg.seq_lens):
        if pcfg.name == "prefill-tiny":
            ts = list(range(S))
        elif pcfg.name == "prefill-ds":
            # early positions, and the last of each quarter: the last is in the
            # heaviest query tile and sees every key
            ts = [0, 1, 63, 64, 200, 333, 1023, 2047, 4095]
        else:
            ts = sorted({0, 1, 31, 32, 127, 128, S - 1} | set(rng.integers(0, S, 3).tolist()))
        picks += [(b, int(cu[b]), t) for t in ts if t < S]
    return picks


@pytest.mark.parametrize("name", ["prefill-tiny", "prefill-mid", "prefill-ds"])
def test_prefill_layer_matches_the_unabsorbed_definition(name):
    pcfg = P[name]
    H.say(f"case {name} lens={pcfg.seq_lens} d={pcfg.d_model} heads={pcfg.n_heads}x{pcfg.d_head} "
          f"d_c={pcfg.d_c} d_R={pcfg.d_rope} d_cq={pcfg.d_cq}")
    model = wl.make_prefill_model(pcfg)
    out, lat, lse = _run_prefill(pcfg, model)
    picks = _positions_to_check(pcfg)
    g_out, r_out, g_lse, r_lse = [], [], [], []
    if name == "prefill-tiny":   # one prompt: O1 over every position at once
        r = oracle.mla_unabsorbed(model, q_len=pcfg.T)
        g_out, r_out = out, r["out"]
        g_lse, r_lse = lse.T, r["lse"]
        c, kR = r["c"], r["kR"]
        ref_lat = np.concatenate([c, kR], axis=1)
        g_lat = lat
    else:   # the output at position t depends on positions 0..t of its prompt only
        for b, s0, t in picks:
            sub = dataclasses.replace(model, H=model.H[s0:s0 + t + 1])
            r = oracle.mla_unabsorbed(sub, q_len=1)
            g_out.append(out[s0 + t]); r_out.append(r["out"][0])
            g_lse.append(lse[:, s0 + t]); r_lse.append(r["lse"][0])
        rows = [s0 + t for _, s0, t in picks]
        c, kR = oracle.cache_append(model.W_DKV, model.W_KR, model.H[rows],
                                    np.array([t for _, _, t in picks]), pcfg.rope_theta)
        ref_lat = np.concatenate([c, kR], axis=1)
        g_lat = lat[rows]
    assert_bf16_gate(np.array(g_out), np.array(r_out), f"{name}-out")
    err = float(np.max(np.abs(np.array(g_lse) - np.array(r_lse))))
    H.say(f"  [{name}] lse max-abs {err:.3e} (gate 2e-2)")
    assert err <= 2e-2
    # the latent rows: one bf16 x bf16 product accumulated in fp32, then RoPE
    K = pcfg.d_model
    Hr = model.H if name == "prefill-tiny" else model.H[[s0 + t for _, s0, t in picks]]
    Wl = np.concatenate([model.W_DKV, model.W_KR], axis=0).astype(np.float64)
    bound = 4 * K * 2.0 ** -24 * (np.abs(Hr.astype(np.float64)) @ np.abs(Wl).T) + 1e-6 * np.abs(ref_lat)
    lat_err = np.abs(g_lat - ref_lat)
    H.say(f"  [{name}] latent max-abs {float(lat_err.max()):.3e}")
    assert np.all(lat_err <= bound + 1e-30)


@pytest.mark.parametrize("name", ["prefill-tiny", "prefill-mid"])
def test_prefill_writes_only_its_outputs(name):
    """The layer with its output, latent rows, log-sum-exp and workspace each
    between guard regions: no guard byte changes, and the results equal those
    of the plain call bitwise (its kernels use no atomics: every sum has a
    fixed order)."""
    m = H.lib()
    pcfg = P[name]
    H.say(f"case prefill guards {name} lens={pcfg.seq_lens}")
    model = wl.make_prefill_model(pcfg)
    out0, lat0, lse0 = _run_prefill(pcfg, model)
    lay = wl.prefill_gpu_layout(model)
    T = pcfg.T
    d = m.prefill_desc(len(pcfg.seq_lens), max(pcfg.seq_lens), pcfg.d_model, pcfg.n_heads,
                       pcfg.d_head, pcfg.d_rope, pcfg.d_c, pcfg.d_cq, pcfg.rope_theta)
    ws = H.Guarded((m.mla_prefill_workspace_size(d, T),), torch.uint8)
    out = H.Guarded((T, pcfg.d_model), torch.float32)
    lat = H.Guarded((T, pcfg.d_c + pcfg.d_rope), torch.float32)
    lse = H.Guarded((pcfg.n_heads, T), torch.float32)
    w = {k: (None if v is None else bf16_dev(v)) for k, v in lay.items() if k != "h"}
    m.mla_prefill(d, bf16_dev(lay["h"]), torch.from_numpy(wl.prefill_cu_seqlens(pcfg.seq_lens)).cuda(),
                  torch.from_numpy(wl.prefill_positions(pcfg.seq_lens)).cuda(), w,
                  pcfg.softmax_scale, out.t, lat.t, lse.t, ws.t)
    torch.cuda.synchronize()
    for buf, nm in ((out, "the output"), (lat, "the latent rows"), (lse, "the log-sum-exp"),
                    (ws, "the workspace")):
        assert buf.guards_intact(), f"a store landed outside {nm}"
    assert np.array_equal(out.t.cpu().numpy().astype(np.float64), out0)
    assert np.array_equal(lat.t.cpu().numpy().astype(np.float64), lat0)
    assert np.array_equal(lse.t.cpu().numpy().astype(np.float64), lse0)
