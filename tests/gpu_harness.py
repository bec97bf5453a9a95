"""Helpers for the GPU tests: move seeded workloads to the device, call the
library through its binding, and compare with the CPU oracle."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
import workloads as wl

TOL = {  # (max-abs, relative Frobenius) gates of the decode output
    "bf16": (2e-2, 1e-2),
    "fp8": (5e-2, 3e-2),
    "fp32": (2e-2, 1e-2),
}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def lib():
    import latent_kv_cache_mla_amd as m
    return m


from workloads.device import device_inputs, to_dev  # noqa: E402,F401


GUARD = 4096          # guard bytes on each side of a guarded buffer
PATTERN = 0x5A


class Guarded:
    """A device buffer of `shape` and `dtype` between two guard regions; the
    inside starts as `fill` (a byte)."""

    def __init__(self, shape, dtype, fill=0xFF):
        esz = torch.empty((), dtype=dtype).element_size()
        self.n = int(np.prod(shape)) * esz
        self.big = torch.full((GUARD + self.n + GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.big[GUARD:GUARD + self.n] = fill
        self.t = self.big[GUARD:GUARD + self.n].view(dtype).view(shape)

    def guards_intact(self):
        g = self.big.cpu().numpy()
        return bool(np.all(g[:GUARD] == PATTERN) and np.all(g[GUARD + self.n:] == PATTERN))


def run_decode(inp: wl.DecodeInputs, num_partitions: int = 0, dev=None, poison: bool = True,
               plan_separately: bool = False, with_lse: bool = True, scale: float | None = None,
               flags: int = 0):
    """Runs mla_decode on the GPU; returns (o float64 [B,q_len,n_h,d_c], lse).
    `scale` overrides the config's softmax scale; `flags` goes to the
    descriptor (MLA_DECODE_FP8_MATH)."""
    m = lib()
    cfg = inp.cfg
    dev = dev or device_inputs(inp)
    q_dt = "fp32" if cfg.cache_dtype == "fp32" else "bf16"
    desc = m.decode_desc(cfg.batch, cfg.q_len, cfg.n_heads, cfg.d_c, cfg.d_rope, dev["max_blocks"],
                         cfg.cache_dtype, q_dt, cfg.out_dtype, num_partitions, flags=flags)
    ws_bytes = m.mla_decode_workspace_size(desc)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    odt = torch.float32 if cfg.out_dtype == "fp32" else torch.bfloat16
    o = torch.empty((cfg.batch, cfg.q_len, cfg.n_heads, cfg.d_c), dtype=odt, device="cuda")
    lse = torch.empty((cfg.batch, cfg.q_len, cfg.n_heads), dtype=torch.float32, device="cuda") \
        if with_lse else None
    if poison:  # NaN everywhere the call must overwrite, and in its scratch
        o.fill_(float("nan"))
        if lse is not None:
            lse.fill_(float("nan"))
        ws.fill_(0xFF)
    if plan_separately:
        m.mla_decode_plan(desc, dev["seq_lens"], ws)
        desc.plan_ready = 1
    m.mla_decode(desc, dev["q_abs"], dev["q_rope"], dev["cache"], dev["cache_scale"],
                 dev["block_table"], dev["seq_lens"],
                 cfg.softmax_scale if scale is None else scale, o, lse, ws)
    torch.cuda.synchronize()
    o64 = o.float().cpu().numpy().astype(np.float64)
    lse64 = None if lse is None else lse.cpu().numpy().astype(np.float64)
    return o64, lse64


def oracle_inputs(inp: wl.DecodeInputs, b: int):
    """fp64 values of what the GPU reads for sequence b (decoded by the oracle)."""
    cfg = inp.cfg
    if cfg.cache_dtype == "fp32":
        lat = inp.lat_f32[b].astype(np.float64)
        return lat[:, :cfg.d_c], lat[:, cfg.d_c:]
    if cfg.cache_dtype == "bf16":
        lat = oracle.bf16_bits_to_f64(inp.lat_bits[b])
        return lat[:, :cfg.d_c], lat[:, cfg.d_c:]
    c = oracle.fp8_cache_dequant(inp.lat_codes[b], inp.lat_scales[b])
    return c, oracle.bf16_bits_to_f64(inp.krope_bits[b])


def oracle_queries(inp: wl.DecodeInputs):
    if inp.cfg.cache_dtype == "fp32":
        return inp.q_abs_f32.astype(np.float64), inp.q_rope_f32.astype(np.float64)
    return oracle.bf16_bits_to_f64(inp.q_abs_bits), oracle.bf16_bits_to_f64(inp.q_rope_bits)


def oracle_decode(inp: wl.DecodeInputs, batches=None, scale: float | None = None):
    """Oracle output for all (or some) sequences: (o, lse) float64."""
    cfg = inp.cfg
    qa, qr = oracle_queries(inp)
    idx = range(cfg.batch) if batches is None else batches
    o = np.zeros((len(idx), cfg.q_len, cfg.n_heads, cfg.d_c))
    lse = np.zeros((len(idx), cfg.q_len, cfg.n_heads))
    for k, b in enumerate(idx):
        c, kr = oracle_inputs(inp, b)
        r = oracle.latent_attention(qa[b], qr[b], c, kr,
                                    cfg.softmax_scale if scale is None else scale)
        o[k], lse[k] = r["o"], r["lse"]
    return o, lse


def errors(g: np.ndarray, r: np.ndarray):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    assert np.all(np.isfinite(g)), "non-finite values in the GPU output"
    max_abs = float(np.max(np.abs(g - r))) if g.size else 0.0
    nr = float(np.linalg.norm(r))
    rel_f = float(np.linalg.norm(g - r) / nr) if nr > 0 else float(np.linalg.norm(g - r))
    return max_abs, rel_f


def assert_close(g, r, kind: str, label: str = ""):
    ma, rf = errors(g, r)
    tma, trf = TOL[kind]
    say(f"  [{label}] max-abs {ma:.3e} (gate {tma}), rel-F {rf:.3e} (gate {trf})")
    assert ma <= tma and rf <= trf, (label, ma, rf)
    return ma, rf


def assert_lse_close(g, r, tol: float, label: str = ""):
    fin = np.isfinite(r)
    assert np.array_equal(np.isfinite(g), fin), f"{label}: -inf pattern differs"
    if fin.any():
        err = float(np.max(np.abs(g[fin] - r[fin])))
        say(f"  [{label}] lse max-abs {err:.3e}")
        assert err <= tol, (label, err)
    assert np.all(g[~fin] == -np.inf)


def fp8_math_lse_tol(inp, batches=None, scale=None):
    """Log-sum-exp gate of the fp8 matrix-core mode (MLA_DECODE_FP8_MATH):
    2e-3 (the gate of the exact paths) plus the largest logit shift the
    query rounding can cause. Rounding to e4m3
    to nearest moves a normal value by at most 2^-4 of itself, and a
    subnormal one (below 2^-6 after the block scaling, which puts the block
    maximum at 128 or more) by at most 2^-10, i.e. 2^-17 of the block
    maximum; so a content logit moves by at most
    |scale| (2^-4 sum_k |q_k c_k| + 2^-17 max|q| sum_k |c_k|), and the
    log-sum-exp by at most the largest of these."""
    cfg = inp.cfg
    sc = abs(cfg.softmax_scale if scale is None else scale)
    qa, _ = oracle_queries(inp)
    worst = 0.0
    for b in (range(cfg.batch) if batches is None else batches):
        c, _ = oracle_inputs(inp, b)
        if len(c) == 0:
            continue
        q = np.abs(qa[b].reshape(-1, cfg.d_c))
        bound = 2.0 ** -4 * (q @ np.abs(c).T) + 2.0 ** -17 * q.max() * np.abs(c).sum(1)[None, :]
        worst = max(worst, float(bound.max()))
    return 2e-3 + sc * worst


def stress_inputs(cfg, variant: str, needle_seed: int = 77):
    """Seeded inputs whose attention is far from uniform (the gated workloads'
    logits have a standard deviation near 0.003):
      sharp        queries x 27.7 (logit standard deviation about 2);
      rope_only    sharp, with the content queries zero;
      content_only sharp, with the rope queries zero;
      needle       rope query e_0 for every head and one token per sequence
                   whose rope key is (20 / scale) e_0: a +20 logit that takes
                   almost all of the weight (the other queries stay sharp)."""
    inp = wl.make_decode_inputs(cfg, q_mult=27.7)
    if variant == "rope_only":
        inp.q_abs_bits[...] = 0
    elif variant == "content_only":
        inp.q_rope_bits[...] = 0
    elif variant == "needle":
        inp.q_rope_bits[...] = 0
        inp.q_rope_bits[..., 0] = wl.to_bf16_bits(np.array([1.0]))[0]
        rng = np.random.default_rng(needle_seed)
        val = wl.to_bf16_bits(np.array([20.0 / cfg.softmax_scale]))[0]
        for b in range(cfg.batch):
            S = int(inp.seq_lens[b])
            if S < cfg.q_len:
                continue
            j = int(rng.integers(0, S - cfg.q_len + 1))
            kr = inp.krope_bits[b] if cfg.cache_dtype == "fp8" else inp.lat_bits[b][:, cfg.d_c:]
            kr[j, :] = 0
            kr[j, 0] = val
    elif variant != "sharp":
        raise ValueError(variant)
    return inp
