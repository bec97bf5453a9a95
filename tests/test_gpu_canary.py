"""Canary tests of the decode path (through the C ABI): what the kernels must
never read or write is filled with a pattern, and the results must not move.

- Canary pages around the cache pool, which no block-table entry names, and
  every slot of a sequence's last page past its length, hold NaN (bf16
  0xFFFF, fp32 NaN, e4m3 0xFF, NaN token scales). A kernel that read any of
  them, even to multiply it by a zero weight, would put a NaN into the output.
- The output, log-sum-exp and workspace buffers sit between guard regions of
  a byte pattern, which a store past either end would change.
The poisoned call must agree bitwise with a call on the clean pool, and
every guard byte must be intact.
"""
import numpy as np
import pytest

import workloads as wl
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

C = wl.CONFIGS
GUARD = 4096          # guard bytes on each side of every output buffer
PATTERN = 0x5A
CANARY_PAGES = 3

_CASES = [
    ("c4-ragged-bf16", wl.scaled(C["c4"], batch=6, ragged=(1, 2000)), 0),
    ("c4-full-bf16", C["c4"], 0),
    ("c5-ragged-fp8", wl.scaled(C["c5"], batch=4, seq_len=None, ragged=(2, 1500)), 0),
    ("c5-ragged-fp8-math", wl.scaled(C["c5"], batch=4, seq_len=None, ragged=(2, 1500)), 1),
    ("tiny-ragged-fp32", wl.scaled(C["tiny"], batch=5, seq_len=None, ragged=(1, 300)), 0),
]


def _pools(inp):
    """(clean pool, poisoned pool, clean scales, poisoned scales, block table of
    the poisoned pool): the poisoned pool has CANARY_PAGES NaN pages on each side
    and NaN in every slot past a sequence's end."""
    cfg = inp.cfg
    pool, spool = wl.paged_cache(inp)
    bt = wl.block_table(inp.seq_lens, inp.page_perm)
    nan_fill = {"bf16": np.uint16(0xFFFF), "fp32": np.float32(np.nan), "fp8": np.uint8(0xFF)}
    bad = pool.copy()
    sbad = None if spool is None else spool.copy()
    for b, S in enumerate(inp.seq_lens):
        S = int(S)
        if S % 64:
            last = bt[b, (S + 63) // 64 - 1]
            bad[last, S % 64:] = nan_fill[cfg.cache_dtype]
            if sbad is not None:
                sbad[last, S % 64:] = np.nan
    canary = np.full((CANARY_PAGES,) + pool.shape[1:], nan_fill[cfg.cache_dtype], dtype=pool.dtype)
    bad = np.concatenate([canary, bad, canary])
    if sbad is not None:
        sc = np.full((CANARY_PAGES,) + spool.shape[1:], np.nan, dtype=np.float32)
        sbad = np.concatenate([sc, sbad, sc])
    bt_bad = np.where(bt >= 0, bt + CANARY_PAGES, bt).astype(np.int32)
    return pool, bad, spool, sbad, bt, bt_bad


def _guarded(torch, nbytes):
    """A uint8 buffer of nbytes between two guard regions, and the middle view."""
    big = torch.full((GUARD + nbytes + GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
    return big, big[GUARD:GUARD + nbytes]


def _run(m, torch, inp, pool, spool, bt, flags):
    cfg = inp.cfg
    dev = H.device_inputs(inp)
    dev["cache"] = H.to_dev(pool)
    dev["cache_scale"] = None if spool is None else H.to_dev(spool.astype(np.float32))
    dev["block_table"] = H.to_dev(bt)
    q_dt = "fp32" if cfg.cache_dtype == "fp32" else "bf16"
    desc = m.decode_desc(cfg.batch, cfg.q_len, cfg.n_heads, cfg.d_c, cfg.d_rope, bt.shape[1],
                         cfg.cache_dtype, q_dt, cfg.out_dtype, flags=flags)
    esz = 4 if cfg.out_dtype == "fp32" else 2
    odt = torch.float32 if cfg.out_dtype == "fp32" else torch.bfloat16
    shape = (cfg.batch, cfg.q_len, cfg.n_heads, cfg.d_c)
    o_big, o_mid = _guarded(torch, int(np.prod(shape)) * esz)
    l_big, l_mid = _guarded(torch, cfg.batch * cfg.q_len * cfg.n_heads * 4)
    ws_bytes = m.mla_decode_workspace_size(desc)
    w_big, w_mid = _guarded(torch, ws_bytes)
    o = o_mid.view(odt).view(shape)
    lse = l_mid.view(torch.float32).view(cfg.batch, cfg.q_len, cfg.n_heads)
    m.mla_decode(desc, dev["q_abs"], dev["q_rope"], dev["cache"], dev["cache_scale"],
                 dev["block_table"], dev["seq_lens"], cfg.softmax_scale, o, lse, w_mid)
    torch.cuda.synchronize()
    for big, n, name in ((o_big, o_mid.numel(), "o_latent"), (l_big, l_mid.numel(), "lse_out"),
                         (w_big, w_mid.numel(), "workspace")):
        g = big.cpu().numpy()
        assert np.all(g[:GUARD] == PATTERN) and np.all(g[GUARD + n:] == PATTERN), \
            f"a store landed outside {name}"
    return o.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("case", _CASES, ids=[c[0] for c in _CASES])
def test_canaries_are_never_read_and_guards_never_written(case):
    import torch
    m = H.lib()
    name, cfg, fp8_math = case
    flags = m.MLA_DECODE_FP8_MATH if fp8_math else 0
    H.say(f"case canary {name} B={cfg.batch} q_len={cfg.q_len} {cfg.cache_dtype} flags={flags}")
    inp = wl.make_decode_inputs(cfg, q_mult=27.7)
    pool, bad, spool, sbad, bt, bt_bad = _pools(inp)
    o1, l1 = _run(m, torch, inp, pool, spool, bt, flags)
    o2, l2 = _run(m, torch, inp, bad, sbad, bt_bad, flags)
    assert not np.isnan(o1).any() and not np.isnan(o2).any(), name
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2), name
