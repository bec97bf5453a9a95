"""The allocation-free decode (mla_decode_noalloc), through the C ABI, against
mla_decode with a caller-owned workspace: two calls in a row on one GPU, the
second smaller than the first (so stale contents of the shared device array
from the first call are present), each compared bitwise with mla_decode and
to the oracle's gate."""
import numpy as np
import pytest
import torch

import workloads as wl
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

C = wl.CONFIGS


def _call(inp, dev, noalloc):
    m = H.lib()
    cfg = inp.cfg
    desc = m.decode_desc(cfg.batch, cfg.q_len, cfg.n_heads, cfg.d_c, cfg.d_rope, dev["max_blocks"],
                         cfg.cache_dtype, "bf16", cfg.out_dtype)
    o = torch.full((cfg.batch, cfg.q_len, cfg.n_heads, cfg.d_c), float("nan"),
                   dtype=torch.bfloat16, device="cuda")
    lse = torch.full((cfg.batch, cfg.q_len, cfg.n_heads), float("nan"), device="cuda")
    if noalloc:
        m.mla_decode_noalloc(desc, dev["q_abs"], dev["q_rope"], dev["cache"], dev["cache_scale"],
                             dev["block_table"], dev["seq_lens"], cfg.softmax_scale, o, lse)
    else:
        ws = torch.empty(m.mla_decode_workspace_size(desc), dtype=torch.uint8, device="cuda")
        m.mla_decode(desc, dev["q_abs"], dev["q_rope"], dev["cache"], dev["cache_scale"],
                     dev["block_table"], dev["seq_lens"], cfg.softmax_scale, o, lse, ws)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def test_noalloc_matches_the_workspace_call_twice_in_a_row():
    first = C["c2"]                                   # 36 MiB of the 72 MiB array
    second = wl.scaled(C["c5"], batch=3, seq_len=1000)  # smaller, another cache type
    for cfg in (first, second):
        H.say(f"case noalloc {cfg.name} B={cfg.batch} S={cfg.seq_len} {cfg.cache_dtype}")
        inp = wl.make_decode_inputs(cfg, q_mult=27.7)
        dev = H.device_inputs(inp)
        a, la = _call(inp, dev, noalloc=True)
        b, lb = _call(inp, dev, noalloc=False)
        assert np.array_equal(a, b) and np.array_equal(la, lb), cfg.name
        ro, rl = H.oracle_decode(inp)
        H.assert_close(a, ro, cfg.cache_dtype, f"noalloc-{cfg.name}")
        H.assert_lse_close(la, rl, 2e-3, f"noalloc-{cfg.name}")
