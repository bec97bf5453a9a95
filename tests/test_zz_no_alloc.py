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


def test_noalloc_under_graph_capture():
    """The allocation-free decode is meant for code under HIP graph capture: a
    captured call is replayed with new queries written into the captured
    buffers and an eager call with its own workspace between replays, and
    every replay matches that eager call bitwise."""
    m = H.lib()
    cfg = wl.scaled(C["c2"], batch=3, seq_len=900)
    H.say(f"case noalloc graph capture B={cfg.batch} S={cfg.seq_len}")
    inp = wl.make_decode_inputs(cfg)
    dev = H.device_inputs(inp)
    desc = m.decode_desc(cfg.batch, cfg.q_len, cfg.n_heads, cfg.d_c, cfg.d_rope, dev["max_blocks"],
                         cfg.cache_dtype, "bf16", cfg.out_dtype)
    ws = torch.empty(m.mla_decode_workspace_size(desc), dtype=torch.uint8, device="cuda")
    qa, qr = dev["q_abs"].clone(), dev["q_rope"].clone()
    shape = (cfg.batch, cfg.q_len, cfg.n_heads, cfg.d_c)
    o_g = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    l_g = torch.empty(shape[:3], dtype=torch.float32, device="cuda")
    args = (dev["cache"], dev["cache_scale"], dev["block_table"], dev["seq_lens"], cfg.softmax_scale)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):   # the first call on the device looks up the array's address
        m.mla_decode_noalloc(desc, qa, qr, *args, o_g, l_g)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        m.mla_decode_noalloc(desc, qa, qr, *args, o_g, l_g)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda").manual_seed(9)
    for rep in range(3):
        qa.copy_((torch.randn(qa.shape, device="cuda", generator=gen) * 0.05).to(qa.dtype))
        qr.copy_((torch.randn(qr.shape, device="cuda", generator=gen) * 0.05).to(qr.dtype))
        o_e = torch.empty_like(o_g)
        l_e = torch.empty_like(l_g)
        m.mla_decode(desc, qa, qr, *args, o_e, l_e, ws)   # eager reference between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e) and torch.equal(l_g, l_e), f"replay {rep}"
