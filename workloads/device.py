"""Device staging of a seeded decode workload: the paged cache, block table,
lengths and queries of one batch as GPU tensors (torch supplies the memory).
Layout only, like the rest of this package: no arithmetic of the method."""
from __future__ import annotations

import numpy as np
import torch

from . import DecodeInputs, block_table, paged_cache


def to_dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def device_inputs(inp: DecodeInputs, max_blocks: int | None = None) -> dict:
    """Device tensors for one decode call: cache pool (and fp8 scales), block
    table, lengths, queries, plus n_pages and max_blocks."""
    cfg = inp.cfg
    pool, spool = paged_cache(inp)
    bt = block_table(inp.seq_lens, inp.page_perm, max_blocks)
    dev = {
        "cache": to_dev(pool),
        "cache_scale": None if spool is None else to_dev(spool.astype(np.float32)),
        "block_table": to_dev(bt),
        "seq_lens": to_dev(inp.seq_lens.astype(np.int32)),
        "n_pages": pool.shape[0],
        "max_blocks": bt.shape[1],
    }
    if cfg.cache_dtype == "fp32":
        dev["q_abs"] = to_dev(inp.q_abs_f32)
        dev["q_rope"] = to_dev(inp.q_rope_f32)
    else:
        dev["q_abs"] = to_dev(inp.q_abs_bits.view(np.int16)).view(torch.bfloat16)
        dev["q_rope"] = to_dev(inp.q_rope_bits.view(np.int16)).view(torch.bfloat16)
    return dev
