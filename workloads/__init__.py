"""Seeded synthetic workloads for the absorbed-MLA decode step.

This module draws random numbers and stores them in the formats the decode
step consumes. It holds none of the method's arithmetic: no scores, no
softmax, no weighted sums, no folds, no decoding of stored codes. Both the
CPU oracle (``oracle/``) and the GPU path are fed from here, and neither is
imported by this module.

The storage conversions done here are input preparation only:

* fp64 -> fp32 -> bf16 with round-to-nearest-even (the stored bf16 bits);
* the fp8 e4m3 (OCP "e4m3fn": bias 7, no infinities, max 448) encoding of a
  latent divided by its per-token scale amax/448, round-to-nearest-even,
  saturating. The scale and the codes are the *stored cache*; whoever reads
  the cache decodes the codes with their own decoder.

Workloads (shapes and value distributions of the DeepSeek-V2/V3 attention
described in llms.blog "Multi-Head Latent Attention: How Low-Rank KV
Compression Scales LLM Serving", section "Quantitative Comparison and
Serving Economics": 128 heads, d_c = 512, d_R = 64):

=====  =====================================================================
tiny   fp32, d_model 512, 8 heads of 64, d_c 64, d_R 16, one sequence of 256
       tokens; random weights N(0, 0.02^2), hidden states N(0, 1)
c2     bf16, batch 32, one query per sequence, context 4096
c3     bf16, batch 4, context 32768 (long context, many splits)
c4     bf16, batch 64, contexts uniform in [512, 16384], pages assigned by a
       random permutation of physical blocks
c5     fp8 e4m3 latent + bf16 rope key + fp32 per-token scale, batch 128,
       context 8192, two query tokens per sequence (causal within the pair)
=====  =====================================================================

Draw order (numpy PCG64, ``np.random.default_rng(seed)``) for c2..c5:
  1. (c4 only) sequence lengths: ``rng.integers(512, 16384, size=64,
     endpoint=True)``;
  2. for each sequence b in order: latents ``rng.standard_normal((S_b, 576))
     / sqrt(576)``;
  3. queries ``rng.standard_normal((B, q_len, n_h, 576)) / sqrt(576)``
     (first d_c lanes: absorbed content query; last d_R lanes: rope query);
  4. (paged with permutation) ``rng.permutation(n_pages)``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

PAGE_SIZE = 64  # tokens per cache page


# ----------------------------------------------------------------------------
# storage-format conversions (input preparation)
# ----------------------------------------------------------------------------

def to_bf16_bits(x) -> np.ndarray:
    """fp64/fp32 array -> bf16 bit patterns (uint16), via fp32, RNE."""
    import torch
    f = torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float32)))
    return f.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_as_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact widening), for building inputs."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def encode_e4m3(x32: np.ndarray) -> np.ndarray:
    """float32 values -> e4m3fn codes (uint8), RNE, saturating to +-448
    (clamped first, then torch's CPU cast, which rounds to nearest even)."""
    import torch
    x = np.clip(np.asarray(x32, dtype=np.float32), -448.0, 448.0)
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def quantize_tokens_e4m3(c: np.ndarray):
    """Per-token fp8 storage of latents c [T, d_c] (fp64).

    scale_j = fp32(amax_j) / 448 in fp32 (1.0 where amax_j == 0);
    code = e4m3(fp32(c) / scale_j) computed in fp32.
    Returns (codes uint8 [T, d_c], scales float32 [T]).
    """
    c32 = np.asarray(c, dtype=np.float32)
    amax = np.max(np.abs(c32), axis=1)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
    codes = encode_e4m3((c32 / scale[:, None]).astype(np.float32))
    return codes, scale


# ----------------------------------------------------------------------------
# configurations
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    q_len: int
    n_heads: int
    d_c: int
    d_rope: int
    cache_dtype: str           # "fp32" | "bf16" | "fp8"
    out_dtype: str             # "fp32" | "bf16"
    seq_len: int | None        # fixed context, or None for ragged
    ragged: tuple | None = None  # (lo, hi) inclusive for ragged contexts
    permute_pages: bool = False
    seed: int = 0
    d_head: int = 128          # per-head content width, only sets the scale
    d_model: int = 0           # tiny only
    rope_theta: float = 10000.0

    @property
    def lanes(self) -> int:
        return self.d_c + self.d_rope

    @property
    def softmax_scale(self) -> float:
        # the score is divided by sqrt(content head width + rope width)
        return 1.0 / math.sqrt(self.d_head + self.d_rope)


CONFIGS = {
    "tiny": DecodeConfig("tiny", 1, 1, 8, 64, 16, "fp32", "fp32", 256, seed=1,
                         d_head=64, d_model=512),
    "c2": DecodeConfig("c2", 32, 1, 128, 512, 64, "bf16", "bf16", 4096, seed=2),
    "c3": DecodeConfig("c3", 4, 1, 128, 512, 64, "bf16", "bf16", 32768, seed=3),
    "c4": DecodeConfig("c4", 64, 1, 128, 512, 64, "bf16", "bf16", None,
                       ragged=(512, 16384), permute_pages=True, seed=4),
    "c5": DecodeConfig("c5", 128, 2, 128, 512, 64, "fp8", "bf16", 8192, seed=5),
}


def scaled(cfg: DecodeConfig, **kw) -> DecodeConfig:
    """A copy of a config with some fields replaced (smaller parity cases)."""
    d = dict(cfg.__dict__)
    d.update(kw)
    return DecodeConfig(**d)


# ----------------------------------------------------------------------------
# decode inputs (c2..c5 and reduced variants)
# ----------------------------------------------------------------------------

@dataclass
class DecodeInputs:
    cfg: DecodeConfig
    seq_lens: np.ndarray                 # int32 [B]
    # stored query, as the GPU consumes it
    q_abs_bits: np.ndarray | None = None  # bf16 bits [B, q_len, n_h, d_c]
    q_rope_bits: np.ndarray | None = None  # bf16 bits [B, q_len, n_h, d_R]
    q_abs_f32: np.ndarray | None = None   # fp32 (tiny)
    q_rope_f32: np.ndarray | None = None
    # stored latents per sequence (contiguous), in stored format
    lat_bits: list = field(default_factory=list)     # bf16: uint16 [S_b, d_c+d_R]
    lat_f32: list = field(default_factory=list)      # fp32: float32 [S_b, d_c+d_R]
    lat_codes: list = field(default_factory=list)    # fp8: uint8 [S_b, d_c]
    lat_scales: list = field(default_factory=list)   # fp8: float32 [S_b]
    krope_bits: list = field(default_factory=list)   # fp8: uint16 [S_b, d_R]
    page_perm: np.ndarray | None = None              # physical page of logical page k


def _seq_lens(cfg: DecodeConfig, rng) -> np.ndarray:
    if cfg.ragged is not None:
        lo, hi = cfg.ragged
        return rng.integers(lo, hi, size=cfg.batch, endpoint=True).astype(np.int32)
    return np.full(cfg.batch, cfg.seq_len, dtype=np.int32)


def make_decode_inputs(cfg: DecodeConfig, seed: int | None = None,
                       q_mult: float = 1.0, seq_lens=None) -> DecodeInputs:
    """Draw one decode batch for `cfg` (see the module docstring for the order).

    q_mult multiplies the drawn queries before rounding (stress variants that
    sharpen the attention); seq_lens overrides the drawn/fixed lengths.
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    lens = _seq_lens(cfg, rng)
    if seq_lens is not None:
        lens = np.asarray(seq_lens, dtype=np.int32)
        assert lens.shape == (cfg.batch,)
    inp = DecodeInputs(cfg=cfg, seq_lens=lens)
    L = cfg.lanes
    norm = 1.0 / math.sqrt(L)
    for b in range(cfg.batch):
        lat = rng.standard_normal((int(lens[b]), L)) * norm
        if cfg.cache_dtype == "bf16":
            inp.lat_bits.append(to_bf16_bits(lat))
        elif cfg.cache_dtype == "fp32":
            inp.lat_f32.append(lat.astype(np.float32))
        elif cfg.cache_dtype == "fp8":
            codes, scales = quantize_tokens_e4m3(lat[:, :cfg.d_c])
            inp.lat_codes.append(codes)
            inp.lat_scales.append(scales)
            inp.krope_bits.append(to_bf16_bits(lat[:, cfg.d_c:]))
        else:
            raise ValueError(cfg.cache_dtype)
    q = rng.standard_normal((cfg.batch, cfg.q_len, cfg.n_heads, L)) * norm * q_mult
    if cfg.cache_dtype == "fp32":
        inp.q_abs_f32 = np.ascontiguousarray(q[..., :cfg.d_c].astype(np.float32))
        inp.q_rope_f32 = np.ascontiguousarray(q[..., cfg.d_c:].astype(np.float32))
    else:
        inp.q_abs_bits = to_bf16_bits(q[..., :cfg.d_c])
        inp.q_rope_bits = to_bf16_bits(q[..., cfg.d_c:])
    n_pages = int(sum(pages_for(int(s)) for s in lens))
    if cfg.permute_pages:
        inp.page_perm = rng.permutation(n_pages).astype(np.int32)
    else:
        inp.page_perm = np.arange(n_pages, dtype=np.int32)
    return inp


def pages_for(seq_len: int) -> int:
    return (seq_len + PAGE_SIZE - 1) // PAGE_SIZE


# ----------------------------------------------------------------------------
# paging (layout only): contiguous per-sequence rows -> page pool + table
# ----------------------------------------------------------------------------

def block_table(seq_lens, page_perm, max_blocks: int | None = None) -> np.ndarray:
    """int32 [B, max_blocks]: logical page k of sequence b -> physical page;
    logical pages are numbered sequence by sequence; padding is -1."""
    lens = [int(s) for s in seq_lens]
    nb = [pages_for(s) for s in lens]
    mb = max(nb + [1]) if max_blocks is None else max_blocks
    bt = np.full((len(lens), mb), -1, dtype=np.int32)
    k = 0
    for b, n in enumerate(nb):
        bt[b, :n] = page_perm[k:k + n]
        k += n
    return bt


def pack_pages(rows_per_seq, page_perm, row_shape, dtype, fill=0):
    """Scatter per-sequence token rows into a page pool [n_pages, 64, *row_shape].

    Slots past a sequence's end inside its last page are set to `fill`.
    """
    n_pages = len(page_perm)
    pool = np.full((n_pages, PAGE_SIZE) + tuple(row_shape), fill, dtype=dtype)
    k = 0
    for rows in rows_per_seq:
        s = rows.shape[0]
        for p in range(pages_for(s)):
            chunk = rows[p * PAGE_SIZE:(p + 1) * PAGE_SIZE]
            pool[page_perm[k], :chunk.shape[0]] = chunk
            k += 1
    return pool


def fp8_token_rows(inp: DecodeInputs):
    """fp8 cache rows as stored: per token 512 code bytes then the rope key's
    bf16 bytes (d_c + 2*d_R bytes per token)."""
    out = []
    for codes, kr in zip(inp.lat_codes, inp.krope_bits):
        out.append(np.concatenate([codes, kr.view(np.uint8).reshape(kr.shape[0], 2 * kr.shape[1])], axis=1))
    return out


def paged_cache(inp: DecodeInputs):
    """(pool, scale_pool_or_None) in the stored page layout for the config."""
    cfg = inp.cfg
    if cfg.cache_dtype == "bf16":
        return pack_pages(inp.lat_bits, inp.page_perm, (cfg.lanes,), np.uint16), None
    if cfg.cache_dtype == "fp32":
        return pack_pages(inp.lat_f32, inp.page_perm, (cfg.lanes,), np.float32), None
    rows = fp8_token_rows(inp)
    pool = pack_pages(rows, inp.page_perm, (cfg.d_c + 2 * cfg.d_rope,), np.uint8)
    spool = pack_pages([s[:, None] for s in inp.lat_scales], inp.page_perm, (1,),
                       np.float32, fill=1.0)[..., 0]
    return pool, spool


# ----------------------------------------------------------------------------
# tiny end-to-end model (weights + hidden states)
# ----------------------------------------------------------------------------

@dataclass
class TinyModel:
    cfg: DecodeConfig
    W_DKV: np.ndarray   # [d_c, d]
    W_KR: np.ndarray    # [d_R, d]
    W_UQ: np.ndarray    # [n_h*d_h, d]   (no query compression in this model)
    W_QR: np.ndarray    # [n_h*d_R, d]
    W_UK: np.ndarray    # [n_h*d_h, d_c]
    W_UV: np.ndarray    # [n_h*d_h, d_c]
    W_O: np.ndarray     # [d, n_h*d_h]
    H: np.ndarray       # [S, d] hidden states of positions 0..S-1
    W_DQ: np.ndarray | None = None  # [d_cq, d] optional query compression


def make_tiny_model(cfg: DecodeConfig | None = None, seed: int | None = None,
                    seq_len: int | None = None, d_cq: int = 0) -> TinyModel:
    """Weights N(0, 0.02^2) and hidden states N(0, 1), rounded to fp32.

    Draw order: W_DKV, W_KR, W_UQ, W_QR, W_UK, W_UV, W_O, H, then W_DQ when
    d_cq > 0 (in which case W_UQ and W_QR take d_cq inputs).
    """
    cfg = cfg or CONFIGS["tiny"]
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    d, nh, dh, dc, dr = cfg.d_model, cfg.n_heads, cfg.d_head, cfg.d_c, cfg.d_rope
    S = cfg.seq_len if seq_len is None else seq_len
    din_q = d_cq if d_cq > 0 else d

    def w(*shape):
        return (rng.standard_normal(shape) * 0.02).astype(np.float32)

    W_DKV, W_KR = w(dc, d), w(dr, d)
    W_UQ, W_QR = w(nh * dh, din_q), w(nh * dr, din_q)
    W_UK, W_UV, W_O = w(nh * dh, dc), w(nh * dh, dc), w(d, nh * dh)
    H = rng.standard_normal((S, d)).astype(np.float32)
    W_DQ = w(d_cq, d) if d_cq > 0 else None
    return TinyModel(cfg, W_DKV, W_KR, W_UQ, W_QR, W_UK, W_UV, W_O, H, W_DQ)


# ----------------------------------------------------------------------------
# prefill (the unabsorbed layer over whole prompts)
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class PrefillConfig:
    """A prompt batch for the unabsorbed layer. Widths of prefill-ds follow
    DeepSeek-V2 as zhangchitc.github.io "Multi-head latent attention",
    section "The definitions: project down, then up", gives them (d 5120,
    query latent 1536, latent 512, 128 heads of 128) with the 64-lane rope
    key of section "Decoupled RoPE"."""
    name: str
    seq_lens: tuple
    d_model: int
    n_heads: int
    d_head: int
    d_rope: int
    d_c: int
    d_cq: int
    seed: int
    rope_theta: float = 10000.0

    @property
    def T(self) -> int:
        return int(sum(self.seq_lens))

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.d_head + self.d_rope)

    def as_decode_config(self) -> DecodeConfig:
        return DecodeConfig(self.name, len(self.seq_lens), 1, self.n_heads, self.d_c, self.d_rope,
                            "fp32", "fp32", self.T, seed=self.seed, d_head=self.d_head,
                            d_model=self.d_model, rope_theta=self.rope_theta)


PREFILL_CONFIGS = {
    # the tiny model's widths, one prompt of 256
    "prefill-tiny": PrefillConfig("prefill-tiny", (256,), 512, 8, 64, 16, 64, 0, seed=11),
    # DeepSeek head widths, fewer heads, query compression, two ragged prompts
    "prefill-mid": PrefillConfig("prefill-mid", (700, 333), 1024, 16, 128, 64, 512, 384, seed=12),
    # DeepSeek-V2 widths, one prompt of 4096
    "prefill-ds": PrefillConfig("prefill-ds", (4096,), 5120, 128, 128, 64, 512, 1536, seed=13),
}


def bf16_round(x) -> np.ndarray:
    """Values rounded to bf16 (RNE), returned as float32 (storage format)."""
    return bf16_bits_as_f32(to_bf16_bits(x))


def make_prefill_model(pcfg: PrefillConfig) -> TinyModel:
    """Weights N(0, 0.02^2) and hidden states N(0, 1) drawn as make_tiny_model
    does (all prompts' rows in one H, in batch order), every array rounded to
    bf16: the values the bf16 prefill path consumes."""
    m = make_tiny_model(pcfg.as_decode_config(), seq_len=pcfg.T, d_cq=pcfg.d_cq)
    for k, v in list(m.__dict__.items()):
        if isinstance(v, np.ndarray):
            setattr(m, k, bf16_round(v))
    return m


def prefill_gpu_layout(model: TinyModel) -> dict:
    """bf16 bit arrays in the prefill entry point's layout: h and the weights
    with the blocks one product shares stacked ([W^DKV; W^KR], [W^UQ; W^QR],
    [W^UK; W^UV])."""
    out = {
        "h": to_bf16_bits(model.H),
        "W_DKVR": to_bf16_bits(np.concatenate([model.W_DKV, model.W_KR], axis=0)),
        "W_UQR": to_bf16_bits(np.concatenate([model.W_UQ, model.W_QR], axis=0)),
        "W_UKV": to_bf16_bits(np.concatenate([model.W_UK, model.W_UV], axis=0)),
        "W_O": to_bf16_bits(model.W_O),
        "W_DQ": None if model.W_DQ is None else to_bf16_bits(model.W_DQ),
    }
    return out


def prefill_cu_seqlens(seq_lens) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(seq_lens, dtype=np.int64))]).astype(np.int32)


def prefill_positions(seq_lens) -> np.ndarray:
    return np.concatenate([np.arange(int(s), dtype=np.int32) for s in seq_lens])
