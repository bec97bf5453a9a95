"""CPU fp64 oracle for weight-absorbed Multi-head Latent Attention decode.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call, link
or execute anything in this package: only the test suite, the entry point's
smoke check and the benchmark's CPU-baseline leg use it. It shares no code,
table or constant generator with the HIP library, and it does not import the
package that wraps that library.

Everything here is plain numpy in float64, written from these pages:

* [Mishra]   Neel Mishra, "Multi-head Latent Attention"
             (neelmishra.github.io), sections "Step 1: a low-rank latent",
             "Step 2: absorb the up-projections", "Step 3: RoPE breaks it",
             "Step 4: decoupled RoPE", "The full accounting".
* [Zhang]    zhangchitc.github.io, "Multi-head latent attention" post,
             sections "The definitions: project down, then up",
             "Matrix absorption: compression that also saves compute",
             "Decoupled RoPE: content and position in separate branches",
             "Value absorption: weight and sum first, project after".
* [LLMsBlog] llms.blog, "Multi-Head Latent Attention: How Low-Rank KV
             Compression Scales LLM Serving", sections "Low-Rank Key-Value
             Joint Compression", "The Positional Problem and Decoupled RoPE",
             "Query Key Absorption", "Value Output Absorption",
             "Quantitative Comparison and Serving Economics".

Modules:
  reference  — the unabsorbed definition (O1), the absorbed CPU form (O2),
               latent attention on given absorbed queries (O3), folds,
               output projections, RoPE, cache append, query absorption.
  formats    — bf16 and fp8 e4m3 decoding/encoding from their definitions.
  closed_forms — per-token cache sizes and operation counts.

Parity unpinned: no page prints a numerical attention output, seed or RNG
stream; agreement with the pages' own numbers is pinned only through their
identities and closed forms. The RoPE pair layout and rotation direction are
a free choice (any fixed choice preserves the relative-position property).
"""
from .reference import (  # noqa: F401
    rope, softmax, mla_unabsorbed, mla_absorbed, latent_attention,
    decode_batch, fold_query, fold_output, output_projection_merged,
    output_projection_two_stage, cache_append, absorb_query,
)
from .formats import (  # noqa: F401
    bf16_bits_to_f64, e4m3_decode, e4m3_encode_f32, fp8_cache_dequant,
    fp8_quantize_tokens,
)
from . import closed_forms  # noqa: F401
