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
               latent attention on given absorbed queries (O3), one head's
               causal attention over expanded keys and values (the prefill
               form), folds, output projections, RoPE, cache append, query
               absorption.
  formats    — bf16 and fp8 e4m3 decoding/encoding from their definitions.
  closed_forms — per-token cache sizes and operation counts.

Pins (tests/test_oracle_pins.py, tests/test_oracle_mutations.py). No page
prints a numerical attention output, seed or RNG stream, so the functions are
pinned to what the pages and the mathematics fix rather than to printed
outputs:
  * mla_unabsorbed (O1): its scores against a pure-Python brute force at the
    DeepSeek head widths, with the score scale pinned to the pages'
    denominator sqrt(d_h + d_R);
  * mla_absorbed (O2), and through it fold_query, fold_output, cache_append,
    absorb_query, latent_attention and output_projection_merged: O2 equals O1
    to 1e-10 on the tiny config and on random shapes (the associativity the
    pages box), so a dropped term or a wrong index in any of them fails;
  * latent_attention (O3): brute force on tiny inputs, single-token, zero
    query, planted spike, empty sequence and causal-pair special cases;
  * output_projection_two_stage: equals the merged form (the same
    reassociation); expanded_attention: equals O1 at every position and a
    written-out three-position case;
  * softmax against scipy; rope against complex rotation, the identity at
    position 0, norm preservation and the relative-position property (the
    pair layout and rotation direction are a free choice that these fix up
    to that choice);
  * formats against torch on all 256 e4m3 codes and on bf16; closed_forms
    against the sizes and ratios the pages print (tests/golden/).
"""
from .reference import (  # noqa: F401
    rope, softmax, score_scale, expanded_attention, mla_unabsorbed, mla_absorbed, latent_attention,
    fold_query, fold_output, output_projection_merged,
    output_projection_two_stage, cache_append, absorb_query,
)
from .formats import (  # noqa: F401
    bf16_bits_to_f64, e4m3_decode, e4m3_encode_f32, fp8_cache_dequant,
    fp8_quantize_tokens,
)
from . import closed_forms  # noqa: F401
