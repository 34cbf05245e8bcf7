"""Float64 CPU oracle for the Block-GTQ packed-KV path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library and its
Python binding) may import, call or link this package; only the tests, the
smoke check and the CPU-baseline leg of the benchmark use it.  It shares no
code, tables or constants with the library: the two agree only through the
specification written down in each function's docstring.

What it follows (sources are the method's public pages):

* "RoPE-Aware Bit Allocation for KV-Cache Quantization", Abstract (arXiv) --
  the RoPE block decomposition of a logit, the label-free per-block energy,
  greedy integer bit allocation by marginal gain, TurboQuant-MSE as the base
  encoder, KxVy budgets, and the packed-cache serving path.
* Block-GTQ README (JIA-Lab-research/blockgtq), introduction, "Bit
  allocation" and calibration paragraphs, and the backend table -- per
  (layer, KV head) Q/K energy over RoPE frequency blocks, a fixed average
  budget, calibration from one forward pass, and the quantize -> dequantize
  -> SDPA reference path that this oracle mirrors.

Where the pages leave a step open (energy formula, distortion model,
rotation, codebook, layout) the reading taken is stated in the docstring of
the function that implements it.

Every function here is pinned by the CPU tests (tests/test_oracle_*.py).
"""
from .codebook import lloyd_max, codebooks, distortion_table
from .rotation import SplitMix64, seeded_stream, haar_rotation, rotation_for
from .alloc import energy, greedy_allocate, exact_sum_squares_f16
from .quant import (groups_for, encode_groups, encode_k, encode_v, f16_bits, f16_value,
                    dequant_k, dequant_v)
from .layout import (k_words_per_token, pack_k, unpack_k, pack_v, unpack_v, k_bit_offsets)
from .attention import decode_attention, softmax_attention, decode_attention_buffered, buffered_positions
from .rope import rope_blocks, block_logits, block_pairs
from .diagnostics import logit_mae

__all__ = [
    "lloyd_max", "codebooks", "distortion_table",
    "SplitMix64", "seeded_stream", "haar_rotation", "rotation_for",
    "energy", "greedy_allocate", "exact_sum_squares_f16",
    "groups_for", "encode_groups", "encode_k", "encode_v", "f16_bits", "f16_value",
    "dequant_k", "dequant_v",
    "k_words_per_token", "pack_k", "unpack_k", "pack_v", "unpack_v", "k_bit_offsets",
    "decode_attention", "softmax_attention", "decode_attention_buffered", "buffered_positions",
    "rope_blocks", "block_logits", "block_pairs", "logit_mae",
]
