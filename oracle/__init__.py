"""CPU oracle (float64 numpy) for paged decode attention and its KV writer.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import it.  It shares no code with the HIP
library (paged_kv_cache_139_amd/) and does not import it.

Pins (tests/test_oracle_*.py, run with -m "not gpu") tie each function to
something other than itself:

  encode_e4m3 / decode_e4m3
      format-definition table values (tests/golden/e4m3_codes.txt), round trip
      of all 256 codes, and agreement with torch's float8_e4m3fn cast after a
      clamp to +-448 on every bf16 bit pattern at four scales.
  reshape_and_cache_ref / gather_ref
      the worked block-table example printed in [L3] "SVG框架图" (logical blocks
      0,1,2 -> physical 7,3,9; tests/golden/worked_example_block_table.txt),
      write-then-gather round trips, untouched-slot invariance, skipped slots.
  paged_attention_ref
      pure-Python scalar loops (brute force), dense attention from
      torch.nn.functional.scaled_dot_product_attention on an identity table,
      closed forms (one token, constant V, zero query, one dominant logit),
      softmax weights sum to one, invariance to any permutation of physical
      blocks, shared prefix == private copies, block size 1 == dense.
      Over FP8 caches (tests/test_oracle_fp8_attention.py): scalar loops
      decoding every code with torch's float8_e4m3fn at k_scale != v_scale,
      one token == decoded value * v_scale, zero query == mean * v_scale,
      (scale s, k_scale 2) == (2s, 1) bitwise, v_scale scales the output;
      swapped or divided scales fail the loops.
  paged_attention_partitioned_ref
      equal to paged_attention_ref to 1e-12, including empty partitions.
  copy_blocks_ref
      block bits equal after copy, other blocks untouched, gather through the
      repointed table unchanged.
  CompactPool (subset.py)
      equal to the full-pool oracle on the sequences it keeps.

No value printed on the pages is an attention output, so no page number pins
the attention arithmetic directly; the pins above do.
"""

from .fp8_e4m3 import (E4M3_MAX, decode_e4m3, e4m3_value_of_code, encode_e4m3,
                       quantize_e4m3)
from .subset import CompactPool
from .paged import (copy_blocks_ref, gather_ref, paged_attention_partitioned_ref,
                    paged_attention_ref, reshape_and_cache_ref, softmax_weights_ref,
                    to_float32, to_float64)

__all__ = [
    "CompactPool",
    "E4M3_MAX", "decode_e4m3", "e4m3_value_of_code", "encode_e4m3", "quantize_e4m3",
    "copy_blocks_ref", "gather_ref", "paged_attention_partitioned_ref",
    "paged_attention_ref", "reshape_and_cache_ref", "softmax_weights_ref",
    "to_float32", "to_float64",
]
