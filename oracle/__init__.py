"""Float64 CPU oracle for the packed joint audio-video DiT hot path.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the bench's CPU
baseline leg may import anything from this package. The HIP library and its
binding never import it, and it imports nothing from them.

Pinned functions (each checked by CPU tests against closed forms,
invariants, special cases or brute force):
  segment_ids, tile_offsets, schedule_ref, rmsnorm, rope_3d,
  qk_norm_rope_ref, attn_varlen_ref, modulation_ref, adaln_modulate_ref,
  silu, swiglu_ref, gated_residual_ref, dit_block_ref, dit_block_rows_ref,
  e4m3_round, fp8_attn_emulated_ref, bf16_round (storage emulation),
  mx_scale_exponents, mx_quantize, mx_dequantize, mx_fake_quant, mx_linear_ref
  (MXFP8 linears, OCP MX v1.0 reading), e2m1_round, mxfp4_scale_exponents,
  mxfp4_quantize, mxfp4_codes, mxfp4_fake_quant, mxfp4_linear_ref (MXFP4), frames_to_uint8_values,
  frames_to_uint8_bthwc (decoded-frame compaction), int8_quantize_qk_blocks,
  keep_count, select_kv_blocks, bsa_attn_emulated_ref, dense_fallback
  (block-sparse attention with INT8 Q/K and FP8 V).

Parity unpinned: agreement of the block structure with the real model's
block (the pages give operator names only, no equations or weights).
"""
from .h3_oracle import (MOD_CHUNKS, adaln_modulate_ref, bf16_round, attn_varlen_ref, check_cu_seqlens,
                        dit_block_ref, dit_block_rows_ref, gated_residual_ref, modulation_ref,
                        qk_norm_rope_ref, rel_frobenius, rmsnorm, rope_3d, schedule_ref,
                        segment_ids, silu, split_modulation, swiglu_ref, tile_offsets)
from .fp8_attention import (e4m3_round, fp8_attn_emulated_ref, quantize_qk_blocks,
                            quantize_v_channels)
from .mx_linear import (E2M1_VALUES, e2m1_round, mx_dequantize, mx_fake_quant, mx_linear_ref,
                        mx_quantize, mx_scale_exponents, mxfp4_codes, mxfp4_fake_quant,
                        mxfp4_linear_ref, mxfp4_quantize, mxfp4_scale_exponents)
from .output_compaction import frames_to_uint8_bthwc, frames_to_uint8_values
from .block_sparse_attention import (bsa_attn_emulated_ref, dense_fallback, int8_quantize_qk_blocks,
                                     keep_count, select_kv_blocks)

__all__ = [
    "MOD_CHUNKS", "adaln_modulate_ref", "bf16_round", "attn_varlen_ref", "check_cu_seqlens", "dit_block_ref",
    "dit_block_rows_ref", "gated_residual_ref", "modulation_ref", "qk_norm_rope_ref",
    "rel_frobenius", "rmsnorm", "rope_3d", "schedule_ref", "segment_ids", "silu",
    "split_modulation", "swiglu_ref", "tile_offsets", "e4m3_round", "fp8_attn_emulated_ref",
    "quantize_qk_blocks", "quantize_v_channels", "mx_dequantize", "mx_fake_quant", "mx_linear_ref",
    "mx_quantize", "mx_scale_exponents", "E2M1_VALUES", "e2m1_round", "mxfp4_codes",
    "mxfp4_fake_quant", "mxfp4_linear_ref", "mxfp4_quantize", "mxfp4_scale_exponents", "frames_to_uint8_bthwc", "frames_to_uint8_values",
    "bsa_attn_emulated_ref", "dense_fallback", "int8_quantize_qk_blocks", "keep_count", "select_kv_blocks",
]
