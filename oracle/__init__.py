"""fp64 CPU oracle (test infrastructure only; never used by the product path)."""
from .codec_oracle import *  # noqa: F401,F403
from .codec_oracle import (F32, BF16, I8, PNG, FORMATS, dct_basis_f64, dct_basis_f32,
                           png_analysis, png_synthesis, analysis, synthesis,  # noqa: F401
                           f32_to_bf16_bits, bf16_bits_to_f64, project_blocks,
                           quantize_rows, encode_rows, encode, dequantize,
                           reconstruct, materialise, round_to, view, crop, select_batch, attention, decode_attention,
                           decode_attention_heads, decode_attention_split, Stream, storage_bytes)
