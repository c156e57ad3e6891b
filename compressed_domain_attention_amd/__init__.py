"""Compressed-domain decode attention for AMD Instinct MI355X (gfx950).

The work is done by a C-ABI shared library of hand-written HIP kernels
(``libcdattn.so``); this package is a thin ctypes binding over it.  Importing
the package does not load the library: the first call that needs it does,
and raises if it is missing.
"""

from .binding import (  # noqa: F401
    CodecError, CodecStream, CodecLayerStack, basis, decode_attention, decode_attention_append, decode_attention_noalloc,
    decode_workspace_bytes, measure_read, timeline_set,
    encode_blocks, append_step, materialise, crop, select_batch, library, library_path,
    FMT_F32, FMT_BF16, FMT_I8, FMT_PNG,
)
