"""EXL3-style trellis-quantized linear layer with 128-point Hadamard rotations
and the padded-width logits projection, as hand-written HIP kernels for
MI355X (gfx950) behind a C ABI (include/exl3.h)."""
from ._lib import (  # noqa: F401
    DEFAULT_PREFILL_MIN_M,
    LAYOUT_KN,
    LAYOUT_NK,
    MAX_CHUNK_COLS,
    NOALLOC_SCRATCH_BYTES,
    Layer,
    decode_states,
    had_r_128,
    head_logits_argmax,
    head_scratch_bytes,
    linear,
    linear_noalloc,
    linear_scratch_bytes,
    logits_pad_mask_argmax,
    logits_padded_width,
    logits_scratch_bytes,
    reconstruct,
)
