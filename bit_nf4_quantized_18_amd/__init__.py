"""MI355X (gfx950) QLoRA NF4 linear layer: HIP kernels behind a C ABI
(include/qlora_nf4.h) and a thin ctypes binding (``binding``)."""
from .binding import (CODEBOOK_INT4, CODEBOOK_NF4, PackedNF4, QloraError, dequantize,  # noqa: F401
                      dropout_mask, dropout_workspace_bytes, grouped_workspace_bytes, levels, linear_bwd,
                      linear_bwd_dropout, linear_bwd_grouped, linear_fwd, linear_fwd_dropout, linear_fwd_grouped,
                      load, load_packed, merge, quantize, requantize, save_packed, status_string, unmerge,
                      workspace_bytes)
