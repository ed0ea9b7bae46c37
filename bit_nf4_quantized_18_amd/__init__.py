"""MI355X (gfx950) QLoRA NF4 linear layer: HIP kernels behind a C ABI
(include/qlora_nf4.h) and a thin ctypes binding (``binding``)."""
from .binding import (PackedNF4, QloraError, dequantize, levels, linear_bwd, linear_fwd, load,  # noqa: F401
                      quantize, status_string, workspace_bytes)
