"""Mixed-adapter LoRA projection for AMD MI355X (gfx950).

Y = X W^T + s (X A_a^T) B_a^T on rows of requests naming adapter a, and
Y = X W^T on all other rows, computed by hand-written HIP kernels behind the
C-ABI declared in include/lora_proj.h.  Importing the package loads nothing;
the first call loads liblora_proj.so and fails if it is not built.
"""
from .binding import (LoraError, lora_proj, lora_proj_raw, path, status_string,  # noqa: F401
                      workspace_bytes, load)
