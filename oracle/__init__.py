"""fp64 CPU oracle of the mixed-adapter LoRA projection — TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The library's product path never calls it, and it shares no code
with the HIP path: it takes plain host arrays of exact input values and returns
float64 results that are never rounded.

Every function here is pinned by tests that do not re-run its own formula
(see tests/test_oracle_pins.py): brute-force merged-weight loops, exact
rational and exact integer results, a one-hot closed form, and invariances.
"""
from .lora_ref import (dequantize_q4, lora_proj_q4_ref, lora_proj_ref, lora_proj_sliced_ref,  # noqa: F401
                       validate_segments)
from .extract_ref import extract_ref  # noqa: F401,E402
