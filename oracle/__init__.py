"""CPU oracle for the STAR-KV decode path (test infrastructure, not product).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the HIP library.
"""

from .starkv_oracle import append, decode, decode_uncompressed, gather_latents, prefill  # noqa: F401
