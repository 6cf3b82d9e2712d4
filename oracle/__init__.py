"""fp64 CPU oracle for Gated MLA.

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The HIP library never does, and this
package never imports the HIP library.
"""
from .gmla_oracle import *  # noqa: F401,F403
from .kv_bytes import kv_bytes_per_token, kv_elements_per_token_layer, decode_step_cache_bytes  # noqa: F401
