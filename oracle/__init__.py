"""CPU oracle for TurboQuant-style KV-cache quantization and attention.

TEST INFRASTRUCTURE, NOT PART OF THE LIBRARY.  Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import, call or run anything under ``oracle/``.  The oracle imports nothing
from ``quantized_kv_cache_tq_amd`` and shares no code, table or constant
generator with it; the two meet only in the tests, on inputs from the seeded
generators in ``quantized_kv_cache_tq_amd.inputs`` (which hold none of the
method's arithmetic).
"""

from .tq_oracle import *  # noqa: F401,F403
