"""The oracle: test infrastructure, not part of the library.

A plain float64 CPU implementation of the paged KV-cache write, the block
manager and PagedAttention decode, written from the pages.  Only the tests, the
smoke check and the benchmark's CPU-baseline leg may import it; the library's
own code path never does, and shares no code with it.
"""
from .paged_attention import *  # noqa: F401,F403
from .paged_attention import __all__  # noqa: F401
