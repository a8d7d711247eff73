"""CPU oracle for batched paged attention over a block-pooled KV cache.

TEST INFRASTRUCTURE: only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The GPU library never does.
"""
from .oracle import Oracle, OracleError, build, get  # noqa: F401
