"""Seeded synthetic inputs for the paged-KV attention workloads.

This package is shared by the tests, the oracle checks and the benchmark.  It
draws random numbers, rounds them to the storage dtype, lays tokens out in a
paged block pool and builds the index arrays (block tables, cumulative lengths,
slot mappings).  It contains none of the attention arithmetic: no logits, no
softmax, no products of q, k or v.
"""

from .workloads import *  # noqa: F401,F403
