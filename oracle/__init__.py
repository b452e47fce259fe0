"""Plain CPU float64 oracle for relative-position attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables or
helpers with the HIP library; the two meet only at the seeded input
generator, which holds none of the method's arithmetic.
"""

from .relpos import (  # noqa: F401
    t5_bucket,
    t5_bucket_array,
    shaw_index,
    deberta_delta,
    skew,
    rel_index_matrices,
    relattn_forward,
    relattn_forward_head,
    relattn_forward_bruteforce,
)
