"""fp64 CPU oracle for exact attention, paged decode and block-skip prefill.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
package: only the test suite, the smoke check and the benchmark's CPU-baseline
leg use it.  It shares no code with the HIP library.

Every function is the plain, materialising definition written out in numpy
float64: build the score matrix, mask it, take the softmax, multiply by V.
See :mod:`oracle.attention` for the citations.
"""
from .attention import (  # noqa: F401
    ref_prefill,
    ref_decode_paged,
    ref_blockskip,
    kv_head_of,
    pool_rows,
    ref_decode_paged_blockskip,
    ref_prefill_paged,
    fp8_e4m3_value,
    fp8_pool_rows,
    ref_decode_paged_fp8,
)
