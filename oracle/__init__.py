"""fp64 CPU oracle for the paged KV-cache decode path.

TEST INFRASTRUCTURE: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library or its Python binding.
"""
from .pagedkv_oracle import (  # noqa: F401
    brute_ref,
    contiguous_ref,
    copy_ref,
    decode_ref,
    dequantize_fp8,
    e4m3_encode,
    e4m3_value,
    gather_sequence,
    prefill_ref,
    softmax_attention,
    splitk_ref,
    transfer_ref,
    widen,
    write_fp8_ref,
    write_ref,
)
