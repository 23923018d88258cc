"""Seeded synthetic inputs for the paged-attention hot path.

This package only builds inputs: random draws, block placement, block tables,
slot numbers and the copy-on-write bookkeeping of a shared prompt.  It holds none
of the attention arithmetic, so both the CPU oracle and the GPU library can be
fed from it without sharing any computation.
"""

from .gen import (  # noqa: F401
    DTYPES,
    Pool,
    DecodeCase,
    ChunkedCase,
    CowCase,
    make_decode_case,
    make_chunked_case,
    make_cow_case,
    config_decode,
    config_cow,
    config_long_mixed,
    append_tokens,
    algorithmic_decode_bytes,
    algorithmic_chunked_flops,
    kv_bytes_per_token,
)
