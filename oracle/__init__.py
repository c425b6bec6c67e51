"""CPU oracle for paged decode attention -- TEST INFRASTRUCTURE ONLY.

``oracle.blocks`` holds the block bookkeeping (tables, reference counts,
copy on write, swapping) and the block copies, as plain Python and numpy.

Only the tests, the smoke check and the CPU-baseline leg of ``bench.py`` may
import this package.  The GPU library and its Python binding never do.
"""
from .oracle import (  # noqa: F401
    F32, F16, BF16, ORACLE_DTYPES,
    build, lib_path, num_threads,
    paged_decode, reshape_and_cache, round_to_dtype, decode_elements,
    f16_bits_to_f64, bf16_bits_to_f64,
)
