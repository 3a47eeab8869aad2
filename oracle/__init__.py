"""CPU oracle for paged attention over a block-table KV cache.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import or call anything here.  The HIP library and its Python binding never
do, and this package never imports them: the two sides share no code, only
the seeded inputs from ``workloads``.

Everything is float64 numpy, written as the plain definition (see
``oracle.attention``).  Every function is pinned by CPU tests against
closed forms, a dense library routine, invariants and brute force
(``tests/test_oracle_pins.py``; the fp8 encoder and the cache writer in
``tests/test_oracle_write_pins.py``).
"""
from .attention import (decode, decode_rows, decode_partials, merge, prefill_chunk,
                        prefill_rows, gather_kv, attend, widen, round_to, write_kv)
from . import fp8_e4m3

__all__ = ["decode", "decode_rows", "decode_partials", "merge", "prefill_chunk", "prefill_rows",
           "gather_kv", "attend", "widen", "round_to", "write_kv", "fp8_e4m3"]
