"""The oracle's process pool gives exactly the single-process oracle's
results (each worker runs the oracle's own per-pair functions)."""
import numpy as np

import oracle
import workloads as W
from oracle.pool import OraclePool


def test_pool_equals_single_process_oracle():
    wl = W.config1()
    pw = W.prefill_workload(seed=7, q_lens=[19, 40, 0, 3], ctx_lens=[30, 5, 8, 0],
                            num_q_heads=8, num_kv_heads=2, head_dim=128, q_dtype="bf16",
                            kv_dtype="fp8")
    dw = W.decode_workload(seed=9, num_seqs=5, num_q_heads=8, num_kv_heads=2, head_dim=128,
                           len_lo=0, len_hi=300, q_dtype="bf16", kv_dtype="fp8")
    with OraclePool(workers=3) as pool:
        for w in (wl, dw):
            args = (w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens, w.scale, w.q_dtype,
                    w.kv_dtype, w.k_scale, w.v_scale)
            a, b = oracle.decode(*args), pool.decode(*args)
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
            items = [(1, 1), (0, 0)]
            a, b = oracle.decode(*args, items=items), pool.decode(*args, items=items)
            assert np.array_equal(np.isnan(a[0]), np.isnan(b[0]))
            m = ~np.isnan(a[0])
            assert np.array_equal(a[0][m], b[0][m])
        args = (pw.q, pw.cu_q_lens, pw.k_cache, pw.v_cache, pw.block_table, pw.seq_lens,
                pw.scale, pw.q_dtype, pw.kv_dtype, pw.k_scale, pw.v_scale)
        a, b = oracle.prefill_chunk(*args), pool.prefill_chunk(*args)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
