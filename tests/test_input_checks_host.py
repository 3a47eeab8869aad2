"""The host-side input checks (paged_kv_cache_22_amd.checks), on the CPU:
every seeded workload the GPU tests build passes them, and each planted
violation of the contract include/pa.h leaves unchecked (a live table entry
outside the pool, a length past its table row or past the host-side bound,
a malformed cu_q_lens, two tokens written to one slot) is named."""
import numpy as np
import pytest

import workloads as W
from gpu_util import check_workload
from paged_kv_cache_22_amd import checks


def small_decode(**kw):
    args = dict(seed=3, num_seqs=6, num_q_heads=8, num_kv_heads=2, head_dim=64, len_lo=1,
                len_hi=200, q_dtype="bf16", kv_dtype="bf16")
    args.update(kw)
    return W.decode_workload(**args)


def small_prefill(**kw):
    args = dict(seed=4, q_lens=[30, 0, 7], ctx_lens=[40, 5, 0], num_q_heads=8, num_kv_heads=2,
                head_dim=64, q_dtype="bf16", kv_dtype="bf16")
    args.update(kw)
    return W.prefill_workload(**args)


@pytest.mark.parametrize("n", [1, 2, 3, 5])
def test_configurations_pass(n):
    check_workload(W.build_config(n, pad=0))


def test_c4_parts_and_padded_tables_pass():
    wl = W.config4()
    check_workload(wl.decode)
    check_workload(wl.prefill)
    # entries past a row's live blocks are never read: padding is allowed
    check_workload(small_decode(pad=-1))
    for bs in (32, 64):
        check_workload(small_decode(block_size=bs))
        check_workload(small_prefill(block_size=bs))


def test_decode_violations_are_named():
    wl = small_decode()
    nb, bs = wl.num_blocks, wl.block_size
    ok = dict(num_blocks=nb, block_size=bs, max_seq_len=wl.max_seq_len)
    checks.check_decode_inputs(wl.block_table, wl.seq_lens, **ok)
    b = int(np.argmax(wl.seq_lens))
    for bad_entry in (nb, -1, 1 << 30):
        t = wl.block_table.copy()
        t[b, 0] = bad_entry
        with pytest.raises(ValueError, match=rf"block_table\[{b}, 0\] = {bad_entry} outside"):
            checks.check_decode_inputs(t, wl.seq_lens, **ok)
    # an entry past the live blocks is not read, so not checked
    t = wl.block_table.copy()
    L = int(wl.seq_lens[b])
    if (L + bs - 1) // bs < t.shape[1]:
        t[b, (L + bs - 1) // bs] = -7
        checks.check_decode_inputs(t, wl.seq_lens, **ok)
    lens = wl.seq_lens.copy()
    lens[0] = wl.block_table.shape[1] * bs + 1
    with pytest.raises(ValueError, match="above max_seq_len"):
        checks.check_decode_inputs(wl.block_table, lens, **ok)
    with pytest.raises(ValueError, match="above max_blocks_per_seq"):
        checks.check_decode_inputs(wl.block_table, lens, num_blocks=nb, block_size=bs,
                                   max_seq_len=int(lens.max()))
    lens = wl.seq_lens.copy()
    lens[1] = -2
    with pytest.raises(ValueError, match="length -2 < 0"):
        checks.check_decode_inputs(wl.block_table, lens, **ok)
    # multi-query: a sequence shorter than its queries
    lens = wl.seq_lens.copy()
    lens[2] = 2
    with pytest.raises(ValueError, match="below q_len 4"):
        checks.check_decode_inputs(wl.block_table, lens, q_len=4, **ok)
    with pytest.raises(ValueError, match="one row per length"):
        checks.check_decode_inputs(wl.block_table[:-1], wl.seq_lens, **ok)


def test_prefill_violations_are_named():
    wl = small_prefill()
    ok = dict(num_blocks=wl.num_blocks, block_size=wl.block_size, max_q_len=wl.max_q_len,
              total_q=wl.total_q)
    checks.check_prefill_inputs(wl.cu_q_lens, wl.block_table, wl.seq_lens, **ok)
    cu = wl.cu_q_lens.copy()
    cu[1], cu[2] = cu[2] + 1, cu[2]
    with pytest.raises(ValueError, match="cu_q_lens decreases"):
        checks.check_prefill_inputs(cu, wl.block_table, wl.seq_lens, **ok)
    with pytest.raises(ValueError, match="above max_q_len"):
        checks.check_prefill_inputs(wl.cu_q_lens, wl.block_table, wl.seq_lens,
                                    **{**ok, "max_q_len": 10})
    with pytest.raises(ValueError, match="past total_q"):
        checks.check_prefill_inputs(wl.cu_q_lens, wl.block_table, wl.seq_lens,
                                    **{**ok, "total_q": wl.total_q - 1})
    with pytest.raises(ValueError, match="needs chunks"):
        checks.check_prefill_inputs(wl.cu_q_lens[:-1], wl.block_table, wl.seq_lens, **ok)
    t = wl.block_table.copy()
    t[0, 0] = wl.num_blocks
    with pytest.raises(ValueError, match="outside"):
        checks.check_prefill_inputs(wl.cu_q_lens, t, wl.seq_lens, **ok)


def test_write_duplicates_are_named():
    checks.check_write_inputs(np.array([5, -1, 7, 10_000, -1, 10_000]), num_blocks=4,
                              block_size=16)   # padding and out-of-pool slots are skipped
    with pytest.raises(ValueError, match="slot 7 written by 2 tokens"):
        checks.check_write_inputs(np.array([7, 3, 7]), num_blocks=4, block_size=16)
    with pytest.raises(ValueError, match="integers"):
        checks.check_write_inputs(np.array([1.0]), num_blocks=4, block_size=16)
