"""One-pass decode with workgroups taking sequences longest first.

With at least 1024 (sequence, kv-head) pairs and at most 1024 sequences the
one-pass kernel hands workgroup x the sequence of rank x / Hkv in the order
(16-token units descending, index ascending), chosen by a selection every
workgroup runs on its own.  Each sequence must still be computed exactly
once and exactly as without the reordering: a batch taken this way must
match, bit for bit, its halves run as separate batches (below the threshold,
in index order), and the oracle.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import Dev, compare, f64, oracle_decode

pytestmark = pytest.mark.gpu


def _run(wl, d, rows):
    import paged_kv_cache_22_amd as pa
    out = pa.decode(d.q[rows].contiguous(), d.k, d.v, d.bt[rows].contiguous(),
                    d.sl[rows].contiguous(), max_seq_len=wl.max_seq_len, scale=wl.scale,
                    partition_size=0, k_scale=d.ks, v_scale=d.vs)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("kv,B,Hkv,G,d", [("bf16", 130, 8, 4, 128), ("fp8", 257, 8, 4, 128),
                                           ("bf16", 1024, 1, 16, 64), ("bf16", 1000, 2, 2, 128)])
def test_longest_first_equals_index_order_bit_for_bit(kv, B, Hkv, G, d):
    rng = np.random.default_rng(900 + B)
    # ties, empty sequences, lengths past the class cap (1023 units), short ones
    lens = rng.integers(1, 600, size=B).astype(np.int32)
    lens[::7] = 256
    lens[3::11] = 0
    lens[5] = lens[6] = 1023 * 16 + 40
    lens[9] = 1024 * 16
    wl = W.decode_workload(seed=901 + B, num_seqs=B, num_q_heads=G * Hkv, num_kv_heads=Hkv,
                           head_dim=d, len_lo=0, len_hi=0, q_dtype="bf16", kv_dtype=kv,
                           seq_lens=lens)
    dv = Dev(wl)
    assert B * Hkv >= 1024
    whole = _run(wl, dv, slice(0, B))
    # the same sequences in batches small enough to run in index order
    step = 1023 // Hkv
    parts = torch.cat([_run(wl, dv, slice(i, min(B, i + step))) for i in range(0, B, step)])
    print(f"[lpt] {kv} B={B} Hkv={Hkv} G={G} d={d}: whole batch vs {-(-B // step)} batches", flush=True)
    assert torch.equal(whole.view(torch.int16), parts.view(torch.int16))
    compare(f64(whole), oracle_decode(wl)[0], "fp8" if kv == "fp8" else "bf16",
            f"longest first {kv} B={B}", out_rounding=True)
