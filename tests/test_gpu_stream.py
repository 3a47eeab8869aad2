"""Fixed-partition decode with several partitions streamed per workgroup
against the kernel that gives each partition a workgroup of its own.

The library streams fixed partitions when the caller's max_seq_len spans at
least 16 of them (include/pa.h) and keeps one workgroup per partition
below that.  Both compute every partition over the same blocks per wave
and combine the waves in the same order, so the two must agree bit for bit:
the merged outputs and every partial a sequence owns.  The streamed results
are also checked against the oracle.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import Dev, compare, f64, oracle_decode

pytestmark = pytest.mark.gpu
STREAM_MIN_PARTS = 16   # include/pa.h, pa_decode: where fixed partitions are streamed

# (kv dtype, head_dim, q-heads, kv-heads, block size, partition size, sequences):
# enough partitions per kv-head that a workgroup streams runs of several,
# across sequence boundaries
CASES = [
    ("bf16", 128, 8, 2, 16, 64, 400),
    ("bf16", 128, 8, 2, 32, 128, 300),
    ("bf16", 128, 8, 2, 64, 256, 120),
    ("bf16", 128, 8, 2, 16, 512, 60),
    ("fp8", 128, 8, 2, 16, 64, 400),
    ("fp8", 128, 16, 1, 32, 64, 600),
    ("bf16", 64, 40, 10, 16, 64, 100),
    ("bf16", 128, 16, 1, 16, 64, 600),
    ("bf16", 128, 8, 1, 32, 128, 300),
    ("fp8", 64, 8, 8, 64, 256, 100),
]


def _lens(P, B, seed):
    """Lengths in [0, (STREAM_MIN_PARTS - 1) P]: runs of many partitions, the
    lengths at and around partition boundaries, and the empty sequence."""
    top = (STREAM_MIN_PARTS - 1) * P
    special = [0, 1, P - 1, P, P + 1, 2 * P - 1, 2 * P, 2 * P + 1, top - 1, top]
    rng = np.random.default_rng(seed)
    rest = rng.integers(1, top, size=B - len(special), endpoint=True)
    lens = np.concatenate([special, rest]).astype(np.int32)
    rng.shuffle(lens)
    return lens


@pytest.mark.parametrize("kv,d,Hq,Hkv,bs,P,B", CASES)
def test_streamed_partitions_bit_identical(kv, d, Hq, Hkv, bs, P, B):
    import paged_kv_cache_22_amd as pa
    lens = _lens(P, B, seed=700 + P + d + bs)
    wl = W.decode_workload(seed=701 + P, num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                           len_lo=0, len_hi=0, q_dtype="bf16", kv_dtype=kv, block_size=bs,
                           seq_lens=lens)
    dv = Dev(wl)
    # a table wide enough for max_seq_len = STREAM_MIN_PARTS * P (columns past
    # a sequence's blocks are never read)
    width = STREAM_MIN_PARTS * P // bs
    bt = torch.zeros((B, width), dtype=torch.int32, device="cuda")
    bt[:, :dv.bt.shape[1]] = dv.bt
    short, long = (STREAM_MIN_PARTS - 1) * P, STREAM_MIN_PARTS * P
    kw = dict(scale=wl.scale, partition_size=P, k_scale=dv.ks, v_scale=dv.vs)
    one = pa.decode(dv.q, dv.k, dv.v, bt, dv.sl, max_seq_len=short, **kw)
    streamed = pa.decode(dv.q, dv.k, dv.v, bt, dv.sl, max_seq_len=long, **kw)
    po1, pl1 = pa.decode_partitions(dv.q, dv.k, dv.v, bt, dv.sl, max_seq_len=short, **kw)
    po2, pl2 = pa.decode_partitions(dv.q, dv.k, dv.v, bt, dv.sl, max_seq_len=long, **kw)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), streamed.view(torch.int16)), "merged outputs differ"
    # the partials each sequence owns: partitions 0 .. ceil(L / P) - 1
    nparts = (lens.astype(np.int64) + P - 1) // P
    for p in range(STREAM_MIN_PARTS - 1):
        rows = torch.from_numpy(nparts > p).to("cuda")
        if not bool(rows.any()):
            continue
        a, b = po1[rows][:, :, p], po2[rows][:, :, p]
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"partial {p} differs"
        a, b = pl1[rows][:, :, p], pl2[rows][:, :, p]
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"partial lse {p} differs"
    print(f"[stream] {kv} d={d} G={Hq // Hkv} bs={bs} P={P} B={B}: bit-identical "
          f"({int(nparts.sum())} partitions)", flush=True)
    ref = oracle_decode(wl)[0]
    compare(f64(streamed), ref, "fp8" if kv == "fp8" else "bf16",
            f"streamed P={P} {kv} d={d}", out_rounding=True)
