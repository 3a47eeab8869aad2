"""Caches larger than 4 GiB: the live blocks sit past the 4 GiB mark of a
large device pool (block ids above 2^20 at 4 KiB tiles), so every tile
offset needs 64-bit arithmetic.  The oracle works on the small pool with
the original block ids; the GPU sees the same blocks at their remapped ids."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import Dev, compare, dev, f64

pytestmark = pytest.mark.gpu

BIG_BLOCKS = 1 << 17          # 131072 blocks x 8 kv-heads x 4 KiB = 4 GiB per cache (bf16, d=128)


def big_copy(small, nb_big, where):
    """A device tensor of nb_big blocks whose blocks `where` hold the small pool."""
    big = torch.empty((nb_big,) + tuple(small.shape[1:]), dtype=small.dtype, device="cuda")
    big[torch.as_tensor(where, device="cuda")] = small
    return big


def test_decode_and_prefill_past_4gib():
    import paged_kv_cache_22_amd as pa
    wl = W.decode_workload(seed=900, num_seqs=12, num_q_heads=32, num_kv_heads=8, head_dim=128,
                           len_lo=1, len_hi=700, q_dtype="bf16", kv_dtype="bf16", name="big")
    nb = wl.num_blocks
    nb_big = BIG_BLOCKS + nb + 64
    where = BIG_BLOCKS + 64 + np.random.default_rng(1).permutation(nb)   # past 4 GiB
    d = Dev(wl)
    kb, vb = big_copy(d.k, nb_big, where), big_copy(d.v, nb_big, where)
    assert kb.numel() * kb.element_size() > (1 << 32)
    remap = np.where(wl.block_table >= 0, where[np.maximum(wl.block_table, 0)], -1).astype(np.int32)
    bt = dev(remap)
    ref, _ = oracle.decode(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, wl.scale,
                           "bf16", "bf16")
    for P in (0, 256, -1):
        print(f"[big] decode P={P}", flush=True)
        out = pa.decode(d.q, kb, vb, bt, d.sl, max_seq_len=wl.max_seq_len, scale=wl.scale,
                        partition_size=P)
        torch.cuda.synchronize()
        compare(f64(out), ref, "bf16", f"decode past 4 GiB P={P}")
    # the same cache as prefill chunks: one query row per sequence = its last token
    cu = torch.arange(0, wl.num_seqs + 1, dtype=torch.int32, device="cuda")
    print("[big] prefill", flush=True)
    out = pa.prefill_chunk(d.q, cu, kb, vb, bt, d.sl, max_q_len=1, scale=wl.scale)
    torch.cuda.synchronize()
    compare(f64(out), ref, "bf16", "prefill past 4 GiB")
    del kb, vb


def test_write_past_4gib():
    import paged_kv_cache_22_amd as pa
    nb_big = BIG_BLOCKS + 64
    slots = W.write_chunks(seed=901, chunk_lens=[100, 37], ctx_lens=[0, 5], num_blocks=32)
    wl = W.write_workload(seed=902, slot_mapping=slots, num_kv_heads=8, head_dim=128,
                          in_dtype="bf16", kv_dtype="fp8", num_blocks=32, fill_cache=False,
                          name="write big")
    off = BIG_BLOCKS + 16                 # the small pool's block 0 lives at block `off`
    kb = torch.zeros((nb_big,) + wl.k_cache.shape[1:], dtype=torch.uint8, device="cuda")
    vb = torch.zeros((nb_big,) + wl.v_cache.shape[1:], dtype=torch.uint8, device="cuda")
    assert kb.numel() > (1 << 31)
    print("[big] write", flush=True)
    pa.write_kv(dev(wl.key, "bf16"), dev(wl.value, "bf16"), kb, vb, dev(slots + off * 16),
                k_scale=dev(wl.k_scale), v_scale=dev(wl.v_scale))
    torch.cuda.synchronize()
    ek, ev = wl.k_cache.copy(), wl.v_cache.copy()
    oracle.write_kv(ek, ev, wl.key, wl.value, slots, "bf16", "fp8", wl.k_scale, wl.v_scale)
    assert (kb[off:off + 32].cpu().numpy() == ek).all()
    assert (vb[off:off + 32].cpu().numpy() == ev).all()
    assert int(kb[:off].count_nonzero()) == 0 and int(vb[:off].count_nonzero()) == 0
