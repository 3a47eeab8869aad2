"""Cache blocks of 32 and 64 tokens (the kernels read them as 2 or 4 units of
16 tokens) against the oracle, which pages with any block size: decode in
every partition mode, prefill chunks, multi-query decode and cache writes."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import Dev, compare, dev, f64, run_decode, run_prefill

pytestmark = pytest.mark.gpu
BS = [32, 64]


def lens_around(bs, rng, n=18, hi=900):
    """Lengths at, just below and just above whole blocks, plus random ones."""
    edge = [1, bs - 1, bs, bs + 1, 2 * bs, 3 * bs + 15, 16, 17, 48]
    return edge + rng.integers(1, hi, n - len(edge)).tolist()


def decode_wl(seed, bs, kv, d, lens, hq=8, hkv=2, q_len=0):
    qd = "f32" if kv == "f32" else "bf16"
    return W.decode_workload(seed=seed, num_seqs=len(lens), num_q_heads=hq, num_kv_heads=hkv,
                             head_dim=d, len_lo=0, len_hi=0, q_dtype=qd, kv_dtype=kv,
                             seq_lens=lens, block_size=bs, q_len=q_len, name=f"bs{bs}")


@pytest.mark.parametrize("bs", BS)
@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("d_head", [64, 128])
def test_decode_all_modes(bs, kv, d_head):
    wl = decode_wl(600 + bs + d_head, bs, kv, d_head,
                   lens_around(bs, np.random.default_rng(bs + d_head)))
    ref, _ = oracle.decode(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, wl.scale,
                           wl.q_dtype, wl.kv_dtype, wl.k_scale, wl.v_scale)
    d = Dev(wl)
    for P in (0, 48, 256, -1):
        print(f"[bs] decode bs={bs} {kv} d={d_head} P={P}", flush=True)
        compare(f64(run_decode(d, partition_size=P)), ref, kv, f"decode bs={bs} {kv} d={d_head} P={P}")


@pytest.mark.parametrize("bs", BS)
def test_decode_llama3_8b_shape_full(bs):
    """C2's batch (64 sequences of 512-4096 tokens, 32/8 heads, d = 128,
    bf16) paged with the larger block size."""
    wl = W.decode_workload(seed=2, num_seqs=64, num_q_heads=32, num_kv_heads=8, head_dim=128,
                           len_lo=512, len_hi=4096, q_dtype="bf16", kv_dtype="bf16",
                           block_size=bs, name=f"C2 bs={bs}")
    ref, _ = oracle.decode(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, wl.scale,
                           "bf16", "bf16")
    d = Dev(wl)
    for P in (1024, -1):
        compare(f64(run_decode(d, partition_size=P)), ref, "bf16", f"C2 shape bs={bs} P={P}")


@pytest.mark.parametrize("bs", BS)
@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8"])
def test_prefill_ragged(bs, kv):
    qd = "f32" if kv == "f32" else "bf16"
    wl = W.prefill_workload(seed=620 + bs, q_lens=[5, 17, 40, 1, 64, 33, 100],
                            ctx_lens=[0, 33, 9, 100, 64, 0, 2 * bs + 3], num_q_heads=8,
                            num_kv_heads=2, head_dim=128, q_dtype=qd, kv_dtype=kv, block_size=bs)
    ref, ref_lse = oracle.prefill_chunk(wl.q, wl.cu_q_lens, wl.k_cache, wl.v_cache,
                                        wl.block_table, wl.seq_lens, wl.scale, qd, kv,
                                        wl.k_scale, wl.v_scale)
    got, lse = run_prefill(Dev(wl), want_lse=True)
    compare(f64(got), ref, kv, f"prefill bs={bs} {kv}")
    assert np.abs(f64(lse) - ref_lse).max() < (1e-3 if kv == "f32" else 2e-3)  # bf16 weights: ln(1 + 2^-9)


@pytest.mark.parametrize("bs", BS)
def test_multi_query(bs):
    import paged_kv_cache_22_amd as pa
    lens = [4, bs, bs + 3, 300, 1000]
    wl = decode_wl(630 + bs, bs, "bf16", 128, lens, hq=32, hkv=8, q_len=4)
    B, qn, Hq, dd = wl.q.shape
    ref, _ = oracle.prefill_chunk(wl.q.reshape(B * qn, Hq, dd), np.arange(0, B * qn + 1, qn),
                                  wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, wl.scale,
                                  "bf16", "bf16")
    d = Dev(wl)
    for P in (0, 64, -1):
        out = pa.decode_multi_query(d.q, d.k, d.v, d.bt, d.sl, max_seq_len=wl.max_seq_len,
                                    scale=wl.scale, partition_size=P)
        torch.cuda.synchronize()
        compare(f64(out), ref.reshape(B, qn, Hq, dd), "bf16", f"multi-query bs={bs} P={P}")


_VIEW = {"f32": (torch.int32, np.uint32), "bf16": (torch.int16, np.uint16),
         "fp8": (torch.uint8, np.uint8)}


@pytest.mark.parametrize("bs", BS)
@pytest.mark.parametrize("in_dtype,kv_dtype", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "fp8")])
def test_write(bs, in_dtype, kv_dtype):
    """Chunks starting on every 16-token unit of a block (whole-unit groups
    inside larger blocks), straddling starts, decode tokens and padding."""
    import paged_kv_cache_22_amd as pa
    nb = 64
    chunk = W.write_chunks(seed=640 + bs, chunk_lens=[64, 48, 40, 7, 100],
                           ctx_lens=[0, 16, 3, bs - 16, 32], num_blocks=nb // 2, block_size=bs)
    dec = W.write_decode_step(seed=641, num_seqs=20, num_blocks=nb // 2, block_size=bs) + (nb // 2) * bs
    slots = np.concatenate([chunk, dec]).astype(np.int32)
    slots[[3, 70]] = -1
    wl = W.write_workload(seed=642, slot_mapping=slots, num_kv_heads=8, head_dim=128,
                          in_dtype=in_dtype, kv_dtype=kv_dtype, num_blocks=nb, block_size=bs,
                          name=f"write bs={bs}")
    kc, vc = dev(wl.k_cache, wl.kv_dtype), dev(wl.v_cache, wl.kv_dtype)
    pa.write_kv(dev(wl.key, in_dtype), dev(wl.value, in_dtype), kc, vc, dev(wl.slot_mapping),
                k_scale=dev(wl.k_scale), v_scale=dev(wl.v_scale))
    torch.cuda.synchronize()
    ek, ev = wl.k_cache.copy(), wl.v_cache.copy()
    oracle.write_kv(ek, ev, wl.key, wl.value, wl.slot_mapping, in_dtype, kv_dtype, wl.k_scale,
                    wl.v_scale)
    tv, nv = _VIEW[kv_dtype]
    assert (kc.view(tv).cpu().numpy().view(nv) == ek.view(nv)).all()
    assert (vc.view(tv).cpu().numpy().view(nv) == ev.view(nv)).all()
