"""Every entry point repeats bit for bit: the same inputs, called again,
give the same output bits (the kernels take no data-dependent or
timing-dependent order anywhere).  Covers decode in every split mode and KV
dtype, multi-query decode (whose kernels are built with the accumulators in
AGPRs: in the VGPR form their outputs varied between calls), prefill chunks,
the mixed step and the shared-prefix cascade, at the Llama-3-8B layer shape
with lengths of 512-4096 tokens."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import Dev, dev

pytestmark = pytest.mark.gpu
REPEATS = 4


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else (
        t.view(torch.int32) if t.dtype == torch.float32 else t)


def assert_repeats(what, fn):
    first = None
    for k in range(REPEATS):
        out = fn()
        torch.cuda.synchronize()
        got = [bits(x).clone() for x in (out if isinstance(out, tuple) else (out,))]
        if first is None:
            first = got
            continue
        bad = sum(int((a != b).sum()) for a, b in zip(first, got))
        assert bad == 0, f"{what}: call {k} differs from the first in {bad} elements"


def decode_wl(kv, q_len=0, B=64):
    return W.decode_workload(seed=2, num_seqs=B, num_q_heads=32, num_kv_heads=8, head_dim=128,
                             len_lo=512, len_hi=4096, q_dtype="f32" if kv == "f32" else "bf16",
                             kv_dtype=kv, q_len=q_len, pad=0)


@pytest.mark.parametrize("kv", ["bf16", "fp8", "f32"])
@pytest.mark.parametrize("P", [-1, 0, 512])
def test_decode_repeats(kv, P):
    import paged_kv_cache_22_amd as pa
    wl = decode_wl(kv, B=64 if kv != "f32" else 16)
    d = Dev(wl)
    print(f"[determinism] decode {kv} P={P}", flush=True)
    assert_repeats(f"decode {kv} P={P}", lambda: pa.decode(
        d.q, d.k, d.v, d.bt, d.sl, max_seq_len=wl.max_seq_len, scale=wl.scale, partition_size=P,
        k_scale=d.ks, v_scale=d.vs))


@pytest.mark.parametrize("kv,q_len", [("bf16", 4), ("bf16", 2), ("fp8", 4), ("f32", 4), ("bf16", 8)])
@pytest.mark.parametrize("P", [-1, 0, 512])
def test_multi_query_repeats(kv, q_len, P):
    import paged_kv_cache_22_amd as pa
    wl = decode_wl(kv, q_len=q_len, B=64 if kv != "f32" else 16)
    d = Dev(wl)
    print(f"[determinism] multi-query {kv} q_len={q_len} P={P}", flush=True)
    assert_repeats(f"multi-query {kv} q_len={q_len} P={P}", lambda: pa.decode_multi_query(
        d.q, d.k, d.v, d.bt, d.sl, max_seq_len=wl.max_seq_len, scale=wl.scale, partition_size=P,
        k_scale=d.ks, v_scale=d.vs))


def test_prefill_mixed_and_shared_prefix_repeat():
    import bench
    import paged_kv_cache_22_amd as pa
    m = W.config4(pad=0)
    dd, dp = bench.mixed_devices(m)
    pre = m.prefill
    print("[determinism] C4 prefill chunks and mixed step", flush=True)
    assert_repeats("C4 prefill", lambda: pa.prefill_chunk(
        dp.q, dp.cu, dp.k, dp.v, dp.bt, dp.sl, max_q_len=pre.max_q_len, scale=pre.scale,
        want_lse=True))
    for P in (-1, 512):
        assert_repeats(f"C4 mixed step P={P}", lambda: pa.mixed_step(
            dd.q, dd.bt, dd.sl, dp.q, dp.cu, dp.bt, dp.sl, dd.k, dd.v,
            max_seq_len=m.decode.max_seq_len, max_q_len=pre.max_q_len, partition_size=P,
            scale=pre.scale))
    sp = W.shared_prefix_workload(seed=2, num_seqs=64, num_q_heads=32, num_kv_heads=8, head_dim=128,
                                  prefix_len=2048, len_lo=512, len_hi=4096, q_dtype="bf16",
                                  kv_dtype="bf16")
    wl = sp.full
    args = (dev(wl.q, wl.q_dtype), dev(wl.k_cache, wl.kv_dtype), dev(wl.v_cache, wl.kv_dtype),
            dev(sp.prefix_table), sp.prefix_len, dev(sp.suffix_table), dev(sp.suffix_lens))
    print("[determinism] shared prefix", flush=True)
    assert_repeats("shared prefix", lambda: pa.decode_shared_prefix(
        *args, max_seq_len=int(sp.suffix_lens.max()), partition_size=512, scale=wl.scale))


SHAPES = [
    # (head_dim, q-heads, kv-heads, block size, KV dtype, queries per sequence)
    (64, 40, 10, 16, "bf16", 1), (64, 40, 10, 32, "fp8", 1), (128, 32, 32, 16, "bf16", 1),
    (128, 64, 4, 64, "bf16", 1), (128, 32, 8, 32, "f32", 1), (64, 16, 2, 16, "bf16", 2),
    (128, 16, 16, 64, "bf16", 4), (64, 32, 8, 16, "f32", 2),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"d{s[0]}-{s[1]}x{s[2]}-bs{s[3]}-{s[4]}-q{s[5]}"
                                                for s in SHAPES])
def test_other_shapes_repeat(shape):
    """Head dims, group sizes 1-16, block sizes 16/32/64 and dtypes beyond the
    Llama-3-8B layer, in the three split modes, and the same caches as
    prefill chunks."""
    import paged_kv_cache_22_amd as pa
    d_, hq, hkv, bs, kv, ql = shape
    qd = "f32" if kv == "f32" else "bf16"
    wl = W.decode_workload(seed=11, num_seqs=24, num_q_heads=hq, num_kv_heads=hkv, head_dim=d_,
                           len_lo=300, len_hi=3000, q_dtype=qd, kv_dtype=kv, block_size=bs,
                           q_len=ql if ql > 1 else 0, pad=0)
    d = Dev(wl)
    for P in (-1, 0, 256):
        print(f"[determinism] {shape} P={P}", flush=True)
        if ql > 1:
            fn = lambda: pa.decode_multi_query(d.q, d.k, d.v, d.bt, d.sl, max_seq_len=wl.max_seq_len,
                                               scale=wl.scale, partition_size=P, k_scale=d.ks,
                                               v_scale=d.vs)
        else:
            fn = lambda: pa.decode(d.q, d.k, d.v, d.bt, d.sl, max_seq_len=wl.max_seq_len,
                                   scale=wl.scale, partition_size=P, k_scale=d.ks, v_scale=d.vs)
        assert_repeats(f"{shape} P={P}", fn)
    pw = W.prefill_workload(seed=12, q_lens=[200, 37, 128], ctx_lens=[900, 15, 2000],
                            num_q_heads=hq, num_kv_heads=hkv, head_dim=d_, q_dtype=qd, kv_dtype=kv,
                            block_size=bs)
    p = Dev(pw)
    assert_repeats(f"{shape} prefill", lambda: pa.prefill_chunk(
        p.q, p.cu, p.k, p.v, p.bt, p.sl, max_q_len=pw.max_q_len, scale=pw.scale, k_scale=p.ks,
        v_scale=p.vs, want_lse=True))
