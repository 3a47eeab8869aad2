"""Multi-query decode (pa_decode_multi_query) against the oracle.

Each sequence's q_len queries are the newest q_len cached tokens, causal
among themselves: exactly a prefill chunk of q_len rows whose context is
seq_len - q_len, which the oracle's causal chunked prefill computes.  Both
kernel routes are covered: q_len * G <= 16 (the decode kernel, columns =
(query, head) pairs, one pass and split-KV) and q_len * G > 16 (the prefill
kernel, one chunk per sequence).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import Dev, compare, dev, f64

pytestmark = pytest.mark.gpu


def oracle_mq(wl):
    """[B, q_len, Hq, d] reference; sequences with seq_len 0 (no queries in
    the cache) are left out and expected to come back as zeros."""
    B, qn, Hq, d = wl.q.shape
    q = wl.q.reshape(B * qn, Hq, d)
    cu = np.arange(0, B * qn + 1, qn, dtype=np.int32)
    items = [(b, h) for b in range(B) if wl.seq_lens[b] > 0 for h in range(wl.num_kv_heads)]
    ref, _ = oracle.prefill_chunk(q, cu, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens,
                                  wl.scale, wl.q_dtype, wl.kv_dtype, wl.k_scale, wl.v_scale,
                                  items=items)
    ref = ref.reshape(B, qn, Hq, d)
    ref[wl.seq_lens == 0] = 0.0
    return ref


def run_mq(d: Dev, P):
    import paged_kv_cache_22_amd as pa
    wl = d.wl
    print(f"[mq] {wl.name}: B={wl.num_seqs} q_len={wl.q_len} Hq={wl.num_q_heads} "
          f"Hkv={wl.num_kv_heads} d={wl.head_dim} {wl.kv_dtype} P={P}", flush=True)
    out = pa.decode_multi_query(d.q, d.k, d.v, d.bt, d.sl, max_seq_len=wl.max_seq_len,
                                scale=wl.scale, partition_size=P, k_scale=d.ks, v_scale=d.vs)
    torch.cuda.synchronize()
    return out


def mq_workload(seed, q_len, G, kv="bf16", d=128, hkv=2, lens=None, B=6, lo=None, hi=300,
                name="mq"):
    qd = "f32" if kv == "f32" else "bf16"
    return W.decode_workload(seed=seed, num_seqs=B, num_q_heads=G * hkv, num_kv_heads=hkv,
                             head_dim=d, len_lo=q_len if lo is None else lo, len_hi=hi,
                             q_dtype=qd, kv_dtype=kv, seq_lens=lens, q_len=q_len, name=name)


@pytest.mark.parametrize("q_len", [2, 3, 4])
@pytest.mark.parametrize("P", [0, 32, 512])
def test_packed_columns_gqa4(q_len, P):
    """Llama-3 grouping (G = 4): q_len * G <= 16 takes the decode kernel.
    Lengths include q_len itself, block edges and several partitions."""
    lens = [q_len, 16, 17, 16 + q_len - 1, 33, 250, 513, 1100]
    wl = mq_workload(400 + q_len, q_len, 4, lens=lens, B=len(lens), name=f"gqa4 q_len={q_len}")
    ref = oracle_mq(wl)
    got = f64(run_mq(Dev(wl), P))
    compare(got, ref, "bf16", f"multi-query q_len={q_len} P={P}")


@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("d_head", [64, 128])
def test_all_dtypes(kv, d_head):
    wl = mq_workload(410 + d_head, 4, 4, kv=kv, d=d_head, B=7, name=f"mq {kv} d={d_head}")
    ref = oracle_mq(wl)
    for P in (0, 64):
        compare(f64(run_mq(Dev(wl), P)), ref, kv, f"multi-query {kv} d={d_head} P={P}")


@pytest.mark.parametrize("G,q_len", [(1, 16), (2, 8), (5, 3), (16, 1), (8, 2)])
def test_column_packings(G, q_len):
    """Every packing up to the 16 columns, non-power-of-two groups included."""
    wl = mq_workload(420 + G, q_len, G, B=5, hi=200, name=f"G={G} q_len={q_len}")
    ref = oracle_mq(wl)
    for P in (0, 48):
        compare(f64(run_mq(Dev(wl), P)), ref, "bf16", f"G={G} q_len={q_len} P={P}")


@pytest.mark.parametrize("G,q_len", [(4, 8), (16, 2), (4, 5)])
def test_more_pairs_than_columns_uses_prefill(G, q_len):
    """q_len * G > 16: the prefill kernel runs each sequence as one chunk
    (partition size and workspace are ignored)."""
    wl = mq_workload(430 + G * q_len, q_len, G, B=5, hi=260, name=f"wide G={G} q_len={q_len}")
    ref = oracle_mq(wl)
    for P in (0, 512):
        compare(f64(run_mq(Dev(wl), P)), ref, "bf16", f"wide G={G} q_len={q_len} P={P}")


@pytest.mark.parametrize("G,q_len", [(4, 4), (4, 8)])
def test_idle_sequences_give_zeros(G, q_len):
    lens = [0, q_len + 3, 0, 40]
    wl = mq_workload(440 + q_len, q_len, G, lens=lens, B=4, name="idle")
    ref = oracle_mq(wl)
    for P in (0, 32):
        got = f64(run_mq(Dev(wl), P))
        assert (got[0] == 0).all() and (got[2] == 0).all()
        compare(got, ref, "bf16", f"idle sequences G={G} q_len={q_len} P={P}")


def test_q_len_one_is_plain_decode_bitwise():
    import paged_kv_cache_22_amd as pa
    wl = mq_workload(450, 1, 4, B=6, hi=700, name="q_len 1")
    d = Dev(wl)
    for P in (0, 64):
        got = run_mq(d, P)
        plain = pa.decode(d.q.reshape(wl.num_seqs, wl.num_q_heads, wl.head_dim), d.k, d.v, d.bt,
                          d.sl, max_seq_len=wl.max_seq_len, scale=wl.scale, partition_size=P)
        torch.cuda.synchronize()
        assert torch.equal(got.reshape(plain.shape).view(torch.int16), plain.view(torch.int16))


def test_last_query_matches_plain_decode():
    """The newest query sees the whole sequence: its row is ordinary decode."""
    import paged_kv_cache_22_amd as pa
    wl = mq_workload(460, 4, 4, B=6, hi=900, name="last query")
    d = Dev(wl)
    got = f64(run_mq(d, 64))[:, -1]
    plain = pa.decode(d.q[:, -1].contiguous(), d.k, d.v, d.bt, d.sl, max_seq_len=wl.max_seq_len,
                      scale=wl.scale, partition_size=64)
    torch.cuda.synchronize()
    assert np.abs(got - f64(plain)).max() <= 2.0 ** -8 * np.abs(f64(plain)).max()


def test_spec_verify_llama3_8b_shape_full():
    """The benchmark's verify step: 64 sequences of 512-4096 tokens, 4 queries
    each (16 columns with GQA 4), 32/8 heads, d = 128, bf16, partitions of
    1024 tokens."""
    wl = W.decode_workload(seed=2, num_seqs=64, num_q_heads=32, num_kv_heads=8, head_dim=128,
                           len_lo=512, len_hi=4096, q_dtype="bf16", kv_dtype="bf16", q_len=4,
                           name="verify C2 shape")
    ref = oracle_mq(wl)
    compare(f64(run_mq(Dev(wl), 1024)), ref, "bf16", "spec verify 64 x 4 queries")


def test_multi_query_in_a_captured_graph():
    """pa_decode_multi_query (balanced and 512-token partitions) captured
    once in a HIP graph and replayed with new queries: every replay equals
    the eager calls bit for bit (the kernels stage their partials in LDS and
    keep no state between calls beyond the workspace they fill)."""
    import paged_kv_cache_22_amd as pa
    wl = W.decode_workload(seed=431, num_seqs=32, num_q_heads=32, num_kv_heads=8, head_dim=128,
                           len_lo=600, len_hi=3000, q_dtype="bf16", kv_dtype="bf16", q_len=4, pad=0)
    d = Dev(wl)
    modes = (-1, 512)
    B, qn, Hq, D = wl.q.shape
    ws = {P: torch.empty(max(pa.decode_workspace_size(B, qn * Hq, D, wl.max_seq_len, P), 256),
                         dtype=torch.uint8, device="cuda") for P in modes}
    outs = {P: torch.empty_like(d.q) for P in modes}

    def step():
        for P in modes:
            pa.decode_multi_query(d.q, d.k, d.v, d.bt, d.sl, max_seq_len=wl.max_seq_len,
                                  scale=wl.scale, partition_size=P, out=outs[P], workspace=ws[P])

    step()                       # eager warm-up: the occupancy query runs outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    rng = np.random.default_rng(432)
    for rep in range(3):
        d.q.copy_(torch.from_numpy(W.to_bf16_bits(
            rng.standard_normal(wl.q.shape).astype(np.float32)).view(np.int16)).view(torch.bfloat16))
        torch.cuda.synchronize()
        print(f"[graph] multi-query replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        got = {P: outs[P].clone() for P in modes}
        step()
        torch.cuda.synchronize()
        for P in modes:
            assert torch.equal(got[P].view(torch.int16), outs[P].view(torch.int16)), (rep, P)
