"""Balanced split-KV decode (partition_size = PA_PARTITION_BALANCED) against
the oracle.  Each kv-head's blocks, laid end to end over the batch, are cut
into equal ranges, one per resident workgroup; a range may hold pieces of
several sequences and a sequence may be spread over many ranges.  The cases
stress both: batches of many short sequences, one long sequence among short
ones, empty sequences in between, and batches longer than one 64-lane scan.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import Dev, compare, f64, run_decode

pytestmark = pytest.mark.gpu
BAL = -1


def oracle_decode(wl):
    return oracle.decode(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, wl.scale,
                         wl.q_dtype, wl.kv_dtype, wl.k_scale, wl.v_scale)[0]


def wl_of(seed, lens, kv="bf16", d=128, hq=32, hkv=8, name="balanced"):
    qd = "f32" if kv == "f32" else "bf16"
    return W.decode_workload(seed=seed, num_seqs=len(lens), num_q_heads=hq, num_kv_heads=hkv,
                             head_dim=d, len_lo=0, len_hi=0, q_dtype=qd, kv_dtype=kv,
                             seq_lens=lens, name=name)


def check(wl, what, kv=None):
    kv = kv or wl.kv_dtype
    print(f"[balanced] {what}: B={wl.num_seqs} Hkv={wl.num_kv_heads} total={wl.total_tokens}",
          flush=True)
    ref = oracle_decode(wl)
    got = f64(run_decode(Dev(wl), partition_size=BAL))
    compare(got, ref, kv, what)
    return got, ref


def test_c1_tiny_fp32():
    check(W.config1(), "C1 balanced", "f32")


def test_c2_llama3_8b_full():
    check(W.config2(), "C2 balanced")


def test_c5_fp8_full():
    check(W.config5(), "C5 balanced")


@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("d_head", [64, 128])
def test_ragged_all_dtypes(kv, d_head):
    rng = np.random.default_rng(500 + d_head)
    lens = rng.integers(1, 700, 23).tolist()
    check(wl_of(501 + d_head, lens, kv=kv, d=d_head, hq=8, hkv=2), f"ragged {kv} d={d_head}", kv)


def test_many_short_sequences_per_split():
    """300 sequences of 1-40 tokens: each range covers many whole sequences
    (direct writes) plus pieces at its two ends; the batch scan runs over
    five 64-lane chunks."""
    rng = np.random.default_rng(510)
    lens = rng.integers(1, 41, 300).tolist()
    check(wl_of(510, lens), "300 short sequences")


def test_batch_beyond_4096_sequences():
    """8200 sequences of 0-24 tokens, 8 kv-heads: each lane's run of the
    start-up scan holds 129 sequences (the search inside a run takes three
    64-wide windows), and each workgroup's range covers more than 64
    sequences (the piece loop reloads its window of lengths)."""
    rng = np.random.default_rng(512)
    lens = rng.integers(0, 25, 8200)
    wl = wl_of(512, lens.tolist(), hq=8, hkv=8, name="8200 short sequences")
    print(f"[balanced] 8200 short sequences: total={wl.total_tokens}", flush=True)
    ref = oracle_decode(wl)
    got = f64(run_decode(Dev(wl), partition_size=BAL))
    # outputs of sequences this short reach |out| ~ 5, where the bf16 output
    # rounding alone is up to 2^-6: the bar adds it per element
    compare(got, ref, "bf16", "8200 short sequences", out_rounding=True)


def test_one_long_sequence_over_many_splits():
    """One 60000-token sequence among short ones: it is spread over most
    ranges, so its merge combines dozens of pieces."""
    lens = [5, 60000, 17, 1, 300]
    check(wl_of(520, lens, hq=16, hkv=4), "long among short")


def test_empty_sequences_in_between():
    lens = [0, 33, 0, 0, 1, 1000, 0, 16, 17, 0]
    got, _ = check(wl_of(530, lens, hq=8, hkv=2), "empty in between")
    for b in (0, 2, 3, 6, 9):
        assert (got[b] == 0).all()


def test_all_empty():
    got, _ = check(wl_of(531, [0, 0, 0], hq=8, hkv=2), "all empty")
    assert (got == 0).all()


def test_fewer_units_than_splits():
    """A few blocks in total: most ranges are empty and return at once."""
    check(wl_of(540, [3, 20, 1], hq=8, hkv=2), "fewer units than splits")


@pytest.mark.parametrize("G", [1, 5, 16])
def test_group_sizes(G):
    rng = np.random.default_rng(550 + G)
    lens = rng.integers(1, 900, 40).tolist()
    check(wl_of(550 + G, lens, hq=2 * G, hkv=2), f"G={G}")


def test_logos_shape_d64_10_kv_heads():
    rng = np.random.default_rng(560)
    lens = rng.integers(100, 3000, 50).tolist()
    check(wl_of(560, lens, d=64, hq=40, hkv=10), "Logos shape")


def test_agrees_with_partition_modes():
    """Same batch through one-pass, fixed partitions and balanced: all three
    within rounding of each other."""
    wl = W.config2()
    d = Dev(wl)
    outs = {P: f64(run_decode(d, partition_size=P)) for P in (0, 1024, BAL)}
    scale = np.abs(outs[0]).max()
    for P in (1024, BAL):
        assert np.abs(outs[P] - outs[0]).max() <= 2.0 ** -8 * scale


def test_workspace_reuse_deterministic():
    import paged_kv_cache_22_amd as pa
    wl = W.config2()
    d = Dev(wl)
    ws = torch.empty(pa.decode_workspace_size(wl.num_seqs, wl.num_q_heads, wl.head_dim,
                                              wl.max_seq_len, BAL), dtype=torch.uint8, device="cuda")
    a = run_decode(d, partition_size=BAL, workspace=ws).clone()
    ws.fill_(0x7F)                                   # garbage partials and piece records
    b = run_decode(d, partition_size=BAL, workspace=ws)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("q_len", [2, 4])
def test_multi_query_balanced(q_len):
    import paged_kv_cache_22_amd as pa
    rng = np.random.default_rng(570 + q_len)
    lens = [q_len] + rng.integers(q_len, 2000, 30).tolist() + [0]
    wl = W.decode_workload(seed=570 + q_len, num_seqs=len(lens), num_q_heads=32, num_kv_heads=8,
                           head_dim=128, len_lo=0, len_hi=0, q_dtype="bf16", kv_dtype="bf16",
                           seq_lens=lens, q_len=q_len, name="mq balanced")
    B, qn, Hq, dd = wl.q.shape
    items = [(b, h) for b in range(B) if lens[b] > 0 for h in range(8)]
    ref, _ = oracle.prefill_chunk(wl.q.reshape(B * qn, Hq, dd), np.arange(0, B * qn + 1, qn),
                                  wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, wl.scale,
                                  "bf16", "bf16", items=items)
    ref = ref.reshape(B, qn, Hq, dd)
    ref[-1] = 0.0
    d = Dev(wl)
    out = pa.decode_multi_query(d.q, d.k, d.v, d.bt, d.sl, max_seq_len=wl.max_seq_len,
                                scale=wl.scale, partition_size=BAL)
    torch.cuda.synchronize()
    compare(f64(out), ref, "bf16", f"multi-query balanced q_len={q_len}")


@pytest.mark.parametrize("P", [BAL, 1024, 0])
def test_stages_equal_one_call(P):
    """Attention stage, then merge stage (pa_decode_stages) = one pa_decode,
    bit for bit, for the balanced, fixed-partition and one-pass modes."""
    import paged_kv_cache_22_amd as pa
    wl = W.config2()
    d = Dev(wl)
    ws = torch.empty(max(pa.decode_workspace_size(wl.num_seqs, wl.num_q_heads, wl.head_dim,
                                                  wl.max_seq_len, P), 256),
                     dtype=torch.uint8, device="cuda")
    whole = run_decode(d, partition_size=P, workspace=ws).clone()
    out = torch.full_like(whole, float("nan"))
    kw = dict(max_seq_len=wl.max_seq_len, out=out, workspace=ws, partition_size=P, scale=wl.scale)
    pa.decode_stages(d.q, d.k, d.v, d.bt, d.sl, stages=pa.PA_STAGE_ATTENTION, **kw)
    pa.decode_stages(d.q, d.k, d.v, d.bt, d.sl, stages=pa.PA_STAGE_MERGE, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), whole.view(torch.int16))
