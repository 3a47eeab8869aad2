"""Pins of the CPU oracle against things other than itself (no GPU needed).

* the pages' printed figures (tests/golden/pages_facts.json);
* torch's float8_e4m3fn and bfloat16 casts (library routines);
* dense attention by torch's scaled_dot_product_attention in fp64 on
  contiguous K/V, with an explicit bottom-right causal mask;
* closed forms (uniform scores -> mean of V, one token -> V[0], a 2-token
  worked example, two-partition merges);
* invariants (physical permutation, split == unsplit, chunking);
* exact selection (one key wins by a logit gap that underflows the others).

The mutation tests at the end plant plausible mistakes into the oracle and
check that at least one pin then fails.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A
from oracle import fp8_e4m3
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")
with open(GOLD) as _f:
    FACTS = json.load(_f)


# ---------------------------------------------------------------------------
# helpers that build a paged cache from contiguous K/V (test-side scatter)
# ---------------------------------------------------------------------------
def scatter_to_pages(Ks, Vs, bs, rng, extra_blocks=3, fill=np.nan, x=None):
    """Ks[b]: [L_b, Hkv, d] float64.  Returns pools, table, lens with a random
    physical placement; unused slots hold ``fill``.  K chunks hold x dims
    (4 when d allows, else d).  The layout, written out here on its own: a
    block of bs tokens is bs / 16 sub-blocks of 16 slots; K element
    (block, sub-block, kv-head, chunk, slot, lane) is dim chunk * x + lane of
    the token at slot 16 * sub-block + slot, V element (block, sub-block,
    kv-head, dim, slot) likewise; 16-token blocks drop the sub-block axis."""
    B = len(Ks)
    Hkv, d = Ks[0].shape[1], Ks[0].shape[2]
    if x is None:
        x = 4 if d % 4 == 0 else d
    n = bs // 16
    lens = np.array([k.shape[0] for k in Ks], dtype=np.int32)
    nblk = [-(-int(L) // bs) for L in lens]
    nb = sum(nblk) + extra_blocks
    perm = rng.permutation(nb)
    kp = np.full((nb, n, Hkv, d // x, 16, x), fill)
    vp = np.full((nb, n, Hkv, d, 16), fill)
    table = np.full((B, max(max(nblk), 1)), -1, dtype=np.int32)
    pos = 0
    for b in range(B):
        for jb in range(nblk[b]):
            phys = perm[pos]; pos += 1
            table[b, jb] = phys
            for slot in range(bs):
                t = jb * bs + slot
                if t < lens[b]:
                    kp[phys, slot // 16, :, :, slot % 16, :] = Ks[b][t].reshape(Hkv, d // x, x)
                    vp[phys, slot // 16, :, :, slot % 16] = Vs[b][t]
    if n == 1:
        kp, vp = kp[:, 0], vp[:, 0]
    return kp, vp, table, lens


def kvh(kp):
    """kv-heads of a K pool built above."""
    return kp.shape[1] if kp.ndim == 5 else kp.shape[2]


def sdpa(q, K, V, scale, mask=None):
    """torch SDPA in float64. q [Hq, n, d], K/V [Hq, L, d], mask [n, L] bool."""
    qt, Kt, Vt = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, K, V))
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(
        qt, Kt, Vt, attn_mask=m, scale=scale).numpy()


def expand_gqa(X, G):
    """[Hkv, L, d] -> [Hkv*G, L, d]: kv-head h serves q-heads h*G .. h*G+G-1."""
    return np.repeat(X, G, axis=0)


def rand_decode_case(seed, B=3, Hq=8, Hkv=2, d=16, bs=16, lo=1, hi=70):
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi, size=B, endpoint=True)
    Ks = [rng.standard_normal((int(L), Hkv, d)) for L in lens]
    Vs = [rng.standard_normal((int(L), Hkv, d)) for L in lens]
    q = rng.standard_normal((B, Hq, d))
    kp, vp, table, lens = scatter_to_pages(Ks, Vs, bs, rng)
    return q, Ks, Vs, kp, vp, table, lens


def f32(x):
    """float64 test data rounded to fp32 storage (so the oracle's widening is exact)."""
    return np.asarray(x, dtype=np.float32)


# ---------------------------------------------------------------------------
# pages' figures
# ---------------------------------------------------------------------------
def test_pages_kv_bytes_per_token():
    f = FACTS["kv_bytes_per_token"]
    got = W.kv_bytes_per_token(f["kv_heads"], f["head_dim"], f["dtype_bytes"],
                               num_layers=f["kv_layers"])
    assert got == f["bytes_per_token"] == 15 * 1024


def test_pages_fp8_max_is_table_max():
    t = fp8_e4m3.table()
    assert np.nanmax(t) == FACTS["fp8_scale_divisor"]["value"] == 448.0
    assert np.nanmin(t) == -448.0


# ---------------------------------------------------------------------------
# P10: e4m3fn table and widening against torch's casts
# ---------------------------------------------------------------------------
def test_fp8_table_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = fp8_e4m3.table()
    nan_ref, nan_ours = np.isnan(ref), np.isnan(ours)
    assert (nan_ref == nan_ours).all()
    assert nan_ours.sum() == 2 and nan_ours[0x7F] and nan_ours[0xFF]
    assert (ref[~nan_ref] == ours[~nan_ours]).all()
    pos = ours[(ours > 0) & ~nan_ours]
    assert pos.min() == 2.0 ** -9          # smallest subnormal
    assert ours[0x08] == 2.0 ** -6         # smallest normal


def test_bf16_widen_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 16, size=20000, dtype=np.uint32).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]        # drop inf/NaN patterns
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert (A.widen(bits, "bf16") == ref).all()


def test_quantiser_maps_amax_to_448():
    wl = W.decode_workload(seed=11, num_seqs=3, num_q_heads=8, num_kv_heads=2, head_dim=32,
                           len_lo=20, len_hi=60, q_dtype="bf16", kv_dtype="fp8")
    for cache, sc in ((wl.k_cache, wl.k_scale), (wl.v_cache, wl.v_scale)):
        for h in range(wl.num_kv_heads):
            vals = np.abs(fp8_e4m3.decode(cache[:, h]))
            assert vals.max() == 448.0
            assert np.isfinite(vals).all()
        assert sc.dtype == np.float32 and (sc > 0).all()


# ---------------------------------------------------------------------------
# P1: dense library routine (decode and prefill, GQA)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed,bs", [(0, 16), (1, 16), (2, 16), (3, 32), (4, 64)])
def test_decode_matches_dense_sdpa(seed, bs):
    q, Ks, Vs, kp, vp, table, lens = rand_decode_case(seed, bs=bs)
    B, Hq, d = q.shape
    Hkv = kvh(kp)
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    out, lse = oracle.decode(f32(q), f32(kp), f32(vp), table, lens, scale, "f32", "f32")
    for b in range(B):
        K = expand_gqa(f32(Ks[b]).astype(np.float64).transpose(1, 0, 2), G)
        V = expand_gqa(f32(Vs[b]).astype(np.float64).transpose(1, 0, 2), G)
        qb = f32(q[b]).astype(np.float64)[:, None, :]
        ref = sdpa(qb, K, V, scale)[:, 0, :]
        assert np.abs(out[b] - ref).max() < 1e-12
        s = scale * np.einsum("hd,hld->hl", qb[:, 0], K)
        ref_lse = np.log(np.exp(s - s.max(1, keepdims=True)).sum(1)) + s.max(1)
        assert np.abs(lse[b] - ref_lse).max() < 1e-12


def _prefill_case(seed, q_lens, ctx_lens, Hq=8, Hkv=2, d=16, bs=16):
    rng = np.random.default_rng(seed)
    Ls = [c + n for c, n in zip(ctx_lens, q_lens)]
    Ks = [rng.standard_normal((L, Hkv, d)) for L in Ls]
    Vs = [rng.standard_normal((L, Hkv, d)) for L in Ls]
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    q = rng.standard_normal((int(cu[-1]), Hq, d))
    kp, vp, table, lens = scatter_to_pages(Ks, Vs, bs, rng)
    return q, cu, Ks, Vs, kp, vp, table, lens


def bottom_right_mask(n, L):
    """mask[i, k] = key k visible to query i of a chunk of n over L tokens."""
    ctx = L - n
    return np.arange(L)[None, :] <= (ctx + np.arange(n))[:, None]


@pytest.mark.parametrize("seed,bs", [(0, 16), (1, 16), (2, 32), (3, 64)])
def test_prefill_matches_dense_sdpa_bottom_right(seed, bs):
    q_lens, ctx_lens = [5, 17, 40], [0, 33, 9]
    q, cu, Ks, Vs, kp, vp, table, lens = _prefill_case(seed, q_lens, ctx_lens, bs=bs)
    Hq, d = q.shape[1], q.shape[2]
    G = Hq // kvh(kp)
    scale = 1.0 / math.sqrt(d)
    out, _ = oracle.prefill_chunk(f32(q), cu, f32(kp), f32(vp), table, lens, scale, "f32", "f32")
    for c in range(len(q_lens)):
        q0, q1 = cu[c], cu[c + 1]
        K = expand_gqa(f32(Ks[c]).astype(np.float64).transpose(1, 0, 2), G)
        V = expand_gqa(f32(Vs[c]).astype(np.float64).transpose(1, 0, 2), G)
        qc = f32(q[q0:q1]).astype(np.float64).transpose(1, 0, 2)
        ref = sdpa(qc, K, V, scale, bottom_right_mask(q1 - q0, int(lens[c])))
        assert np.abs(out[q0:q1] - ref.transpose(1, 0, 2)).max() < 1e-12


def test_prefill_without_context_is_plain_causal():
    """ctx = 0: bottom-right and top-left alignment coincide, so torch's own
    is_causal path is a second, mask-free pin."""
    q, cu, Ks, Vs, kp, vp, table, lens = _prefill_case(3, [23], [0])
    G = q.shape[1] // kvh(kp)
    scale = 0.3
    out, _ = oracle.prefill_chunk(f32(q), cu, f32(kp), f32(vp), table, lens, scale, "f32", "f32")
    K = expand_gqa(f32(Ks[0]).astype(np.float64).transpose(1, 0, 2), G)
    V = expand_gqa(f32(Vs[0]).astype(np.float64).transpose(1, 0, 2), G)
    qc = torch.from_numpy(f32(q).astype(np.float64).transpose(1, 0, 2).copy())
    ref = torch.nn.functional.scaled_dot_product_attention(
        qc, torch.from_numpy(K), torch.from_numpy(V), is_causal=True, scale=scale).numpy()
    assert np.abs(out - ref.transpose(1, 0, 2)).max() < 1e-12


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------
def test_worked_example_two_tokens():
    """q = (1, 0), keys (1, 0) and (0, 0), values e1 and e2, scale 1:
    scores (1, 0) -> weights e/(1+e), 1/(1+e); lse = ln(1 + e)."""
    kp = np.zeros((1, 1, 1, 16, 2), np.float32); vp = np.zeros((1, 1, 2, 16), np.float32)
    kp[0, 0, 0, 0] = [1, 0]; kp[0, 0, 0, 1] = [0, 0]
    vp[0, 0, :, 0] = [1, 0]; vp[0, 0, :, 1] = [0, 1]
    q = np.array([[[1.0, 0.0]]], np.float32)
    out, lse = oracle.decode(q, kp, vp, np.zeros((1, 1), np.int32), np.array([2], np.int32),
                             1.0, "f32", "f32")
    e = math.e
    assert abs(out[0, 0, 0] - e / (1 + e)) < 1e-15
    assert abs(out[0, 0, 1] - 1 / (1 + e)) < 1e-15
    assert abs(lse[0, 0] - math.log(1 + e)) < 1e-15


@pytest.mark.parametrize("L", [1, 15, 16, 17, 200])
def test_uniform_scores_give_mean_of_v(L):
    rng = np.random.default_rng(L)
    Ks = [rng.standard_normal((L, 2, 8))]
    Vs = [rng.standard_normal((L, 2, 8))]
    kp, vp, table, lens = scatter_to_pages(Ks, Vs, 16, rng)
    q = np.zeros((1, 8, 8))
    out, lse = oracle.decode(f32(q), f32(kp), f32(vp), table, lens, 0.125, "f32", "f32")
    for j in range(8):
        mean = f32(Vs[0]).astype(np.float64)[:, j // 4].sum(0) / L
        assert np.abs(out[0, j] - mean).max() < 1e-13
        assert abs(lse[0, j] - math.log(L)) < 1e-13


def test_equal_keys_at_huge_logits_give_mean_of_v():
    """All keys equal and logits near 1e5: the softmax is still uniform."""
    L, d = 45, 8
    rng = np.random.default_rng(17)
    Ks = [np.ones((L, 2, d))]
    Vs = [rng.standard_normal((L, 2, d))]
    kp, vp, table, lens = scatter_to_pages(Ks, Vs, 16, rng)
    q = np.full((1, 8, d), 4096.0)
    out, lse = oracle.decode(f32(q), f32(kp), f32(vp), table, lens, 4.0, "f32", "f32")
    for j in range(8):
        mean = f32(Vs[0]).astype(np.float64)[:, j // 4].sum(0) / L
        assert np.abs(out[0, j] - mean).max() < 1e-13
        assert abs(lse[0, j] - (4.0 * 4096.0 * d + math.log(L))) < 1e-9


def test_one_token_returns_v0_exactly():
    rng = np.random.default_rng(5)
    Ks = [rng.standard_normal((1, 2, 8))]
    Vs = [rng.standard_normal((1, 2, 8))]
    kp, vp, table, lens = scatter_to_pages(Ks, Vs, 16, rng)
    q = rng.standard_normal((1, 8, 8))
    out, _ = oracle.decode(f32(q), f32(kp), f32(vp), table, lens, 0.3, "f32", "f32")
    for j in range(8):
        assert (out[0, j] == f32(Vs[0][0, j // 4]).astype(np.float64)).all()


def test_zero_length_sequence():
    kp = np.zeros((2, 1, 1, 16, 4), np.float32); vp = np.zeros((2, 1, 4, 16), np.float32)
    q = np.ones((1, 2, 4), np.float32)
    out, lse = oracle.decode(q, kp, vp, np.full((1, 1), -1, np.int32), np.array([0], np.int32),
                             0.5, "f32", "f32")
    assert (out == 0).all() and (lse == -np.inf).all()


def test_merge_closed_forms():
    o = np.zeros((1, 1, 3, 2)); lse = np.full((1, 1, 3), -np.inf)
    o[0, 0, 0] = [1.0, 0.0]; o[0, 0, 1] = [0.0, 1.0]
    lse[0, 0, :2] = [0.7, 0.7]
    out, l = oracle.merge(o, lse, [2], 1)          # two partitions of one token each
    assert np.allclose(out[0, 0], [0.5, 0.5], rtol=0, atol=1e-15)
    assert abs(l[0, 0] - (0.7 + math.log(2))) < 1e-15
    lse[0, 0, :2] = [math.log(3.0), 0.0]            # weights 3 : 1
    out, l = oracle.merge(o, lse, [2], 1)
    assert np.allclose(out[0, 0], [0.75, 0.25], rtol=0, atol=1e-15)
    assert abs(l[0, 0] - math.log(4.0)) < 1e-15
    lse[0, 0, 2] = 50.0                              # past ceil(L/P): ignored
    out2, _ = oracle.merge(o, lse, [2], 1)
    assert (out2 == out).all()


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------
def test_block_size_invariance():
    """The same token rows paged with 16-, 32- and 64-token blocks: the
    oracle's decode and prefill results are bit-identical."""
    rng = np.random.default_rng(9)
    Ls = [1, 16, 17, 63, 64, 65, 200]
    Ks = [rng.standard_normal((L, 2, 16)) for L in Ls]
    Vs = [rng.standard_normal((L, 2, 16)) for L in Ls]
    q = f32(rng.standard_normal((len(Ls), 8, 16)))
    cu = np.arange(len(Ls) + 1, dtype=np.int32)             # one query per sequence
    outs = []
    for bs in (16, 32, 64):
        kp, vp, table, lens = scatter_to_pages(Ks, Vs, bs, np.random.default_rng(bs))
        dec, _ = oracle.decode(q, f32(kp), f32(vp), table, lens, 0.25, "f32", "f32")
        pre, _ = oracle.prefill_chunk(q, cu, f32(kp), f32(vp), table, lens, 0.25, "f32", "f32")
        outs.append((dec, pre))
    for dec, pre in outs[1:]:
        assert (dec == outs[0][0]).all() and (pre == outs[0][1]).all()


def test_physical_permutation_invariance():
    wl = W.decode_workload(seed=21, num_seqs=4, num_q_heads=8, num_kv_heads=2, head_dim=32,
                           len_lo=1, len_hi=90, q_dtype="bf16", kv_dtype="bf16", pool_blocks=40)
    out, lse = oracle.decode(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens,
                             wl.scale, "bf16", "bf16")
    pi = np.random.default_rng(7).permutation(wl.num_blocks)
    k2 = np.empty_like(wl.k_cache); v2 = np.empty_like(wl.v_cache)
    k2[pi] = wl.k_cache; v2[pi] = wl.v_cache
    t2 = np.where(wl.block_table >= 0, pi[np.maximum(wl.block_table, 0)], -1).astype(np.int32)
    out2, lse2 = oracle.decode(wl.q, k2, v2, t2, wl.seq_lens, wl.scale, "bf16", "bf16")
    assert (out == out2).all() and (lse == lse2).all()


@pytest.mark.parametrize("P", [16, 32, 48, 512])
def test_split_equals_unsplit(P):
    wl = W.decode_workload(seed=31, num_seqs=3, num_q_heads=8, num_kv_heads=2, head_dim=32,
                           len_lo=1, len_hi=300, q_dtype="bf16", kv_dtype="bf16")
    args = (wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, wl.scale, "bf16", "bf16")
    out, lse = oracle.decode(*args)
    pmax = -(-wl.max_seq_len // P)
    o_p, l_p = oracle.decode_partials(*args, partition_size=P, max_partitions=pmax)
    m, ml = oracle.merge(o_p, l_p, wl.seq_lens, P)
    assert np.abs(m - out).max() < 1e-12
    assert np.abs(ml - lse).max() < 1e-12
    if P >= wl.max_seq_len:                     # one partition: the identity
        assert (m == out).all()


def test_chunking_equals_one_pass():
    """A sequence fed as chunks [0,a), [a,b), [b,L), each seeing the earlier
    tokens through its block table, equals one causal pass over all L."""
    L, a, b = 150, 64, 128        # 64-token chunks, as the parity runs on the pages used
    rng = np.random.default_rng(9)
    Ks = [rng.standard_normal((L, 2, 16))]; Vs = [rng.standard_normal((L, 2, 16))]
    kp, vp, table, _ = scatter_to_pages(Ks, Vs, 16, rng)
    q = f32(rng.standard_normal((L, 8, 16)))
    kp, vp = f32(kp), f32(vp)
    whole, _ = oracle.prefill_chunk(q, np.array([0, L], np.int32), kp, vp, table,
                                    np.array([L], np.int32), 0.25, "f32", "f32")
    parts = []
    for lo, hi in ((0, a), (a, b), (b, L)):
        o, _ = oracle.prefill_chunk(q[lo:hi], np.array([0, hi - lo], np.int32), kp, vp, table,
                                    np.array([hi], np.int32), 0.25, "f32", "f32")
        parts.append(o)
    assert np.abs(np.concatenate(parts) - whole).max() < 1e-12
    # the last query of the whole pass is a decode step over all L tokens
    dec, _ = oracle.decode(q[L - 1:L], kp, vp, table, np.array([L], np.int32), 0.25, "f32", "f32")
    assert np.abs(dec[0] - whole[L - 1]).max() < 1e-12


def test_verify_queries_equal_truncated_decodes():
    """Draft verification: the newest q_len cached tokens of a sequence of L
    tokens as queries.  Query i sits at position L - q_len + i, so it is an
    ordinary decode step over the first L - q_len + 1 + i tokens; the
    oracle's reference for it (one prefill chunk of q_len rows per
    sequence) must equal those decode steps exactly, for every query."""
    rng = np.random.default_rng(21)
    q_len, Hkv, G, d = 4, 2, 4, 16
    lens = [37, 64, 5, 4]
    Ks = [rng.standard_normal((L, Hkv, d)) for L in lens]
    Vs = [rng.standard_normal((L, Hkv, d)) for L in lens]
    kp, vp, table, sl = scatter_to_pages(Ks, Vs, 16, rng)
    kp, vp = f32(kp), f32(vp)
    B = len(lens)
    q = f32(rng.standard_normal((B * q_len, Hkv * G, d)))
    cu = np.arange(0, B * q_len + 1, q_len, dtype=np.int32)
    ref, _ = oracle.prefill_chunk(q, cu, kp, vp, table, sl, 0.3, "f32", "f32")
    for b, L in enumerate(lens):
        for i in range(q_len):
            row = b * q_len + i
            dec, _ = oracle.decode(q[row:row + 1], kp, vp, table[b:b + 1],
                                   np.array([L - q_len + 1 + i], np.int32), 0.3, "f32", "f32")
            assert np.abs(dec[0] - ref[row]).max() < 1e-12, (b, i)


def test_prefix_sharing_equals_private_copies():
    wl = W.config4()
    pre = wl.prefill
    # shrink: two chunks, one kv-head, to keep the CPU test fast
    items = [(0, 0), (1, 0)]
    args = (pre.q, pre.cu_q_lens, pre.k_cache, pre.v_cache)
    shared, _ = oracle.prefill_chunk(*args, pre.block_table, pre.seq_lens, pre.scale,
                                     "bf16", "bf16", items=items)
    # private copy of the prefix for chunk 1: new physical blocks, same contents
    nb = pre.num_blocks
    k2 = np.concatenate([pre.k_cache, pre.k_cache[pre.block_table[1, :128]]])
    v2 = np.concatenate([pre.v_cache, pre.v_cache[pre.block_table[1, :128]]])
    t2 = pre.block_table.copy()
    t2[1, :128] = nb + np.arange(128)
    private, _ = oracle.prefill_chunk(pre.q, pre.cu_q_lens, k2, v2, t2, pre.seq_lens, pre.scale,
                                      "bf16", "bf16", items=items)
    rows = slice(0, 1024)
    assert np.array_equal(shared[rows, :4], private[rows, :4])


# ---------------------------------------------------------------------------
# exact selection
# ---------------------------------------------------------------------------
def test_exact_selection_decode_and_causal_boundary():
    d, bs, L = 32, 16, 70
    rng = np.random.default_rng(13)
    tau = 37
    K = -np.ones((L, 1, d)); K[tau] = 1.0
    V = rng.integers(0, 16, size=(L, 1, d)).astype(np.float64)
    kp, vp, table, lens = scatter_to_pages([K], [V], bs, rng)
    scale = 1.0 / math.sqrt(d)
    q = 8.0 * np.ones((1, 4, d))
    out, _ = oracle.decode(f32(q), f32(kp), f32(vp), table, lens, scale, "f32", "f32")
    assert np.abs(out[0] - V[tau, 0]).max() < 1e-30     # others weigh e^-90 each
    # prefill over the same sequence: rows at or past tau see V[tau]; earlier
    # rows see only keys with equal scores, i.e. the mean of their V
    qp = 8.0 * np.ones((L, 4, d))
    o, _ = oracle.prefill_chunk(f32(qp), np.array([0, L], np.int32), f32(kp), f32(vp), table,
                                lens, scale, "f32", "f32")
    for i in range(L):
        want = V[tau, 0] if i >= tau else V[:i + 1, 0].mean(0)
        assert np.abs(o[i] - want).max() < 1e-12, i


# ---------------------------------------------------------------------------
# generator facts
# ---------------------------------------------------------------------------
def test_config_shapes_and_tables():
    c1 = W.config1()
    assert c1.q.shape == (4, 8, 64) and c1.k_cache.shape == (64, 2, 16, 16, 4)
    assert c1.v_cache.shape == (64, 2, 64, 16)
    assert (c1.seq_lens >= 1).all() and (c1.seq_lens <= 200).all()
    used = np.concatenate([c1.block_table[b, :-(-int(L) // 16)] for b, L in enumerate(c1.seq_lens)])
    assert len(set(used.tolist())) == len(used)          # no block used twice
    assert (c1.block_table[c1.block_table >= 0] < 64).all()
    c1b = W.config1()
    assert np.array_equal(c1.q, c1b.q) and np.array_equal(c1.k_cache, c1b.k_cache)


def test_config4_prefix_is_shared():
    wl = W.config4()
    t = wl.prefill.block_table
    assert (t[:, :128] == t[0, :128]).all()
    private = t[:, 128:].ravel()
    assert len(set(private.tolist())) == private.size
    assert not set(private.tolist()) & set(t[0, :128].tolist())
    assert wl.prefill.pairs() == 4 * (512 * 2048 + 512 * 513 // 2)
    assert wl.prefill.flops() == pytest.approx(77.3e9, rel=1e-3)


# ---------------------------------------------------------------------------
# mutation tests: planted mistakes must trip a pin
# ---------------------------------------------------------------------------
def _pins_pass():
    try:
        test_decode_matches_dense_sdpa(0, 16)
        test_decode_matches_dense_sdpa(4, 64)
        test_prefill_matches_dense_sdpa_bottom_right(0, 16)
        test_prefill_matches_dense_sdpa_bottom_right(3, 64)
        test_split_equals_unsplit(16)
        test_uniform_scores_give_mean_of_v(17)
        test_equal_keys_at_huge_logits_give_mean_of_v()
        test_worked_example_two_tokens()
        test_verify_queries_equal_truncated_decodes()
    except Exception:          # a wrong shape counts as a caught mistake too
        return False
    return True


def test_pins_pass_unmutated():
    assert _pins_pass()


def test_mutation_wrong_gqa_mapping(monkeypatch):
    def bad_decode(q, k_cache, v_cache, block_table, seq_lens, scale, q_dtype, kv_dtype,
                   k_scale=None, v_scale=None, items=None):
        B, Hq, d = q.shape
        Hkv = A.kv_heads(k_cache)
        qf = A.widen(q, q_dtype)
        out = np.zeros((B, Hq, d)); lse = np.zeros((B, Hq))
        for b in range(B):
            for j in range(Hq):
                K, V = A.gather_kv(k_cache, v_cache, block_table[b], int(seq_lens[b]),
                                   j % Hkv, kv_dtype)           # interleaved, not contiguous
                out[b, j], lse[b, j] = A.attend(qf[b, j], K, V, scale)
        return out, lse
    monkeypatch.setattr(oracle, "decode", bad_decode)
    assert not _pins_pass()


def test_mutation_transposed_v_layout(monkeypatch):
    monkeypatch.setattr(A, "v_block", lambda v, phys, h, n: v[phys, h, :n, :])
    assert not _pins_pass()


def test_mutation_causal_off_by_one(monkeypatch):
    orig = A.attend

    def prefill_bad(q, cu, kc, vc, bt, sl, scale, qd, kd, k_scale=None, v_scale=None, items=None):
        total_q, Hq, d = q.shape
        G = Hq // kc.shape[1]
        qf = A.widen(q, qd)
        out = np.zeros((total_q, Hq, d)); lse = np.zeros((total_q, Hq))
        for c in range(len(sl)):
            q0, q1 = int(cu[c]), int(cu[c + 1]); L = int(sl[c]); ctx = L - (q1 - q0)
            for h in range(kc.shape[1]):
                K, V = A.gather_kv(kc, vc, bt[c], L, h, kd)
                for i in range(q1 - q0):
                    vis = max(ctx + i, 1)                   # drops the diagonal key
                    for g in range(G):
                        out[q0 + i, h * G + g], lse[q0 + i, h * G + g] = orig(
                            qf[q0 + i, h * G + g], K[:vis], V[:vis], scale)
        return out, lse
    monkeypatch.setattr(oracle, "prefill_chunk", prefill_bad)
    assert not _pins_pass()


def test_mutation_merge_drops_last_partition(monkeypatch):
    orig = A.merge

    def merge_bad(o_p, lse_p, seq_lens, P):
        return orig(o_p, lse_p, [max(int(L) - P, 0) for L in seq_lens], P)
    monkeypatch.setattr(oracle, "merge", merge_bad)
    assert not _pins_pass()


def test_mutation_missing_max_subtraction(monkeypatch):
    def attend_bad(qrow, K, V, scale):
        if K.shape[0] == 0:
            return np.zeros(V.shape[1]), -math.inf
        e = np.exp(scale * (K @ qrow))                 # no max subtracted
        return (e @ V) / e.sum(), float(np.log(e.sum()))
    monkeypatch.setattr(A, "attend", attend_bad)
    with np.errstate(all="ignore"):
        assert not _pins_pass()


def test_mutation_scale_dropped(monkeypatch):
    orig = A.attend
    monkeypatch.setattr(A, "attend", lambda q, K, V, scale: orig(q, K, V, 1.0))
    assert not _pins_pass()


# ---------------------------------------------------------------------------
# round_to: fp64 results rounded to the output storage type
# ---------------------------------------------------------------------------
def _round_to_cases():
    """fp32 bit patterns: random ones, exact ties (both parities of the kept
    last bit), subnormals, the neighbourhood of the largest finite bf16, and
    the special values."""
    rng = np.random.default_rng(77)
    rand = rng.integers(0, 2 ** 32, 200_000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 2 ** 16, 4000, dtype=np.uint64).astype(np.uint32) << np.uint32(16)) \
        | np.uint32(0x8000)
    sub = rng.integers(1, 2 ** 23, 4000, dtype=np.uint64).astype(np.uint32)
    sub = np.concatenate([sub, sub | np.uint32(0x80000000)])
    top = np.uint32(0x7F7F0000) + np.arange(0, 0x10000, 7, dtype=np.uint32)
    top = np.concatenate([top, top | np.uint32(0x80000000), [np.uint32(0x7F7F8000)]])
    special = np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0x7F800001,
                        0x3F800000, 0x3F808000, 0x3F818000], dtype=np.uint32)
    return np.concatenate([rand, ties, sub, top, special]).astype(np.uint32).view(np.float32)


def test_round_to_bf16_matches_torch_cast():
    """oracle.round_to(x, "bf16") on fp32 values is round to nearest even to
    bf16: bit for bit what torch's CPU cast gives, signed zeros, overflow to
    infinity and NaN included."""
    x = _round_to_cases()
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).float().numpy().astype(np.float64)
    with np.errstate(invalid="ignore"):    # signalling NaN patterns among the inputs
        got = A.round_to(x.astype(np.float64), "bf16")
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint64), want[~nan].view(np.uint64))


def test_round_to_worked_ties():
    """bf16 keeps 7 fraction bits: 1 + 2^-8 lies halfway between 1 and
    1 + 2^-7 and goes to the even one, 1; 1 + 3 * 2^-8 lies halfway between
    1 + 2^-7 and 1 + 2^-6 and goes to 1 + 2^-6; just past a tie rounds up."""
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20, -(1 + 2.0 ** -8)])
    assert list(A.round_to(x, "bf16")) == [1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -1.0]


def test_round_to_fp64_rounds_through_fp32():
    """fp64 inputs are first rounded to fp32 (as the kernels hold them), then
    to bf16: equal to torch casting float64 -> float32 -> bfloat16."""
    rng = np.random.default_rng(78)
    x = rng.standard_normal(100_000) * np.exp2(rng.integers(-30, 30, 100_000))
    want = torch.from_numpy(x).to(torch.float32).to(torch.bfloat16).double().numpy()
    assert np.array_equal(A.round_to(x, "bf16"), want)
    assert np.array_equal(A.round_to(x, "f32"), x.astype(np.float32).astype(np.float64))


def test_mutation_round_to_truncates(monkeypatch):
    """A round_to that truncates instead of rounding fails the pin."""
    def trunc(x, dtype):
        f = np.asarray(x, dtype=np.float32)
        b = f.view(np.uint32) & np.uint32(0xFFFF0000)
        return b.view(np.float32).astype(np.float64)
    monkeypatch.setattr(A, "round_to", trunc)
    with pytest.raises(AssertionError):
        test_round_to_bf16_matches_torch_cast()


def test_mutation_verify_queries_see_the_whole_sequence(monkeypatch):
    """A chunk's queries all attending to every cached token (the causal
    limit inside the chunk forgotten) must fail a pin."""
    orig = A.attend

    def prefill_bad(q, cu, kc, vc, bt, sl, scale, qd, kd, k_scale=None, v_scale=None, items=None):
        total_q, Hq, d = q.shape
        G = Hq // kc.shape[1]
        qf = A.widen(q, qd)
        out = np.zeros((total_q, Hq, d)); lse = np.zeros((total_q, Hq))
        for c in range(len(sl)):
            q0, q1 = int(cu[c]), int(cu[c + 1]); L = int(sl[c])
            for h in range(kc.shape[1]):
                K, V = A.gather_kv(kc, vc, bt[c], L, h, kd)
                for i in range(q1 - q0):
                    for g in range(G):
                        out[q0 + i, h * G + g], lse[q0 + i, h * G + g] = orig(
                            qf[q0 + i, h * G + g], K, V, scale)
        return out, lse
    monkeypatch.setattr(oracle, "prefill_chunk", prefill_bad)
    assert not _pins_pass()
