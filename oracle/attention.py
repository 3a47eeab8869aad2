"""Plain fp64 paged attention over a block-table KV cache (CPU oracle).

Test infrastructure only: imported by tests, the smoke check and the bench's
CPU-baseline leg, never by the product path.  It shares no code with the HIP
library and does not import it.

What the pages fix and what is read into them
---------------------------------------------
The pages name paged attention over block tables and sequence lengths held as
device tensors (vllm-metal architecture article, sections 三 and 四), prefix
caching and chunked prefill (vllm-metis 0.1.0, intro and "How the model maps
onto vLLM"), GQA 4:1 (vllm-metis 0.1.0, "Status") and FP8 with scale
amax / 448 (same section).  They print no formula, layout or merge rule, so
this oracle writes out the plain definition of each step:

* attention of one query row:  out = softmax(scale * q . K^T) V over the
  visible keys, scale = 1/sqrt(d) passed explicitly;
* GQA: q-head j reads kv-head j // G, G = Hq / Hkv (contiguous groups);
* decode: the query is the newest token, already in the cache, so it sees
  keys 0 .. L-1 (L counts that token);
* prefill chunk of n queries over a sequence of L tokens: context
  ctx = L - n, query i sits at position ctx + i and sees keys 0 .. ctx + i
  (causal, aligned to the bottom-right of the score matrix);
* split-KV: partition p of size P covers tokens [pP, min((p+1)P, L)); it
  yields its normalised output o_p and lse_p = ln sum exp(s); the merge is
  out = sum_p w_p o_p / sum_p w_p with w_p = exp(lse_p - max lse);
* FP8 KV: value = e4m3fn(code) * scale[kv_head], per K and per V.

Layouts (see ``k_block`` / ``v_block``, the only places that read them, and
``write_kv``): a block of bs tokens is n = bs / 16 consecutive 16-token
sub-blocks, k_cache[num_blocks, n, Hkv, d/X, 16, X] (X dims per chunk) and
v_cache[num_blocks, n, Hkv, d, 16]; with 16-token blocks the n axis is left
out, k_cache[num_blocks, Hkv, d/X, 16, X] and v_cache[num_blocks, Hkv, d, 16].
Storage dtypes: "f32" float32, "bf16" uint16 bit patterns, "fp8" uint8 codes.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Tuple

import numpy as np

from . import fp8_e4m3

NEG_INF = -math.inf


# ---------------------------------------------------------------------------
# widening of stored values to float64 (exact for every storage type)
# ---------------------------------------------------------------------------
def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> float64.  bf16 bits are the top half of an fp32."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "fp8":
        return fp8_e4m3.decode(x)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# the block-table walk
# ---------------------------------------------------------------------------
def block_size(v_cache) -> int:
    """Tokens per cache block: 16 times the sub-blocks per block."""
    return 16 if v_cache.ndim == 4 else 16 * v_cache.shape[1]


def kv_heads(k_cache) -> int:
    """kv-heads of a K cache (the axis after the block, or after the sub-block)."""
    return k_cache.shape[1] if k_cache.ndim == 5 else k_cache.shape[2]


def k_block(k_cache, phys: int, h: int, n: int) -> np.ndarray:
    """Keys of slots 0..n-1 of (physical block, kv-head), as rows [n, d].

    Slot t is slot t mod 16 of sub-block t // 16.  A sub-block's K tile is
    stored as [d / X][16][X]: chunks of X consecutive dims, the slot index
    inside a chunk (X is the array's last extent)."""
    ns = -(-n // 16)
    tiles = k_cache[phys:phys + 1, h] if k_cache.ndim == 5 else k_cache[phys, :ns, h]
    rows = tiles.transpose(0, 2, 1, 3)                 # [sub-block, slot, d/X, X]
    return rows.reshape(-1, rows.shape[2] * rows.shape[3])[:n]


def v_block(v_cache, phys: int, h: int, n: int) -> np.ndarray:
    """Values of slots 0..n-1 of (physical block, kv-head), as rows [n, d]:
    each sub-block's V tile is stored dim-major [d][16]."""
    ns = -(-n // 16)
    tiles = v_cache[phys:phys + 1, h] if v_cache.ndim == 4 else v_cache[phys, :ns, h]
    rows = tiles.transpose(0, 2, 1)                    # [sub-block, slot, d]
    return rows.reshape(-1, rows.shape[2])[:n]


def gather_kv(k_cache, v_cache, table_row, seq_len: int, h: int, kv_dtype: str,
              k_scale=None, v_scale=None) -> Tuple[np.ndarray, np.ndarray]:
    """Walk one sequence's block table, one logical block at a time, for kv-head h.

    Logical token t lives in physical block table_row[t // bs] at slot t % bs.
    Entries at or past ceil(L / bs) are never read, nor are slots past L in
    the last block.  Returns float64 K [L, d] and V [L, d] (fp8 values
    multiplied by the head's scale).
    """
    bs = block_size(v_cache)
    d = v_cache.shape[-2]
    K = np.empty((seq_len, d), dtype=np.float64)
    V = np.empty((seq_len, d), dtype=np.float64)
    for j in range(-(-seq_len // bs)):
        phys = int(table_row[j])
        n = min(bs, seq_len - j * bs)
        K[j * bs:j * bs + n] = widen(k_block(k_cache, phys, h, n), kv_dtype)
        V[j * bs:j * bs + n] = widen(v_block(v_cache, phys, h, n), kv_dtype)
    if kv_dtype == "fp8":
        K *= float(k_scale[h])
        V *= float(v_scale[h])
    return K, V


# ---------------------------------------------------------------------------
# attention of query rows against gathered keys
# ---------------------------------------------------------------------------
def attend(qrow: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> Tuple[np.ndarray, float]:
    """softmax(scale * K q) V for one query row; returns (out[d], lse).

    With no visible key the output is zeros and lse = -inf.
    """
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64), NEG_INF
    s = scale * (K @ qrow)
    m = s.max()
    e = np.exp(s - m)
    den = e.sum()
    return (e @ V) / den, float(m + math.log(den))


def _heads(Hq: int, Hkv: int) -> int:
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return Hq // Hkv


def decode_rows(q, k_cache, v_cache, block_table, seq_lens, scale: float, q_dtype: str,
                kv_dtype: str, b: int, h: int, k_scale=None, v_scale=None):
    """Decode attention of one (sequence b, kv-head h) pair: the G query heads
    h*G .. h*G+G-1 of sequence b against its keys 0 .. L-1.  Returns
    (out[G, d], lse[G]) in float64."""
    Hq = q.shape[1]
    G = _heads(Hq, kv_heads(k_cache))
    qf = widen(q[b, h * G:(h + 1) * G], q_dtype)
    K, V = gather_kv(k_cache, v_cache, block_table[b], int(seq_lens[b]), h, kv_dtype,
                     k_scale, v_scale)
    out = np.empty((G, q.shape[2]))
    lse = np.empty(G)
    for g in range(G):
        out[g], lse[g] = attend(qf[g], K, V, scale)
    return out, lse


def decode(q, k_cache, v_cache, block_table, seq_lens, scale: float, q_dtype: str,
           kv_dtype: str, k_scale=None, v_scale=None,
           items: Optional[Iterable[Tuple[int, int]]] = None):
    """Decode attention; returns (out[B, Hq, d], lse[B, Hq]) in float64.

    ``items`` restricts the work to (sequence, kv-head) pairs; the other rows
    are left NaN so that a caller cannot mistake them for results.
    """
    B, Hq, d = q.shape
    Hkv = kv_heads(k_cache)
    G = _heads(Hq, Hkv)
    out = np.full((B, Hq, d), np.nan)
    lse = np.full((B, Hq), np.nan)
    todo = items if items is not None else [(b, h) for b in range(B) for h in range(Hkv)]
    for b, h in todo:
        out[b, h * G:(h + 1) * G], lse[b, h * G:(h + 1) * G] = decode_rows(
            q, k_cache, v_cache, block_table, seq_lens, scale, q_dtype, kv_dtype, b, h,
            k_scale, v_scale)
    return out, lse


def decode_partials(q, k_cache, v_cache, block_table, seq_lens, scale: float, q_dtype: str,
                    kv_dtype: str, partition_size: int, max_partitions: int,
                    k_scale=None, v_scale=None):
    """Per-partition (o_p, lse_p) of decode attention, float64.

    Returns o [B, Hq, Pmax, d] and lse [B, Hq, Pmax]; partitions that hold no
    token have o = 0 and lse = -inf.
    """
    B, Hq, d = q.shape
    Hkv = kv_heads(k_cache)
    G = _heads(Hq, Hkv)
    P = partition_size
    qf = widen(q, q_dtype)
    o = np.zeros((B, Hq, max_partitions, d))
    lse = np.full((B, Hq, max_partitions), NEG_INF)
    for b in range(B):
        L = int(seq_lens[b])
        for h in range(Hkv):
            K, V = gather_kv(k_cache, v_cache, block_table[b], L, h, kv_dtype, k_scale, v_scale)
            for p in range(-(-L // P)):
                lo, hi = p * P, min((p + 1) * P, L)
                for g in range(G):
                    j = h * G + g
                    o[b, j, p], lse[b, j, p] = attend(qf[b, j], K[lo:hi], V[lo:hi], scale)
    return o, lse


def merge(o_p: np.ndarray, lse_p: np.ndarray, seq_lens, partition_size: int):
    """Log-sum-exp merge of partition results; returns (out[B,Hq,d], lse[B,Hq]).

    Only partitions p < ceil(L / P) of a sequence take part; a sequence with
    no partition gets zeros and lse = -inf.
    """
    B, Hq, _, d = o_p.shape
    out = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), NEG_INF)
    for b in range(B):
        n = -(-int(seq_lens[b]) // partition_size)
        if n == 0:
            continue
        for j in range(Hq):
            ls = lse_p[b, j, :n]
            M = ls.max()
            if M == NEG_INF:
                continue
            w = np.exp(ls - M)
            out[b, j] = (w[:, None] * o_p[b, j, :n]).sum(axis=0) / w.sum()
            lse[b, j] = M + math.log(w.sum())
    return out, lse


def prefill_rows(q, cu_q_lens, k_cache, v_cache, block_table, seq_lens, scale: float,
                 q_dtype: str, kv_dtype: str, c: int, h: int, k_scale=None, v_scale=None):
    """Causal prefill of one (chunk c, kv-head h) pair: the chunk's n query
    rows, heads h*G .. h*G+G-1.  Query i sits at position ctx + i
    (ctx = seq_lens[c] - n) and sees keys 0 .. ctx + i.  Returns
    (out[n, G, d], lse[n, G]) in float64."""
    Hq, d = q.shape[1], q.shape[2]
    G = _heads(Hq, kv_heads(k_cache))
    q0, q1 = int(cu_q_lens[c]), int(cu_q_lens[c + 1])
    L = int(seq_lens[c])
    ctx = L - (q1 - q0)
    if ctx < 0:
        raise ValueError("seq_len smaller than the chunk")
    qf = widen(q[q0:q1, h * G:(h + 1) * G], q_dtype)
    K, V = gather_kv(k_cache, v_cache, block_table[c], L, h, kv_dtype, k_scale, v_scale)
    out = np.empty((q1 - q0, G, d))
    lse = np.empty((q1 - q0, G))
    for i in range(q1 - q0):
        visible = ctx + i + 1
        for g in range(G):
            out[i, g], lse[i, g] = attend(qf[i, g], K[:visible], V[:visible], scale)
    return out, lse


def prefill_chunk(q, cu_q_lens, k_cache, v_cache, block_table, seq_lens, scale: float,
                  q_dtype: str, kv_dtype: str, k_scale=None, v_scale=None,
                  items: Optional[Iterable[Tuple[int, int]]] = None):
    """Causal chunked prefill; returns (out[total_q, Hq, d], lse[total_q, Hq]).

    Chunk c holds queries cu[c] .. cu[c+1]-1 of a sequence of seq_lens[c]
    tokens whose K/V (context and the chunk itself) are in the cache.  Query i
    of the chunk sits at position ctx + i and attends to keys 0 .. ctx + i.
    ``items`` restricts the work to (chunk, kv-head) pairs (others stay NaN).
    """
    total_q, Hq, d = q.shape
    Hkv = kv_heads(k_cache)
    G = _heads(Hq, Hkv)
    out = np.full((total_q, Hq, d), np.nan)
    lse = np.full((total_q, Hq), np.nan)
    n_chunks = len(seq_lens)
    todo = items if items is not None else [(c, h) for c in range(n_chunks) for h in range(Hkv)]
    for c, h in todo:
        q0, q1 = int(cu_q_lens[c]), int(cu_q_lens[c + 1])
        out[q0:q1, h * G:(h + 1) * G], lse[q0:q1, h * G:(h + 1) * G] = prefill_rows(
            q, cu_q_lens, k_cache, v_cache, block_table, seq_lens, scale, q_dtype, kv_dtype,
            c, h, k_scale, v_scale)
    return out, lse


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 results to the output storage type and widen back (for
    comparing against values a kernel had to round): round to nearest even to
    fp32, then to bf16 (add half an ulp of the kept part, minus one unless the
    kept part is odd, and drop the low 16 bits).  Overflow gives an infinity
    of the right sign; a NaN stays a NaN."""
    with np.errstate(invalid="ignore", over="ignore"):
        f = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return f.astype(np.float64)
    if dtype == "bf16":
        bits = f.view(np.uint32).astype(np.uint64)
        lsb = (bits >> np.uint64(16)) & np.uint64(1)
        r = ((bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
        out = r.astype(np.uint32).view(np.float32).astype(np.float64)
        return np.where(np.isnan(f), np.nan, out)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# writing new tokens into the paged cache
# ---------------------------------------------------------------------------
def write_kv(k_cache, v_cache, key, value, slot_mapping, in_dtype: str, kv_dtype: str,
             k_scale=None, v_scale=None):
    """Store the K/V rows of new tokens into their cache slots (in place).

    Token t goes to slot s = slot_mapping[t] = physical block * bs + offset;
    s < 0 marks a padding token that is skipped.  bf16 / fp32 caches receive
    the values as they are (same storage type as the input).  An fp8 cache
    receives e4m3fn(x / scale[kv_head]): fp32 true division, then round to
    nearest even with saturation at 448 (the amax / 448 scale rule of
    vllm-metis 0.1.0, "Status", applied on write).
    """
    bs = block_size(v_cache)
    T, Hkv, d = key.shape
    kx = k_cache.shape[-1]
    for t in range(T):
        s = int(slot_mapping[t])
        if s < 0:
            continue
        phys, off = s // bs, s % bs
        sub, o = off // 16, off % 16
        for h in range(Hkv):
            kr, vr = key[t, h], value[t, h]
            if kv_dtype == "fp8":
                kq = fp8_e4m3.encode(widen(kr, in_dtype).astype(np.float32) / np.float32(k_scale[h]))
                vq = fp8_e4m3.encode(widen(vr, in_dtype).astype(np.float32) / np.float32(v_scale[h]))
            elif kv_dtype == in_dtype:
                kq, vq = kr, vr
            else:
                raise ValueError("a bf16 / fp32 cache takes inputs of its own type")
            kt = k_cache[phys, h] if k_cache.ndim == 5 else k_cache[phys, sub, h]
            vt = v_cache[phys, h] if v_cache.ndim == 4 else v_cache[phys, sub, h]
            kt[:, o, :] = np.asarray(kq).reshape(d // kx, kx)
            vt[:, o] = vq
    return k_cache, v_cache
