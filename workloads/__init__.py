"""Seeded synthetic inputs for paged attention over a block-table KV cache.

This module only draws and lays out inputs; it holds none of the attention
arithmetic.  Both the HIP path (through the Python binding) and the CPU
oracle consume exactly the arrays built here, so quantisation of the inputs
never enters a parity error.

Storage conventions (raw bits, so that each consumer widens them itself):

* ``"f32"``  -> ``numpy.float32``
* ``"bf16"`` -> ``numpy.uint16``  (bfloat16 bit patterns, round-to-nearest-even
  from an fp32 draw, done by torch's CPU cast)
* ``"fp8"``  -> ``numpy.uint8``   (OCP e4m3fn codes; one fp32 scale per kv-head)

Cache layout: a block of ``block_size`` tokens (16, 32 or 64) is
``n = block_size / 16`` consecutive 16-token sub-blocks, each holding one
contiguous tile per kv-head:

* ``k_cache[num_blocks, n, num_kv_heads, head_dim/X, 16, X]`` with X the dims
  in 16 bytes (4 fp32, 8 bf16, 16 fp8): 16-byte chunks of consecutive dims,
  the token index inside each chunk
* ``v_cache[num_blocks, n, num_kv_heads, head_dim, 16]``  dim-major

For 16-token blocks (n = 1) the arrays are stored without the ``n`` axis:
``k_cache[num_blocks, num_kv_heads, head_dim/X, 16, X]``,
``v_cache[num_blocks, num_kv_heads, head_dim, 16]`` (the same bytes).

The pages name block tables and sequence lengths as the metadata of the paged
cache and say the platform fixes the cache layout (vllm-metal architecture
article, sections 二 and 四) but never give one; the layout above is this
library's choice and is used identically by every consumer.

Draw order per workload: ``numpy.random.default_rng(seed)`` draws the
sequence lengths, then the pool permutation, then q; the K and V pools are
drawn in fp32 N(0, 1) in chunks of 1024 blocks, chunk k of K from
``default_rng([seed, 1, k])`` and of V from ``default_rng([seed, 2, k])``.  Sequence ``b`` takes the
next ``ceil(L_b / block_size)`` entries of the permutation as its block-table
row; unused table entries are padding (``-1`` by default).
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

BLOCK_SIZE = 16
FP8_MAX = 448.0  # OCP e4m3fn largest finite value; scale rule amax / 448
_CHUNK_BLOCKS = 1024
_THREADS = min(16, os.cpu_count() or 1)

__all__ = [
    "DecodeWorkload", "PrefillWorkload", "MixedWorkload",
    "config1", "config2", "config3", "config4", "config5", "build_config",
    "decode_workload", "prefill_workload", "to_bf16_bits", "to_fp8_codes",
    "WriteWorkload", "write_workload", "write_chunks", "write_decode_step",
    "SharedPrefixWorkload", "shared_prefix_workload",
    "kv_bytes_per_token", "CONFIG_NAMES", "cache_shapes", "block_size_of", "to_cache_layout",
]

CONFIG_NAMES = {
    1: "tiny fp32 decode: 4 seqs, 8/2 heads, d=64, lens 1-200",
    2: "Llama-3-8B-shaped layer decode bf16: 64 seqs, 32/8 heads, d=128, lens 512-4096",
    3: "long-context split-KV decode bf16: 8 seqs, 32/8 heads, d=128, lens 32768-131072, partitions of 512",
    4: "mixed chunked-prefill + prefix sharing bf16: 16 decode seqs (1024-8192) + 4 chunks of 512 over a 2048-token shared prefix",
    5: "fp8-e4m3 KV decode: 256 seqs, 32/8 heads, d=128, lens 256-2048, per-kv-head scales",
}


# ---------------------------------------------------------------------------
# dtype helpers (input preparation only)
# ---------------------------------------------------------------------------
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> bfloat16 bit patterns (RNE), via torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_fp8_codes(x: np.ndarray, scale: np.ndarray, axis_scale: int) -> np.ndarray:
    """Quantise fp32 ``x`` to e4m3fn codes with ``x / scale`` (true division).

    ``scale`` is broadcast along ``axis_scale`` of ``x``.  Values are clamped to
    +-448 before the cast (torch's cast does not saturate).
    """
    import torch
    shape = [1] * x.ndim
    shape[axis_scale] = -1
    s = np.asarray(scale, dtype=np.float32).reshape(shape)
    y = torch.from_numpy(np.ascontiguousarray(x / s, dtype=np.float32))
    y = y.clamp_(-FP8_MAX, FP8_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def cache_shapes(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int,
                 kv_dtype: str):
    """Shapes of k_cache and v_cache (see the module docstring)."""
    x = chunk_dims(kv_dtype)
    n = block_size // 16
    if block_size not in (16, 32, 64):
        raise ValueError("block_size must be 16, 32 or 64")
    if n == 1:
        return ((num_blocks, num_kv_heads, head_dim // x, 16, x),
                (num_blocks, num_kv_heads, head_dim, 16))
    return ((num_blocks, n, num_kv_heads, head_dim // x, 16, x),
            (num_blocks, n, num_kv_heads, head_dim, 16))


def block_size_of(v_cache) -> int:
    """Tokens per block of a v_cache array in this layout."""
    return 16 if v_cache.ndim == 4 else 16 * int(v_cache.shape[1])


def to_cache_layout(k, v, block_size: int):
    """Pools drawn as [NB, Hkv, d/X, block_size, X] / [NB, Hkv, d, block_size]
    (the token index running over the whole block) -> the sub-block layout."""
    if block_size == 16:
        return k, v
    nb, hkv, nck, bs, x = k.shape
    d = v.shape[2]
    n = bs // 16
    k = np.ascontiguousarray(k.reshape(nb, hkv, nck, n, 16, x).transpose(0, 3, 1, 2, 4, 5))
    v = np.ascontiguousarray(v.reshape(nb, hkv, d, n, 16).transpose(0, 3, 1, 2, 4))
    return k, v


def chunk_dims(kv_dtype: str) -> int:
    """Dims per 16-byte chunk of the K tile layout."""
    return {"f32": 4, "bf16": 8, "fp8": 16}[kv_dtype]


def kv_bytes_per_token(num_kv_heads: int, head_dim: int, kv_bytes: float,
                       num_layers: int = 1) -> float:
    """K plus V bytes one token occupies: 2 * layers * kv-heads * d * bytes.

    vllm-metis 0.1.0 ("How the model maps onto vLLM") prices its 6 KV layers
    of 10 heads of 64 in BF16 at 15 KiB per token, which this formula gives.
    """
    return 2.0 * num_layers * num_kv_heads * head_dim * kv_bytes


# ---------------------------------------------------------------------------
# containers
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class DecodeWorkload:
    """Decode queries over a paged KV cache: one per sequence, or (q_len > 1)
    the newest q_len cached tokens of each sequence."""
    name: str
    q: np.ndarray                 # [B, Hq, d], or [B, q_len, Hq, d]; f32 / bf16 bits
    k_cache: np.ndarray           # [NB, Hkv, d/X, bs, X]
    v_cache: np.ndarray           # [NB, Hkv, d, bs]
    block_table: np.ndarray       # int32 [B, max_blocks_per_seq]
    seq_lens: np.ndarray          # int32 [B]
    q_dtype: str                  # "f32" | "bf16"
    kv_dtype: str                 # "f32" | "bf16" | "fp8"
    scale: float                  # softmax scale, 1/sqrt(d)
    k_scale: Optional[np.ndarray] = None   # f32 [Hkv] (fp8 only)
    v_scale: Optional[np.ndarray] = None
    partition_size: int = 0       # 0 = one pass per sequence

    @property
    def num_seqs(self) -> int: return int(self.q.shape[0])
    @property
    def q_len(self) -> int: return int(self.q.shape[1]) if self.q.ndim == 4 else 1
    @property
    def num_q_heads(self) -> int: return int(self.q.shape[-2])
    @property
    def head_dim(self) -> int: return int(self.q.shape[-1])
    @property
    def num_kv_heads(self) -> int: return int(self.k_cache.shape[1 if self.k_cache.ndim == 5 else 2])
    @property
    def block_size(self) -> int: return block_size_of(self.v_cache)
    @property
    def num_blocks(self) -> int: return int(self.k_cache.shape[0])
    @property
    def max_blocks_per_seq(self) -> int: return int(self.block_table.shape[1])
    @property
    def max_seq_len(self) -> int: return int(self.seq_lens.max()) if self.seq_lens.size else 0
    @property
    def total_tokens(self) -> int: return int(self.seq_lens.astype(np.int64).sum())

    def kv_elem_bytes(self) -> int:
        return {"f32": 4, "bf16": 2, "fp8": 1}[self.kv_dtype]

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes: live tokens only, all kv-heads."""
        return int(self.total_tokens * kv_bytes_per_token(
            self.num_kv_heads, self.head_dim, self.kv_elem_bytes()))


@dataclasses.dataclass
class PrefillWorkload:
    """Causal prefill chunks over a paged context (bottom-right aligned)."""
    name: str
    q: np.ndarray                 # [total_q, Hq, d]
    cu_q_lens: np.ndarray         # int32 [num_chunks + 1]
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_table: np.ndarray       # int32 [num_chunks, max_blocks_per_seq]
    seq_lens: np.ndarray          # int32 [num_chunks] = context + chunk length
    q_dtype: str
    kv_dtype: str
    scale: float
    k_scale: Optional[np.ndarray] = None
    v_scale: Optional[np.ndarray] = None

    @property
    def num_chunks(self) -> int: return int(self.seq_lens.shape[0])
    @property
    def total_q(self) -> int: return int(self.q.shape[0])
    @property
    def num_q_heads(self) -> int: return int(self.q.shape[1])
    @property
    def head_dim(self) -> int: return int(self.q.shape[2])
    @property
    def num_kv_heads(self) -> int: return int(self.k_cache.shape[1 if self.k_cache.ndim == 5 else 2])
    @property
    def block_size(self) -> int: return block_size_of(self.v_cache)
    @property
    def num_blocks(self) -> int: return int(self.k_cache.shape[0])
    @property
    def max_blocks_per_seq(self) -> int: return int(self.block_table.shape[1])
    @property
    def q_lens(self) -> np.ndarray: return np.diff(self.cu_q_lens).astype(np.int64)
    @property
    def max_q_len(self) -> int: return int(self.q_lens.max()) if self.num_chunks else 0

    def pairs(self) -> int:
        """Visible (query, key) pairs per head: sum over queries of ctx + i + 1."""
        total = 0
        for c in range(self.num_chunks):
            n = int(self.q_lens[c]); ctx = int(self.seq_lens[c]) - n
            total += n * ctx + n * (n + 1) // 2
        return total

    def flops(self) -> float:
        """QK^T and PV multiply-adds at 2 flops each, all q-heads."""
        return 4.0 * self.pairs() * self.num_q_heads * self.head_dim


@dataclasses.dataclass
class MixedWorkload:
    """Decode rows and prefill chunks sharing one physical pool."""
    name: str
    decode: DecodeWorkload
    prefill: PrefillWorkload


# ---------------------------------------------------------------------------
# drawing
# ---------------------------------------------------------------------------
def _draw_pool(seed, stream, num_blocks, num_kv_heads, head_dim, block_size, dtype):
    """Draw one N(0,1) pool of num_blocks tiles; returns the storage array
    (f32 or bf16 bits) or, for fp8, the fp32 pool (quantised later).

    Chunk k of 4096 blocks comes from its own generator
    ``default_rng([seed, stream, k])``, so chunks are drawn in parallel
    threads and the result does not depend on the thread count."""
    tile = num_kv_heads * head_dim * block_size
    out = np.empty(num_blocks * tile, dtype=np.uint16 if dtype == "bf16" else np.float32)

    def one(k):
        b0 = k * _CHUNK_BLOCKS
        b1 = min(num_blocks, b0 + _CHUNK_BLOCKS)
        x = np.random.default_rng([seed, stream, k]).standard_normal((b1 - b0) * tile,
                                                                      dtype=np.float32)
        out[b0 * tile:b1 * tile] = to_bf16_bits(x) if dtype == "bf16" else x

    n_chunks = -(-num_blocks // _CHUNK_BLOCKS)
    with ThreadPoolExecutor(max_workers=min(_THREADS, max(1, n_chunks))) as ex:
        list(ex.map(one, range(n_chunks)))
    return out


def _quantise_pool_fp8(pool_f32, num_kv_heads):
    """Per-kv-head amax/448 scale, then e4m3fn codes.  pool: [NB, Hkv, ...].
    Works in block chunks on a thread pool (numpy and torch release the GIL)."""
    nb = pool_f32.shape[0]
    flat = pool_f32.reshape(nb, num_kv_heads, -1)
    chunks = [(b0, min(nb, b0 + _CHUNK_BLOCKS)) for b0 in range(0, nb, _CHUNK_BLOCKS)]
    with ThreadPoolExecutor(max_workers=_THREADS) as ex:
        parts = list(ex.map(lambda c: np.abs(flat[c[0]:c[1]]).max(axis=(0, 2)), chunks))
    amax = np.max(np.stack(parts), axis=0)
    scale = (amax.astype(np.float32) / np.float32(FP8_MAX)).astype(np.float32)
    codes = np.empty(pool_f32.shape, dtype=np.uint8)

    def one(c):
        codes[c[0]:c[1]] = to_fp8_codes(pool_f32[c[0]:c[1]], scale, axis_scale=1)

    with ThreadPoolExecutor(max_workers=_THREADS) as ex:
        list(ex.map(one, chunks))
    return codes, scale


def _tables_from_perm(perm, lens, block_size, max_blocks, pad):
    table = np.full((len(lens), max_blocks), pad, dtype=np.int32)
    pos = 0
    for b, L in enumerate(lens):
        n = -(-int(L) // block_size)
        table[b, :n] = perm[pos:pos + n]
        pos += n
    return table, pos


def _make_pools(seed, nb, hkv, d, bs, kv_dtype):
    k = _draw_pool(seed, 1, nb, hkv, d, bs, "f32" if kv_dtype == "fp8" else kv_dtype)
    v = _draw_pool(seed, 2, nb, hkv, d, bs, "f32" if kv_dtype == "fp8" else kv_dtype)
    x = chunk_dims(kv_dtype)
    k = k.reshape(nb, hkv, d // x, bs, x)
    v = v.reshape(nb, hkv, d, bs)
    ks = vs = None
    if kv_dtype == "fp8":
        k, ks = _quantise_pool_fp8(k, hkv)
        v, vs = _quantise_pool_fp8(v, hkv)
    k, v = to_cache_layout(k, v, bs)
    return k, v, ks, vs


def _draw_q(rng, shape, q_dtype):
    x = rng.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    return to_bf16_bits(x) if q_dtype == "bf16" else x


def decode_workload(*, seed: int, num_seqs: int, num_q_heads: int, num_kv_heads: int,
                    head_dim: int, len_lo: int, len_hi: int, q_dtype: str, kv_dtype: str,
                    block_size: int = BLOCK_SIZE, pool_blocks: Optional[int] = None,
                    partition_size: int = 0, pad: int = -1, seq_lens=None, q_len: int = 0,
                    name: str = "decode") -> DecodeWorkload:
    """Generic seeded decode workload (lengths uniform integers in [lo, hi]).
    ``q_len`` > 0 gives q the shape [B, q_len, Hq, d] (several queries per
    sequence); 0 keeps the plain [B, Hq, d]."""
    rng = np.random.default_rng(seed)
    if seq_lens is None:
        lens = rng.integers(len_lo, len_hi, size=num_seqs, endpoint=True).astype(np.int32)
    else:
        lens = np.asarray(seq_lens, dtype=np.int32)
    need = int(sum(-(-int(L) // block_size) for L in lens))
    nb = max(need, 1) if pool_blocks is None else int(pool_blocks)
    if nb < need:
        raise ValueError("pool too small for the drawn lengths")
    perm = rng.permutation(nb).astype(np.int32)
    max_blocks = max(1, -(-int(lens.max(initial=0)) // block_size))
    table, _ = _tables_from_perm(perm, lens, block_size, max_blocks, pad)
    qshape = (num_seqs, num_q_heads, head_dim) if q_len == 0 else \
        (num_seqs, q_len, num_q_heads, head_dim)
    q = _draw_q(rng, qshape, q_dtype)
    k, v, ks, vs = _make_pools(seed, nb, num_kv_heads, head_dim, block_size, kv_dtype)
    return DecodeWorkload(name=name, q=q, k_cache=k, v_cache=v, block_table=table,
                          seq_lens=lens, q_dtype=q_dtype, kv_dtype=kv_dtype,
                          scale=1.0 / math.sqrt(head_dim), k_scale=ks, v_scale=vs,
                          partition_size=partition_size)


def prefill_workload(*, seed: int, q_lens, ctx_lens, num_q_heads: int, num_kv_heads: int,
                     head_dim: int, q_dtype: str, kv_dtype: str, block_size: int = BLOCK_SIZE,
                     pad: int = -1, name: str = "prefill") -> PrefillWorkload:
    """Generic seeded prefill-chunk workload with private blocks per chunk."""
    rng = np.random.default_rng(seed)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    lens = (np.asarray(ctx_lens, dtype=np.int32) + q_lens).astype(np.int32)
    need = int(sum(-(-int(L) // block_size) for L in lens))
    nb = max(need, 1)
    perm = rng.permutation(nb).astype(np.int32)
    max_blocks = max(1, -(-int(lens.max(initial=0)) // block_size))
    table, _ = _tables_from_perm(perm, lens, block_size, max_blocks, pad)
    cu = np.zeros(len(q_lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    q = _draw_q(rng, (int(cu[-1]), num_q_heads, head_dim), q_dtype)
    k, v, ks, vs = _make_pools(seed, nb, num_kv_heads, head_dim, block_size, kv_dtype)
    return PrefillWorkload(name=name, q=q, cu_q_lens=cu, k_cache=k, v_cache=v,
                           block_table=table, seq_lens=lens, q_dtype=q_dtype,
                           kv_dtype=kv_dtype, scale=1.0 / math.sqrt(head_dim),
                           k_scale=ks, v_scale=vs)


# ---------------------------------------------------------------------------
# the five configurations
# ---------------------------------------------------------------------------
def config1(pad: int = -1) -> DecodeWorkload:
    """Tiny fp32: 4 seqs, 8/2 heads (GQA 4), d=64, lens U{1..200}, pool of 64."""
    return decode_workload(seed=1, num_seqs=4, num_q_heads=8, num_kv_heads=2, head_dim=64,
                           len_lo=1, len_hi=200, q_dtype="f32", kv_dtype="f32",
                           pool_blocks=64, pad=pad, name="C1")


def config2(pad: int = -1, partition_size: int = 512) -> DecodeWorkload:
    """Llama-3-8B layer decode, bf16: 64 seqs, 32/8 heads, d=128, lens U{512..4096}."""
    return decode_workload(seed=2, num_seqs=64, num_q_heads=32, num_kv_heads=8, head_dim=128,
                           len_lo=512, len_hi=4096, q_dtype="bf16", kv_dtype="bf16",
                           pad=pad, partition_size=partition_size, name="C2")


def config3(pad: int = -1) -> DecodeWorkload:
    """Long-context split-KV, bf16: 8 seqs, lens U{32768..131072}, partitions of 512."""
    return decode_workload(seed=3, num_seqs=8, num_q_heads=32, num_kv_heads=8, head_dim=128,
                           len_lo=32768, len_hi=131072, q_dtype="bf16", kv_dtype="bf16",
                           pad=pad, partition_size=512, name="C3")


def config4(pad: int = -1, partition_size: int = 512) -> MixedWorkload:
    """Mixed step: 16 decode seqs (U{1024..8192}) + 4 prefill chunks of 512 new tokens
    over a 2048-token prefix whose 128 blocks every chunk table references.

    Pool order: prefix blocks, then each chunk's 32 private blocks, then the
    decode sequences' blocks, all taken from one permutation.
    """
    bs, hq, hkv, d = BLOCK_SIZE, 32, 8, 128
    rng = np.random.default_rng(4)
    dec_lens = rng.integers(1024, 8192, size=16, endpoint=True).astype(np.int32)
    n_chunks, q_len, ctx = 4, 512, 2048
    prefix_blocks, private_blocks = ctx // bs, q_len // bs
    dec_blocks = int(sum(-(-int(L) // bs) for L in dec_lens))
    nb = prefix_blocks + n_chunks * private_blocks + dec_blocks
    perm = rng.permutation(nb).astype(np.int32)
    pos = 0
    prefix = perm[pos:pos + prefix_blocks]; pos += prefix_blocks
    ptab = np.full((n_chunks, prefix_blocks + private_blocks), pad, dtype=np.int32)
    for c in range(n_chunks):
        ptab[c, :prefix_blocks] = prefix
        ptab[c, prefix_blocks:] = perm[pos:pos + private_blocks]; pos += private_blocks
    dtab, _ = _tables_from_perm(perm[pos:], dec_lens, bs,
                                -(-int(dec_lens.max()) // bs), pad)
    q_dec = _draw_q(rng, (16, hq, d), "bf16")
    q_pre = _draw_q(rng, (n_chunks * q_len, hq, d), "bf16")
    k, v, _, _ = _make_pools(4, nb, hkv, d, bs, "bf16")
    scale = 1.0 / math.sqrt(d)
    dec = DecodeWorkload(name="C4-decode", q=q_dec, k_cache=k, v_cache=v, block_table=dtab,
                         seq_lens=dec_lens, q_dtype="bf16", kv_dtype="bf16", scale=scale,
                         partition_size=partition_size)
    cu = np.arange(n_chunks + 1, dtype=np.int32) * q_len
    pre = PrefillWorkload(name="C4-prefill", q=q_pre, cu_q_lens=cu, k_cache=k, v_cache=v,
                          block_table=ptab, seq_lens=np.full(n_chunks, ctx + q_len, np.int32),
                          q_dtype="bf16", kv_dtype="bf16", scale=scale)
    return MixedWorkload(name="C4", decode=dec, prefill=pre)


def config5(pad: int = -1, partition_size: int = 512) -> DecodeWorkload:
    """fp8-e4m3 KV decode: 256 seqs, lens U{256..2048}, per-kv-head amax/448 scales,
    q and output bf16."""
    return decode_workload(seed=5, num_seqs=256, num_q_heads=32, num_kv_heads=8, head_dim=128,
                           len_lo=256, len_hi=2048, q_dtype="bf16", kv_dtype="fp8",
                           pad=pad, partition_size=partition_size, name="C5")


def build_config(n: int, **kw):
    return {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}[n](**kw)


# ---------------------------------------------------------------------------
# cache writes: new tokens' K/V rows and the slots they go to
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class WriteWorkload:
    """K/V rows of new tokens, their slot mapping and the cache they are
    written into (its initial contents are random bytes, so that untouched
    slots can be told apart)."""
    name: str
    key: np.ndarray               # [T, Hkv, d] in in_dtype storage
    value: np.ndarray
    slot_mapping: np.ndarray      # int32 [T]; -1 = padding token
    k_cache: np.ndarray           # [NB, Hkv, d/X, bs, X] in kv_dtype storage
    v_cache: np.ndarray           # [NB, Hkv, d, bs]
    in_dtype: str
    kv_dtype: str
    k_scale: Optional[np.ndarray] = None
    v_scale: Optional[np.ndarray] = None

    @property
    def num_tokens(self) -> int: return int(self.key.shape[0])
    @property
    def num_kv_heads(self) -> int: return int(self.key.shape[1])
    @property
    def head_dim(self) -> int: return int(self.key.shape[2])
    @property
    def num_blocks(self) -> int: return int(self.k_cache.shape[0])
    @property
    def block_size(self) -> int: return block_size_of(self.v_cache)

    def bytes_moved(self) -> int:
        """Algorithmic HBM bytes of one write: every token's K and V rows and
        its slot number are read; every token with a slot inside the pool has
        its K and V rows written."""
        ein = 2 if self.in_dtype == "bf16" else 4
        ekv = {"f32": 4, "bf16": 2, "fp8": 1}[self.kv_dtype]
        row = self.num_kv_heads * self.head_dim
        live = int(((self.slot_mapping >= 0) &
                    (self.slot_mapping < self.num_blocks * self.block_size)).sum())
        return self.num_tokens * (2 * row * ein + 4) + live * 2 * row * ekv


_STORAGE = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}


def write_workload(*, seed: int, slot_mapping, num_kv_heads: int, head_dim: int,
                   in_dtype: str, kv_dtype: str, num_blocks: int, block_size: int = BLOCK_SIZE,
                   fill_cache: bool = True, name: str = "write") -> WriteWorkload:
    """Rows N(0,1) (cast to bf16 for bf16 input); an fp8 cache gets the
    per-kv-head amax/448 scale of the rows drawn here.  ``fill_cache`` draws
    random bytes for the initial cache, else zeros."""
    slots = np.asarray(slot_mapping, dtype=np.int32)
    T = len(slots)
    shape = (T, num_kv_heads, head_dim)
    # rows drawn in chunks of 1024 tokens, chunk k of K from default_rng([seed, 7, 1, k])
    # and of V from default_rng([seed, 7, 2, k]), on a thread pool
    k32 = np.empty(shape, np.float32)
    v32 = np.empty(shape, np.float32)
    row = num_kv_heads * head_dim

    def draw(job):
        which, k = job
        t0, t1 = k * 1024, min(T, (k + 1) * 1024)
        dst = k32 if which == 1 else v32
        r = np.random.default_rng([seed, 7, which, k])
        dst[t0:t1] = r.standard_normal((t1 - t0) * row, dtype=np.float32).reshape(t1 - t0, *shape[1:])

    jobs = [(w, k) for w in (1, 2) for k in range(-(-T // 1024))]
    with ThreadPoolExecutor(max_workers=_THREADS) as ex:
        list(ex.map(draw, jobs))
    if in_dtype == "bf16":
        key, value = to_bf16_bits(k32), to_bf16_bits(v32)
        kf = (key.astype(np.uint32) << 16).view(np.float32)
        vf = (value.astype(np.uint32) << 16).view(np.float32)
    else:
        key, value, kf, vf = k32, v32, k32, v32
    ks = vs = None
    if kv_dtype == "fp8":
        amax = lambda x: np.abs(x).max(axis=(0, 2)) if T else np.ones(num_kv_heads, np.float32)
        ks = (amax(kf).astype(np.float32) / np.float32(FP8_MAX)).astype(np.float32)
        vs = (amax(vf).astype(np.float32) / np.float32(FP8_MAX)).astype(np.float32)
    st = _STORAGE[kv_dtype]
    kshape, vshape = cache_shapes(num_blocks, num_kv_heads, head_dim, block_size, kv_dtype)
    nbytes = int(np.prod(kshape)) * np.dtype(st).itemsize
    if fill_cache:
        crng = np.random.default_rng([seed, 8])
        kc = crng.integers(0, 256, nbytes, dtype=np.uint8).view(st).reshape(kshape)
        vc = crng.integers(0, 256, nbytes, dtype=np.uint8).view(st).reshape(vshape)
    else:
        kc, vc = np.zeros(kshape, st), np.zeros(vshape, st)
    return WriteWorkload(name=name, key=key, value=value, slot_mapping=slots, k_cache=kc,
                         v_cache=vc, in_dtype=in_dtype, kv_dtype=kv_dtype, k_scale=ks,
                         v_scale=vs)


def write_chunks(*, seed: int, chunk_lens, ctx_lens, num_blocks: int,
                 block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Slot mapping of prefill chunks: chunk c appends chunk_lens[c] tokens
    after ctx_lens[c] tokens of context, its sequence's blocks taken from a
    random permutation of the pool (disjoint between chunks), so a chunk
    starts mid-block whenever its context is not a multiple of the block size."""
    rng = np.random.default_rng([seed, 9])
    perm = rng.permutation(num_blocks)
    slots, pos = [], 0
    for n, ctx in zip(chunk_lens, ctx_lens):
        nblk = -(-(int(ctx) + int(n)) // block_size)
        table = perm[pos:pos + nblk]
        pos += nblk
        if pos > num_blocks:
            raise ValueError("pool too small for the chunks")
        t = np.arange(int(ctx), int(ctx) + int(n))
        slots.append(table[t // block_size] * block_size + t % block_size)
    return np.concatenate(slots).astype(np.int32) if slots else np.zeros(0, np.int32)


def write_decode_step(*, seed: int, num_seqs: int, num_blocks: int,
                      block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Slot mapping of one decode step: one new token per sequence, each in
    its sequence's last block (distinct blocks), at a uniform offset."""
    rng = np.random.default_rng([seed, 10])
    blocks = rng.permutation(num_blocks)[:num_seqs]
    if len(blocks) < num_seqs:
        raise ValueError("pool too small for the sequences")
    offs = rng.integers(0, block_size, num_seqs)
    return (blocks * block_size + offs).astype(np.int32)


# ---------------------------------------------------------------------------
# decode batches whose sequences share a cached prefix
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class SharedPrefixWorkload:
    """Decode sequences that all start with the same prefix_len cached tokens
    (the same physical blocks), each followed by its own tokens.  ``full`` is
    the plain view (whole block tables, whole lengths); the prefix table and
    the suffix tables / lengths are the cascade's view of the same cache."""
    full: DecodeWorkload
    prefix_len: int
    prefix_table: np.ndarray      # int32 [1, prefix_len / block_size]
    suffix_table: np.ndarray      # int32 [B, max suffix blocks]
    suffix_lens: np.ndarray       # int32 [B]


def shared_prefix_workload(*, seed: int, num_seqs: int, num_q_heads: int, num_kv_heads: int,
                           head_dim: int, prefix_len: int, len_lo: int, len_hi: int,
                           q_dtype: str, kv_dtype: str, q_len: int = 0,
                           block_size: int = BLOCK_SIZE, suffix_lens=None,
                           name: str = "shared prefix") -> SharedPrefixWorkload:
    """Suffix lengths uniform integers in [len_lo, len_hi] (after the
    prefix_len-token prefix, a multiple of block_size).  Pool order: the
    prefix's blocks, then each sequence's own blocks, all from one
    permutation; K/V/q drawn as for decode_workload."""
    if prefix_len % block_size:
        raise ValueError("the prefix must be whole blocks")
    rng = np.random.default_rng(seed)
    if suffix_lens is None:
        suffix_lens = rng.integers(len_lo, len_hi, size=num_seqs, endpoint=True)
    sfx = np.asarray(suffix_lens, dtype=np.int32)
    npre = prefix_len // block_size
    nsfx = [-(-int(L) // block_size) for L in sfx]
    nb = max(npre + sum(nsfx), 1)
    perm = rng.permutation(nb).astype(np.int32)
    prefix_table = perm[:npre].reshape(1, npre) if npre else np.zeros((1, 1), np.int32)
    max_sfx = max(max(nsfx, default=0), 1)
    suffix_table = np.full((num_seqs, max_sfx), -1, dtype=np.int32)
    full_table = np.full((num_seqs, npre + max_sfx), -1, dtype=np.int32)
    pos = npre
    for b, n in enumerate(nsfx):
        suffix_table[b, :n] = perm[pos:pos + n]
        full_table[b, :npre] = perm[:npre]
        full_table[b, npre:npre + n] = perm[pos:pos + n]
        pos += n
    qshape = (num_seqs, num_q_heads, head_dim) if q_len == 0 else \
        (num_seqs, q_len, num_q_heads, head_dim)
    q = _draw_q(rng, qshape, q_dtype)
    k, v, ks, vs = _make_pools(seed, nb, num_kv_heads, head_dim, block_size, kv_dtype)
    full = DecodeWorkload(name=name, q=q, k_cache=k, v_cache=v, block_table=full_table,
                          seq_lens=(sfx + prefix_len).astype(np.int32), q_dtype=q_dtype,
                          kv_dtype=kv_dtype, scale=1.0 / math.sqrt(head_dim), k_scale=ks,
                          v_scale=vs)
    return SharedPrefixWorkload(full=full, prefix_len=prefix_len, prefix_table=prefix_table,
                                suffix_table=suffix_table, suffix_lens=sfx)
