"""Cache-write parity (pa_write_kv): both caches, byte for byte, equal the
oracle's writer on the same seeded inputs.  Integer-exact bar: the fp8 codes
(rounding, ties to even, saturation) and every slot the call must leave alone
are compared bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from workloads.device import dev

pytestmark = pytest.mark.gpu

_VIEW = {"f32": (torch.int32, np.uint32), "bf16": (torch.int16, np.uint16),
         "fp8": (torch.uint8, np.uint8)}


def raw(t, dtype):
    """Tensor -> numpy array of its bit patterns."""
    tv, nv = _VIEW[dtype]
    return t.view(tv).cpu().numpy().view(nv)


def as_bits(a, dtype):
    return np.ascontiguousarray(a).view(_VIEW[dtype][1])


def run(wl, key=None, value=None):
    import paged_kv_cache_22_amd as pa
    kc, vc = dev(wl.k_cache, wl.kv_dtype), dev(wl.v_cache, wl.kv_dtype)
    if key is None:
        key, value = dev(wl.key, wl.in_dtype), dev(wl.value, wl.in_dtype)
    print(f"[write] {wl.name}: T={wl.num_tokens} Hkv={wl.num_kv_heads} d={wl.head_dim} "
          f"{wl.in_dtype}->{wl.kv_dtype} NB={wl.num_blocks}", flush=True)
    pa.write_kv(key, value, kc, vc, dev(wl.slot_mapping), k_scale=dev(wl.k_scale),
                v_scale=dev(wl.v_scale))
    torch.cuda.synchronize()
    return raw(kc, wl.kv_dtype), raw(vc, wl.kv_dtype)


def expected(wl, tokens=None):
    """The oracle's write into a copy of the initial cache.  Slots outside
    the pool are skipped by the library (its documented behaviour), so they
    reach the oracle as padding; ``tokens`` restricts the write to a sample."""
    kc, vc = wl.k_cache.copy(), wl.v_cache.copy()
    slots = wl.slot_mapping.copy()
    slots[slots >= wl.num_blocks * wl.block_size] = -1
    if tokens is not None:
        keep = np.zeros(len(slots), bool)
        keep[tokens] = True
        slots[~keep] = -1
    oracle.write_kv(kc, vc, wl.key, wl.value, slots, wl.in_dtype, wl.kv_dtype,
                    wl.k_scale, wl.v_scale)
    return as_bits(kc, wl.kv_dtype), as_bits(vc, wl.kv_dtype)


def assert_same(got, want, what):
    bad = int((got != want).sum())
    print(f"[parity] {what}: {bad} of {got.size} elements differ", flush=True)
    assert bad == 0, f"{what}: {bad} elements differ"


def mixed_slots(seed, nb, chunk_lens, ctx_lens, decode_seqs):
    """Chunks (mid-block starts included), decode tokens in other blocks,
    padding tokens and one slot beyond the pool."""
    half = nb // 2
    chunk = W.write_chunks(seed=seed, chunk_lens=chunk_lens, ctx_lens=ctx_lens, num_blocks=half)
    dec = W.write_decode_step(seed=seed, num_seqs=decode_seqs, num_blocks=nb - half) + half * 16
    slots = np.concatenate([chunk, dec]).astype(np.int32)
    rng = np.random.default_rng(seed)
    slots[rng.choice(len(slots), size=3, replace=False)] = -1
    slots[rng.integers(len(slots))] = nb * 16 + 5           # outside the pool: skipped
    return slots


DTYPES = [("f32", "f32"), ("bf16", "bf16"), ("bf16", "fp8"), ("f32", "fp8")]


@pytest.mark.parametrize("in_dtype,kv_dtype", DTYPES)
@pytest.mark.parametrize("hkv,d", [(8, 128), (10, 64), (2, 64)])
def test_write_matches_oracle(in_dtype, kv_dtype, hkv, d):
    nb = 96
    slots = mixed_slots(11 + d + hkv, nb, [1, 15, 16, 17, 100, 63], [0, 5, 16, 31, 7, 1], 37)
    wl = W.write_workload(seed=3, slot_mapping=slots, num_kv_heads=hkv, head_dim=d,
                          in_dtype=in_dtype, kv_dtype=kv_dtype, num_blocks=nb,
                          name=f"mixed {in_dtype}->{kv_dtype}")
    kc, vc = run(wl)
    ek, ev = expected(wl)
    assert_same(kc, ek, f"{wl.name} K")
    assert_same(vc, ev, f"{wl.name} V")


@pytest.mark.parametrize("in_dtype,kv_dtype", DTYPES)
@pytest.mark.parametrize("hkv,d", [(8, 128), (10, 64)])
def test_whole_blocks_and_partial_groups(in_dtype, kv_dtype, hkv, d):
    """Token groups that fill whole blocks in order (chunks starting on a
    block boundary) next to groups that straddle blocks or end early, and a
    whole-looking group broken by one padding token."""
    nb = 80
    slots = W.write_chunks(seed=70 + d, chunk_lens=[64, 32, 40, 7, 48], ctx_lens=[0, 16, 3, 32, 0],
                           num_blocks=nb)
    slots[-20] = -1                       # inside the last chunk's second block
    wl = W.write_workload(seed=8, slot_mapping=slots, num_kv_heads=hkv, head_dim=d,
                          in_dtype=in_dtype, kv_dtype=kv_dtype, num_blocks=nb,
                          name=f"whole blocks {in_dtype}->{kv_dtype}")
    kc, vc = run(wl)
    ek, ev = expected(wl)
    assert_same(kc, ek, f"{wl.name} K")
    assert_same(vc, ev, f"{wl.name} V")


def ties_workload(in_dtype):
    """Scale 1: inputs are every e4m3 value, every midpoint between two
    neighbours (the ties), values past 448 and the negatives of all of them."""
    vals = oracle.fp8_e4m3.table()[:0x7F]
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([vals, mids, [450.0, 464.0, 480.0, 512.0, 9984.0, 2.0 ** 127]])
    x = np.concatenate([x, -x]).astype(np.float32)
    d, hkv = 128, 2
    T = -(-x.size // (d * hkv))
    flat = np.zeros(T * hkv * d, np.float32)
    flat[:x.size] = x
    key = flat.reshape(T, hkv, d)
    value = key[::-1].copy()
    if in_dtype == "bf16":
        bits = W.to_bf16_bits(key)
        assert (bits.astype(np.uint32) << 16).view(np.float32).reshape(-1)[:x.size].tolist() \
            == x.tolist()                                    # every tie is exact in bf16
        key, value = bits, W.to_bf16_bits(value)
    slots = np.arange(T, dtype=np.int32) * 3                 # scattered offsets
    nb = -(-(3 * T) // 16)
    wl = W.write_workload(seed=5, slot_mapping=slots, num_kv_heads=hkv, head_dim=d,
                          in_dtype=in_dtype, kv_dtype="fp8", num_blocks=nb, name="ties")
    wl.key, wl.value = key, value
    wl.k_scale = np.ones(hkv, np.float32)
    wl.v_scale = np.ones(hkv, np.float32)
    return wl


@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
def test_fp8_ties_and_saturation(in_dtype):
    wl = ties_workload(in_dtype)
    kc, vc = run(wl)
    ek, ev = expected(wl)
    assert_same(kc, ek, f"ties {in_dtype} K")
    assert_same(vc, ev, f"ties {in_dtype} V")


def _scale_sets():
    """Two sets of 8 per-head scales: powers of two and their fp32
    neighbours (significands of all ones and of 1 + ulp, where a quotient
    through the reciprocal is hardest to round), amax / 448 values, and
    scales far from 1, two of them outside [2^-60, 2^60]."""
    nx = np.nextafter
    f = np.float32
    a = [f(1.0), f(2.0 ** -7), nx(f(2.0 ** -7), f(0)), nx(f(8.0), f(100)), f(3.0 / 448), f(0.1),
         f(2.7 / 448), f(7.0)]
    b = [nx(f(1.0), f(0)), f(2.0 ** 20), f(2.0 ** -70), nx(f(2.0 ** -20), f(1)), f(1.0 / 3),
         f(5.5 / 448), f(123.456), f(2.0 ** 70)]   # 2^-70, 2^70: outside the fast quotient's range
    return np.array(a, np.float32), np.array(b, np.float32)


def _quant_workload(key, value, in_dtype, k_scale, v_scale, name):
    T, hkv, d = key.shape
    slots = np.arange(T, dtype=np.int32)
    nb = -(-T // 16)
    wl = W.write_workload(seed=9, slot_mapping=slots, num_kv_heads=hkv, head_dim=d,
                          in_dtype=in_dtype, kv_dtype="fp8", num_blocks=nb, name=name)
    wl.key, wl.value = key, value
    wl.k_scale, wl.v_scale = k_scale, v_scale
    return wl


def test_fp8_quantise_every_bf16_value():
    """Every bf16 bit pattern except the NaNs, quantised with each of 16
    scales (8 per head for K, 8 for V): the codes equal the oracle's
    (e4m3fn of the correctly rounded fp32 quotient), so the kernel's quotient
    matches the true division wherever it can move a code.  NaN inputs are
    outside the write's contract."""
    bits = np.arange(65536, dtype=np.uint32)
    nan = ((bits & 0x7F80) == 0x7F80) & ((bits & 0x7F) != 0)
    vals = bits[~nan].astype(np.uint16)
    d, hkv = 128, 8
    rows = -(-vals.size // d)
    flat = np.zeros(rows * d, np.uint16)
    flat[:vals.size] = vals
    flat = flat.reshape(rows, d)
    key = np.repeat(flat[:, None, :], hkv, axis=1)                       # every value in every head
    value = np.repeat(np.roll(flat, 37, axis=0)[:, None, :], hkv, axis=1)
    ks, vs = _scale_sets()
    wl = _quant_workload(np.ascontiguousarray(key), np.ascontiguousarray(value), "bf16", ks, vs,
                         "every bf16 value")
    kc, vc = run(wl)
    with np.errstate(over="ignore"):      # the largest values over small scales: inf, saturated to 448
        ek, ev = expected(wl)
    assert_same(kc, ek, "every bf16 value K")
    assert_same(vc, ev, "every bf16 value V")


def test_fp8_quantise_near_rounding_midpoints():
    """fp32 inputs whose quotient lands within 3 fp32 ulps of an e4m3
    rounding midpoint (every midpoint between neighbouring codes, the one
    between 0 and the smallest subnormal, and 464 past the largest code),
    both signs, for each head's scale: where the fp32 rounding of the
    quotient decides the code."""
    table = oracle.fp8_e4m3.table()[:0x7F].astype(np.float64)
    mids = np.concatenate([(table[:-1] + table[1:]) / 2, [464.0]])
    d, hkv = 128, 8
    ks, vs = _scale_sets()

    def rows_for(scales):
        per_head = []
        for sc in scales:
            x0 = (mids * np.float64(sc)).astype(np.float32)
            xs = [x0]
            up, dn = x0.copy(), x0.copy()
            for _ in range(3):
                up = np.nextafter(up, np.float32(np.inf))
                dn = np.nextafter(dn, np.float32(-np.inf))
                xs += [up, dn]
            v = np.concatenate(xs)
            v = np.concatenate([v, -v]).astype(np.float32)
            per_head.append(v)
        n = max(v.size for v in per_head)
        T = -(-n // d)
        out = np.zeros((T, hkv, d), np.float32)
        for h, v in enumerate(per_head):
            col = np.zeros(T * d, np.float32)
            col[:v.size] = v
            out[:, h, :] = col.reshape(T, d)
        return out

    key, value = rows_for(ks), rows_for(vs)
    T = max(key.shape[0], value.shape[0])
    key = np.concatenate([key, np.zeros((T - key.shape[0], hkv, d), np.float32)])
    value = np.concatenate([value, np.zeros((T - value.shape[0], hkv, d), np.float32)])
    wl = _quant_workload(key, value, "f32", ks, vs, "near midpoints")
    kc, vc = run(wl)
    ek, ev = expected(wl)
    assert_same(kc, ek, "near midpoints K")
    assert_same(vc, ev, "near midpoints V")


@pytest.mark.parametrize("in_dtype,kv_dtype", [("bf16", "bf16"), ("bf16", "fp8")])
def test_strided_views_of_fused_projection(in_dtype, kv_dtype):
    """key / value as column slices of a fused [T, (Hq + 2 Hkv) d] tensor."""
    nb, hkv, hq, d = 48, 8, 32, 128
    slots = mixed_slots(21, nb, [33, 70], [3, 0], 20)
    wl = W.write_workload(seed=4, slot_mapping=slots, num_kv_heads=hkv, head_dim=d,
                          in_dtype=in_dtype, kv_dtype=kv_dtype, num_blocks=nb, name="strided")
    T = wl.num_tokens
    qpart = torch.zeros((T, hq * d), dtype=torch.bfloat16, device="cuda")
    fused = torch.cat([qpart, dev(wl.key, in_dtype).reshape(T, -1),
                       dev(wl.value, in_dtype).reshape(T, -1)], dim=1)
    key = fused[:, hq * d:(hq + hkv) * d].view(T, hkv, d)
    value = fused[:, (hq + hkv) * d:].view(T, hkv, d)
    assert not key.is_contiguous() and key.stride(0) == (hq + 2 * hkv) * d
    kc, vc = run(wl, key, value)
    ek, ev = expected(wl)
    assert_same(kc, ek, "strided K")
    assert_same(vc, ev, "strided V")


def test_empty_write_leaves_cache():
    wl = W.write_workload(seed=6, slot_mapping=np.zeros(0, np.int32), num_kv_heads=8,
                          head_dim=128, in_dtype="bf16", kv_dtype="fp8", num_blocks=4,
                          name="empty")
    kc, vc = run(wl)
    assert_same(kc, wl.k_cache, "empty K")
    assert_same(vc, wl.v_cache, "empty V")


def test_all_padding_leaves_cache():
    wl = W.write_workload(seed=6, slot_mapping=np.full(130, -1, np.int32), num_kv_heads=8,
                          head_dim=128, in_dtype="bf16", kv_dtype="bf16", num_blocks=4,
                          name="padding")
    kc, vc = run(wl)
    assert_same(kc, wl.k_cache, "padding K")
    assert_same(vc, wl.v_cache, "padding V")


# ---------------------------------------------------------------------------
# the sizes the benchmark times
# ---------------------------------------------------------------------------
def test_mixed_step_chunk_write_full_size():
    """4 prefill chunks of 512 tokens appended after a 2048-token prefix,
    32/8 heads, d = 128, bf16 (the mixed chunked-prefill step)."""
    nb = 4 * (2048 + 512) // 16
    slots = W.write_chunks(seed=40, chunk_lens=[512] * 4, ctx_lens=[2048] * 4, num_blocks=nb)
    wl = W.write_workload(seed=40, slot_mapping=slots, num_kv_heads=8, head_dim=128,
                          in_dtype="bf16", kv_dtype="bf16", num_blocks=nb, name="chunks 4x512")
    kc, vc = run(wl)
    ek, ev = expected(wl)
    assert_same(kc, ek, "chunks K")
    assert_same(vc, ev, "chunks V")


def test_fp8_decode_step_full_size():
    """One decode step of 256 sequences into an fp8 cache (bf16 input)."""
    nb = 4096
    slots = W.write_decode_step(seed=50, num_seqs=256, num_blocks=nb)
    wl = W.write_workload(seed=50, slot_mapping=slots, num_kv_heads=8, head_dim=128,
                          in_dtype="bf16", kv_dtype="fp8", num_blocks=nb, name="decode 256 fp8")
    kc, vc = run(wl)
    ek, ev = expected(wl)
    assert_same(kc, ek, "decode step K")
    assert_same(vc, ev, "decode step V")


@pytest.mark.parametrize("in_dtype,kv_dtype,hkv,d,T", [
    ("bf16", "fp8", 8, 128, 32768),      # the context-fill workload the benchmark times
    ("bf16", "bf16", 8, 128, 32768),
    ("f32", "f32", 2, 64, 65536),
])
def test_large_fill_sampled(in_dtype, kv_dtype, hkv, d, T):
    """Large writes, where each lane handles several tokens: one long chunk
    from a block boundary, a second one starting mid-block and a few padding
    tokens.  The oracle writes a sample of 2048 tokens spread over the whole
    call (one in every T/2048), and those slots are compared byte for byte."""
    nb = -(-T // 16) + 8
    slots = W.write_chunks(seed=60 + d, chunk_lens=[T - 100, 100], ctx_lens=[0, 5], num_blocks=nb)
    slots[[7, T // 2, T - 3]] = -1
    wl = W.write_workload(seed=60, slot_mapping=slots, num_kv_heads=hkv, head_dim=d,
                          in_dtype=in_dtype, kv_dtype=kv_dtype, num_blocks=nb, fill_cache=False,
                          name=f"fill {T} {in_dtype}->{kv_dtype}")
    kc, vc = run(wl)
    step = T // 2048
    sample = np.arange(0, T, step) + np.random.default_rng(60).integers(0, step, 2048)
    sample = np.union1d(sample, [7, T - 100, T - 97, T - 1])      # padding, second chunk
    ek, ev = expected(wl, tokens=sample)
    live = sample[slots[sample] >= 0]
    blk, off = slots[live] // 16, slots[live] % 16
    assert_same(kc[blk, :, :, off, :], ek[blk, :, :, off, :], "fill K (sample)")
    assert_same(vc[blk, :, :, off], ev[blk, :, :, off], "fill V (sample)")
    # the padding tokens' slots were never written: zeros from the initial cache
    untouched = np.setdiff1d(np.arange(nb * 16), slots[slots >= 0])
    ub, uo = untouched // 16, untouched % 16
    assert not kc[ub, :, :, uo, :].any() and not vc[ub, :, :, uo].any()
