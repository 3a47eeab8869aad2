"""Pins of the oracle's e4m3fn encoder and KV-cache writer (CPU only).

* the encoder against torch's float8_e4m3fn cast (a library routine) on
  random values, every representable value, every midpoint between
  neighbours (the ties) and out-of-range magnitudes (after clamping, since
  torch's cast does not saturate);
* closed forms: saturation to 448, ties to the even code, round trip of
  every finite code;
* the writer: cache positions checked with the layout formula written out
  here, independently of the oracle's reader, and a write-then-attend round
  trip against dense attention on the original rows.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8_e4m3 as F
import workloads as W


def torch_e4m3(x):
    t = torch.from_numpy(np.clip(np.asarray(x, np.float32), -448, 448))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def finite_values():
    return F.table()[:0x7F]          # +0 .. 448, increasing


def test_encode_matches_torch_random_and_exact():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100000) * 64, rng.standard_normal(5000) * 1e-3,
                        finite_values(), -finite_values(), [0.0, -0.0, 1e-30, 500.0, -1e6]])
    x = x.astype(np.float32)
    assert (F.encode(x) == torch_e4m3(x)).all()


def test_encode_ties_go_to_even_code():
    v = finite_values()
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    assert (mids.astype(np.float64) == (v[:-1] + v[1:]) / 2).all()    # exact in fp32
    codes = F.encode(mids)
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)                           # the even neighbour
    assert (codes == want).all()
    assert (codes == torch_e4m3(mids)).all()
    assert (F.encode(-mids) == (want | 0x80)).all()


def test_encode_closed_forms():
    assert F.encode(np.float32(448.0)) == 0x7E
    assert F.encode(np.float32(1e9)) == 0x7E and F.encode(np.float32(-1e9)) == 0xFE
    assert F.encode(np.float32(2.0 ** -10)) == 0x00                     # half the least subnormal
    assert F.encode(np.float32(3 * 2.0 ** -10)) == 0x02                 # between 2^-9 (odd) and 2^-8
    assert F.encode(np.float32(1.0)) == 0x38
    codes = np.arange(0x7F, dtype=np.uint8)
    assert (F.encode(F.decode(codes).astype(np.float32)) == codes).all()
    assert (F.encode(-F.decode(codes[1:]).astype(np.float32)) == (codes[1:] | 0x80)).all()


def test_write_positions_by_layout_formula():
    """Each written row lands where the documented layout puts it:
    K element (t, h, dim) at k_cache[blk, h, dim // X, off, dim % X],
    V element at v_cache[blk, h, dim, off], with slot = blk * 16 + off."""
    rng = np.random.default_rng(2)
    T, Hkv, d, bs, NB, X = 7, 2, 32, 16, 5, 4
    key = rng.standard_normal((T, Hkv, d)).astype(np.float32)
    val = rng.standard_normal((T, Hkv, d)).astype(np.float32)
    slots = np.array([3, 17, -1, 79, 16, 40, 0], np.int32)
    kc = np.full((NB, Hkv, d // X, bs, X), np.nan, np.float32)
    vc = np.full((NB, Hkv, d, bs), np.nan, np.float32)
    oracle.write_kv(kc, vc, key, val, slots, "f32", "f32")
    for t, s in enumerate(slots):
        if s < 0:
            continue
        blk, off = divmod(int(s), bs)
        for h in range(Hkv):
            for dim in range(d):
                assert kc[blk, h, dim // X, off, dim % X] == key[t, h, dim]
                assert vc[blk, h, dim, off] == val[t, h, dim]
    written = {int(s) for s in slots if s >= 0}
    untouched = [s for s in range(NB * bs) if s not in written]
    for s in untouched:
        blk, off = divmod(s, bs)
        assert np.isnan(kc[blk, :, :, off, :]).all() and np.isnan(vc[blk, :, :, off]).all()


@pytest.mark.parametrize("bs", [32, 64])
def test_write_positions_by_layout_formula_sub_blocks(bs):
    """Blocks of 32 or 64 tokens are 16-token sub-blocks: K element (t, h,
    dim) of slot = blk * bs + off lands at k_cache[blk, off // 16, h,
    dim // X, off % 16, dim % X], the V element at v_cache[blk, off // 16, h,
    dim, off % 16]; every other position is left alone."""
    rng = np.random.default_rng(3)
    T, Hkv, d, NB, X = 9, 2, 32, 3, 4
    n = bs // 16
    key = rng.standard_normal((T, Hkv, d)).astype(np.float32)
    val = rng.standard_normal((T, Hkv, d)).astype(np.float32)
    slots = rng.permutation(NB * bs)[:T].astype(np.int32)
    slots[2] = -1
    kc = np.full((NB, n, Hkv, d // X, 16, X), np.nan, np.float32)
    vc = np.full((NB, n, Hkv, d, 16), np.nan, np.float32)
    oracle.write_kv(kc, vc, key, val, slots, "f32", "f32")
    for t, s in enumerate(slots):
        if s < 0:
            continue
        blk, off = divmod(int(s), bs)
        for h in range(Hkv):
            for dim in range(d):
                assert kc[blk, off // 16, h, dim // X, off % 16, dim % X] == key[t, h, dim]
                assert vc[blk, off // 16, h, dim, off % 16] == val[t, h, dim]
    written = {int(s) for s in slots if s >= 0}
    for s in range(NB * bs):
        if s not in written:
            blk, off = divmod(s, bs)
            assert np.isnan(kc[blk, off // 16, :, :, off % 16, :]).all()
            assert np.isnan(vc[blk, off // 16, :, :, off % 16]).all()


def test_write_fp8_codes_and_round_trip_attention():
    """fp8 write = encode(x / scale) per kv-head; attention over the written
    cache equals dense attention over the dequantised rows."""
    rng = np.random.default_rng(3)
    T, Hkv, Hq, d, bs = 40, 2, 8, 32, 16
    key = rng.standard_normal((T, Hkv, d)).astype(np.float32)
    val = rng.standard_normal((T, Hkv, d)).astype(np.float32)
    ks = (np.abs(key).max(axis=(0, 2)) / 448).astype(np.float32)
    vs = (np.abs(val).max(axis=(0, 2)) / 448).astype(np.float32)
    nb = 4
    perm = rng.permutation(nb * bs)[:T].astype(np.int32)          # scattered slots
    kc = np.zeros((nb, Hkv, d // 16, bs, 16), np.uint8)
    vc = np.zeros((nb, Hkv, d, bs), np.uint8)
    oracle.write_kv(kc, vc, key, val, perm, "f32", "fp8", ks, vs)
    for t in (0, 17, 39):
        blk, off = divmod(int(perm[t]), bs)
        for h in range(Hkv):
            want = F.encode(key[t, h] / ks[h])
            assert (kc[blk, h, :, off, :].reshape(-1) == want).all()
            assert (vc[blk, h, :, off] == F.encode(val[t, h] / vs[h])).all()
    # a block table that lists the slots' blocks in logical order: write one
    # sequence contiguously and read it back through decode
    kc2 = np.zeros_like(kc); vc2 = np.zeros_like(vc)
    table = np.array([[2, 0, 3]], np.int32)
    slots = np.array([table[0, t // bs] * bs + t % bs for t in range(T)], np.int32)
    oracle.write_kv(kc2, vc2, key, val, slots, "f32", "fp8", ks, vs)
    q = rng.standard_normal((1, Hq, d)).astype(np.float32)
    out, _ = oracle.decode(q, kc2, vc2, table, np.array([T], np.int32), 0.2, "f32", "fp8", ks, vs)
    Kd = F.decode(F.encode(key / ks[None, :, None])) * ks[None, :, None]
    Vd = F.decode(F.encode(val / vs[None, :, None])) * vs[None, :, None]
    G = Hq // Hkv
    for j in range(Hq):
        h = j // G
        s = 0.2 * (Kd[:, h] @ q[0, j].astype(np.float64))
        p = np.exp(s - s.max()); p /= p.sum()
        assert np.abs(out[0, j] - p @ Vd[:, h]).max() < 1e-12


def test_write_bf16_is_exact_copy():
    rng = np.random.default_rng(4)
    key = W.to_bf16_bits(rng.standard_normal((9, 2, 64)).astype(np.float32)).reshape(9, 2, 64)
    val = W.to_bf16_bits(rng.standard_normal((9, 2, 64)).astype(np.float32)).reshape(9, 2, 64)
    kc = np.zeros((2, 2, 8, 16, 8), np.uint16); vc = np.zeros((2, 2, 64, 16), np.uint16)
    slots = np.arange(9, dtype=np.int32) + 5
    oracle.write_kv(kc, vc, key, val, slots, "bf16", "bf16")
    K, V = oracle.gather_kv(kc, vc, np.array([0, 1]), 14, 1, "bf16")
    assert (K[5:14] == oracle.widen(key[:, 1], "bf16")).all()
    assert (V[5:14] == oracle.widen(val[:, 1], "bf16")).all()
