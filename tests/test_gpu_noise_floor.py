"""Noise floor of the GPU results: their error against the fp64 oracle is of
the order the admitted roundings alone produce.

The pages fix no rounding; the kernels round the softmax weights to bf16 for
the output product and the output to bf16 (readings R10 and R22).  A
"rounding model" computes attention in fp64 with exactly those roundings:

* decode: o = sum_t bf16(p_t) V_t / sum_t p_t (the running sum takes the
  unrounded fp32 weights), output rounded to bf16;
* prefill: o = sum_t bf16(p_t) V_t / sum_t bf16(p_t) (the normaliser is the
  sum of the weights as they enter the product), output rounded to bf16.

Its error against the oracle is the floor the GPU error is measured
against.  The GPU's weights are not bitwise the model's (its running max lags
the true max, so each weight is the model's times a non-integer power of two
and rounds to bf16 independently), so the two errors are independent draws
of one distribution: their root-mean-square over all outputs must agree
(GPU within RMS_RATIO of the model), and the largest, where one flipped
rounding of a dominant weight can move an output by an ulp, within
MAX_RATIO.  An extra error source spread over the outputs (a dropped term, a
wrong rounding) raises the RMS far past the model's.  Diagnostic, in
addition to the graded parity tests; computed on the full C2 and C5 batches
and on sampled rows of the C4 prefill chunks.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import Dev, f64, run_decode, run_prefill

pytestmark = pytest.mark.gpu

RMS_RATIO = 1.5
MAX_RATIO = 3.0


def bf16_round(x):
    """fp64 -> fp32 (nearest) -> bf16 (nearest, ties to even), back to fp64:
    the path the kernels' values take."""
    x32 = np.asarray(x, dtype=np.float32)
    bits = x32.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32).astype(np.float64)


def _gather(wl, b, h):
    return oracle.gather_kv(wl.k_cache, wl.v_cache, wl.block_table[b], int(wl.seq_lens[b]), h,
                            wl.kv_dtype, wl.k_scale, wl.v_scale)


def decode_model(wl):
    """Decode under the rounding model, [B, Hq, d]."""
    B, Hq, d = wl.q.shape
    Hkv = wl.k_cache.shape[1]
    G = Hq // Hkv
    q = oracle.widen(wl.q, wl.q_dtype)
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(Hkv):
            K, V = _gather(wl, b, h)
            s = q[b, h * G:(h + 1) * G] @ K.T * wl.scale          # [G, L]
            p = np.exp(s - s.max(axis=1, keepdims=True))
            o = (bf16_round(p) @ V) / p.sum(axis=1, keepdims=True)
            out[b, h * G:(h + 1) * G] = bf16_round(o)
    return out


def prefill_rows(wl, rows):
    """The oracle (its per-row attention on the gathered keys) and the
    rounding model for the (token row, q-head) pairs in ``rows``."""
    cu = wl.cu_q_lens
    Hq = wl.q.shape[1]
    Hkv = wl.k_cache.shape[1]
    G = Hq // Hkv
    q = oracle.widen(wl.q, wl.q_dtype)
    ref, model, cache = {}, {}, {}
    for (t, j) in rows:
        c = int(np.searchsorted(cu, t, side="right") - 1)
        i = t - int(cu[c])
        n = int(cu[c + 1] - cu[c])
        vis = int(wl.seq_lens[c]) - n + i + 1          # keys 0 .. ctx + i
        h = j // G
        if (c, h) not in cache:
            cache[(c, h)] = _gather(wl, c, h)
        K, V = cache[(c, h)]
        ref[(t, j)] = oracle.attend(q[t, j], K[:vis], V[:vis], wl.scale)[0]
        s = K[:vis] @ q[t, j] * wl.scale
        pb = bf16_round(np.exp(s - s.max()))
        model[(t, j)] = bf16_round(pb @ V[:vis] / pb.sum())
    return ref, model


def _check(d_gpu, d_model, what):
    """d_*: arrays of (result - oracle) over the same outputs."""
    rg, rm = float(np.sqrt(np.mean(d_gpu ** 2))), float(np.sqrt(np.mean(d_model ** 2)))
    mg, mm = float(np.abs(d_gpu).max()), float(np.abs(d_model).max())
    print(f"[noise] {what}: rms err gpu {rg:.3e} / model {rm:.3e} (ratio {rg / max(rm, 1e-30):.2f}); "
          f"max err gpu {mg:.3e} / model {mm:.3e} (ratio {mg / max(mm, 1e-30):.2f})", flush=True)
    assert rm > 0.0 and mm > 0.0
    assert rg <= RMS_RATIO * rm, f"{what}: GPU rms error {rg} above {RMS_RATIO}x the rounding floor {rm}"
    assert mg <= MAX_RATIO * mm, f"{what}: GPU max error {mg} above {MAX_RATIO}x the rounding floor {mm}"


@pytest.mark.parametrize("cfg,P", [(2, -1), (5, 1024)])
def test_decode_error_at_rounding_floor(cfg, P):
    wl = W.config2() if cfg == 2 else W.config5()
    got = f64(run_decode(Dev(wl), partition_size=P))
    ref = oracle.decode(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, wl.scale,
                        wl.q_dtype, wl.kv_dtype, wl.k_scale, wl.v_scale)[0]
    model = decode_model(wl)
    _check(got - ref, model - ref, f"C{cfg} decode")


def test_prefill_error_at_rounding_floor():
    wl = W.config4().prefill
    got = f64(run_prefill(Dev(wl)))
    rng = np.random.default_rng(7)
    total, Hq = wl.q.shape[0], wl.q.shape[1]
    rows = sorted({(int(t), int(j)) for t, j in zip(rng.integers(0, total, 96), rng.integers(0, Hq, 96))})
    ref, model = prefill_rows(wl, rows)
    d_gpu = np.stack([got[t, j] - ref[(t, j)] for t, j in rows])
    d_model = np.stack([model[(t, j)] - ref[(t, j)] for t, j in rows])
    _check(d_gpu, d_model, "C4 prefill rows")
