"""The entry points inside a captured HIP graph (torch.cuda.CUDAGraph).

A serving step's decode runs under captured graphs (vllm-metis 0.1.0, "How
the model maps onto vLLM": CUDA graphs) and its kernels join the step with no
host synchronisation (vllm-metal architecture article, section 三).  The
library's calls enqueue kernels only -- no allocation, no memset, no host
read of device data -- so they can be captured.  Here one step is captured
once: the cache write of each sequence's newest token, decode in the
balanced mode, at 512-token partitions and at 128-token partitions (up to
24 per sequence: the streamed kernel), a causal prefill chunk, and a mixed
step (decode rows and chunks in one call).  Its
inputs (q, the new K/V rows and their slots, the sequence lengths) are then
rewritten in place and the graph replayed several times, with eager work
and synchronisations between the replays; every replay must equal, bit for
bit, the same calls made eagerly on the same inputs, and the oracle within
the graded tolerance.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import compare, dev, f64, oracle_decode

pytestmark = pytest.mark.gpu
BAL = -1
MODES = (BAL, 512, 128)


def test_step_captured_in_a_graph_replays_like_eager_calls():
    import paged_kv_cache_22_amd as pa
    B, Hq, Hkv, D = 16, 32, 8, 128
    wl = W.decode_workload(seed=410, num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                           len_lo=600, len_hi=3000, q_dtype="bf16", kv_dtype="bf16", pad=0)
    pw = W.prefill_workload(seed=411, q_lens=[100, 37], ctx_lens=[300, 61], num_q_heads=Hq,
                            num_kv_heads=Hkv, head_dim=D, q_dtype="bf16", kv_dtype="bf16", pad=0)
    max_len = int(wl.seq_lens.max())
    base_lens = wl.seq_lens.copy()
    # static device buffers the graph reads and writes
    k, v = dev(wl.k_cache, "bf16"), dev(wl.v_cache, "bf16")
    bt = dev(wl.block_table)
    q = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    new_k = torch.empty((B, Hkv, D), dtype=torch.bfloat16, device="cuda")
    new_v = torch.empty_like(new_k)
    slots = torch.empty(B, dtype=torch.int32, device="cuda")
    lens = torch.empty(B, dtype=torch.int32, device="cuda")
    pq, pcu = dev(pw.q, "bf16"), dev(pw.cu_q_lens)
    pk, pv, pbt, psl = dev(pw.k_cache, "bf16"), dev(pw.v_cache, "bf16"), dev(pw.block_table), \
        dev(pw.seq_lens)
    ws = {P: torch.empty(max(pa.decode_workspace_size(B, Hq, D, max_len, P), 256),
                         dtype=torch.uint8, device="cuda") for P in MODES}
    outs = {P: torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda") for P in MODES}
    pout = torch.empty_like(pq)
    # a mixed step over the decode cache: the decode rows (balanced) and the
    # chunks, their tables naming blocks of the decode pool
    mbt = dev(np.random.default_rng(413).integers(0, wl.num_blocks, size=pw.block_table.shape)
              .astype(np.int32))
    mws = torch.empty_like(ws[BAL])
    m_dec, m_pre = torch.empty_like(outs[BAL]), torch.empty_like(pq)

    def step():
        pa.write_kv(new_k, new_v, k, v, slots)
        for P in MODES:
            pa.decode(q, k, v, bt, lens, max_seq_len=max_len, scale=wl.scale, partition_size=P,
                      out=outs[P], workspace=ws[P])
        pa.prefill_chunk(pq, pcu, pk, pv, pbt, psl, max_q_len=int(pw.max_q_len), scale=pw.scale,
                         out=pout)
        pa.mixed_step(q, bt, lens, pq, pcu, mbt, psl, k, v, max_seq_len=max_len,
                      max_q_len=int(pw.max_q_len), partition_size=BAL, scale=wl.scale,
                      dec_out=m_dec, pre_out=m_pre, workspace=mws)

    rng = np.random.default_rng(412)

    def new_inputs():
        """Fresh q and new rows; each sequence keeps 1 .. its full length
        tokens, the newest written at its slot by the step itself."""
        L = rng.integers(1, base_lens + 1).astype(np.int32)
        s = np.array([wl.block_table[b, (L[b] - 1) // 16] * 16 + (L[b] - 1) % 16
                      for b in range(B)], np.int32)
        q.copy_(dev(W.to_bf16_bits(rng.standard_normal((B, Hq, D)).astype(np.float32)), "bf16"))
        new_k.copy_(dev(W.to_bf16_bits(rng.standard_normal((B, Hkv, D)).astype(np.float32)), "bf16"))
        new_v.copy_(dev(W.to_bf16_bits(rng.standard_normal((B, Hkv, D)).astype(np.float32)), "bf16"))
        slots.copy_(torch.from_numpy(s))
        lens.copy_(torch.from_numpy(L))
        torch.cuda.synchronize()
        return L

    # eager warm-up: the balanced and streamed kernels' one-time occupancy
    # queries run here, outside the capture
    new_inputs()
    step()
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(4):
        L = new_inputs()
        print(f"[graph] replay {rep}: lens {L.min()}..{L.max()}", flush=True)
        k0, v0 = k.clone(), v.clone()
        g.replay()
        torch.cuda.synchronize()
        got = {P: outs[P].clone() for P in outs}
        got_p = pout.clone()
        got_m = (m_dec.clone(), m_pre.clone())
        k_after, v_after = k.clone(), v.clone()
        # the same calls eagerly, on the same inputs and the same starting cache
        k.copy_(k0)
        v.copy_(v0)
        torch.cuda.synchronize()
        step()
        torch.cuda.synchronize()
        for P in outs:
            assert torch.equal(got[P].view(torch.int16), outs[P].view(torch.int16)), (rep, P)
        assert torch.equal(got_p.view(torch.int16), pout.view(torch.int16)), rep
        assert torch.equal(got_m[0].view(torch.int16), m_dec.view(torch.int16)), rep
        assert torch.equal(got_m[1].view(torch.int16), m_pre.view(torch.int16)), rep
        # the mixed step's decode rows are pa_decode's, bit for bit
        assert torch.equal(got_m[0].view(torch.int16), got[BAL].view(torch.int16)), rep
        assert torch.equal(k_after.view(torch.int16), k.view(torch.int16)), rep
        assert torch.equal(v_after.view(torch.int16), v.view(torch.int16)), rep
        # and the oracle, on the cache as the step left it
        ref_wl = W.DecodeWorkload(name="graph step", q=W.to_bf16_bits(f64(q).astype(np.float32)),
                                  k_cache=k.view(torch.int16).cpu().numpy().view(np.uint16),
                                  v_cache=v.view(torch.int16).cpu().numpy().view(np.uint16),
                                  block_table=wl.block_table, seq_lens=L, q_dtype="bf16",
                                  kv_dtype="bf16", scale=wl.scale)
        ref = oracle_decode(ref_wl)[0]
        for P in outs:
            compare(f64(got[P]), ref, "bf16", f"graph replay {rep} P={P}")
