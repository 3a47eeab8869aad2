#!/usr/bin/env python3
"""Paged-attention decode benchmark on one MI355X.

Headline: KV GB/s (and % of the 8 TB/s HBM peak) plus tokens-attended/s of
bf16 decode at the Llama-3-8B layer shape: 64 sequences, 32 q-heads / 8
kv-heads, head_dim 128, block_size 16, lengths uniform in [512, 4096] (seed
2), block tables a random permutation of one pool.  A step is one pass of
the decode path over that batch: pa_decode in its balanced split-KV mode
(the attention kernel over equal block ranges, one per resident workgroup,
then the log-sum-exp merge for sequences split over several ranges), inputs
resident in HBM.  Before
every timed step a 1 GiB buffer is read (a reduction into one scalar) so no
input survives in the L2 or the 256 MB Infinity Cache; a read leaves clean
lines behind, so no write-back of the flush lands inside the next timed
kernel.  Step times come from HIP events on the launch stream.

The other workloads (long-context split-KV, the mixed chunked-prefill step
timed as one step, fp8 KV, the cache writes that precede attention, and draft
verification with several queries per sequence) are timed the same way and
reported under "per_config".  The CPU-baseline leg times the fp64 oracle on
the host's cores (a process pool over its (sequence, kv-head) pairs) over the
whole headline batch, repeated for at least 10 s.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged-attn decode KV GB/s (% HBM peak) + tokens-attended/s, Llama-3-8B shape"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, AMD published
FLUSH_BYTES = 1 << 30
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_PROFILE = os.path.join(PROFILES, "decode_kernel_bf16_llama3_8b_c2_traffic.txt")
KERNEL_SOURCES = ["decode_kernels.h", "decode.hip", "tiles.h", "device.h"]


def kernel_source_hash():
    """sha256 over the sources of the decode kernel (so a stored counter
    reading is used only for the kernel it was taken on)."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_22_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(partition_size):
    """HBM bytes per launch of the decode kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None if that summary was
    taken on other kernel sources or another partition size."""
    try:
        kv = dict(line.split(":", 1) for line in open(TRAFFIC_PROFILE) if ":" in line)
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("source_sha256") != kernel_source_hash():
        return None
    if int(kv.get("partition_size", -1)) != partition_size:
        return None
    return int(kv["traffic_bytes_per_launch"])


def host_info():
    """CPU model and core count of the host, ROCm / HIP runtime / driver versions."""
    info = {"cpu_model": None, "host_cores": os.cpu_count()}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm_version"] = f.read().strip()
    except OSError:
        info["rocm_version"] = None
    try:
        with open("/sys/module/amdgpu/version") as f:
            info["amdgpu_driver_version"] = f.read().strip()
    except OSError:
        # an amdgpu built with the kernel carries no module version of its own
        info["amdgpu_driver_version"] = None
    info["linux_kernel"] = os.uname().release
    return info


def gpu_info(torch):
    """Device name, arch and HIP runtime / driver versions (after the GPU is initialised)."""
    import ctypes
    p = torch.cuda.get_device_properties(0)
    info = {"gpu": p.name, "arch": getattr(p, "gcnArchName", None), "torch_hip": torch.version.hip}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        if hip.hipDriverGetVersion(ctypes.byref(v)) == 0:
            info["hip_driver_version"] = v.value
        if hip.hipRuntimeGetVersion(ctypes.byref(v)) == 0:
            info["hip_runtime_version"] = v.value
    except OSError:
        pass
    return info


def cpu_baseline(wl, min_seconds=10.0):
    """The oracle as it stands, on the host's cores: its (sequence, kv-head)
    pairs spread over a process pool (one worker per core, at most 16, BLAS
    at one thread each); the whole batch repeated until at least
    min_seconds, the mean pass reported.  Started before any GPU use."""
    from oracle.pool import OraclePool
    with OraclePool() as pool:
        args = (wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, wl.scale,
                wl.q_dtype, wl.kv_dtype, wl.k_scale, wl.v_scale)
        # inputs written once where the workers map them, and the workers
        # started: neither is timed
        staged = pool.stage({"q": wl.q, "k_cache": wl.k_cache, "v_cache": wl.v_cache,
                             "block_table": wl.block_table, "seq_lens": wl.seq_lens})
        try:
            pool.decode(*args, items=[(0, 0)], staged=staged)
            passes = 0
            t0 = time.perf_counter()
            while True:
                pool.decode(*args, staged=staged)
                passes += 1
                total = time.perf_counter() - t0
                if total >= min_seconds:
                    break
        finally:
            pool.release(staged)
        workers = pool.workers
    dt = total / passes
    info = host_info()
    return {"value": round(wl.kv_bytes() / dt / 1e9, 4), "unit": "GB/s", "cores": workers,
            "kind": "oracle", "seconds_per_pass": round(dt, 3), "passes": passes,
            "seconds": round(total, 2),
            "tokens_attended_per_s": round(wl.total_tokens / dt, 1),
            "cpu_model": info["cpu_model"], "host_cores": info["host_cores"],
            "sample": f"the whole batch ({wl.num_seqs} sequences, {wl.total_tokens} tokens, "
                      f"all {wl.num_kv_heads} kv-heads), {passes} passes, fp64 numpy oracle "
                      f"over {workers} worker processes (one BLAS thread each), inputs "
                      f"memory-mapped from one staged copy"}


class CacheFlush:
    """Evicts the caches between timed steps by reading a 1 GiB buffer.
    Reading (not rewriting) leaves no dirty lines whose write-back would be
    charged to the next kernel."""

    def __init__(self, torch):
        self.torch = torch
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        self.out = torch.zeros((), dtype=torch.float32, device="cuda")

    def __call__(self):
        self.torch.sum(self.buf, dim=(0,), out=self.out)


def time_stream_read(torch, pa, flush, reps=20):
    """The measured HBM read rate (pa_stream_read over a 1 GiB buffer, both
    load forms), the context for the peak-relative figures: median of
    `reps` reads, each after a cache flush, timed with HIP events."""
    buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(pa.STREAM_READ_SINK_WORDS, dtype=torch.int32, device="cuda")
    res = {"bytes": FLUSH_BYTES}
    for name, nt in (("nontemporal", True), ("plain", False)):
        for _ in range(3):
            pa.stream_read(buf, nontemporal=nt, sink=sink)
        ms = []
        for _ in range(reps):
            flush()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            pa.stream_read(buf, nontemporal=nt, sink=sink)
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        med = sorted(ms)[len(ms) // 2]
        res[f"{name}_ms"] = round(med, 5)
        res[f"{name}_GBps"] = round(FLUSH_BYTES / med / 1e6, 1)
    best = max(res["nontemporal_GBps"], res["plain_GBps"])
    res["GBps"] = best
    res["pct_hbm_peak"] = round(100 * best / HBM_PEAK_GBS, 2)
    res["note"] = ("a front-to-back read of 1 GiB (pa_stream_read: 16-byte loads, one contiguous "
                   "span per workgroup), after a cache flush: what a linear read reaches on this "
                   "device, beside the 8 TB/s specification the percentages use")
    del buf
    return res


class Timer:
    """Per-step HIP events on the current stream, around each launch group."""

    def __init__(self, torch, n, marks):
        self.ev = [[torch.cuda.Event(enable_timing=True) for _ in range(marks)] for _ in range(n)]

    def ms(self, i, a, b):
        return self.ev[i][a].elapsed_time(self.ev[i][b])


def time_decode(torch, pa, d, wl, P, steps, warmup, flush):
    """Per-step ms of pa_decode (the partition kernel, then the merge kernel
    for sequences split into several partitions)."""
    out = torch.empty_like(d.q)
    ws_bytes = pa.decode_workspace_size(wl.num_seqs, wl.num_q_heads, wl.head_dim,
                                        wl.max_seq_len, P)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")

    def launch(ev):
        ev[0].record()
        pa.decode(d.q, d.k, d.v, d.bt, d.sl, max_seq_len=wl.max_seq_len, scale=wl.scale,
                  partition_size=P, k_scale=d.ks, v_scale=d.vs, out=out, workspace=ws)
        ev[1].record()

    wt = Timer(torch, warmup, 2)
    for i in range(warmup):
        flush()
        launch(wt.ev[i])
    torch.cuda.synchronize()
    t = Timer(torch, steps, 2)
    for i in range(steps):
        flush()
        launch(t.ev[i])
    torch.cuda.synchronize()
    ms = [t.ms(i, 0, 1) for i in range(steps)]
    return ms, ms


def time_partition_kernel(torch, pa, d, wl, P, steps, warmup, flush):
    """Per-launch ms of the attention kernel alone (the attention stage of
    pa_decode_stages, without the merge), HIP events on the launch stream."""
    out = torch.empty_like(d.q)
    ws = torch.empty(max(pa.decode_workspace_size(wl.num_seqs, wl.num_q_heads, wl.head_dim,
                                                  wl.max_seq_len, P), 256),
                     dtype=torch.uint8, device="cuda")

    def launch(ev):
        ev[0].record()
        pa.decode_stages(d.q, d.k, d.v, d.bt, d.sl, max_seq_len=wl.max_seq_len,
                         stages=pa.PA_STAGE_ATTENTION, out=out, workspace=ws,
                         partition_size=P, scale=wl.scale, k_scale=d.ks, v_scale=d.vs)
        ev[1].record()

    for i in range(warmup):
        flush()
        launch(Timer(torch, 1, 2).ev[0])
    torch.cuda.synchronize()
    t = Timer(torch, steps, 2)
    for i in range(steps):
        flush()
        launch(t.ev[i])
    torch.cuda.synchronize()
    return [t.ms(i, 0, 1) for i in range(steps)]


def checked(wl):
    """Device copies of a workload, made after the host-side checks of what
    the kernels read without validating it (every live block-table entry
    inside the pool, lengths within their rows and the host-side bounds)."""
    from paged_kv_cache_22_amd import checks
    from workloads.device import Dev
    if hasattr(wl, "cu_q_lens"):
        checks.check_prefill_inputs(wl.cu_q_lens, wl.block_table, wl.seq_lens,
                                    num_blocks=wl.num_blocks, block_size=wl.block_size,
                                    max_q_len=wl.max_q_len, total_q=wl.total_q)
    else:
        checks.check_decode_inputs(wl.block_table, wl.seq_lens, num_blocks=wl.num_blocks,
                                   block_size=wl.block_size, max_seq_len=wl.max_seq_len,
                                   q_len=wl.q_len)
    return Dev(wl)


def mixed_devices(m):
    """Device copies of the mixed step: one KV cache shared by its decode rows
    and its chunks (they are one pool), with each part's own q, tables and
    lengths."""
    from paged_kv_cache_22_amd import checks
    from workloads.device import Dev
    dd = checked(m.decode)
    checks.check_prefill_inputs(m.prefill.cu_q_lens, m.prefill.block_table, m.prefill.seq_lens,
                                num_blocks=m.decode.num_blocks, block_size=m.decode.block_size,
                                max_q_len=m.prefill.max_q_len, total_q=m.prefill.total_q)
    dp = Dev.__new__(Dev)
    dp.wl = m.prefill
    dp.q = dev_like(m.prefill.q, m.prefill.q_dtype)
    dp.k, dp.v, dp.ks, dp.vs = dd.k, dd.v, dd.ks, dd.vs
    dp.bt = dev_like(m.prefill.block_table)
    dp.sl = dev_like(m.prefill.seq_lens)
    dp.cu = dev_like(m.prefill.cu_q_lens)
    return dd, dp


def dev_like(arr, tag=None):
    from workloads.device import dev
    return dev(arr, tag)


def time_mixed(torch, pa, dd, dp, m, P, steps, warmup, flush):
    """The mixed step as one step: after one cache flush, pa_decode on the
    decode rows and pa_prefill_chunk on the chunks, back to back on one
    stream, between one pair of events (a third event between the two gives
    the split).  Returns per-step (step, decode part, prefill part) ms."""
    dec, pre = m.decode, m.prefill
    out_d = torch.empty_like(dd.q)
    out_p = torch.empty_like(dp.q)
    ws = torch.empty(max(pa.decode_workspace_size(dec.num_seqs, dec.num_q_heads, dec.head_dim,
                                                  dec.max_seq_len, P), 256),
                     dtype=torch.uint8, device="cuda")

    def launch(ev):
        ev[0].record()
        pa.decode(dd.q, dd.k, dd.v, dd.bt, dd.sl, max_seq_len=dec.max_seq_len, scale=dec.scale,
                  partition_size=P, out=out_d, workspace=ws)
        ev[1].record()
        pa.prefill_chunk(dp.q, dp.cu, dp.k, dp.v, dp.bt, dp.sl, max_q_len=pre.max_q_len,
                         scale=pre.scale, out=out_p)
        ev[2].record()

    wt = Timer(torch, warmup, 3)
    for i in range(warmup):
        flush()
        launch(wt.ev[i])
    torch.cuda.synchronize()
    t = Timer(torch, steps, 3)
    for i in range(steps):
        flush()
        launch(t.ev[i])
    torch.cuda.synchronize()
    return ([t.ms(i, 0, 2) for i in range(steps)], [t.ms(i, 0, 1) for i in range(steps)],
            [t.ms(i, 1, 2) for i in range(steps)])


def time_mixed_one_call(torch, pa, dd, dp, m, P, steps, warmup, flush):
    """The mixed step through pa_mixed_step (the decode rows' merge inside
    the chunks' launch): one flush, one call, between one pair of events."""
    dec, pre = m.decode, m.prefill
    out_d = torch.empty_like(dd.q)
    out_p = torch.empty_like(dp.q)
    ws = torch.empty(max(pa.decode_workspace_size(dec.num_seqs, dec.num_q_heads, dec.head_dim,
                                                  dec.max_seq_len, P), 256),
                     dtype=torch.uint8, device="cuda")

    def launch(ev):
        ev[0].record()
        pa.mixed_step(dd.q, dd.bt, dd.sl, dp.q, dp.cu, dp.bt, dp.sl, dd.k, dd.v,
                      max_seq_len=dec.max_seq_len, max_q_len=pre.max_q_len, partition_size=P,
                      scale=dec.scale, dec_out=out_d, pre_out=out_p, workspace=ws)
        ev[1].record()

    wt = Timer(torch, warmup, 2)
    for i in range(warmup):
        flush()
        launch(wt.ev[i])
    torch.cuda.synchronize()
    t = Timer(torch, steps, 2)
    for i in range(steps):
        flush()
        launch(t.ev[i])
    torch.cuda.synchronize()
    return [t.ms(i, 0, 1) for i in range(steps)]


def mixed_summary(m, P, one_call, step, dec, pre):
    mean = lambda xs: sum(xs) / len(xs)
    sm, dm, pm = mean(step), mean(dec), mean(pre)
    om = mean(one_call)
    tflops = m.prefill.flops() / pm / 1e9
    attended = m.decode.total_tokens + m.prefill.pairs()
    return {
        "workload": "mixed step: 16 decode seqs (1024-8192) + 4 chunks of 512 over a 2048-token "
                    "shared prefix, 32/8 heads, d=128, bf16, seed 4",
        "decode_partition_size": P,
        "step_ms": round(om, 5),
        "p10_ms": round(sorted(one_call)[len(one_call) // 10], 5),
        "p90_ms": round(sorted(one_call)[(9 * len(one_call)) // 10], 5),
        "tokens_attended_per_s": round(attended / om * 1e3, 1),
        "note": "step: one flush, then one pa_mixed_step call (decode rows' attention, then the "
                "chunks with the decode rows' merge in their launch) between one pair of HIP "
                "events; two_calls: pa_decode and pa_prefill_chunk back to back on one stream, "
                "split at an event between them",
        "two_calls": {
            "step_ms": round(sm, 5),
            "decode": {"ms": round(dm, 5), "kv_bytes": m.decode.kv_bytes(),
                       "kv_GBps": round(m.decode.kv_bytes() / dm / 1e6, 2),
                       "pct_hbm_peak": round(100 * m.decode.kv_bytes() / dm / 1e6 / HBM_PEAK_GBS,
                                             2)},
            "prefill": {"ms": round(pm, 5), "TFLOPs": round(tflops, 2),
                        "pct_bf16_mfma_peak": round(100 * tflops / BF16_MFMA_PEAK_TFLOPS, 2),
                        "pairs": m.prefill.pairs(), "flops": m.prefill.flops()},
        },
    }


def time_verify(torch, pa, W, steps, warmup, flush, partition_size):
    """Draft verification at the Llama-3-8B layer shape: 64 sequences of
    512-4096 tokens, 4 queries each (pa_decode_multi_query, the 16 MFMA
    columns filled by 4 queries x 4 heads), against the same work done as 64
    prefill chunks of 4 rows (pa_prefill_chunk)."""
    wl = W.decode_workload(seed=2, num_seqs=64, num_q_heads=32, num_kv_heads=8, head_dim=128,
                           len_lo=512, len_hi=4096, q_dtype="bf16", kv_dtype="bf16", q_len=4,
                           pad=0, name="verify")
    d = checked(wl)
    B, qn = wl.num_seqs, wl.q_len
    out = torch.empty_like(d.q)
    ws = torch.empty(max(pa.decode_workspace_size(B, qn * wl.num_q_heads, wl.head_dim,
                                                  wl.max_seq_len, partition_size), 256),
                     dtype=torch.uint8, device="cuda")
    q3 = d.q.reshape(B * qn, wl.num_q_heads, wl.head_dim)
    out3 = torch.empty_like(q3)
    cu = torch.arange(0, B * qn + 1, qn, dtype=torch.int32, device="cuda")

    def mq(ev):
        ev[0].record()
        pa.decode_multi_query(d.q, d.k, d.v, d.bt, d.sl, max_seq_len=wl.max_seq_len,
                              scale=wl.scale, partition_size=partition_size, out=out, workspace=ws)
        ev[1].record()

    def pf(ev):
        ev[0].record()
        pa.prefill_chunk(q3, cu, d.k, d.v, d.bt, d.sl, max_q_len=qn, scale=wl.scale, out=out3)
        ev[1].record()

    res = {"workload": "draft verification: 64 seqs x 4 queries, lens U[512,4096] seed 2, "
                       "32/8 heads, d=128, bf16", "partition_size": partition_size}
    for name, fn in (("multi_query_decode", mq), ("as_prefill_chunks", pf)):
        wt = Timer(torch, warmup, 2)
        for i in range(warmup):
            flush()
            fn(wt.ev[i])
        torch.cuda.synchronize()
        t = Timer(torch, steps, 2)
        for i in range(steps):
            flush()
            fn(t.ev[i])
        torch.cuda.synchronize()
        ms = sum(t.ms(i, 0, 1) for i in range(steps)) / steps
        res[name] = {"ms": round(ms, 5), "kv_GBps": round(wl.kv_bytes() / ms / 1e6, 2),
                     "pct_hbm_peak": round(100 * wl.kv_bytes() / ms / 1e6 / HBM_PEAK_GBS, 2),
                     "queries_per_s": round(B * qn / ms * 1e3, 1)}
    res["kv_bytes"] = wl.kv_bytes()
    return res


def time_block_sizes(torch, pa, W, steps, warmup, flush):
    """The headline batch (C2's lengths, heads and data recipe) paged with
    32- and 64-token blocks, balanced split-KV."""
    res = {}
    for bs in (32, 64):
        w = W.decode_workload(seed=2, num_seqs=64, num_q_heads=32, num_kv_heads=8, head_dim=128,
                              len_lo=512, len_hi=4096, q_dtype="bf16", kv_dtype="bf16",
                              block_size=bs, pad=0, name=f"C2 bs={bs}")
        d = checked(w)
        s, _ = time_decode(torch, pa, d, w, -1, steps, warmup, flush)
        ms = sum(s) / len(s)
        res[str(bs)] = {"ms_per_step": round(ms, 5), "kv_GBps": round(w.kv_bytes() / ms / 1e6, 2),
                        "pct_hbm_peak": round(100 * w.kv_bytes() / ms / 1e6 / HBM_PEAK_GBS, 2)}
        del d
    return res


def time_shared_prefix(torch, pa, W, steps, warmup, flush):
    """64 sequences (32/8 heads, d=128, bf16) sharing a 2048-token prefix,
    each with U[512, 4096] tokens of its own (seed 2): pa_decode (balanced)
    over the whole tables, which reads the prefix once per sequence, against
    pa_decode_shared_prefix, which reads it once for the batch."""
    import numpy as np
    from workloads.device import dev
    sp = W.shared_prefix_workload(seed=2, num_seqs=64, num_q_heads=32, num_kv_heads=8,
                                  head_dim=128, prefix_len=2048, len_lo=512, len_hi=4096,
                                  q_dtype="bf16", kv_dtype="bf16", name="shared prefix")
    wl = sp.full
    q, k, v = dev(wl.q, "bf16"), dev(wl.k_cache, "bf16"), dev(wl.v_cache, "bf16")
    bt, sl = dev(wl.block_table), dev(wl.seq_lens)
    pt, st, sfl = dev(sp.prefix_table), dev(sp.suffix_table), dev(sp.suffix_lens)
    out = torch.empty_like(q)
    ws = torch.empty(max(pa.decode_workspace_size(wl.num_seqs, wl.num_q_heads, wl.head_dim,
                                                  wl.max_seq_len, -1), 256),
                     dtype=torch.uint8, device="cuda")
    smax = int(sp.suffix_lens.max())
    ws2 = torch.empty(max(int(pa.lib.pa_decode_shared_prefix_workspace_size(
        wl.num_seqs, 1, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, 2048, smax, 1024)), 256),
        dtype=torch.uint8, device="cuda")

    def plain(ev):
        ev[0].record()
        pa.decode(q, k, v, bt, sl, max_seq_len=wl.max_seq_len, scale=wl.scale, partition_size=-1,
                  out=out, workspace=ws)
        ev[1].record()

    def cascade(ev):
        ev[0].record()
        pa.decode_shared_prefix(q, k, v, pt, 2048, st, sfl, max_seq_len=smax, partition_size=1024,
                                scale=wl.scale, out=out, workspace=ws2)
        ev[1].record()

    unique = 2048 * 8 * 128 * 2 * 2 + int(sp.suffix_lens.astype(np.int64).sum()) * 8 * 128 * 2 * 2
    res = {"workload": "64 seqs sharing a 2048-token prefix + U[512,4096] own tokens, seed 2, "
                       "32/8 heads, d=128, bf16",
           "kv_bytes_attended": wl.kv_bytes(), "kv_bytes_unique": unique}
    for name, fn in (("plain_balanced", plain), ("cascade", cascade)):
        wt = Timer(torch, warmup, 2)
        for i in range(warmup):
            flush()
            fn(wt.ev[i])
        torch.cuda.synchronize()
        t = Timer(torch, steps, 2)
        for i in range(steps):
            flush()
            fn(t.ev[i])
        torch.cuda.synchronize()
        ms = sum(t.ms(i, 0, 1) for i in range(steps)) / steps
        res[name] = {"ms": round(ms, 5),
                     "tokens_attended_per_s": round(wl.total_tokens / ms * 1e3, 1),
                     "attended_kv_GBps": round(wl.kv_bytes() / ms / 1e6, 2),
                     "unique_kv_GBps": round(unique / ms / 1e6, 2)}
    return res


def write_cases(W):
    """Cache writes of the decode and prefill steps above, and a long-context
    fill: (label, WriteWorkload, pool blocks).  The caches are allocated on
    the device (zeros); only the new rows and slot maps come from the host."""
    cases = []
    for label, seed, T, ind, kvd, nb in (("decode step, 64 seqs, bf16", 2, 64, "bf16", "bf16", 9216),
                                         ("decode step, 256 seqs, bf16->fp8", 5, 256, "bf16", "fp8",
                                          18432)):
        slots = W.write_decode_step(seed=seed, num_seqs=T, num_blocks=nb)
        cases.append((label, slots, ind, kvd, nb))
    nb = 4 * (2048 + 512) // 16
    cases.append(("4 prefill chunks of 512 after a 2048-token prefix, bf16",
                  W.write_chunks(seed=4, chunk_lens=[512] * 4, ctx_lens=[2048] * 4, num_blocks=nb),
                  "bf16", "bf16", nb))
    for kvd in ("bf16", "fp8"):
        cases.append((f"32768-token context fill, bf16->{kvd}",
                       W.write_chunks(seed=6, chunk_lens=[32768], ctx_lens=[0], num_blocks=2048),
                       "bf16", kvd, 2048))
    out = []
    for label, slots, ind, kvd, nb in cases:
        wl = W.write_workload(seed=len(out) + 1, slot_mapping=slots, num_kv_heads=8, head_dim=128,
                              in_dtype=ind, kv_dtype=kvd, num_blocks=nb, fill_cache=False,
                              name=label)
        out.append(wl)
    return out


def time_write(torch, pa, wl, steps, warmup, flush):
    """Per-call ms of pa_write_kv on one write workload (caches on the device)."""
    from workloads.device import dev
    cdt = {"bf16": torch.bfloat16, "fp8": torch.uint8, "f32": torch.float32}[wl.kv_dtype]
    kc = torch.zeros(wl.k_cache.shape, dtype=cdt, device="cuda")
    vc = torch.zeros(wl.v_cache.shape, dtype=cdt, device="cuda")
    key, value = dev(wl.key, wl.in_dtype), dev(wl.value, wl.in_dtype)
    slots, ks, vs = dev(wl.slot_mapping), dev(wl.k_scale), dev(wl.v_scale)

    def launch(ev):
        ev[0].record()
        pa.write_kv(key, value, kc, vc, slots, k_scale=ks, v_scale=vs)
        ev[1].record()

    wt = Timer(torch, warmup, 2)
    for i in range(warmup):
        flush()
        launch(wt.ev[i])
    torch.cuda.synchronize()
    t = Timer(torch, steps, 2)
    for i in range(steps):
        flush()
        launch(t.ev[i])
    torch.cuda.synchronize()
    ms = sum(t.ms(i, 0, 1) for i in range(steps)) / steps
    gbs = wl.bytes_moved() / ms / 1e6
    return {"workload": wl.name, "tokens": wl.num_tokens, "ms": round(ms, 5),
            "bytes": wl.bytes_moved(), "GBps": round(gbs, 2),
            "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}


def med(xs):
    s = sorted(xs)
    return s[len(s) // 2]


def decode_summary(wl, step_ms, kern_ms):
    kv = wl.kv_bytes()
    ms = sum(step_ms) / len(step_ms)
    kms = sum(kern_ms) / len(kern_ms)
    return {
        "ms_per_step": round(ms, 5), "kv_GBps": round(kv / ms / 1e6, 2),
        "pct_hbm_peak": round(100 * kv / ms / 1e6 / HBM_PEAK_GBS, 2),
        "tokens_attended_per_s": round(wl.total_tokens / ms * 1e3, 1),
        "partition_kernel_ms": round(kms, 5),
        "partition_kernel_GBps": round(kv / kms / 1e6, 2),
        "p10_ms": round(sorted(step_ms)[len(step_ms) // 10], 5),
        "p50_ms": round(med(step_ms), 5),
        "p90_ms": round(sorted(step_ms)[(9 * len(step_ms)) // 10], 5),
        "kv_bytes": kv, "total_tokens": wl.total_tokens,
    }


def copy_calibration():
    """Three plain copies of 512 MiB: each reads and writes exactly 512 MiB."""
    import torch
    n = 512 << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                      "copies": 3}))


def profile_one(args, W):
    """Time one non-headline workload alone (for per-kernel profiling)."""
    import torch
    import paged_kv_cache_22_amd as pa
    flush = CacheFlush(torch)
    if args.workload == "VERIFY":
        print(json.dumps(time_verify(torch, pa, W, args.steps, args.warmup, flush,
                                     args.partition_size)), flush=True)
        return
    if args.partition_size < 0 and args.workload == "C5":
        args.partition_size = 0   # its best: one pass (sequences of 256-2048 tokens, no merge)
    if args.workload == "PREFIX":
        print(json.dumps(time_shared_prefix(torch, pa, W, args.steps, args.warmup, flush)), flush=True)
        return
    if args.workload == "BLOCKS":
        print(json.dumps(time_block_sizes(torch, pa, W, args.steps, args.warmup, flush)), flush=True)
        return
    if args.workload == "STREAM":
        print(json.dumps(time_stream_read(torch, pa, flush, reps=args.steps)), flush=True)
        return
    if args.workload == "WRITE":
        for wl in write_cases(W):
            print(json.dumps(time_write(torch, pa, wl, args.steps, args.warmup, flush)), flush=True)
        return
    n = int(args.workload[1])
    res = {"workload": W.CONFIG_NAMES[n]}
    if n == 4:
        m = W.config4(pad=0, partition_size=args.partition_size)
        dd, dp = mixed_devices(m)
        one = time_mixed_one_call(torch, pa, dd, dp, m, args.partition_size, args.steps,
                                  args.warmup, flush)
        step, dec, pre = time_mixed(torch, pa, dd, dp, m, args.partition_size, args.steps,
                                    args.warmup, flush)
        res.update(mixed_summary(m, args.partition_size, one, step, dec, pre))
    else:
        w = W.config3(pad=0) if n == 3 else W.config5(pad=0, partition_size=args.partition_size)
        dd = checked(w)
        s, k = time_decode(torch, pa, dd, w, w.partition_size, args.steps, args.warmup, flush)
        res.update(decode_summary(w, s, k))
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--partition-size", type=int, default=-1,
                    help="split-KV partition size in tokens for the headline; -1 = the "
                         "balanced split (equal work per resident workgroup), 0 = one pass")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true", help="skip the other workloads")
    ap.add_argument("--workload", default="C2", choices=["C2", "C3", "C4", "C5", "WRITE", "VERIFY", "BLOCKS", "PREFIX",
                             "STREAM"],
                    help="time only this workload (default: the Llama-3-8B-shaped C2 headline "
                         "plus the others under per_config; WRITE = the cache writes, VERIFY = draft "
                         "verification, BLOCKS = 32/64-token blocks, PREFIX = a shared-prefix batch, "
                         "STREAM = the linear read rate of a 1 GiB buffer)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy three times (a known byte count "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the kernels "
              f"run on one GPU's share of the batch; the multi-GPU split is not built)",
              file=sys.stderr)
        sys.exit(2)

    import workloads as W
    if args.workload != "C2":
        return profile_one(args, W)
    wl = W.config2(pad=0, partition_size=args.partition_size)
    cpu = None if args.no_cpu_baseline else cpu_baseline(wl)   # before any GPU use

    import torch
    import paged_kv_cache_22_amd as pa

    torch.cuda.init()
    flush = CacheFlush(torch)
    d = checked(wl)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step_ms, _ = time_decode(torch, pa, d, wl, args.partition_size, args.steps,
                             args.warmup, flush)
    wall = time.perf_counter() - t0
    if args.partition_size != 0:   # the dominant kernel on its own
        kern_ms = time_partition_kernel(torch, pa, d, wl, args.partition_size, args.steps,
                                        args.warmup, flush)
    else:
        kern_ms = step_ms
    head = decode_summary(wl, step_ms, kern_ms)
    del d

    per_config = {}
    if not args.headline_only:
        # C3 at its stated 512-token partitions, C5 in one pass (its best:
        # sequences of 256-2048 tokens, no merge), each also balanced
        for n, P in ((3, 512), (5, 0)):
            w = W.build_config(n, pad=0) if n == 3 else W.build_config(n, pad=0, partition_size=P)
            dd = checked(w)
            s, k = time_decode(torch, pa, dd, w, P, 20, 3, flush)
            per_config[w.name] = decode_summary(w, s, k)
            per_config[w.name]["workload"] = W.CONFIG_NAMES[n]
            per_config[w.name]["partition_size"] = P
            s, k = time_decode(torch, pa, dd, w, -1, 20, 3, flush)
            per_config[w.name]["balanced"] = {kk: vv for kk, vv in decode_summary(w, s, k).items()
                                              if kk in ("ms_per_step", "kv_GBps", "pct_hbm_peak")}
            del dd
        # the mixed step, timed as one step (decode rows balanced across the chip)
        m = W.config4(pad=0, partition_size=-1)
        dd, dp = mixed_devices(m)
        one = time_mixed_one_call(torch, pa, dd, dp, m, -1, 20, 3, flush)
        step, dec, pre = time_mixed(torch, pa, dd, dp, m, -1, 20, 3, flush)
        per_config["C4"] = mixed_summary(m, -1, one, step, dec, pre)
        del dd, dp
        per_config["kv_write"] = [time_write(torch, pa, wl, 20, 3, flush) for wl in write_cases(W)]
        per_config["verify"] = time_verify(torch, pa, W, 20, 3, flush, args.partition_size)
        per_config["block_size"] = time_block_sizes(torch, pa, W, 20, 3, flush)
        per_config["shared_prefix"] = time_shared_prefix(torch, pa, W, 20, 3, flush)
    stream = None if args.headline_only else time_stream_read(torch, pa, flush)

    kv = head["kv_GBps"]
    line = {
        "metric": METRIC,
        "value": kv,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Llama-3-8B-shaped layer decode, bf16: 64 seqs, 32 q-heads / 8 "
                               "kv-heads, head_dim 128, block_size 16, lens U[512,4096] seed 2, "
                               "block tables a random permutation of one pool",
                   "global_batch": wl.num_seqs, "seq_len": "512-4096",
                   "total_tokens": wl.total_tokens, "partition_size": args.partition_size,
                   "parallelism": "none (1 GPU)"},
        "pct_hbm_peak": head["pct_hbm_peak"],
        "tokens_attended_per_s": head["tokens_attended_per_s"],
        "timing": {"p10_ms": head["p10_ms"], "p50_ms": head["p50_ms"], "p90_ms": head["p90_ms"],
                   "wall_s_incl_cache_flush": round(wall, 3),
                   "note": "per-step HIP events around the launches; a 1 GiB read before "
                           "each step evicts the Infinity Cache and is not timed"},
        "roofline": {
            "kernel": ("decode_balanced_kernel<128, bf16>" if args.partition_size < 0 else
                       "decode_kernel<128, bf16, split>") + " (attention stage of pa_decode_stages)",
            "bound": "hbm",
            "achieved": head["partition_kernel_GBps"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(head["partition_kernel_GBps"] / HBM_PEAK_GBS, 4),
            "traffic": stored_traffic(args.partition_size),
            "algorithmic_bytes_per_launch": head["kv_bytes"],
            "avg_launch_ms": head["partition_kernel_ms"],
            "note": "achieved = live K+V bytes / mean HIP-event duration of the attention "
                    "kernel launched alone (without the merge); traffic = HBM bytes "
                    "read+written per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE "
                    "summary (copy-calibrated), null if the kernel sources or the partition "
                    "mode changed since",
        },
        "stream_read": stream,
        "cpu_baseline": cpu,
        "host": {**host_info(), **gpu_info(torch)},
        "per_config": per_config,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
