"""Copy a seeded workload to the GPU as torch tensors (bf16 bit patterns are
reinterpreted as torch.bfloat16, fp8 codes stay uint8).  Plumbing only."""
import numpy as np


def dev(arr, tag=None):
    """numpy storage array -> GPU tensor."""
    import torch
    if arr is None:
        return None
    if tag == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.cuda()


class Dev:
    """Device copies of a decode or prefill workload."""

    def __init__(self, wl):
        self.wl = wl
        self.q = dev(wl.q, wl.q_dtype)
        self.k = dev(wl.k_cache, wl.kv_dtype)
        self.v = dev(wl.v_cache, wl.kv_dtype)
        self.bt = dev(wl.block_table)
        self.sl = dev(wl.seq_lens)
        self.ks = dev(wl.k_scale)
        self.vs = dev(wl.v_scale)
        self.cu = dev(wl.cu_q_lens) if hasattr(wl, "cu_q_lens") else None
