"""Host-side checks of the device arrays whose contents the C ABI does not
validate (include/pa.h, "Errors": an out-of-range block-table entry or a
sequence longer than its table row is undefined behaviour, and on the GPU an
out-of-range entry is a memory fault).

The entry points never read device memory from the host, so these checks
are separate, opt-in calls for tests and debugging: they copy the arrays to
the host (a synchronising copy for GPU tensors) and raise ValueError naming
the first violations.  They read only what the kernels read: the table
entries below ceil(seq_len / block_size) of each row.
"""
from __future__ import annotations

import numpy as np

__all__ = ["check_decode_inputs", "check_prefill_inputs", "check_write_inputs"]

_SHOW = 5   # violations listed per message


def _host(a, name):
    if a is None:
        raise ValueError(f"{name} is required")
    if hasattr(a, "detach"):   # a torch tensor, on any device
        a = a.detach().cpu().numpy()
    a = np.asarray(a)
    if a.dtype.kind not in "iu":
        raise ValueError(f"{name} must hold integers, not {a.dtype}")
    return a.astype(np.int64)


def _fail(what, bad):
    if bad:
        more = f" (and {len(bad) - _SHOW} more)" if len(bad) > _SHOW else ""
        raise ValueError(f"{what}: " + "; ".join(bad[:_SHOW]) + more)


def _check_tables(table, lens, num_blocks, block_size, what):
    """Every table entry a row's length makes live lies in [0, num_blocks)."""
    if table.ndim != 2 or table.shape[0] != lens.shape[0]:
        raise ValueError(f"{what}: block_table must be [rows, max_blocks], one row per length")
    bad = []
    width = table.shape[1] * block_size
    for b, L in enumerate(lens):
        if L < 0:
            bad.append(f"row {b}: length {L} < 0")
            continue
        if L > width:
            bad.append(f"row {b}: length {L} above max_blocks_per_seq * block_size = {width}")
            continue
        live = table[b, :(L + block_size - 1) // block_size]
        off = np.flatnonzero((live < 0) | (live >= num_blocks))
        bad += [f"row {b}: block_table[{b}, {j}] = {live[j]} outside [0, {num_blocks})"
                for j in off]
    _fail(what, bad)


def check_decode_inputs(block_table, seq_lens, *, num_blocks: int, block_size: int,
                        max_seq_len: int, q_len: int = 1) -> None:
    """pa_decode / pa_decode_multi_query / a mixed step's decode part:
    0 <= seq_len <= max_seq_len (the host-side bound that sizes the grid),
    every live table entry inside the pool, and with q_len > 1 no sequence
    of 0 < seq_len < q_len (its rows are unspecified)."""
    lens = _host(seq_lens, "seq_lens").reshape(-1)
    table = _host(block_table, "block_table")
    bad = [f"seq {b}: seq_len {L} above max_seq_len {max_seq_len}"
           for b, L in enumerate(lens) if L > max_seq_len]
    if q_len > 1:
        bad += [f"seq {b}: seq_len {L} below q_len {q_len}"
                for b, L in enumerate(lens) if 0 < L < q_len]
    _fail("decode inputs", bad)
    _check_tables(table, lens, num_blocks, block_size, "decode inputs")


def check_prefill_inputs(cu_q_lens, block_table, seq_lens, *, num_blocks: int,
                         block_size: int, max_q_len: int, total_q: int) -> None:
    """pa_prefill_chunk / a mixed step's chunk part: cu_q_lens starts at 0,
    never decreases and ends within total_q; every chunk's length is at most
    max_q_len (the host-side bound that sizes the grid); every live table
    entry inside the pool.  (A chunk whose seq_len is below its length is
    allowed: its rows get zeros.)"""
    cu = _host(cu_q_lens, "cu_q_lens").reshape(-1)
    lens = _host(seq_lens, "seq_lens").reshape(-1)
    table = _host(block_table, "block_table")
    if cu.size != lens.size + 1:
        raise ValueError(f"prefill inputs: cu_q_lens has {cu.size} entries for "
                         f"{lens.size} chunks (needs chunks + 1)")
    bad = []
    if cu.size and cu[0] != 0:
        bad.append(f"cu_q_lens[0] = {cu[0]}, not 0")
    q = np.diff(cu)
    bad += [f"chunk {c}: cu_q_lens decreases ({cu[c]} -> {cu[c + 1]})"
            for c in np.flatnonzero(q < 0)]
    bad += [f"chunk {c}: length {q[c]} above max_q_len {max_q_len}"
            for c in np.flatnonzero(q > max_q_len)]
    if cu.size and cu[-1] > total_q:
        bad.append(f"cu_q_lens ends at {cu[-1]}, past total_q {total_q}")
    _fail("prefill inputs", bad)
    _check_tables(table, lens, num_blocks, block_size, "prefill inputs")


def check_write_inputs(slot_mapping, *, num_blocks: int, block_size: int) -> None:
    """pa_write_kv: no two tokens mapped to one slot (their writes race).
    Negative slots (padding) and slots past the pool are skipped by the
    kernel, so they are allowed."""
    s = _host(slot_mapping, "slot_mapping").reshape(-1)
    live = s[(s >= 0) & (s < num_blocks * block_size)]
    vals, counts = np.unique(live, return_counts=True)
    _fail("write inputs", [f"slot {v} written by {n} tokens" for v, n in zip(vals, counts)
                           if n > 1])
