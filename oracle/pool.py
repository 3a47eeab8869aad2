"""Run the oracle over its independent work items on all host cores.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT (like the rest of ``oracle``):
used by the GPU parity tests, to compute full-size references in seconds,
and by the bench's CPU-baseline leg.

No arithmetic lives here.  Decode attention of one (sequence, kv-head) pair
and causal prefill of one (chunk, kv-head) pair are independent of every
other pair, so each worker process calls the oracle's own per-pair functions
(``decode_rows``, ``prefill_rows``) and the parent only places the returned
rows.  The result is bit-identical to the single-process oracle's.

Workers are started with the "spawn" method (fresh interpreters that import
numpy and this package only; they never touch a GPU), each with its BLAS
pinned to one thread.  The input arrays -- caches of several GB at the long
context -- are written once per call as ``.npy`` files into a temporary
directory (``/dev/shm`` when it has room) and memory-mapped read-only by the
workers, so no worker holds a private copy; a worker keeps the maps of the
directory it last read.
"""
from __future__ import annotations

import atexit
import multiprocessing as mp
import os
import shutil
import tempfile
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

from . import attention

# at most this many workers (the share of host cores one GPU's jobs may use)
MAX_WORKERS = 16

_NAMES = ("q", "k_cache", "v_cache", "block_table", "seq_lens", "cu_q_lens")


def default_workers() -> int:
    return max(1, min(MAX_WORKERS, os.cpu_count() or 1))


# ---------------------------------------------------------------------------
# worker side
# ---------------------------------------------------------------------------
_LIMITS = None


def _init_worker():
    global _LIMITS
    try:
        from threadpoolctl import threadpool_limits
        _LIMITS = threadpool_limits(limits=1)   # kept alive for the worker's lifetime
    except ImportError:   # the environment variables below still pin OpenBLAS / MKL
        pass


_OPENED = {"key": None, "arrays": None}


def _open(dirpath: str):
    """The staged arrays of ``dirpath`` as read-only ndarrays over the mapped
    files; the last directory's maps are kept for the tasks that follow."""
    key = (dirpath, os.stat(os.path.join(dirpath, "q.npy")).st_mtime_ns)
    if _OPENED["key"] != key:
        arrs = {}
        for n in _NAMES:
            f = os.path.join(dirpath, n + ".npy")
            if os.path.exists(f):
                arrs[n] = np.asarray(np.load(f, mmap_mode="r"))
        _OPENED["key"], _OPENED["arrays"] = key, arrs
    return _OPENED["arrays"]


def _decode_task(task):
    dirpath, scale, q_dtype, kv_dtype, k_scale, v_scale, b, h = task
    a = _open(dirpath)
    out, lse = attention.decode_rows(a["q"], a["k_cache"], a["v_cache"], a["block_table"],
                                     a["seq_lens"], scale, q_dtype, kv_dtype, b, h,
                                     k_scale, v_scale)
    return b, h, out, lse


def _prefill_task(task):
    dirpath, scale, q_dtype, kv_dtype, k_scale, v_scale, c, h = task
    a = _open(dirpath)
    out, lse = attention.prefill_rows(a["q"], a["cu_q_lens"], a["k_cache"], a["v_cache"],
                                      a["block_table"], a["seq_lens"], scale, q_dtype, kv_dtype,
                                      c, h, k_scale, v_scale)
    return c, h, out, lse


# ---------------------------------------------------------------------------
# parent side
# ---------------------------------------------------------------------------
class OraclePool:
    """A pool of oracle worker processes.  ``decode`` and ``prefill_chunk``
    take the oracle's arguments and return what the oracle returns."""

    def __init__(self, workers: Optional[int] = None):
        self.workers = workers or default_workers()
        # BLAS thread count of the spawned interpreters, fixed before numpy loads there
        saved = {k: os.environ.get(k) for k in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS",
                                                "MKL_NUM_THREADS")}
        for k in saved:
            os.environ[k] = "1"
        try:
            self._pool = mp.get_context("spawn").Pool(self.workers, initializer=_init_worker)
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v

    def close(self):
        if self._pool is not None:
            self._pool.close()
            self._pool.join()
            self._pool = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # -- shared inputs -------------------------------------------------------
    @staticmethod
    def stage(arrays: dict) -> str:
        """Write the named input arrays where the workers map them; returns
        the directory, to pass as ``staged`` to calls on the same inputs and
        to ``release`` afterwards."""
        need = sum(a.nbytes for a in arrays.values() if a is not None)
        base = None
        try:
            st = os.statvfs("/dev/shm")
            if st.f_bavail * st.f_frsize > 2 * need + (1 << 30):
                base = "/dev/shm"
        except OSError:
            pass
        d = tempfile.mkdtemp(prefix="pa_oracle_", dir=base)
        for n, a in arrays.items():
            if a is not None:
                np.save(os.path.join(d, n + ".npy"), np.ascontiguousarray(a))
        return d

    @staticmethod
    def release(dirpath: str) -> None:
        shutil.rmtree(dirpath, ignore_errors=True)

    def _run(self, fn, tasks: Sequence[tuple]):
        return list(self._pool.imap_unordered(fn, tasks, chunksize=1))

    # -- the oracle's entry points -------------------------------------------
    def decode(self, q, k_cache, v_cache, block_table, seq_lens, scale: float, q_dtype: str,
               kv_dtype: str, k_scale=None, v_scale=None,
               items: Optional[Iterable[Tuple[int, int]]] = None, staged: Optional[str] = None):
        """oracle.decode, its (sequence, kv-head) pairs spread over the workers.
        ``staged``: a directory from ``stage`` holding these same inputs."""
        B, Hq, d = q.shape
        Hkv = attention.kv_heads(k_cache)
        G = Hq // Hkv
        todo = list(items) if items is not None else [(b, h) for b in range(B) for h in range(Hkv)]
        # longest sequences first, so no worker is left with a long one at the end
        todo.sort(key=lambda it: -int(seq_lens[it[0]]))
        ks = None if k_scale is None else np.asarray(k_scale, np.float32).copy()
        vs = None if v_scale is None else np.asarray(v_scale, np.float32).copy()
        out = np.full((B, Hq, d), np.nan)
        lse = np.full((B, Hq), np.nan)
        dirpath = staged or self.stage({"q": q, "k_cache": k_cache, "v_cache": v_cache,
                                        "block_table": block_table, "seq_lens": seq_lens})
        try:
            tasks = [(dirpath, scale, q_dtype, kv_dtype, ks, vs, int(b), int(h)) for b, h in todo]
            for b, h, o, l in self._run(_decode_task, tasks):
                out[b, h * G:(h + 1) * G] = o
                lse[b, h * G:(h + 1) * G] = l
        finally:
            if staged is None:
                self.release(dirpath)
        return out, lse

    def prefill_chunk(self, q, cu_q_lens, k_cache, v_cache, block_table, seq_lens, scale: float,
                      q_dtype: str, kv_dtype: str, k_scale=None, v_scale=None,
                      items: Optional[Iterable[Tuple[int, int]]] = None):
        """oracle.prefill_chunk, its (chunk, kv-head) pairs spread over the workers."""
        total_q, Hq, d = q.shape
        Hkv = attention.kv_heads(k_cache)
        G = Hq // Hkv
        n_chunks = len(seq_lens)
        todo = list(items) if items is not None else [(c, h) for c in range(n_chunks)
                                                      for h in range(Hkv)]
        ks = None if k_scale is None else np.asarray(k_scale, np.float32).copy()
        vs = None if v_scale is None else np.asarray(v_scale, np.float32).copy()
        out = np.full((total_q, Hq, d), np.nan)
        lse = np.full((total_q, Hq), np.nan)
        dirpath = self.stage({"q": q, "cu_q_lens": cu_q_lens, "k_cache": k_cache,
                               "v_cache": v_cache, "block_table": block_table,
                               "seq_lens": seq_lens})
        try:
            tasks = [(dirpath, scale, q_dtype, kv_dtype, ks, vs, int(c), int(h)) for c, h in todo]
            for c, h, o, l in self._run(_prefill_task, tasks):
                q0, q1 = int(cu_q_lens[c]), int(cu_q_lens[c + 1])
                out[q0:q1, h * G:(h + 1) * G] = o
                lse[q0:q1, h * G:(h + 1) * G] = l
        finally:
            self.release(dirpath)
        return out, lse


_SHARED: Optional[OraclePool] = None


def shared_pool() -> OraclePool:
    """One pool per process, started on first use and closed at exit."""
    global _SHARED
    if _SHARED is None:
        _SHARED = OraclePool()
        atexit.register(_SHARED.close)
    return _SHARED
