"""Synthetic workloads for benchmarks and GPU tests: seeded matrices from
``synth``, packed by libwal's C++ packer.

The 252-matrix body sweep (36 layers of q, k, v, o, gate, up, down shapes of
Qwen3-8B) is drawn and packed by a pool of worker processes, one matrix per
task, so setting it up takes seconds rather than minutes.
"""
from __future__ import annotations

import multiprocessing as mp
import os
from typing import List, Optional, Tuple

import numpy as np

import synth

from . import pack_matrix, wal_inspect


def _pack_one(args) -> Tuple[bytes, bytes]:
    cfg, mid = args
    m = synth.config_matrix(cfg, mid)
    blob, _ = pack_matrix(m)
    _, xbits = synth.config_x(cfg, mid)
    return blob.tobytes(), xbits.tobytes()


def default_workers() -> int:
    """Packing processes: WAL_PACK_WORKERS if set (1 packs in-process, e.g.
    under a profiler that would follow every child), else the usable CPUs up
    to 16."""
    env = os.environ.get("WAL_PACK_WORKERS")
    if env:
        return max(1, int(env))
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def packed_config(cfg: int, ids: List[int], workers: Optional[int] = None):
    """[(blob uint8, info, x bf16 bits uint16)] for matrices ``ids`` of config ``cfg``."""
    workers = workers or default_workers()
    tasks = [(cfg, i) for i in ids]
    if workers > 1 and len(tasks) > 1:
        # spawn: fresh interpreters, safe even after the parent has used the GPU
        ctx = mp.get_context("spawn")
        with ctx.Pool(workers) as pool:
            res = pool.map(_pack_one, tasks, chunksize=1)
    else:
        res = [_pack_one(t) for t in tasks]
    out = []
    for b, xb in res:
        blob = np.frombuffer(b, dtype=np.uint8).copy()
        out.append((blob, wal_inspect(blob), np.frombuffer(xb, dtype=np.uint16).copy()))
    return out


def sweep(layers: int = 36, workers: Optional[int] = None):
    """The body sweep (first ``layers`` layers, 7 matrices each), packed."""
    return packed_config(2, list(range(7 * layers)), workers)
