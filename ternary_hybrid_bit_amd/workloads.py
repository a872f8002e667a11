"""Synthetic workloads for benchmarks and GPU tests: seeded matrices from
``synth``, packed by libwal's C++ packer.

The 252-matrix body sweep (36 layers of q, k, v, o, gate, up, down shapes of
Qwen3-8B) is drawn and packed by a pool of worker processes, one matrix per
task, so setting it up takes seconds rather than minutes (about 75 s in one
process).

Worker rule.  A GPU machine admits at most 16 of a user's processes on its card
at once.  A profiler that preloads its tool library into every process (as
rocprofv3 does) makes each pool worker such a process, so under a profiler
packing runs in-process, and otherwise the pool is capped at 8 workers
(parent + 8 stays under the limit even if the workers were counted).
Profiled runs can skip packing altogether: ``WAL_SWEEP_CACHE=<path>`` makes
``sweep`` load the packed sweep from that .npz file when it exists and
write it there after packing when it does not, so a plain run can pack once
and every profiler pass of the same session load the file.
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


MAX_WORKERS = 8


def under_profiler() -> bool:
    """True when a profiler has preloaded its tool into this process (it
    would follow every child process as well)."""
    if any(k.startswith("ROCPROF") for k in os.environ):
        return True
    return "rocprofiler" in os.environ.get("LD_PRELOAD", "")


def default_workers() -> int:
    """Packing processes: WAL_PACK_WORKERS if set (1 packs in-process), 1
    under a profiler, else the usable CPUs up to MAX_WORKERS."""
    env = os.environ.get("WAL_PACK_WORKERS")
    if env:
        return max(1, min(MAX_WORKERS, int(env)))
    if under_profiler():
        return 1
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(MAX_WORKERS, n))


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


def _save(path: str, items) -> None:
    tmp = path + ".tmp.npz"
    np.savez(tmp, blobs=np.concatenate([b for b, _, _ in items]),
             blob_sizes=np.array([b.size for b, _, _ in items], np.int64),
             xs=np.concatenate([x for _, _, x in items]),
             x_sizes=np.array([x.size for _, _, x in items], np.int64))
    os.replace(tmp, path)


def _load(path: str):
    with np.load(path, allow_pickle=False) as f:
        blobs, bs, xs, xsz = f["blobs"], f["blob_sizes"], f["xs"], f["x_sizes"]
    out, ob, ox = [], 0, 0
    for nb, nx in zip(bs.tolist(), xsz.tolist()):
        blob = blobs[ob:ob + nb].copy()
        out.append((blob, wal_inspect(blob), xs[ox:ox + nx].copy()))
        ob += nb
        ox += nx
    return out


def base3_body(workers: Optional[int] = None):
    """The 27B-shaped base-3 body (synth.BASE3_BODY, about 2.1 GB packed).
    With WAL_BASE3_CACHE set, loaded from / saved to that file."""
    ids = list(range(synth.BASE3_BODY_MATRICES))
    cache = os.environ.get("WAL_BASE3_CACHE")
    if cache and os.path.exists(cache):
        return _load(cache)
    items = packed_config(synth.BASE3_BODY, ids, workers)
    if cache:
        _save(cache, items)
    return items


def sweep(layers: int = 36, workers: Optional[int] = None):
    """The body sweep (first ``layers`` layers, 7 matrices each), packed.
    With WAL_SWEEP_CACHE set, loaded from / saved to that file (its blobs
    pass wal_inspect's header checks on load)."""
    cache = os.environ.get("WAL_SWEEP_CACHE")
    if cache and layers == 36:
        if os.path.exists(cache):
            return _load(cache)
        items = packed_config(2, list(range(7 * layers)), workers)
        _save(cache, items)
        return items
    return packed_config(2, list(range(7 * layers)), workers)
