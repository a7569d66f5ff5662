"""The oracle's encode and decode over millions of groups, split into chunks
across worker processes (test helper).

Workers are started with the spawn method and import only NumPy and the
oracle: they never touch the GPU.  Chunks are processed in order and their
results concatenated, so the output is exactly that of one call over all
groups (the oracle treats every group on its own).
"""

import multiprocessing as mp
import os

import numpy as np

CHUNK = 32768


def workers():
    return max(1, min(8, os.cpu_count() or 1))


def _encode(job):
    from oracle import codec
    x, c, l, t = job
    blocks, info = codec.encode_groups(x, codec.Tables(c, l), t, return_info=True)
    return blocks, info["clipped"], info["stats"]


def _decode(job):
    from oracle import codec
    b, c, l, t = job
    return codec.decode_blocks(b, codec.Tables(c, l), t)


def _map(fn, jobs):
    if len(jobs) == 1 or workers() == 1:
        return [fn(j) for j in jobs]
    with mp.get_context("spawn").Pool(min(workers(), len(jobs))) as pool:
        return pool.map(fn, jobs, chunksize=1)


def encode(x_groups, tables, t):
    """Oracle blocks [G, 64], clipped flags [G] and summed statistics."""
    x = np.ascontiguousarray(x_groups)
    jobs = [(x[i:i + CHUNK], tables.centroids, tables.code_len, np.float32(t)) for i in range(0, x.shape[0], CHUNK)]
    res = _map(_encode, jobs)
    stats = {}
    for _, _, st in res:
        for k, v in st.items():
            stats[k] = stats.get(k, 0) + v
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res]), stats


def decode(blocks, tables, t):
    """Oracle FP16 values [G, 128] of the given blocks."""
    b = np.ascontiguousarray(blocks)
    jobs = [(b[i:i + CHUNK], tables.centroids, tables.code_len, np.float32(t)) for i in range(0, b.shape[0], CHUNK)]
    return np.concatenate(_map(_decode, jobs))
