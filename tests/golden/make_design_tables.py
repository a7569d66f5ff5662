"""Write the table sets of the S x H design points the v1 block can hold.

Calls only the oracle (``oracle.study.design_tables``) on the seeded
calibration samples of ``workloads``; the GPU path never produces these.

    python tests/golden/make_design_tables.py     # writes tests/golden/design_tables.npz

For each workload -- the 1024x1024 weight (c1), the LLaMA-3-8B gate
projection (gate) and the KV cache's K and V -- and each S in {16, 32, 64},
H in {1, 2, 4}: <wl>_S<S>_H<H>_centroids [S, 15] and <wl>_S<S>_H<H>_code_len
[S, H, 16], learned from the workload's calibration sample with the
trainer's steps (the 1-D k-means once per workload, Lloyd k-means for S
patterns, H codebooks per pattern).  oracle.study.v1_tables writes a point
into the block's 64 x 4 table slots.
"""

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import codec, study  # noqa: E402
import workloads as W  # noqa: E402

S_LIST = (16, 32, 64)
H_LIST = (1, 2, 4)


def samples():
    yield "c1", W.c1_sample()
    yield "gate", W.c2_sample("gate")
    yield "k", W.kv_sample("k")
    yield "v", W.kv_sample("v")


def main(out=os.path.join(HERE, "design_tables.npz")):
    arrays = {}
    for name, s in samples():
        t0 = time.time()
        x = s.numpy().reshape(-1, W.GROUP)
        ts = codec.tensor_scale(float(np.max(np.abs(x.astype(np.float32)))))[0]
        tabs = study.design_tables(x, ts, S_LIST, H_LIST)
        for (S, H), (c, L) in tabs.items():
            study.v1_tables(c, L).check()
            arrays["%s_S%d_H%d_centroids" % (name, S, H)] = c.astype(np.float32)
            arrays["%s_S%d_H%d_code_len" % (name, S, H)] = L.astype(np.uint8)
        print("%s: %d design points in %.1f s" % (name, len(tabs), time.time() - t0), flush=True)
    np.savez_compressed(out, **arrays)
    print("wrote", out)


if __name__ == "__main__":
    main()
