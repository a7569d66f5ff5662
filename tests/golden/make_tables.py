"""Write the pattern/codebook table sets used by the parity tests.

Calls only the oracle's training (``oracle.train.train_tables``) on seeded
calibration samples from ``workloads``; the GPU path never produces these.

    python tests/golden/make_tables.py            # writes tests/golden/tables.npz

Table sets (one per tensor type, each learned from a separate 2**20-value
sample with the tensor's own recipe):
  c1            1024x1024 N(0, 0.02) weight with Laplace outliers
  c2_<name>     the seven LLaMA-3-8B layer matrices (q k v o gate up down)
  c3_k, c3_v    KV cache head vectors (8192-vector samples); for these the
                per-tensor scale t is fixed from the sample (online codec) and
                stored as c3_<kind>_t
  c5_w1, c5_w2  70B-shaped FFN matrices
  act           LLaMA-3-8B hidden states in the 2x activation format (groups
                of 64; a 256-token sample); activations take their per-tensor
                scale from each tensor's own amax
"""

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads as W  # noqa: E402


def samples():
    yield "c1", W.c1_sample()
    for nm in W.LAYER_ORDER:
        yield "c2_" + nm, W.c2_sample(nm)
    for kind in ("k", "v"):
        yield "c3_" + kind, W.kv_sample(kind)
    for nm in ("w1", "w2"):
        yield "c5_" + nm, W.c5_sample(nm)
    yield "act", W.act_sample()


def main(out=os.path.join(HERE, "tables.npz"), only=None):
    arrays = {}
    if os.path.exists(out):
        arrays.update(dict(np.load(out)))
    for name, s in samples():
        if only and name not in only:
            continue
        t0 = time.time()
        x = s.numpy().reshape(-1)
        group = W.ACT_GROUP if name == "act" else W.GROUP
        tab = oracle.train.train_tables(x, seed=0, group=group)
        tab.check()
        arrays[name + "_centroids"] = tab.centroids
        arrays[name + "_code_len"] = tab.code_len
        if name.startswith("c3_"):
            t, _ = oracle.codec.tensor_scale(float(np.max(np.abs(x.astype(np.float32)))))
            arrays[name + "_t"] = np.float32(t)
        print("%-10s %d values  %.1fs" % (name, x.size, time.time() - t0), flush=True)
        np.savez(out, **arrays)


if __name__ == "__main__":
    main(only=set(sys.argv[1:]) or None)
