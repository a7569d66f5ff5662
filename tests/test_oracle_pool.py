"""The pooled oracle helper used by the full-size GPU tests gives exactly what
one oracle call over all groups gives (CPU only)."""

import numpy as np

from oracle import codec
import oracle_pool
import workloads as W


def test_pool_equals_one_call(monkeypatch):
    monkeypatch.setattr(oracle_pool, "CHUNK", 700)
    z = np.load(__file__.replace("test_oracle_pool.py", "golden/tables.npz"))
    tb = codec.Tables(z["c1_centroids"], z["c1_code_len"])
    x = W.c1_weight().numpy().reshape(-1, 128)[:2000]
    t = codec.tensor_scale(float(np.max(np.abs(x.astype(np.float32)))))[0]
    blocks, info = codec.encode_groups(x, tb, t, return_info=True)
    pb, clipped, stats = oracle_pool.encode(x, tb, t)
    assert np.array_equal(pb, blocks) and np.array_equal(clipped, info["clipped"]) and stats == info["stats"]
    y = codec.decode_blocks(blocks, tb, t)
    assert np.array_equal(oracle_pool.decode(blocks, tb, t).view(np.uint16), y.view(np.uint16))
