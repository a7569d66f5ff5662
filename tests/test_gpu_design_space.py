"""GPU parity at the S x H design points the v1 block can hold (S patterns in
{16, 32, 64}, H codebooks in {1, 2, 4}; Ecco review, "Assumptions & free
parameters": S and H chosen by design-space exploration; Fig. 5 caption).

Each point's tables (tests/golden/design_tables.npz, learned by the oracle)
are written into the block's 64 x 4 table slots by repetition
(oracle.study.v1_tables), so blocks carry p < S and h < H.  For the
1024x1024 weight, the LLaMA-3-8B gate projection, and the KV cache's K and
V (8,192 groups each): blocks, encode statistics and decoded FP16 values
bit for bit equal to the oracle's, and the pattern and codebook fields
inside the design point's range."""

import os
import sys

import numpy as np
import pytest

from oracle import codec, study
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ecco = pytest.importorskip("entropy_coded_group_amd")

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "design_tables.npz")


def say(msg):
    print("[gpu-design] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    name = torch.cuda.get_device_properties(0).gcnArchName
    if not name.startswith("gfx950"):
        pytest.skip("not gfx950: %s" % name)
    ecco.lib()
    return torch.device("cuda:0")


def workload(name):
    """(groups [8192, 128] FP16, per-tensor scale t)."""
    if name == "c1":
        x = W.c1_weight().numpy()
        return x.reshape(-1, 128), codec.tensor_scale(float(np.max(np.abs(x.astype(np.float32)))))[0]
    if name == "gate":
        x = W.c2_layer(0, names=["gate"])["gate"].numpy()
        t = codec.tensor_scale(float(np.max(np.abs(x.astype(np.float32)))))[0]
        return x.reshape(-1, 128)[:8192], t
    smp = W.kv_sample(name).numpy()
    t = codec.tensor_scale(float(np.max(np.abs(smp.astype(np.float32)))))[0]     # fixed ahead of time
    return W.kv_tensor(name, shape=(1, 8, 1024, 128)).numpy().reshape(-1, 128), t


@pytest.mark.parametrize("name", ["c1", "gate", "k", "v"])
def test_design_points_encode_decode_exact(dev, name):
    z = np.load(GOLD)
    x, t = workload(name)
    G = x.shape[0]
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    for S in (16, 32, 64):
        for H in (1, 2, 4):
            key = "%s_S%d_H%d" % (name, S, H)
            tb = study.v1_tables(z[key + "_centroids"], z[key + "_code_len"])
            tdev = ecco.tables_to_device(ecco.ecco_tables_build(tb.centroids, tb.code_len))
            bd = torch.full((G, 64), 0xAB, dtype=torch.uint8, device="cuda")
            st = torch.zeros(7, dtype=torch.int64, device="cuda")
            say("%s S=%d H=%d" % (name, S, H))
            ecco.ecco_encode(xd, 1, G, G * 128, G, tdev, t, bd, st)
            yd = torch.full((G, 128), 0x7FFF, dtype=torch.int16, device="cuda")
            ecco.ecco_decode(bd, 1, G, G, G * 128, tdev, t, yd)
            torch.cuda.synchronize()
            ob, info = codec.encode_groups(x, tb, t, return_info=True)
            gb = bd.cpu().numpy()
            bad = np.nonzero(np.any(gb != ob, axis=1))[0]
            assert bad.size == 0, "%s: %d blocks differ, first %d" % (key, bad.size, bad[0])
            assert dict(zip(ecco.STATS_FIELDS, st.cpu().tolist())) == info["stats"], key
            assert np.all((gb[:, 0] & 63) < S) and np.all((gb[:, 0] >> 6) < H), key
            y = yd.cpu().numpy().view(np.uint16)
            assert np.array_equal(y, codec.decode_blocks(ob, tb, t).view(np.uint16)), key
