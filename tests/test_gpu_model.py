"""GPU parity on the 32-layer LLaMA-3-8B-shaped weight set, as the benchmark
runs it: layers 0 and 31 drawn on the GPU (workloads.c4_matrix), each
matrix type's tables learned by ecco_train_patterns from its calibration
sample, the seven per-tensor scales from one ecco_amax_many call, the layer
encoded by one ecco_encode_many launch and decoded by one ecco_decode_many
launch into slices of one reused FP16 buffer.

Checked against the oracle: every block of the layer bit for bit (1.7 M
groups, the oracle's encode split over worker processes), the encode
statistics, and the decoded FP16 values of every group the oracle clips plus
every 97th group and the first and last 64 of each matrix.
"""

import sys

import numpy as np
import pytest

from oracle import codec
import oracle_pool
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ecco = pytest.importorskip("entropy_coded_group_amd")


def say(msg):
    print("[gpu-model] " + msg, flush=True)
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


@pytest.fixture(scope="module")
def tables(dev):
    out = {}
    for nm in W.LAYER_ORDER:
        blob = ecco.ecco_train_patterns(W.c2_sample(nm), threads=8)
        c, l = ecco.ecco_tables_get(blob)
        out[nm] = (codec.Tables(c, l), ecco.tables_to_device(blob))
    return out


def sample_index(G, stride=97):
    return np.unique(np.r_[np.arange(0, G, stride), np.arange(min(64, G)), np.arange(max(0, G - 64), G)])


@pytest.mark.parametrize("layer", [0, W.N_LAYERS - 1])
def test_model_layer_matches_oracle(dev, tables, layer):
    say("layer %d: generate on the device" % layer)
    mats = {nm: W.c4_matrix(layer, nm) for nm in W.LAYER_ORDER}
    amax = torch.full((len(mats),), -1.0, dtype=torch.float32, device="cuda")
    ecco.ecco_amax_many([(w, w.numel(), amax[i:i + 1]) for i, w in enumerate(mats.values())])
    torch.cuda.synchronize()
    host = {nm: w.cpu().numpy() for nm, w in mats.items()}
    for i, (nm, x) in enumerate(host.items()):
        assert amax[i].item() == np.max(np.abs(x.astype(np.float32))), nm
    ts = {nm: np.float32(ecco.ecco_tensor_scale_from_amax(amax[i].item())) for i, nm in enumerate(mats)}
    for nm in mats:
        assert ts[nm] == codec.tensor_scale(float(np.max(np.abs(host[nm].astype(np.float32)))))[0]
    blocks = {nm: torch.full((w.shape[0], w.shape[1] // 128, 64), 0xAB, dtype=torch.uint8, device="cuda")
              for nm, w in mats.items()}
    stats = torch.zeros((len(mats), 7), dtype=torch.int64, device="cuda")
    say("layer %d: encode (one launch), decode (one launch) into one reused buffer" % layer)
    ecco.ecco_encode_many([(w, w.shape[0], w.shape[1] // 128, w.shape[1], w.shape[1] // 128, tables[nm][1], ts[nm],
                            blocks[nm], stats[i]) for i, (nm, w) in enumerate(mats.items())])
    offs, o = {}, 0
    for nm, w in mats.items():
        offs[nm] = o
        o += w.numel()
    ybuf = torch.full((o,), 0x7FFF, dtype=torch.int16, device="cuda")
    ecco.ecco_decode_many([(blocks[nm], w.shape[0], w.shape[1] // 128, w.shape[1] // 128, w.shape[1],
                            tables[nm][1], ts[nm], ybuf[offs[nm]:]) for nm, w in mats.items()])
    torch.cuda.synchronize()
    gst = stats.cpu().numpy()
    yall = ybuf.cpu().numpy().view(np.float16)
    del mats, ybuf
    for i, (nm, x) in enumerate(host.items()):
        tb = tables[nm][0]
        xg = x.reshape(-1, 128)
        G = xg.shape[0]
        say("layer %d %s: oracle encode of %d groups" % (layer, nm, G))
        ob, clipped, ost = oracle_pool.encode(xg, tb, ts[nm])
        gb = blocks[nm].cpu().numpy().reshape(-1, 64)
        bad = np.nonzero(np.any(gb != ob, axis=1))[0]
        assert bad.size == 0, "layer %d %s: %d of %d blocks differ, first group %d" % (layer, nm, bad.size, G, bad[0])
        assert dict(zip(ecco.STATS_FIELDS, gst[i].tolist())) == ost, nm
        idx = np.union1d(sample_index(G), np.nonzero(clipped)[0])
        say("layer %d %s: oracle decode of %d groups (%d clipped)" % (layer, nm, idx.size, int(clipped.sum())))
        assert clipped.sum() > 0
        want = oracle_pool.decode(ob[idx], tb, ts[nm])
        got = yall[offs[nm]:offs[nm] + G * 128].reshape(G, 128)[idx]
        diff = np.nonzero(np.any(got.view(np.uint16) != want.view(np.uint16), axis=1))[0]
        assert diff.size == 0, "layer %d %s: %d decoded groups differ, first group %d" % (
            layer, nm, diff.size, idx[diff[0]])
