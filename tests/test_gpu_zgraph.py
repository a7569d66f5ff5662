"""The codec calls under HIP graph capture: one step of a layer (amax of every
matrix, encode, decode, fused decode+GEMV at batch 1, through the _many entry
points) captured with torch.cuda.graph and replayed.  The library allocates
nothing, never synchronizes and clears its outputs with kernels, so a
captured step must give exactly the eager step's results.  Each replay runs
after eager work that overwrites every output, with synchronizations between;
the inputs are then changed in place and the replays must follow them."""

import os
import sys

import numpy as np
import pytest

from oracle import codec
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ecco = pytest.importorskip("entropy_coded_group_amd")

# (name of the golden tables, shape): rows of 8 blocks (one row per wave),
# 32 blocks (two rows per batch) and 16 blocks (four rows per batch)
MATS = [("c2_q", (512, 1024)), ("c2_k", (256, 4096)), ("c2_gate", (1024, 2048))]


def say(msg):
    print("[gpu-graph] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950"):
        pytest.skip("not gfx950")
    ecco.lib()
    return torch.device("cuda:0")


def test_layer_step_replays_like_eager(dev):
    z = np.load(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tables.npz"))
    m = []
    for k, (tname, shape) in enumerate(MATS):
        out_f, in_f = shape
        w = W.llama_matrix(shape, 700 + k).cuda()
        blob = ecco.ecco_tables_build(z[tname + "_centroids"], z[tname + "_code_len"])
        t = float(codec.tensor_scale(float(w.float().abs().max().item()))[0])
        m.append(dict(w=w, out_f=out_f, in_f=in_f, gpr=in_f // 128, t=t, tdev=ecco.tables_to_device(blob),
                      blocks=torch.empty((out_f, in_f // 128, 64), dtype=torch.uint8, device="cuda"),
                      y=torch.empty((out_f, in_f), dtype=torch.float16, device="cuda"),
                      x=torch.randn((1, in_f), generator=torch.Generator().manual_seed(710 + k)).half().cuda(),
                      gy=torch.empty((1, out_f), dtype=torch.float32, device="cuda")))
    amax = torch.empty(len(m), dtype=torch.float32, device="cuda")
    amax_jobs = [(d["w"], d["w"].numel(), amax[k:k + 1]) for k, d in enumerate(m)]
    enc_jobs = [(d["w"], d["out_f"], d["gpr"], d["in_f"], d["gpr"], d["tdev"], d["t"], d["blocks"], None) for d in m]
    dec_jobs = [(d["blocks"], d["out_f"], d["gpr"], d["gpr"], d["in_f"], d["tdev"], d["t"], d["y"]) for d in m]
    gemv_jobs = [(d["blocks"], d["tdev"], d["t"], d["out_f"], d["in_f"], d["x"], d["gy"]) for d in m]

    def step():
        ecco.ecco_amax_many(amax_jobs)
        ecco.ecco_encode_many(enc_jobs)
        ecco.ecco_decode_many(dec_jobs)
        ecco.ecco_decode_gemv_many(gemv_jobs, 1)

    def outputs():
        return [amax.clone()] + [d[k].clone() for d in m for k in ("blocks", "y", "gy")]

    def scribble():
        # eager work that overwrites every output before a replay
        amax.fill_(-1.0)
        for d in m:
            d["blocks"].fill_(0xA5)
            d["y"].fill_(3.0)
            d["gy"].fill_(float("nan"))

    def check(ref, what):
        got = outputs()
        for i, (a, b) in enumerate(zip(ref, got)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "%s: output %d differs" % (what, i)

    say("eager step")
    step()
    torch.cuda.synchronize()
    ref = outputs()
    # the amax outputs are the tensors' maxima (the scales above came from them)
    assert all(float(ref[0][k]) == float(d["w"].float().abs().max()) for k, d in enumerate(m))

    say("capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                        # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for r in range(3):
        say("replay %d" % r)
        scribble()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(ref, "replay %d" % r)

    say("inputs changed in place")
    for d in m:
        d["w"].neg_()
        d["x"].mul_(0.5)
    step()
    torch.cuda.synchronize()
    ref2 = outputs()
    assert not all(torch.equal(a, b) for a, b in zip(ref, ref2))
    for r in range(2):
        scribble()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(ref2, "replay %d after the input change" % r)
