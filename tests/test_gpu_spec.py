"""GPU parity of the speculative decoders (ecco_decode_speculative, the pages'
segment-parallel method on one wavefront per block, and ecco_decode_segmented
with 2, 4 and 8 lanes per block) against the oracle and against ecco_decode:
decoded FP16 bits identical.  Cases: the 1024x1024 weight
matrix, random and clipping tables over ragged sizes, special groups, 40,000
random blocks (invalid windows, clipping, NaN scale bytes), strided rows."""

import os
import sys

import numpy as np
import pytest

import oracle
from oracle import codec
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ecco = pytest.importorskip("entropy_coded_group_amd")

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tables.npz")


def say(msg):
    print("[gpu-spec] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950"):
        pytest.skip("not gfx950")
    ecco.lib()
    return torch.device("cuda:0")


def golden(name):
    z = np.load(GOLD)
    return codec.Tables(z[name + "_centroids"], z[name + "_code_len"])


def dev_tables(tb):
    return ecco.tables_to_device(ecco.ecco_tables_build(tb.centroids, tb.code_len))


def scale_of(x):
    return codec.tensor_scale(float(np.max(np.abs(np.asarray(x, np.float32)))))[0]


def random_tables(seed, adversarial=False):
    rng = np.random.default_rng(seed)
    c = np.sort(rng.uniform(-1, 1, (64, 15)), axis=1).astype(np.float16).astype(np.float32)
    if adversarial:
        base = np.array([2, 3, 4, 5, 6, 7, 8, 8] + [4] * 8, np.uint8)
        L = np.stack([np.stack([rng.permutation(base) for _ in range(4)]) for _ in range(64)])
    else:
        L = np.zeros((64, 4, 16), np.uint8)
        for p in range(64):
            for h in range(4):
                L[p, h] = oracle.huffman.limited_lengths(rng.integers(1, 300, 16) ** (1 + (h & 1)))
    return codec.Tables(c, L)


def incomplete_tables(seed):
    """Random lengths with one to three codewords per book made one or two
    bits longer (at most 8): Kraft sums below 1, so random bits often start
    with no codeword, where decoding stops."""
    tb = random_tables(seed, adversarial=True)
    rng = np.random.default_rng(seed + 1)
    L = tb.code_len.copy()
    for p in range(64):
        for h in range(4):
            for s in rng.choice(16, int(rng.integers(1, 4)), replace=False):
                L[p, h, s] = min(8, int(L[p, h, s]) + int(rng.integers(1, 3)))
    return codec.Tables(tb.centroids, L)


SEG_LANES = (2, 4, 8)


def spec_decode(bd, n_rows, gpr, bs, ys, tdev, t, y, lanes):
    """lanes 64: ecco_decode_speculative; 2, 4, 8: ecco_decode_segmented."""
    if lanes == 64:
        ecco.ecco_decode_speculative(bd, n_rows, gpr, bs, ys, tdev, t, y)
    else:
        ecco.ecco_decode_segmented(bd, n_rows, gpr, bs, ys, tdev, t, y, lanes)


def both_decodes(blocks, tdev, t, lanes=64):
    G = blocks.shape[0]
    bd = torch.from_numpy(np.ascontiguousarray(blocks)).cuda()
    ys = torch.full((G, 128), 0x7FFF, dtype=torch.int16, device="cuda")
    yl = torch.full((G, 128), 0x7FFF, dtype=torch.int16, device="cuda")
    spec_decode(bd, 1, G, G, G * 128, tdev, t, ys, lanes)
    ecco.ecco_decode(bd, 1, G, G, G * 128, tdev, t, yl)
    torch.cuda.synchronize()
    return ys.cpu().numpy().view(np.float16), yl.cpu().numpy().view(np.float16)


def assert_fp16_equal(a, b, what):
    a = np.asarray(a, np.float16)
    b = np.asarray(b, np.float16)
    na, nb = np.isnan(a), np.isnan(b)
    assert np.array_equal(na, nb), "%s: NaN positions differ" % what
    ua, ub = a.view(np.uint16)[~na], b.view(np.uint16)[~nb]
    bad = np.nonzero(ua != ub)[0]
    assert bad.size == 0, "%s: %d mismatches, first at flat index %d: gpu %04x oracle %04x" % (
        what, bad.size, bad[0], ua[bad[0]], ub[bad[0]])


def check(blocks, tb, t, what):
    tdev = dev_tables(tb)
    ref = codec.decode_blocks(blocks, tb, t)
    for lanes in (64,) + SEG_LANES:
        say("  %d lanes per block" % lanes)
        ys, yl = both_decodes(blocks, tdev, t, lanes)
        assert_fp16_equal(ys, ref, "%s, %d lanes per block, vs oracle" % (what, lanes))
        assert_fp16_equal(ys, yl, "%s, %d lanes per block, vs ecco_decode" % (what, lanes))


def test_spec_c1_weight(dev):
    tb = golden("c1")
    x = W.c1_weight().numpy().reshape(-1, 128)
    t = scale_of(x)
    say("speculative decode, 8192 groups")
    check(codec.encode_groups(x, tb, t), tb, t, "c1")


@pytest.mark.parametrize("adv,seed,n", [(False, 1, 1), (False, 2, 63), (True, 3, 65), (True, 4, 1000),
                                        (False, 5, 4097)])
def test_spec_random_tables(dev, adv, seed, n):
    tb = random_tables(700 + seed, adversarial=adv)
    x = W.random_groups(n, 710 + seed, ("normal", "laplace", "wide")[seed % 3]).numpy()
    t = scale_of(x)
    blocks, info = codec.encode_groups(x, tb, t, return_info=True)
    if adv:
        assert info["clipped"].any()
    say("speculative decode, random tables n=%d adversarial=%s" % (n, adv))
    check(blocks, tb, t, "random %d" % n)


def test_spec_special_groups(dev):
    tb = golden("c1")
    c = tb.centroids[9]
    rows = [np.zeros(128), np.full(128, 0.25), np.full(128, -3.0), np.r_[1.0, np.resize(c, 127)],
            np.linspace(-1, 1, 128), np.r_[np.zeros(127), 5e-6], np.r_[65504.0, np.zeros(127)]]
    x = np.array(rows, dtype=np.float16)
    for t in (np.float32(1.0), scale_of(x), np.float32(1e-3)):
        say("speculative decode, special groups t=%g" % t)
        check(codec.encode_groups(x, tb, t), tb, t, "special t=%g" % t)


def test_spec_random_blocks(dev):
    for name, tb in (("c1", golden("c1")), ("adversarial", random_tables(720, adversarial=True)),
                     ("incomplete", incomplete_tables(722))):
        blocks = W.random_blocks(40000, 721).numpy()
        for t in (np.float32(1.0), np.float32(0.0173)):
            say("speculative decode, random blocks %s t=%g" % (name, t))
            check(blocks, tb, t, "fuzz %s t=%g" % (name, t))


@pytest.mark.parametrize("lanes", (64,) + SEG_LANES)
def test_spec_strided_rows(dev, lanes):
    tb = golden("c1")
    tdev = dev_tables(tb)
    rows, gpr, bs, ys = 3, 50, 53, 50 * 128 + 40
    x = W.random_groups(rows * gpr, 730, "laplace").numpy()
    t = scale_of(x)
    ob = codec.encode_groups(x, tb, t)
    bfull = np.zeros((rows, bs, 64), np.uint8)
    bfull[:, :gpr] = ob.reshape(rows, gpr, 64)
    bd = torch.from_numpy(bfull).cuda()
    yd = torch.full((rows, ys), 0x7FFF, dtype=torch.int16, device="cuda")
    say("speculative decode, strided rows, %d lanes per block" % lanes)
    spec_decode(bd, rows, gpr, bs, ys, tdev, t, yd, lanes)
    torch.cuda.synchronize()
    got = yd.cpu().numpy()
    assert_fp16_equal(got[:, :gpr * 128].view(np.float16).reshape(-1, 128), codec.decode_blocks(ob, tb, t),
                      "strided")
    assert np.all(got[:, gpr * 128:] == 0x7FFF)
