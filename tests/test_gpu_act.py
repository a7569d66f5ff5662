"""GPU parity of the 2x activation format (groups of 64 values, 14-bit outlier
records): ecco_encode_act / ecco_decode_act through the C ABI against the
oracle coder with group=64.

Bar: block bytes, encode statistics and decoded FP16 bits identical to the
oracle.  Small cases element by element (one group to several 64-block batches
with ragged tails, random and clipping tables, special groups, random blocks,
strided rows); the full 16384 x 4096 hidden-state tensor on a deterministic
sample of groups.
"""

import os
import sys

import numpy as np
import pytest

import oracle
from oracle import codec, huffman
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ecco = pytest.importorskip("entropy_coded_group_amd")

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tables.npz")
G64 = 64


def say(msg):
    print("[gpu-act] " + msg, flush=True)
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


def act_tables():
    z = np.load(GOLD)
    return codec.Tables(z["act_centroids"], z["act_code_len"])


def dev_tables(tb):
    return ecco.tables_to_device(ecco.ecco_tables_build(tb.centroids, tb.code_len))


def scale_of(x):
    return codec.tensor_scale(float(np.max(np.abs(np.asarray(x, np.float32)))))[0]


def random_tables(seed):
    rng = np.random.default_rng(seed)
    c = np.sort(rng.uniform(-1, 1, (64, 15)), axis=1).astype(np.float16).astype(np.float32)
    L = np.zeros((64, 4, 16), np.uint8)
    for p in range(64):
        for h in range(4):
            L[p, h] = huffman.limited_lengths(rng.integers(1, 300, 16) ** (1 + (h & 1)))
    return codec.Tables(c, L)


def clipping_tables(seed):
    """Symbol 7 coded in 8 bits by every codebook of every pattern (all patterns
    alike), so groups sitting at centroid 7 need more than 496 bits."""
    rng = np.random.default_rng(seed)
    c = np.tile(np.linspace(-1, 1, 15).astype(np.float16).astype(np.float32), (64, 1))
    L = np.zeros((64, 4, 16), np.uint8)
    for p in range(64):
        for h in range(4):
            order = [s for s in rng.permutation(16) if s != 7] + [7]
            rank = np.empty(16, np.int64)
            rank[order] = np.arange(16)
            L[p, h] = huffman.limited_lengths(2.0 ** (15 - rank))
    return codec.Tables(c, L)


def groups64(n, seed, kind):
    return W.random_groups((n + 1) // 2, seed, kind).numpy().reshape(-1, G64)[:n]


def gpu_encode(x, tdev, t, stats=False):
    G = x.shape[0]
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    bd = torch.full((G, 64), 0xAB, dtype=torch.uint8, device="cuda")
    sd = torch.zeros(7, dtype=torch.int64, device="cuda") if stats else None
    ecco.ecco_encode_act(xd, 1, G, G * G64, G, tdev, t, bd, sd)
    torch.cuda.synchronize()
    if stats:
        return bd.cpu().numpy(), dict(zip(ecco.STATS_FIELDS, sd.cpu().tolist()))
    return bd.cpu().numpy()


def gpu_decode(blocks, tdev, t):
    G = blocks.shape[0]
    bd = torch.from_numpy(np.ascontiguousarray(blocks)).cuda()
    yd = torch.full((G, G64), 0x7FFF, dtype=torch.int16, device="cuda")
    ecco.ecco_decode_act(bd, 1, G, G, G * G64, tdev, t, yd)
    torch.cuda.synchronize()
    return yd.cpu().numpy().view(np.float16)


def assert_fp16_equal(a, b, what):
    a = np.asarray(a, np.float16)
    b = np.asarray(b, np.float16)
    na, nb = np.isnan(a), np.isnan(b)
    assert np.array_equal(na, nb), "%s: NaN positions differ" % what
    ua, ub = a.view(np.uint16)[~na], b.view(np.uint16)[~nb]
    bad = np.nonzero(ua != ub)[0]
    assert bad.size == 0, "%s: %d mismatches, first at flat index %d: gpu %04x oracle %04x" % (
        what, bad.size, bad[0], ua[bad[0]], ub[bad[0]])


def assert_blocks_equal(g, o, what):
    bad = np.nonzero(np.any(g != o, axis=1))[0]
    assert bad.size == 0, "%s: %d of %d blocks differ, first group %d\n gpu %s\n ora %s" % (
        what, bad.size, g.shape[0], bad[0], g[bad[0]].tobytes().hex(), o[bad[0]].tobytes().hex())


def check_roundtrip(x, tb, t, what, min_clipped=None):
    tdev = dev_tables(tb)
    g_blocks, g_stats = gpu_encode(x, tdev, t, stats=True)
    o_blocks, info = codec.encode_groups(x, tb, t, return_info=True, group=G64)
    if min_clipped is not None:
        assert info["clipped"].mean() >= min_clipped
    assert_blocks_equal(g_blocks, o_blocks, what + " encode")
    assert g_stats == info["stats"], what
    assert_fp16_equal(gpu_decode(o_blocks, tdev, t), codec.decode_blocks(o_blocks, tb, t, group=G64),
                      what + " decode")


def test_act_hidden_states_exact(dev):
    tb = act_tables()
    x = W.act_tensor((256, 4096), seed=620).numpy().reshape(-1, G64)     # 16384 groups
    t = scale_of(x)
    say("act hidden states 16384 groups")
    check_roundtrip(x, tb, t, "hidden states")


@pytest.mark.parametrize("kind,seed,n", [("normal", 1, 1), ("normal", 2, 63), ("laplace", 3, 64),
                                         ("wide", 4, 65), ("normal", 5, 129), ("laplace", 6, 1000),
                                         ("wide", 7, 4097)])
def test_act_random_groups_random_tables(dev, kind, seed, n):
    tb = random_tables(100 + seed)
    x = groups64(n, 110 + seed, kind)
    say("act random %s n=%d" % (kind, n))
    check_roundtrip(x, tb, scale_of(x), "random %s %d" % (kind, n))


def test_act_clipped_groups(dev):
    tb = clipping_tables(7)
    rng = np.random.default_rng(8)
    n = 700
    amp = rng.uniform(0.5, 2.0, (n, 1))
    x = tb.centroids[0, 7] * amp * (1.0 + rng.uniform(-0.02, 0.02, (n, G64)))
    x[:, 5] = amp[:, 0]                                    # the scale element
    x = np.concatenate([x.astype(np.float16), groups64(300, 9, "normal")])
    say("act clipping tables, 1000 groups")
    check_roundtrip(x, tb, scale_of(x), "clipped", min_clipped=0.5)


def test_act_repeated_pattern_tables(dev):
    base = random_tables(130)
    tb = codec.Tables(base.centroids[np.arange(64) % 16], base.code_len)
    x = groups64(2000, 131, "laplace")
    say("act 16 distinct patterns")
    check_roundtrip(x, tb, scale_of(x), "16 patterns")


def test_act_special_groups(dev):
    tb = act_tables()
    c = tb.centroids[9]
    rows = [np.zeros(64), np.full(64, 0.25), np.full(64, -3.0), np.r_[1.0, np.resize(c, 63)],
            np.r_[-1.0, np.resize(c[::-1], 63)], np.linspace(-1, 1, 64), np.r_[np.zeros(63), 5e-6],
            np.r_[65504.0, np.zeros(63)], np.r_[np.full(32, 1e-7), np.full(32, -1e-7)]]
    x = np.array(rows, dtype=np.float16)
    tdev = dev_tables(tb)
    for t in (np.float32(1.0), scale_of(x), np.float32(1e-3)):
        say("act special groups t=%g" % t)
        o_blocks = codec.encode_groups(x, tb, t, group=G64)
        assert_blocks_equal(gpu_encode(x, tdev, t), o_blocks, "special encode t=%g" % t)
        assert_fp16_equal(gpu_decode(o_blocks, tdev, t), codec.decode_blocks(o_blocks, tb, t, group=G64),
                          "special decode t=%g" % t)


def incomplete_act_tables(seed):
    """The activation tables with one to three codewords of each book made
    one or two bits longer (at most 8): Kraft sums below 1, so random bits
    often start with no codeword, where decoding stops."""
    tb = act_tables()
    rng = np.random.default_rng(seed)
    L = tb.code_len.copy()
    for p in range(64):
        for h in range(4):
            for s in rng.choice(16, int(rng.integers(1, 4)), replace=False):
                L[p, h, s] = min(8, int(L[p, h, s]) + int(rng.integers(1, 3)))
    return codec.Tables(tb.centroids, L)


def test_act_fuzz_decode_random_blocks(dev):
    for name, tb in (("act", act_tables()), ("clipping", clipping_tables(3)), ("incomplete", incomplete_act_tables(4))):
        tdev = dev_tables(tb)
        blocks = W.random_blocks(40000, 140).numpy()
        for t in (np.float32(1.0), np.float32(0.0173)):
            say("act fuzz decode %s t=%g" % (name, t))
            assert_fp16_equal(gpu_decode(blocks, tdev, t), codec.decode_blocks(blocks, tb, t, group=G64),
                              "fuzz %s t=%g" % (name, t))


def test_act_strided_rows(dev):
    """Rows of a wider buffer: x and y row strides beyond the row, blocks with
    a row stride beyond the groups per row; nothing outside is touched."""
    tb = act_tables()
    tdev = dev_tables(tb)
    rows, gpr, xs, bs = 37, 11, 11 * 64 + 40, 13
    x = W.act_tensor((rows, 1024), seed=150).numpy()[:, :xs]
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    t = scale_of(x[:, :gpr * 64])
    say("act strided encode")
    bd = torch.full((rows, bs, 64), 0xAB, dtype=torch.uint8, device="cuda")
    ecco.ecco_encode_act(xd, rows, gpr, xs, bs, tdev, t, bd)
    torch.cuda.synchronize()
    gb = bd.cpu().numpy()
    ob = codec.encode_groups(x[:, :gpr * 64].reshape(-1, G64), tb, t, group=G64)
    assert_blocks_equal(gb[:, :gpr].reshape(-1, 64), ob, "strided encode")
    assert np.all(gb[:, gpr:] == 0xAB)
    say("act strided decode")
    ys = gpr * 64 + 24
    yd = torch.full((rows, ys), 0x7FFF, dtype=torch.int16, device="cuda")
    ecco.ecco_decode_act(bd, rows, gpr, bs, ys, tdev, t, yd)
    torch.cuda.synchronize()
    gy = yd.cpu().numpy()
    assert_fp16_equal(gy[:, :gpr * 64].view(np.float16).reshape(-1, G64),
                      codec.decode_blocks(ob, tb, t, group=G64), "strided decode")
    assert np.all(gy[:, gpr * 64:] == 0x7FFF)


def test_act_full_size_sampled(dev):
    """The 16384 x 4096 hidden-state tensor (1,048,576 groups) as the bench
    runs it: amax, encode and decode on the GPU; every 97th group against the
    oracle."""
    tb = act_tables()
    tdev = dev_tables(tb)
    T, D = W.ACT_SHAPE
    say("act full size: generate %dx%d" % (T, D))
    x = W.act_tensor()
    xd = x.cuda()
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    ecco.ecco_amax(xd, xd.numel(), amax)
    torch.cuda.synchronize()
    xn = x.numpy().reshape(-1, G64)
    assert amax.item() == np.max(np.abs(xn.astype(np.float32)))
    t = np.float32(ecco.ecco_tensor_scale_from_amax(amax.item()))
    assert t == scale_of(xn)
    G = xn.shape[0]
    say("act full size: encode + decode %d groups" % G)
    bd = torch.empty((G, 64), dtype=torch.uint8, device="cuda")
    ecco.ecco_encode_act(xd, 1, G, G * G64, G, tdev, t, bd)
    yd = torch.empty((T, D), dtype=torch.float16, device="cuda")
    ecco.ecco_decode_act(bd, 1, G, G, G * G64, tdev, t, yd)
    torch.cuda.synchronize()
    idx = np.arange(0, G, 97)
    idx = np.unique(np.r_[idx, G - 1])
    gb = bd.cpu().numpy()[idx]
    ob = codec.encode_groups(xn[idx], tb, t, group=G64)
    assert_blocks_equal(gb, ob, "full-size encode (sampled)")
    gy = yd.cpu().numpy().reshape(-1, G64)[idx]
    assert_fp16_equal(gy, codec.decode_blocks(ob, tb, t, group=G64), "full-size decode (sampled)")


def test_act_pattern_choice_near_bisectors(dev):
    """64-value groups whose (min, max) lie on the bisector of two patterns'
    end centroids (in units of a), where the binary32 fitness decides: the
    encoder tries only the pattern grid's candidates for these, and its blocks
    must equal the oracle's (trained and random tables)."""
    rng = np.random.default_rng(47)
    for name, tb in (("trained", act_tables()), ("random", random_tables(49))):
        c0, c14 = tb.centroids[:, 0].astype(np.float64), tb.centroids[:, 14].astype(np.float64)
        rows = []
        for a in (1.0, 0.0625, 4.0):
            for _ in range(400):
                p, q = rng.choice(64, 2, replace=False)
                mid = np.array([c0[p] + c0[q], c14[p] + c14[q]]) / 2
                dirn = np.array([-(c14[q] - c14[p]), c0[q] - c0[p]])
                lo, hi = sorted(mid + rng.uniform(-0.2, 0.2) * dirn)
                lo, hi = max(lo, -0.99), min(hi, 0.99)
                body = np.r_[lo, hi, rng.uniform(lo, hi, G64 - 3)] * a
                sign = a if rng.random() < 0.5 else -a
                rows.append(np.r_[sign, body])
        x = np.array(rows, dtype=np.float16)
        say("act bisector groups, %s tables, %d groups" % (name, len(x)))
        check_roundtrip(x, tb, np.float32(1.0), "act bisectors, %s" % name)
