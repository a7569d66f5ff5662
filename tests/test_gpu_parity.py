"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: block bytes and decoded FP16 bits identical to the oracle (NaN compared
as NaN: only garbage blocks produce it), encode statistics identical, and the
fused decode+GEMV within |y - y_ref| <= 1e-3 * max(|y_ref|, sum|w x| / sqrt(in))
of a float64 GEMV over oracle-decoded weights.  Small cases are compared
element by element over several tiles and ragged tails; the full-size
workloads (a LLaMA-3-8B layer's matrices, a 16x8x8192x128 KV cache, 70B FFN
matrices) have every block compared (the oracle's encode split over worker
processes), and their decoded values on a deterministic sample of groups
plus every group the oracle clips; the fused GEMV on sampled rows plus the
rows holding the most clipped groups.
"""

import os
import sys

import numpy as np
import pytest

import oracle
from oracle import codec, gemv as ogemv
import oracle_pool
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ecco = pytest.importorskip("entropy_coded_group_amd")

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tables.npz")


def say(msg):
    print("[gpu-parity] " + msg, flush=True)
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


def golden(name):
    z = np.load(GOLD)
    return codec.Tables(z[name + "_centroids"], z[name + "_code_len"])


def golden_t(name):
    return np.float32(np.load(GOLD)[name + "_t"])


def dev_tables(tb):
    return ecco.tables_to_device(ecco.ecco_tables_build(tb.centroids, tb.code_len))


def scale_of(x):
    return codec.tensor_scale(float(np.max(np.abs(np.asarray(x, np.float32)))))[0]


def gpu_encode(x_groups, tdev, t, stats=False):
    """x_groups: [G, 128] float16 (numpy) -> blocks [G, 64] uint8 (numpy)."""
    G = x_groups.shape[0]
    xd = torch.from_numpy(np.ascontiguousarray(x_groups)).cuda()
    bd = torch.full((G, 64), 0xAB, dtype=torch.uint8, device="cuda")
    sd = torch.zeros(7, dtype=torch.int64, device="cuda") if stats else None
    ecco.ecco_encode(xd, 1, G, G * 128, G, tdev, t, bd, sd)
    torch.cuda.synchronize()
    if stats:
        return bd.cpu().numpy(), dict(zip(ecco.STATS_FIELDS, sd.cpu().tolist()))
    return bd.cpu().numpy()


def gpu_decode(blocks, tdev, t):
    G = blocks.shape[0]
    bd = torch.from_numpy(np.ascontiguousarray(blocks)).cuda()
    yd = torch.full((G, 128), 0x7FFF, dtype=torch.int16, device="cuda")
    ecco.ecco_decode(bd, 1, G, G, G * 128, tdev, t, yd)
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


def adversarial_tables(seed):
    """Complete codes whose lengths are assigned at random: long codes for common
    symbols, so many groups clip."""
    rng = np.random.default_rng(seed)
    base = np.array([2, 3, 4, 5, 6, 7, 8, 8] + [4] * 8, np.uint8)
    L = np.stack([np.stack([rng.permutation(base) for _ in range(4)]) for _ in range(64)])
    c = np.sort(rng.uniform(-1, 1, (64, 15)), axis=1).astype(np.float16).astype(np.float32)
    return codec.Tables(c, L)


def incomplete_tables(seed, base=None):
    """Codebooks with Kraft sum below 1: one to three codewords of each book
    made one or two bits longer (at most 8), so random bits often start with
    no codeword, where decoding stops.  Books whose lengthened codewords were
    all 8 bits already stay complete."""
    tb = base if base is not None else adversarial_tables(seed)
    rng = np.random.default_rng(seed + 1000)
    L = tb.code_len.copy()
    for p in range(64):
        for h in range(4):
            for s in rng.choice(16, int(rng.integers(1, 4)), replace=False):
                L[p, h, s] = min(8, int(L[p, h, s]) + int(rng.integers(1, 3)))
    out = codec.Tables(tb.centroids, L)
    ks = [oracle.huffman.kraft_sum(L[p, h]) for p in range(64) for h in range(4)]
    assert max(ks) <= 1 and sum(k < 1 for k in ks) > 200
    return out


def random_tables(seed):
    rng = np.random.default_rng(seed)
    c = np.sort(rng.uniform(-1, 1, (64, 15)), axis=1).astype(np.float16).astype(np.float32)
    L = np.zeros((64, 4, 16), np.uint8)
    for p in range(64):
        for h in range(4):
            L[p, h] = oracle.huffman.limited_lengths(rng.integers(1, 300, 16) ** (1 + (h & 1)))
    return codec.Tables(c, L)


# ------------------------------------------------------------------ small, exact

def test_amax_and_tensor_scale(dev):
    x = W.c1_weight()
    say("amax c1")
    out = torch.zeros(1, dtype=torch.float32, device="cuda")
    xd = x.cuda()
    ecco.ecco_amax(xd, xd.numel(), out)
    torch.cuda.synchronize()
    ref = np.max(np.abs(x.numpy().astype(np.float32)))
    assert out.item() == ref
    assert np.float32(ecco.ecco_tensor_scale_from_amax(out.item())) == scale_of(x.numpy())
    for n in (1, 7, 8, 9, 1000, 4099):                    # tails of the vector loop
        y = W.random_groups(40, n, "wide").numpy().ravel()[:n].copy()
        yd = torch.from_numpy(y).cuda()
        ecco.ecco_amax(yd, n, out)
        torch.cuda.synchronize()
        assert out.item() == np.max(np.abs(y.astype(np.float32))), n


def test_amax_many_matches_one_call_per_tensor(dev):
    """ecco_amax_many: sixteen tensors of ragged sizes (1 value to 2^20 + 3)
    in one call, outputs pre-filled with garbage, one tensor with NaNs (ignored)
    and one whose extreme is negative; then a second, smaller call in which two
    jobs share an output (it gets the maximum over both)."""
    say("amax_many 16 jobs")
    rng = np.random.default_rng(41)
    sizes = [1, 7, 8, 9, 1000, 4099, 65536, 1 << 20, (1 << 20) + 3, 12345, 777, 3, 2048, 100003, 64, 5]
    xs = []
    for k, n in enumerate(sizes):
        y = (rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 2)).astype(np.float16)
        if k == 4:
            y[[3, 500]] = np.float16("nan")
        if k == 5:
            y[77] = -np.abs(y).max() * 2
        xs.append(y)
    xd = [torch.from_numpy(y).cuda() for y in xs]
    out = torch.full((16,), 1e30, dtype=torch.float32, device="cuda")
    ecco.ecco_amax_many([(xd[k], sizes[k], out[k:k + 1]) for k in range(16)])
    one = torch.full((16,), -1.0, dtype=torch.float32, device="cuda")
    for k in range(16):
        ecco.ecco_amax(xd[k], sizes[k], one[k:k + 1])
    torch.cuda.synchronize()
    ref = np.array([np.nanmax(np.abs(y.astype(np.float32))) for y in xs], np.float32)
    assert np.array_equal(out.cpu().numpy(), ref)
    assert np.array_equal(one.cpu().numpy(), ref)
    # second call: fewer jobs, jobs 0 and 2 share out[0]
    out2 = torch.full((2,), 1e30, dtype=torch.float32, device="cuda")
    ecco.ecco_amax_many([(xd[7], sizes[7], out2[0:1]), (xd[9], sizes[9], out2[1:2]), (xd[13], sizes[13], out2[0:1])])
    torch.cuda.synchronize()
    assert out2[0].item() == max(ref[7], ref[13]) and out2[1].item() == ref[9]


def test_c1_encode_decode_bitexact(dev):
    tb = golden("c1")
    tdev = dev_tables(tb)
    x = W.c1_weight().numpy().reshape(-1, 128)
    t = scale_of(x)
    say("c1 encode 8192 groups")
    g_blocks, g_stats = gpu_encode(x, tdev, t, stats=True)
    o_blocks, info = codec.encode_groups(x, tb, t, return_info=True)
    assert_blocks_equal(g_blocks, o_blocks, "c1 encode")
    assert g_stats == info["stats"]
    say("c1 decode 8192 groups")
    assert_fp16_equal(gpu_decode(o_blocks, tdev, t), codec.decode_blocks(o_blocks, tb, t), "c1 decode")


@pytest.mark.parametrize("kind,seed,n", [("normal", 1, 1), ("normal", 2, 63), ("laplace", 3, 64),
                                         ("wide", 4, 65), ("normal", 5, 129), ("laplace", 6, 1000),
                                         ("wide", 7, 4097), ("ties", 8, 2051), ("ties", 9, 17)])
def test_random_groups_random_tables(dev, kind, seed, n):
    tb = random_tables(seed)
    tdev = dev_tables(tb)
    x = W.random_groups(n, seed, kind).numpy()
    t = scale_of(x)
    say("random %s n=%d" % (kind, n))
    g_blocks, g_stats = gpu_encode(x, tdev, t, stats=True)
    o_blocks, info = codec.encode_groups(x, tb, t, return_info=True)
    assert_blocks_equal(g_blocks, o_blocks, "encode %s %d" % (kind, n))
    assert g_stats == info["stats"]
    assert_fp16_equal(gpu_decode(o_blocks, tdev, t), codec.decode_blocks(o_blocks, tb, t), "decode")


@pytest.mark.parametrize("distinct", [16, 32])
def test_repeated_pattern_tables_encode_exact(dev, distinct):
    """Tables whose 64 slots repeat 16 or 32 patterns: the encoder searches only
    the distinct ones and must still give the oracle's blocks (which search
    all 64)."""
    base = random_tables(50 + distinct)
    tb = codec.Tables(base.centroids[np.arange(64) % distinct], base.code_len)
    tdev = dev_tables(tb)
    x = np.concatenate([W.random_groups(1500, 51, "normal").numpy(), W.random_groups(500, 52, "laplace").numpy()])
    t = scale_of(x)
    say("repeated patterns %d" % distinct)
    g_blocks, g_stats = gpu_encode(x, tdev, t, stats=True)
    o_blocks, info = codec.encode_groups(x, tb, t, return_info=True)
    assert info["p"].max() < distinct
    assert_blocks_equal(g_blocks, o_blocks, "encode, %d distinct patterns" % distinct)
    assert g_stats == info["stats"]


def test_heavily_clipped_groups(dev):
    tb = adversarial_tables(11)
    tdev = dev_tables(tb)
    x = np.concatenate([W.random_groups(700, 12, "normal").numpy(), W.random_groups(300, 13, "wide").numpy()])
    t = scale_of(x)
    say("clipping tables, 1000 groups")
    g_blocks, g_stats = gpu_encode(x, tdev, t, stats=True)
    o_blocks, info = codec.encode_groups(x, tb, t, return_info=True)
    assert info["clipped"].mean() > 0.3
    assert_blocks_equal(g_blocks, o_blocks, "clipped encode")
    assert g_stats == info["stats"]
    assert_fp16_equal(gpu_decode(o_blocks, tdev, t), codec.decode_blocks(o_blocks, tb, t), "clipped decode")


def test_special_groups(dev):
    tb = golden("c1")
    tdev = dev_tables(tb)
    c = tb.centroids[9]
    rows = [np.zeros(128), np.full(128, 0.25), np.full(128, -3.0), np.r_[1.0, np.resize(c, 127)],
            np.r_[-1.0, np.resize(c[::-1], 127)], np.linspace(-1, 1, 128), np.r_[np.zeros(127), 5e-6],
            np.r_[65504.0, np.zeros(127)], np.r_[np.full(64, 1e-7), np.full(64, -1e-7)]]
    x = np.array(rows, dtype=np.float16)
    for t in (np.float32(1.0), scale_of(x), np.float32(1e-3)):
        say("special groups t=%g" % t)
        g_blocks = gpu_encode(x, tdev, t)
        o_blocks = codec.encode_groups(x, tb, t)
        assert_blocks_equal(g_blocks, o_blocks, "special encode t=%g" % t)
        assert_fp16_equal(gpu_decode(o_blocks, tdev, t), codec.decode_blocks(o_blocks, tb, t), "special decode")


QBINS_OK_AT = 108800        # byte offset of the blob's quantiser-bins flag (Tables::qbins_ok)


def _near_threshold_groups(tb, scales, rng):
    """Groups whose values sit on the quantiser's thresholds m_k * a and on
    their FP16 neighbours: value 0 is the scale element +-a (an exact FP8
    value, t = 1), values 1 and 2 are pattern p's end centroids times a (so
    that p is the pattern chosen), the rest FP16 values at, just above and
    just below each threshold, in a shuffled order."""
    rows = []
    mids = tb.midpoints()
    for a in scales:
        for p in rng.choice(64, 16, replace=False):
            thr = (mids[p] * np.float32(a)).astype(np.float32)
            near = []
            for tk in thr:
                h = np.float16(tk)
                near += [h, np.nextafter(h, np.float16(np.inf)), np.nextafter(h, np.float16(-np.inf))]
            body = np.resize(np.array(near, np.float16), 125)
            rng.shuffle(body)
            ends = (tb.centroids[p, [0, 14]] * np.float32(a)).astype(np.float16)
            sign = np.float16(a) if rng.random() < 0.5 else -np.float16(a)
            rows.append(np.r_[sign, ends, body].astype(np.float16))
    return np.array(rows, np.float16)


def test_quantiser_bins_at_thresholds(dev):
    """Values on and beside every threshold, through the binned quantiser
    (trained tables have bins) and through the threshold tree (tables whose
    crowded midpoints leave them without bins): blocks equal the oracle's."""
    rng = np.random.default_rng(23)
    tb = golden("c1")
    assert ecco.ecco_tables_build(tb.centroids, tb.code_len)[QBINS_OK_AT] == 1          # bins on
    crowded = codec.Tables(tb.centroids.copy(), tb.code_len)
    crowded.centroids[3, 5] = crowded.centroids[3, 6] = crowded.centroids[3, 7]
    assert ecco.ecco_tables_build(crowded.centroids, crowded.code_len)[QBINS_OK_AT] == 0  # bins off
    scales = (1.0, 0.0625, 4.0, 448.0, 2.0 ** -9)       # exact FP8 values: a = |x_0| with t = 1
    for name, tables in (("bins", tb), ("tree", crowded)):
        tdev = dev_tables(tables)
        x = _near_threshold_groups(tables, scales, rng)
        t = np.float32(1.0)
        say("threshold groups, %s, %d groups" % (name, len(x)))
        g_blocks, g_stats = gpu_encode(x, tdev, t, stats=True)
        o_blocks, info = codec.encode_groups(x, tables, t, return_info=True)
        assert_blocks_equal(g_blocks, o_blocks, "threshold groups, %s" % name)
        assert g_stats == info["stats"]


def test_pattern_choice_near_bisectors(dev):
    """Groups whose (min, max) lie on the bisector of two patterns' end
    centroids (in units of a), where the binary32 fitness decides: blocks
    equal the oracle's whether the grid's candidates or the full search
    choose (random tables, golden tables)."""
    rng = np.random.default_rng(41)
    for name, tb in (("golden", golden("c1")), ("random", random_tables(43))):
        tdev = dev_tables(tb)
        c0, c14 = tb.centroids[:, 0].astype(np.float64), tb.centroids[:, 14].astype(np.float64)
        rows = []
        for a in (1.0, 0.0625, 4.0):
            for _ in range(300):
                p, q = rng.choice(64, 2, replace=False)
                mid = np.array([c0[p] + c0[q], c14[p] + c14[q]]) / 2
                dirn = np.array([-(c14[q] - c14[p]), c0[q] - c0[p]])
                lo, hi = sorted(mid + rng.uniform(-0.2, 0.2) * dirn)
                lo, hi = max(lo, -0.99), min(hi, 0.99)
                body = np.r_[lo, hi, rng.uniform(lo, hi, 125)] * a
                sign = a if rng.random() < 0.5 else -a
                rows.append(np.r_[sign, body])
        x = np.array(rows, dtype=np.float16)
        t = np.float32(1.0)
        say("bisector groups, %s tables, %d groups" % (name, len(x)))
        g_blocks, g_stats = gpu_encode(x, tdev, t, stats=True)
        o_blocks, info = codec.encode_groups(x, tb, t, return_info=True)
        assert_blocks_equal(g_blocks, o_blocks, "bisector groups, %s" % name)
        assert g_stats == info["stats"]


def test_nonfinite_groups_counted_and_contained(dev):
    """Groups holding NaN or +-Inf: their blocks are unspecified, but the
    launch completes, the statistics count them as the oracle does, every
    finite group of the same launch is still bit-exact, and every block
    decodes."""
    tb = golden("c1")
    tdev = dev_tables(tb)
    x = W.random_groups(600, 12, "normal").numpy()
    bad = np.arange(3, 600, 37)
    for i, g in enumerate(bad):
        x[g, (i * 13) % 128] = (np.float16("nan"), np.float16("inf"), np.float16("-inf"))[i % 3]
    x[bad[-1], :] = np.float16("nan")                       # a group of nothing but NaN
    t = np.float32(0.01)
    say("non-finite groups")
    g_blocks, g_stats = gpu_encode(x, tdev, t, stats=True)
    o_blocks, info = codec.encode_groups(x, tb, t, return_info=True)
    assert g_stats["nonfinite_groups"] == info["stats"]["nonfinite_groups"] == len(bad)
    good = np.setdiff1d(np.arange(600), bad)
    assert_blocks_equal(g_blocks[good], o_blocks[good], "finite groups beside non-finite ones")
    y = gpu_decode(g_blocks, tdev, t)
    assert y.shape == (600, 128)
    assert_fp16_equal(y[good], codec.decode_blocks(o_blocks[good], tb, t), "finite groups decode")


def test_fuzz_decode_random_blocks(dev):
    for name, tb in (("c1", golden("c1")), ("adversarial", adversarial_tables(5)),
                     ("incomplete", incomplete_tables(6))):
        tdev = dev_tables(tb)
        blocks = W.random_blocks(40000, 99).numpy()
        for t in (np.float32(1.0), np.float32(0.0173)):
            say("fuzz decode %s t=%g" % (name, t))
            assert_fp16_equal(gpu_decode(blocks, tdev, t), codec.decode_blocks(blocks, tb, t),
                              "fuzz %s t=%g" % (name, t))


def test_incomplete_codebooks_encode_and_decode(dev):
    """Trained centroids with incomplete codebooks: the GPU's blocks and
    statistics equal the oracle's, and the blocks decode to the oracle's
    values; so do random blocks, most of which stop at a window with no
    codeword (k below 128, no records applied)."""
    tb = incomplete_tables(8, base=golden("c1"))
    tdev = dev_tables(tb)
    x = W.c1_weight().numpy().reshape(-1, 128)
    t = scale_of(x)
    say("incomplete codebooks: encode %d groups" % len(x))
    g_blocks, g_stats = gpu_encode(x, tdev, t, stats=True)
    o_blocks, info = codec.encode_groups(x, tb, t, return_info=True)
    assert_blocks_equal(g_blocks, o_blocks, "incomplete codebooks")
    assert g_stats == info["stats"]
    say("incomplete codebooks: decode")
    assert_fp16_equal(gpu_decode(g_blocks, tdev, t), codec.decode_blocks(o_blocks, tb, t), "incomplete decode")
    blocks = W.random_blocks(20000, 123).numpy()
    _, dinfo = codec.decode_blocks(blocks, tb, t, return_info=True)
    k = np.asarray(dinfo["k"])
    assert np.mean(k < 128) > 0.5                       # most random streams stop early
    assert_fp16_equal(gpu_decode(blocks, tdev, t), codec.decode_blocks(blocks, tb, t), "incomplete random blocks")


@pytest.mark.parametrize("out_f,in_f,batch", [(300, 1024, 1), (64, 4096, 4), (9, 2048, 8)])
def test_gemv_over_incomplete_codebooks(dev, out_f, in_f, batch):
    """The fused decode+GEMV over random blocks of incomplete codebooks (many
    streams stop early): within tolerance of the float64 product over the
    oracle's decode."""
    tb = incomplete_tables(9)
    tdev = dev_tables(tb)
    blocks = W.random_blocks(out_f * in_f // 128, 400 + out_f).numpy()
    blocks[:, 1] = 0x38                                 # scale byte 1.0: weights of moderate size
    t = np.float32(0.5)
    w_hat = codec.decode_blocks(blocks, tb, t)
    blocks[~np.all(np.isfinite(w_hat.astype(np.float32)), axis=1)] = 0   # no NaN records (an all-zero block decodes to 0)
    x = W.c5_x(batch, in_f, seed=402).numpy()
    say("gemv incomplete %dx%d b=%d" % (out_f, in_f, batch))
    y = torch.full((batch, out_f), float("nan"), dtype=torch.float32, device="cuda")
    ecco.ecco_decode_gemv(torch.from_numpy(blocks).cuda(), tdev, t, out_f, in_f,
                          torch.from_numpy(x).cuda(), batch, y)
    torch.cuda.synchronize()
    w_hat = codec.decode_blocks(blocks, tb, t).reshape(out_f, in_f)
    assert np.all(np.isfinite(w_hat.astype(np.float32)))
    y_ref, mag = ogemv.gemv_ref(w_hat, x)
    ok, worst = ogemv.gemv_tolerance_ok(y.cpu().numpy(), y_ref, mag, in_f)
    assert ok, "worst error / bound = %g" % worst


def test_kv_append_k_and_v_in_one_call(dev):
    """The K and V rows of a decode step appended by one ecco_encode_many call
    (strided rows of the [B, H, S, 128] caches, each tensor with its own tables
    and fixed scale): the same blocks as one ecco_encode call per tensor and as
    the oracle."""
    B, H, S, D = 2, 3, 512, 128
    first, ntok = 300, 37
    jobs, sep, data = [], [], []
    for kind, seed in (("k", 31), ("v", 32)):
        tb, t = golden("c3_" + kind), golden_t("c3_" + kind)
        tdev = dev_tables(tb)
        kv = W.kv_tensor(kind, shape=(B, H, S, D), seed=seed)
        kvd = kv.cuda()
        b1 = torch.full((B, H, S, 64), 0xAB, dtype=torch.uint8, device="cuda")
        b2 = torch.full((B, H, S, 64), 0xAB, dtype=torch.uint8, device="cuda")
        jobs.append((kvd[:, :, first:], B * H, ntok, S * D, S, tdev, t, b1[:, :, first:], None))
        ecco.ecco_encode(kvd[:, :, first:], B * H, ntok, S * D, S, tdev, t, b2[:, :, first:])
        data.append((kind, kv, tb, t, tdev, kvd, b1, b2))
    say("kv append K+V in one call")
    ecco.ecco_encode_many(jobs)
    torch.cuda.synchronize()
    for kind, kv, tb, t, _, _, b1, b2 in data:
        g1, g2 = b1.cpu().numpy(), b2.cpu().numpy()
        assert np.array_equal(g1, g2), kind
        ob = codec.encode_groups(kv.numpy()[:, :, first:first + ntok].reshape(-1, 128), tb, t)
        assert_blocks_equal(g1[:, :, first:first + ntok].reshape(-1, 64), ob, "kv append %s" % kind)
        assert np.all(g1[:, :, :first] == 0xAB) and np.all(g1[:, :, first + ntok:] == 0xAB)


def test_strided_kv_append_and_decode(dev):
    tb = golden("c3_k")
    t = golden_t("c3_k")
    tdev = dev_tables(tb)
    B, H, S, D = 2, 3, 512, 128
    kv = W.kv_tensor("k", shape=(B, H, S, D), seed=21)
    first, ntok = 256, 200
    say("strided KV append")
    kvd = kv.cuda()
    blocks = torch.full((B, H, S, 64), 0xAB, dtype=torch.uint8, device="cuda")
    xs = kvd[:, :, first:, :]
    bs = blocks[:, :, first:, :]
    ecco.ecco_encode(xs, B * H, ntok, S * D, S, tdev, t, bs)
    torch.cuda.synchronize()
    gb = blocks.cpu().numpy()
    new = kv.numpy()[:, :, first:first + ntok, :].reshape(-1, 128)
    ob = codec.encode_groups(new, tb, t)
    assert_blocks_equal(gb[:, :, first:first + ntok, :].reshape(-1, 64), ob, "kv append")
    assert np.all(gb[:, :, :first] == 0xAB) and np.all(gb[:, :, first + ntok:] == 0xAB)
    say("strided KV decode")
    y = torch.full((B, H, S, D), 0x7FFF, dtype=torch.int16, device="cuda")
    ecco.ecco_decode(bs, B * H, ntok, S, S * D, tdev, t, y[:, :, first:, :])
    torch.cuda.synchronize()
    gy = y.cpu().numpy().view(np.float16)
    assert_fp16_equal(gy[:, :, first:first + ntok].reshape(-1, 128), codec.decode_blocks(ob, tb, t), "kv decode")
    assert np.all(y.cpu().numpy()[:, :, :first] == 0x7FFF) and np.all(y.cpu().numpy()[:, :, first + ntok:] == 0x7FFF)


def test_decode_many_mixed_jobs_exact(dev):
    """Several tensors with their own tables, scales and layouts in one launch:
    sizes from one group to several batches with ragged tails, a strided job,
    clipping tables; every output element against the oracle, and nothing
    written outside the jobs' outputs."""
    specs = [("golden", 1, 1), ("random", 63, 2), ("adversarial", 64, 3), ("random", 65, 4),
             ("golden", 1000, 5), ("random", 4097, 6), ("adversarial", 777, 7)]
    jobs, refs, keep = [], [], []
    for i, (kind, n, seed) in enumerate(specs):
        tb = {"golden": lambda s: golden("c1"), "random": random_tables,
              "adversarial": adversarial_tables}[kind](seed)
        x = W.random_groups(n, 300 + seed, ("normal", "laplace", "wide")[i % 3]).numpy()
        t = scale_of(x) * np.float32(1.0 + 0.25 * i)
        ob = codec.encode_groups(x, tb, t)
        tdev = dev_tables(tb)
        bd = torch.from_numpy(ob).cuda()
        yd = torch.full((n + 2, 128), 0x7FFF, dtype=torch.int16, device="cuda")
        jobs.append((bd, 1, n, n, n * 128, tdev, t, yd[1:n + 1]))
        refs.append(codec.decode_blocks(ob, tb, t))
        keep.append((tdev, yd))
    # a strided job: 5 rows of 300 groups inside rows of 320 blocks / 320*128 + 64 elements
    tb = random_tables(8)
    rows, gpr, bstride, ystride = 5, 300, 320, 320 * 128 + 64
    x = W.random_groups(rows * gpr, 308, "laplace").numpy()
    t = scale_of(x)
    ob = codec.encode_groups(x, tb, t)
    bfull = np.zeros((rows, bstride, 64), np.uint8)
    bfull[:, :gpr] = ob.reshape(rows, gpr, 64)
    tdev = dev_tables(tb)
    bd = torch.from_numpy(bfull).cuda()
    yd = torch.full((rows * ystride,), 0x7FFF, dtype=torch.int16, device="cuda")
    # random blocks under tables with incomplete codebooks: this job's
    # workgroups take the decode core's stopping instance, the others not
    tbi = incomplete_tables(10)
    rbi = W.random_blocks(3000, 311).numpy()
    tdi = dev_tables(tbi)
    ydi = torch.full((3002, 128), 0x7FFF, dtype=torch.int16, device="cuda")
    jobs.insert(2, (torch.from_numpy(rbi).cuda(), 1, 3000, 3000, 3000 * 128, tdi, np.float32(0.5), ydi[1:3001]))
    refs.insert(2, codec.decode_blocks(rbi, tbi, np.float32(0.5)))
    keep.insert(2, (tdi, ydi))
    jobs.append((bd, rows, gpr, bstride, ystride, tdev, t, yd))
    keep.append((tdev, yd))
    say("decode_many %d jobs" % len(jobs))
    ecco.ecco_decode_many(jobs)
    torch.cuda.synchronize()
    for i, (ref, (_, yd)) in enumerate(zip(refs, keep)):
        got = yd.cpu().numpy()
        assert np.all(got[0] == 0x7FFF) and np.all(got[-1] == 0x7FFF), "job %d wrote outside its output" % i
        assert_fp16_equal(got[1:-1].view(np.float16), ref, "decode_many job %d" % i)
    got = keep[-1][1].cpu().numpy()
    g2 = got.reshape(rows, ystride)
    assert_fp16_equal(g2[:, :gpr * 128].reshape(-1, 128).view(np.float16), codec.decode_blocks(ob, tb, t),
                      "decode_many strided job")
    assert np.all(g2[:, gpr * 128:] == 0x7FFF)


def test_encode_many_mixed_jobs_exact(dev):
    """Several tensors with their own tables, scales and layouts encoded in one
    launch (one group to several units with ragged tails, clipping tables, a
    strided job); every block against the oracle, nothing written outside the
    jobs' blocks, and statistics summed over the jobs that share a buffer."""
    specs = [("golden", 1, 1), ("random", 3, 2), ("adversarial", 64, 3), ("random", 65, 4),
             ("golden", 1000, 5), ("random", 4097, 6), ("adversarial", 777, 7)]
    jobs, refs, keep = [], [], []
    stats = torch.zeros(7, dtype=torch.int64, device="cuda")
    want = dict.fromkeys(ecco.STATS_FIELDS, 0)
    for i, (kind, n, seed) in enumerate(specs):
        tb = {"golden": lambda s: golden("c1"), "random": random_tables,
              "adversarial": adversarial_tables}[kind](seed)
        x = W.random_groups(n, 400 + seed, ("normal", "laplace", "wide")[i % 3]).numpy()
        t = scale_of(x) * np.float32(1.0 + 0.25 * i)
        ob, info = codec.encode_groups(x, tb, t, return_info=True)
        for k, v in info["stats"].items():
            want[k] += v
        tdev = dev_tables(tb)
        xd = torch.from_numpy(x).cuda()
        bd = torch.full((n + 2, 64), 0xAB, dtype=torch.uint8, device="cuda")
        jobs.append((xd, 1, n, n * 128, n, tdev, t, bd[1:n + 1], stats))
        refs.append(ob)
        keep.append((tdev, xd, bd))
    # a strided job: 5 rows of 300 groups inside rows of 320*128 + 64 elements / 320 blocks
    tb = random_tables(8)
    rows, gpr, xstride, bstride = 5, 300, 320 * 128 + 64, 320
    xs = W.random_groups(rows * gpr, 408, "laplace").numpy()
    t = scale_of(xs)
    xfull = np.zeros((rows, xstride), np.float16)
    xfull[:, :gpr * 128] = xs.reshape(rows, gpr * 128)
    ob_s = codec.encode_groups(xs, tb, t)
    tdev = dev_tables(tb)
    xd = torch.from_numpy(xfull).cuda()
    bd = torch.full((rows, bstride, 64), 0xAB, dtype=torch.uint8, device="cuda")
    jobs.append((xd, rows, gpr, xstride, bstride, tdev, t, bd, None))
    keep.append((tdev, xd, bd))
    say("encode_many %d jobs" % len(jobs))
    ecco.ecco_encode_many(jobs)
    torch.cuda.synchronize()
    for i, (ref, (_, _, bd)) in enumerate(zip(refs, keep)):
        got = bd.cpu().numpy()
        assert np.all(got[0] == 0xAB) and np.all(got[-1] == 0xAB), "job %d wrote outside its blocks" % i
        assert_blocks_equal(got[1:-1], ref, "encode_many job %d" % i)
    assert dict(zip(ecco.STATS_FIELDS, stats.cpu().tolist())) == want
    got = keep[-1][2].cpu().numpy()
    assert_blocks_equal(got[:, :gpr].reshape(-1, 64), ob_s, "encode_many strided job")
    assert np.all(got[:, gpr:] == 0xAB)


def test_many_calls_at_the_job_limit(dev):
    """ecco_encode_many, ecco_decode_many and ecco_decode_gemv_many with the
    maximum of 16 jobs, each with its own tables and size (1 to 301 groups):
    every job's result equal to the oracle's (blocks, FP16) or within the GEMV
    bound."""
    n_jobs = 16
    assert n_jobs == ecco.DECODE_MAX_JOBS == ecco.GEMV_MAX_JOBS
    enc, dec, gem, refs = [], [], [], []
    for i in range(n_jobs):
        tb = random_tables(600 + i)
        n = 1 + 20 * i
        x = W.random_groups(n, 610 + i, ("normal", "laplace", "wide")[i % 3]).numpy()
        t = scale_of(x)
        ob = codec.encode_groups(x, tb, t)
        tdev = dev_tables(tb)
        xd = torch.from_numpy(x).cuda()
        bd = torch.full((n, 64), 0xAB, dtype=torch.uint8, device="cuda")
        yd = torch.full((n, 128), 0x7FFF, dtype=torch.int16, device="cuda")
        enc.append((xd, 1, n, n * 128, n, tdev, t, bd, None))
        dec.append((torch.from_numpy(ob).cuda(), 1, n, n, n * 128, tdev, t, yd))
        # GEMV: the job's groups as a [rows, 128] matrix times one x vector
        xv = W.c5_x(1, 128, seed=620 + i).numpy()
        gy = torch.full((1, n), float("nan"), dtype=torch.float32, device="cuda")
        gem.append((dec[-1][0], tdev, t, n, 128, torch.from_numpy(xv).cuda(), gy))
        refs.append((tb, t, ob, xv, bd, yd, gy))
    say("encode_many / decode_many / gemv_many with %d jobs" % n_jobs)
    ecco.ecco_encode_many(enc)
    ecco.ecco_decode_many(dec)
    ecco.ecco_decode_gemv_many(gem, 1)
    torch.cuda.synchronize()
    for i, (tb, t, ob, xv, bd, yd, gy) in enumerate(refs):
        assert_blocks_equal(bd.cpu().numpy(), ob, "encode_many job %d" % i)
        w_hat = codec.decode_blocks(ob, tb, t)
        assert_fp16_equal(yd.cpu().numpy().view(np.float16), w_hat, "decode_many job %d" % i)
        y_ref, mag = ogemv.gemv_ref(w_hat, xv)
        ok, worst = ogemv.gemv_tolerance_ok(gy.cpu().numpy(), y_ref, mag, 128)
        assert ok, "gemv_many job %d worst error / bound = %g" % (i, worst)


def test_decode_many_full_layer_sampled(dev):
    """The layer workload's step as the bench issues it: the seven matrices of
    a LLaMA-3-8B layer reduced by one ecco_amax_many call, encoded by one
    ecco_encode_many launch and decoded by one ecco_decode_many launch, each
    with its own tables and scale; sampled groups against the oracle."""
    ws, tbs, tdevs = {}, {}, {}
    for name in W.LAYER_ORDER:
        tbs[name] = golden("c2_" + name)
        tdevs[name] = dev_tables(tbs[name])
        say("layer %s generate" % name)
        ws[name] = W.c2_layer(0, names=[name])[name]
    wds = {name: ws[name].cuda() for name in W.LAYER_ORDER}
    amax = torch.full((len(W.LAYER_ORDER),), -1.0, dtype=torch.float32, device="cuda")
    say("layer amax_many")
    ecco.ecco_amax_many([(wds[name], wds[name].numel(), amax[k:k + 1]) for k, name in enumerate(W.LAYER_ORDER)])
    torch.cuda.synchronize()
    enc_jobs, dec_jobs, checks = [], [], []
    for k, name in enumerate(W.LAYER_ORDER):
        w = ws[name]
        out_f, in_f = w.shape
        t = scale_of(w.numpy())
        assert np.float32(ecco.ecco_tensor_scale_from_amax(amax[k].item())) == t, name
        bd = torch.empty((out_f, in_f // 128, 64), dtype=torch.uint8, device="cuda")
        yd = torch.empty((out_f, in_f), dtype=torch.int16, device="cuda")
        enc_jobs.append((wds[name], out_f, in_f // 128, in_f, in_f // 128, tdevs[name], t, bd, None))
        dec_jobs.append((bd, out_f, in_f // 128, in_f // 128, in_f, tdevs[name], t, yd))
        G = out_f * in_f // 128
        idx = sample_index(G, 211)
        checks.append((name, tbs[name], t, idx, w.numpy().reshape(-1, 128)[idx], bd, yd))
    say("layer encode_many")
    ecco.ecco_encode_many(enc_jobs)
    torch.cuda.synchronize()
    del enc_jobs, wds
    say("layer decode_many")
    ecco.ecco_decode_many(dec_jobs)
    torch.cuda.synchronize()
    for name, tb, t, idx, xg, bd, yd in checks:
        ob = codec.encode_groups(xg, tb, t)
        assert_blocks_equal(bd.cpu().numpy().reshape(-1, 64)[idx], ob, "layer %s encode_many (sampled)" % name)
        assert_fp16_equal(yd.cpu().numpy().reshape(-1, 128)[idx].view(np.float16), codec.decode_blocks(ob, tb, t),
                          "layer %s decode_many (sampled)" % name)


@pytest.mark.parametrize("out_f,in_f,batch", [(1, 128, 1), (37, 1024, 3), (300, 1024, 8), (64, 8192, 4),
                                              (20, 28672, 2), (1, 4096, 1), (999, 4096, 1), (5, 2048, 1),
                                              (1000, 2048, 1), (33, 8192, 1), (50, 14336, 1), (7, 12416, 1),
                                              (3, 8320, 1), (1, 16384, 1), (300, 14336, 1),
                                              (4, 2048, 8), (8, 4096, 5), (12, 6144, 7), (1024, 2048, 2),
                                              (500, 10240, 4)])
def test_gemv_small(dev, out_f, in_f, batch):
    tb = golden("c5_w1")
    tdev = dev_tables(tb)
    w = W.llama_matrix((out_f, in_f), seed=700 + out_f).numpy()
    t = scale_of(w)
    blocks = codec.encode_groups(w.reshape(-1, 128), tb, t)
    x = W.c5_x(batch, in_f, seed=701).numpy()
    say("gemv %dx%d b=%d" % (out_f, in_f, batch))
    y = torch.full((batch, out_f), float("nan"), dtype=torch.float32, device="cuda")
    ecco.ecco_decode_gemv(torch.from_numpy(blocks).cuda(), tdev, t, out_f, in_f,
                          torch.from_numpy(x).cuda(), batch, y)
    torch.cuda.synchronize()
    w_hat = codec.decode_blocks(blocks, tb, t).reshape(out_f, in_f)
    y_ref, mag = ogemv.gemv_ref(w_hat, x)
    ok, worst = ogemv.gemv_tolerance_ok(y.cpu().numpy(), y_ref, mag, in_f)
    assert ok, "worst error / bound = %g" % worst


GEMV_MANY_SHAPES = [(37, 4096), (1000, 2048), (33, 8192), (50, 14336), (5, 1024), (1, 128), (300, 4096)]


@pytest.mark.parametrize("batch", [1, 3, 8])
def test_gemv_many_mixed_jobs(dev, batch):
    """Seven matrices of different shapes, tables and scales in one call (at
    batch 1 they split four ways: 1, 2 or 4 whole rows per batch and one row
    per wave): every y within the bound of the float64 reference, and bit for
    bit what a call per matrix gives."""
    names = ["c5_w1", "c5_w2", "c1"]
    cases = []
    for i, (out_f, in_f) in enumerate(GEMV_MANY_SHAPES):
        tb = golden(names[i % 3])
        w = W.llama_matrix((out_f, in_f), seed=720 + i).numpy()
        t = scale_of(w)
        blocks = codec.encode_groups(w.reshape(-1, 128), tb, t)
        x = W.c5_x(batch, in_f, seed=730 + i).numpy()
        cases.append(dict(tb=tb, tdev=dev_tables(tb), t=t, blocks=blocks, bd=torch.from_numpy(blocks).cuda(),
                          x=x, xd=torch.from_numpy(x).cuda(), out_f=out_f, in_f=in_f,
                          y=torch.full((batch, out_f), float("nan"), dtype=torch.float32, device="cuda"),
                          y1=torch.full((batch, out_f), float("nan"), dtype=torch.float32, device="cuda")))
    say("gemv_many %d jobs b=%d" % (len(cases), batch))
    ecco.ecco_decode_gemv_many([(c["bd"], c["tdev"], c["t"], c["out_f"], c["in_f"], c["xd"], c["y"]) for c in cases],
                               batch)
    for c in cases:
        ecco.ecco_decode_gemv(c["bd"], c["tdev"], c["t"], c["out_f"], c["in_f"], c["xd"], batch, c["y1"])
    torch.cuda.synchronize()
    for c in cases:
        y = c["y"].cpu().numpy()
        assert np.array_equal(y.view(np.uint32), c["y1"].cpu().numpy().view(np.uint32)), (c["out_f"], c["in_f"])
        w_hat = codec.decode_blocks(c["blocks"], c["tb"], c["t"]).reshape(c["out_f"], c["in_f"])
        y_ref, mag = ogemv.gemv_ref(w_hat, c["x"])
        ok, worst = ogemv.gemv_tolerance_ok(y, y_ref, mag, c["in_f"])
        assert ok, "%dx%d b=%d worst error / bound = %g" % (c["out_f"], c["in_f"], batch, worst)


# -------------------------------------------------------------- full-size, sampled

def sample_index(G, stride=97):
    idx = np.unique(np.r_[np.arange(0, G, stride), np.arange(min(64, G)), np.arange(max(0, G - 64), G)])
    return idx


@pytest.mark.parametrize("name", ["q", "k", "gate", "down"])
def test_llama_layer_matrix_full_size_sampled(dev, name):
    tb = golden("c2_" + name)
    tdev = dev_tables(tb)
    w = W.c2_layer(0, names=[name])[name]
    out_f, in_f = w.shape
    wd = w.cuda()
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    ecco.ecco_amax(wd, wd.numel(), amax)
    torch.cuda.synchronize()
    t = np.float32(ecco.ecco_tensor_scale_from_amax(amax.item()))
    assert t == scale_of(w.numpy())
    G = out_f * in_f // 128
    say("c2 %s encode %d groups" % (name, G))
    bd = torch.empty((out_f, in_f // 128, 64), dtype=torch.uint8, device="cuda")
    ecco.ecco_encode(wd, out_f, in_f // 128, in_f, in_f // 128, tdev, t, bd)
    yd = torch.empty_like(wd)
    ecco.ecco_decode(bd, out_f, in_f // 128, in_f // 128, in_f, tdev, t, yd)
    torch.cuda.synchronize()
    say("c2 %s oracle encode of every group" % name)
    ob, clipped, _ = oracle_pool.encode(w.numpy().reshape(-1, 128), tb, t)
    gb = bd.cpu().numpy().reshape(-1, 64)
    assert_blocks_equal(gb, ob, "c2 %s encode" % name)
    idx = np.union1d(sample_index(G), np.nonzero(clipped)[0])
    say("c2 %s oracle decode of %d groups (%d clipped)" % (name, idx.size, int(clipped.sum())))
    assert_fp16_equal(yd.cpu().numpy().reshape(-1, 128)[idx], oracle_pool.decode(ob[idx], tb, t),
                      "c2 %s decode (sampled + clipped)" % name)


def test_kv_cache_full_size_sampled(dev):
    B, H, S, D = W.KV_SHAPE
    for kind in ("k", "v"):
        tb = golden("c3_" + kind)
        t = golden_t("c3_" + kind)
        tdev = dev_tables(tb)
        say("kv %s generate" % kind)
        kv = W.kv_tensor(kind)
        kvd = kv.cuda()
        blocks = torch.empty((B, H, S, 64), dtype=torch.uint8, device="cuda")
        say("kv %s encode prefix + append" % kind)
        ecco.ecco_encode(kvd, B * H, S - W.KV_APPEND, S * D, S, tdev, t, blocks)
        ecco.ecco_encode(kvd[:, :, S - W.KV_APPEND:], B * H, W.KV_APPEND, S * D, S, tdev, t,
                         blocks[:, :, S - W.KV_APPEND:])
        y = torch.empty_like(kvd)
        say("kv %s decode whole cache" % kind)
        ecco.ecco_decode(blocks, 1, B * H * S, B * H * S, B * H * S * D, tdev, t, y)
        torch.cuda.synchronize()
        gb = blocks.cpu().numpy()
        app = kv.numpy()[:, :, S - W.KV_APPEND:].reshape(-1, 128)
        ob_app = codec.encode_groups(app, tb, t)
        assert_blocks_equal(gb[:, :, S - W.KV_APPEND:].reshape(-1, 64), ob_app, "kv %s append" % kind)
        say("kv %s oracle encode of every group" % kind)
        ob, clipped, _ = oracle_pool.encode(kv.numpy().reshape(-1, 128), tb, t)
        assert_blocks_equal(gb.reshape(-1, 64), ob, "kv %s whole cache" % kind)
        idx = np.union1d(sample_index(B * H * S, 193), np.nonzero(clipped)[0])
        say("kv %s oracle decode of %d groups (%d clipped)" % (kind, idx.size, int(clipped.sum())))
        assert_fp16_equal(y.cpu().numpy().reshape(-1, 128)[idx], oracle_pool.decode(ob[idx], tb, t),
                          "kv %s decode (sampled + clipped)" % kind)
        del kvd, y, blocks
        torch.cuda.empty_cache()


def test_beyond_2_pow_32_elements_strided_sampled(dev):
    """Two strided rows of 16,779,267 groups each: the second row starts past
    2^31 elements and its end lies past 2^32, so every element and block offset
    needs 64-bit arithmetic (8.6 GB of FP16 in and out)."""
    tb = golden("c1")
    tdev = dev_tables(tb)
    gpr = (1 << 24) + 2051
    xs, bs = gpr * 128 + 8, gpr + 1
    say("2^32: generate 2 x %d groups on the device" % gpr)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)
    x = torch.randn(2 * xs, generator=gen, dtype=torch.float16, device="cuda")
    t = np.float32(1.0)
    blocks = torch.full((2 * bs, 64), 0xAB, dtype=torch.uint8, device="cuda")
    say("2^32: encode")
    ecco.ecco_encode(x, 2, gpr, xs, bs, tdev, t, blocks)
    y = torch.full((2 * xs,), 0x7FFF, dtype=torch.int16, device="cuda")
    say("2^32: decode")
    ecco.ecco_decode(blocks, 2, gpr, bs, xs, tdev, t, y)
    torch.cuda.synchronize()
    cols = np.unique(np.r_[np.arange(0, gpr, 104729), gpr - 64 + np.arange(64), np.arange(64)])
    for r in (0, 1):
        say("2^32: check row %d" % r)
        xi = torch.from_numpy(r * xs + cols[:, None] * 128 + np.arange(128)[None, :]).cuda()
        xg = x[xi].cpu().numpy()
        ob = codec.encode_groups(xg, tb, t)
        bi = torch.from_numpy(r * bs + cols).cuda()
        assert_blocks_equal(blocks[bi].cpu().numpy(), ob, "row %d encode (sampled)" % r)
        assert_fp16_equal(y[xi].cpu().numpy().view(np.float16), codec.decode_blocks(ob, tb, t),
                          "row %d decode (sampled)" % r)
    # the gaps between rows are untouched
    assert int(blocks[gpr].min()) == 0xAB and int(blocks[2 * bs - 1].min()) == 0xAB
    assert torch.all(y[gpr * 128:xs] == 0x7FFF) and torch.all(y[xs + gpr * 128:] == 0x7FFF)
    del y, blocks
    # amax over more than 2^32 values: the largest |x| planted past element
    # 2^32, a smaller one in the first half
    say("2^32: amax")
    x[2 * xs - 5] = 60000.0
    x[3] = -59008.0
    out = torch.full((3,), -1.0, dtype=torch.float32, device="cuda")
    ecco.ecco_amax(x, 2 * xs, out[0:1])
    ecco.ecco_amax_many([(x, xs, out[1:2]), (x[xs:], xs, out[2:3])])
    torch.cuda.synchronize()
    assert out.cpu().tolist() == [60000.0, 59008.0, 60000.0]
    del x
    torch.cuda.empty_cache()


def test_gemv_many_layer_groups_full_size_sampled(dev):
    """A LLaMA-3-8B layer's GEMVs as a decode step issues them at batch 1: q, k
    and v in one call (they read the same x), gate and up in another, down (rows
    of 112 blocks, one row per wave) alone; sampled rows against the float64
    reference over oracle-decoded weights, and every row bit for bit what a
    call per matrix gives."""
    for group in (["q", "k", "v"], ["gate", "up"], ["down"]):
        in_f = W.LLAMA3_8B_LAYER[group[0]][1]
        x = W.c5_x(1, in_f, seed=740).numpy()
        xd = torch.from_numpy(x).cuda()
        mats = []
        for nm in group:
            tb = golden("c2_" + nm)
            say("layer %s generate + encode" % nm)
            w = W.c2_layer(0, [nm])[nm]
            out_f = w.shape[0]
            t = scale_of(w.numpy())
            wd = w.cuda()
            bd = torch.empty((out_f, in_f // 128, 64), dtype=torch.uint8, device="cuda")
            tdev = dev_tables(tb)
            ecco.ecco_encode(wd, out_f, in_f // 128, in_f, in_f // 128, tdev, t, bd)
            mats.append(dict(nm=nm, w=w.numpy(), tb=tb, tdev=tdev, t=t, bd=bd, out_f=out_f,
                             y=torch.full((1, out_f), float("nan"), dtype=torch.float32, device="cuda"),
                             y1=torch.full((1, out_f), float("nan"), dtype=torch.float32, device="cuda")))
            del wd
        say("gemv_many %s" % "+".join(group))
        ecco.ecco_decode_gemv_many([(m["bd"], m["tdev"], m["t"], m["out_f"], in_f, xd, m["y"]) for m in mats], 1)
        for m in mats:
            ecco.ecco_decode_gemv(m["bd"], m["tdev"], m["t"], m["out_f"], in_f, xd, 1, m["y1"])
        torch.cuda.synchronize()
        for m in mats:
            y = m["y"].cpu().numpy()
            assert np.array_equal(y.view(np.uint32), m["y1"].cpu().numpy().view(np.uint32)), m["nm"]
            rows = np.unique(np.r_[np.arange(0, m["out_f"], 97), m["out_f"] - 1])
            ob = codec.encode_groups(m["w"][rows].reshape(-1, 128), m["tb"], m["t"])
            w_hat = codec.decode_blocks(ob, m["tb"], m["t"]).reshape(len(rows), in_f)
            y_ref, mag = ogemv.gemv_ref(w_hat, x)
            ok, worst = ogemv.gemv_tolerance_ok(y[:, rows], y_ref, mag, in_f)
            assert ok, "%s worst error / bound = %g" % (m["nm"], worst)
        del mats
        torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["w1", "w2"])
def test_ffn70b_gemv_full_size_sampled(dev, name):
    tb = golden("c5_" + name)
    tdev = dev_tables(tb)
    say("c5 %s generate" % name)
    w = W.c5_matrix(name)
    out_f, in_f = w.shape
    t = scale_of(w.numpy())
    wd = w.cuda()
    bd = torch.empty((out_f, in_f // 128, 64), dtype=torch.uint8, device="cuda")
    say("c5 %s encode" % name)
    ecco.ecco_encode(wd, out_f, in_f // 128, in_f, in_f // 128, tdev, t, bd)
    torch.cuda.synchronize()
    gb = bd.cpu().numpy()
    say("c5 %s oracle encode of every group" % name)
    ob_all, clipped, _ = oracle_pool.encode(w.numpy().reshape(-1, 128), tb, t)
    assert_blocks_equal(gb.reshape(-1, 64), ob_all, "c5 %s encode" % name)
    # sampled rows plus the 16 rows that hold the most clipped groups
    per_row = clipped.reshape(out_f, in_f // 128).sum(axis=1)
    most_clipped = np.argsort(-per_row, kind="stable")[:16]
    rows = np.unique(np.r_[np.arange(0, out_f, 131 if name == "w1" else 41), out_f - 1, most_clipped])
    ob = ob_all.reshape(out_f, in_f // 128, 64)[rows].reshape(-1, 64)
    w_hat = oracle_pool.decode(ob, tb, t).reshape(len(rows), in_f)
    for batch in (1, 4, 8):
        x = W.c5_x(batch, in_f).numpy()
        say("c5 %s gemv b=%d" % (name, batch))
        y = torch.full((batch, out_f), float("nan"), dtype=torch.float32, device="cuda")
        ecco.ecco_decode_gemv(bd, tdev, t, out_f, in_f, torch.from_numpy(x).cuda(), batch, y)
        torch.cuda.synchronize()
        y_ref, mag = ogemv.gemv_ref(w_hat, x)
        ok, worst = ogemv.gemv_tolerance_ok(y.cpu().numpy()[:, rows], y_ref, mag, in_f)
        assert ok, "c5 %s b=%d worst error / bound = %g" % (name, batch, worst)
        assert not np.any(np.isnan(y.cpu().numpy()))


# ------------------------------------------------------------ fused attention

def _attention_case(B, H, G, S, stride, seed, incomplete=False):
    """Oracle-encoded K/V caches [B, H, stride] x 64 B (first S tokens used),
    their oracle-decoded values, q, and the scales.  incomplete: the V tables'
    codebooks made incomplete, and a third of the K blocks replaced by random
    bytes under K tables with incomplete codebooks (their streams mostly stop
    early)."""
    tbk, tbv = golden("c3_k"), golden("c3_v")
    if incomplete:
        tbk, tbv = incomplete_tables(seed, base=tbk), incomplete_tables(seed + 1, base=tbv)
    tk, tv = golden_t("c3_k"), golden_t("c3_v")
    k = W.kv_tensor("k", shape=(B, H, S, 128), seed=seed).numpy()
    v = W.kv_tensor("v", shape=(B, H, S, 128), seed=seed + 1).numpy()
    kb = codec.encode_groups(k.reshape(-1, 128), tbk, tk).reshape(B, H, S, 64)
    vb = codec.encode_groups(v.reshape(-1, 128), tbv, tv).reshape(B, H, S, 64)
    if incomplete:
        rb = W.random_blocks(B * H * S, seed + 3).numpy().reshape(B, H, S, 64)
        rb[..., 1] = 0x30                                   # scale byte 0.5: moderate scores
        pick = (np.arange(S) % 3 == 1)
        kb[:, :, pick] = rb[:, :, pick]
        kd_chk = codec.decode_blocks(kb.reshape(-1, 64), tbk, tk)
        bad = ~np.all(np.isfinite(kd_chk.astype(np.float32)), axis=1).reshape(B, H, S)
        kb[bad] = codec.encode_groups(k.reshape(B, H, S, 128)[bad], tbk, tk)   # no NaN records
    kd = codec.decode_blocks(kb.reshape(-1, 64), tbk, tk).reshape(B, H, S, 128)
    vd = codec.decode_blocks(vb.reshape(-1, 64), tbv, tv).reshape(B, H, S, 128)
    full_k = np.zeros((B, H, stride, 64), np.uint8)
    full_v = np.zeros((B, H, stride, 64), np.uint8)
    full_k[:, :, :S] = kb
    full_v[:, :, :S] = vb
    q = W.c5_x(B * H * G, 128, seed=seed + 2).numpy().reshape(B, H * G, 128)
    return dict(tbk=tbk, tbv=tbv, tk=tk, tv=tv, kb=full_k, vb=full_v, kd=kd, vd=vd, q=q)


def _gpu_attention(c, B, H, G, S, stride, scale):
    ws = torch.empty(ecco.ecco_attention_workspace_size(B, H, G, S), dtype=torch.uint8, device="cuda")
    out = torch.full((B, H * G, 128), float("nan"), dtype=torch.float32, device="cuda")
    ecco.ecco_attention_decode(torch.from_numpy(c["kb"]).cuda(), dev_tables(c["tbk"]), c["tk"],
                               torch.from_numpy(c["vb"]).cuda(), dev_tables(c["tbv"]), c["tv"],
                               torch.from_numpy(np.ascontiguousarray(c["q"])).cuda(), B, H, G, S, stride, scale,
                               ws, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("B,H,G,S,extra", [(1, 1, 1, 1, 0), (2, 3, 4, 63, 5), (2, 2, 2, 200, 0),
                                           (1, 3, 8, 1000, 37), (3, 1, 4, 129, 0), (1, 2, 1, 4096, 64)])
def test_attention_small(dev, B, H, G, S, extra):
    from oracle import attention
    stride = S + extra
    c = _attention_case(B, H, G, S, stride, 60 + S)
    scale = 1.0 / np.sqrt(128.0)
    say("attention B=%d H=%d G=%d S=%d" % (B, H, G, S))
    got = _gpu_attention(c, B, H, G, S, stride, scale)
    ref, mag = attention.attention_ref(c["kd"], c["vd"], c["q"], scale)
    ok, worst = attention.attention_tolerance_ok(got, ref, mag)
    assert ok, "attention outside tolerance: worst error / bound = %g" % worst


def test_attention_incomplete_codebooks(dev):
    """Attention over caches whose tables have incomplete codebooks (K: a third
    of the blocks random bytes, whose streams mostly stop early): the kernels
    take the decode core's stopping instance; within tolerance of the float64
    oracle over the oracle's decode."""
    from oracle import attention
    B, H, G, S = 2, 2, 4, 700
    c = _attention_case(B, H, G, S, S + 3, 90, incomplete=True)
    scale = 1.0 / np.sqrt(128.0)
    say("attention, incomplete codebooks")
    got = _gpu_attention(c, B, H, G, S, S + 3, scale)
    ref, mag = attention.attention_ref(c["kd"], c["vd"], c["q"], scale)
    ok, worst = attention.attention_tolerance_ok(got, ref, mag)
    assert ok, "attention outside tolerance: worst error / bound = %g" % worst


def test_attention_kv_cache_full_size_sampled(dev):
    """The full [16, 8, 8192, 128] caches encoded on the GPU, attention for all
    512 query heads; three (sequence, kv head) pairs checked against the oracle
    (blocks re-encoded by the oracle from the same values)."""
    from oracle import attention
    B, H, S, D = W.KV_SHAPE
    G = 4
    tbk, tbv = golden("c3_k"), golden("c3_v")
    tk, tv = golden_t("c3_k"), golden_t("c3_v")
    say("attention full size: generate + encode")
    k = W.kv_tensor("k")
    v = W.kv_tensor("v")
    kb = torch.empty((B, H, S, 64), dtype=torch.uint8, device="cuda")
    vb = torch.empty((B, H, S, 64), dtype=torch.uint8, device="cuda")
    tkd, tvd = dev_tables(tbk), dev_tables(tbv)
    kd_ = k.cuda()
    ecco.ecco_encode(kd_, 1, B * H * S, B * H * S * D, B * H * S, tkd, tk, kb)
    del kd_
    vd_ = v.cuda()
    ecco.ecco_encode(vd_, 1, B * H * S, B * H * S * D, B * H * S, tvd, tv, vb)
    del vd_
    q = W.c5_x(B * H * G, 128, seed=77).numpy().reshape(B, H * G, 128)
    ws = torch.empty(ecco.ecco_attention_workspace_size(B, H, G, S), dtype=torch.uint8, device="cuda")
    out = torch.full((B, H * G, 128), float("nan"), dtype=torch.float32, device="cuda")
    scale = 1.0 / np.sqrt(128.0)
    say("attention full size: run")
    ecco.ecco_attention_decode(kb, tkd, tk, vb, tvd, tv, torch.from_numpy(q).cuda(), B, H, G, S, S, scale, ws, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    gkb, gvb = kb.cpu().numpy(), vb.cpu().numpy()
    kn, vn = k.numpy(), v.numpy()
    for (b, h) in [(0, 0), (7, 3), (15, 7)]:
        say("attention full size: oracle pair (%d, %d)" % (b, h))
        okb = codec.encode_groups(kn[b, h], tbk, tk)
        ovb = codec.encode_groups(vn[b, h], tbv, tv)
        assert_blocks_equal(gkb[b, h], okb, "K blocks (%d, %d)" % (b, h))
        assert_blocks_equal(gvb[b, h], ovb, "V blocks (%d, %d)" % (b, h))
        kd = codec.decode_blocks(okb, tbk, tk).reshape(1, 1, S, D)
        vd = codec.decode_blocks(ovb, tbv, tv).reshape(1, 1, S, D)
        ref, mag = attention.attention_ref(kd, vd, q[b:b + 1, h * G:(h + 1) * G], scale)
        ok, worst = attention.attention_tolerance_ok(got[b:b + 1, h * G:(h + 1) * G], ref, mag)
        assert ok, "pair (%d, %d): worst error / bound = %g" % (b, h, worst)
