"""Pins for the oracle's block encode / decode (CPU only).

What the pages fix and these tests check:
  * every group becomes exactly one 512-bit block (Ecco review, "Core claim";
    circularity check);
  * the pattern is the one whose min and max best match the group's min and
    max by squared error ("What carries the argument"), checked by brute force
    in float64 over all 64 patterns on 6561 tiny groups;
  * values map to the nearest of the pattern's 15 centroids;
  * the codebook giving the shortest encoding is used;
  * the index stream round-trips losslessly whenever nothing is clipped, and a
    clipped block decodes exactly its whole codewords;
  * spare bits hold the largest remaining values, at most 16 of them, 15 bits
    each, 240 bits at most ("free parameters": padded outlier slots);
  * special groups (constant, all-zero, exact centroid values, forced clip).
The spec-literal per-group oracle and the vectorised one must agree bit for bit,
and mutation tests plant plausible mistakes in a copy of the vectorised oracle
and check that one of these pins catches each.
"""

import itertools
import types

import numpy as np
import pytest

import oracle
from oracle import codec, fp, literal, huffman, metrics
import workloads as W

F32 = np.float32


def random_tables(seed, lens_kind="trained"):
    rng = np.random.default_rng(seed)
    c = np.sort(rng.uniform(-1, 1, (64, 15)), axis=1)
    c[:, 0] = -rng.uniform(0.2, 1.0, 64)
    c[:, -1] = rng.uniform(0.2, 1.0, 64)
    c = np.sort(c, axis=1).astype(np.float16).astype(np.float32)
    L = np.zeros((64, 4, 16), np.uint8)
    for p in range(64):
        for h in range(4):
            L[p, h] = huffman.limited_lengths(rng.integers(1, 200, 16) ** (1 + h % 2))
    return codec.Tables(c, L)


@pytest.fixture(scope="module")
def tabs():
    return random_tables(0)


@pytest.fixture(scope="module")
def trained():
    sample = W.c1_sample(n_values=256 * 128).numpy()
    return oracle.train.train_tables(sample, kmeans_iters=8, huff_iters=4)


@pytest.fixture(scope="module")
def c1_groups():
    return W.c1_weight().numpy().reshape(-1, 128)[:2048]


def _t_for(x):
    return codec.tensor_scale(float(np.max(np.abs(x.astype(np.float32)))))[0]


# ---------------------------------------------------------------- invariants

def check_roundtrip(enc, dec, x, tables, t):
    blocks, info = enc(x, tables, t, return_info=True)
    assert blocks.shape == (x.shape[0], 64) and blocks.dtype == np.uint8
    _, dinfo = dec(blocks, tables, t, return_info=True)
    assert np.array_equal(blocks[:, 0] & 63, info["p"])
    assert np.array_equal(blocks[:, 0] >> 6, info["h"])
    assert np.array_equal(blocks[:, 1], info["s8"])
    unc = ~info["clipped"]
    assert np.array_equal(dinfo["k"], info["k"])
    assert np.all(dinfo["k"][unc] == 128)
    assert np.all(info["k"][info["clipped"]] < 128)
    assert np.array_equal(dinfo["sym"][unc], info["sym"][unc])
    for g in np.nonzero(info["clipped"])[0]:
        k = info["k"][g]
        assert np.array_equal(dinfo["sym"][g, :k], info["sym"][g, :k])
    assert np.array_equal(dinfo["end"][unc], 16 + info["L"][unc])
    return blocks, info


def test_roundtrip_c1(trained, c1_groups):
    blocks, info = check_roundtrip(codec.encode_groups, codec.decode_blocks, c1_groups, trained,
                                   _t_for(c1_groups))
    assert np.any(info["clipped"]) and np.any(~info["clipped"])


def test_roundtrip_random_tables(tabs):
    for kind in ("normal", "laplace", "wide"):
        x = W.random_groups(300, 5, kind).numpy()
        check_roundtrip(codec.encode_groups, codec.decode_blocks, x, tabs, _t_for(x))


def check_pattern_choice(enc, tables, t, x):
    """Brute force: the chosen pattern minimises the squared distance between
    (min, max) of the 127 non-scale values and the pattern's (first, last)
    centroid times a, evaluated in float64 from sorted Python lists."""
    _, info = enc(x, tables, t, return_info=True)
    bad = 0
    for g in range(x.shape[0]):
        xs = [float(v) for v in x[g].astype(np.float32)]
        i = info["istar"][g]
        rest = sorted(xs[:i] + xs[i + 1:])
        a = float(info["a"][g])
        d = [(rest[0] - float(tables.centroids[p][0]) * a) ** 2 +
             (rest[-1] - float(tables.centroids[p][-1]) * a) ** 2 for p in range(64)]
        best = min(d)
        got = d[int(info["p"][g])]
        if not got <= best + 1e-5 * max(best, 1e-30) + 1e-12:
            bad += 1
        # and no lower-index pattern is strictly better by a clear margin
    return bad == 0


def tiny_grid_groups(seed=0):
    levels = np.float16([-0.875, -0.6, -0.35, -0.1, 0.0, 0.15, 0.4, 0.65, 0.875])
    combos = np.array(list(itertools.product(range(9), repeat=4)))
    vals = levels[combos]                                             # [6561, 4]
    x = np.repeat(vals, 32, axis=1)[:, :127]
    scale = np.full((x.shape[0], 1), np.float16(1.0))
    return np.concatenate([scale, x], axis=1).astype(np.float16)


def test_pattern_choice_brute_force_tiny_groups(tabs):
    x = tiny_grid_groups()
    assert check_pattern_choice(codec.encode_groups, tabs, F32(1.0), x)
    assert check_pattern_choice(codec.encode_groups, tabs, F32(0.37), x)


def test_pattern_choice_brute_force_random(trained, c1_groups):
    assert check_pattern_choice(codec.encode_groups, trained, _t_for(c1_groups), c1_groups[:400])


def check_quantiser(enc, tables, t, x):
    """Each non-scale value maps to a nearest centroid of the chosen pattern."""
    _, info = enc(x, tables, t, return_info=True)
    c = tables.centroids.astype(np.float64)
    for g in range(x.shape[0]):
        a = float(info["a"][g])
        cc = c[info["p"][g]] * a
        for j in range(128):
            s = info["sym"][g, j]
            if j == info["istar"][g]:
                if s != 15:
                    return False
                continue
            v = float(x[g, j])
            if s > 14:
                return False
            err = abs(v - cc[s])
            if err > np.min(np.abs(v - cc)) + 1e-6 * abs(v) + 1e-30:
                return False
    return True


def check_midpoint_ties(enc):
    """A value exactly on a midpoint goes to the lower centroid: centroids
    k/8 - 7/8 have FP16-exact midpoints, and with t = 1 and a scale element of
    1.0, a = 1 so the thresholds are the midpoints themselves."""
    c = np.tile((np.arange(15) / 8.0 - 0.875).astype(np.float32), (64, 1))
    tb = codec.Tables(c, np.full((64, 4, 16), 4, np.uint8))
    mids = (c[0, :-1] + c[0, 1:]) / 2
    vals = np.resize(mids, 127)
    x = np.concatenate([[1.0], vals]).astype(np.float16)[None]
    _, info = enc(x, tb, F32(1.0), return_info=True)
    want = np.concatenate([[15], np.resize(np.arange(14), 127)])
    return bool(info["a"][0] == 1.0 and np.array_equal(info["sym"][0], want))


def test_midpoint_ties_go_to_lower_centroid():
    assert check_midpoint_ties(codec.encode_groups)


def test_quantiser_nearest_centroid(trained, c1_groups, tabs):
    assert check_quantiser(codec.encode_groups, trained, _t_for(c1_groups), c1_groups[:200])
    x = W.random_groups(100, 2, "laplace").numpy()
    assert check_quantiser(codec.encode_groups, tabs, _t_for(x), x)


def check_codebook_and_scale(enc, tables, t, x):
    blocks, info = enc(x, tables, t, return_info=True)
    inv_t = F32(F32(1) / F32(t))
    for g in range(x.shape[0]):
        xs = x[g].astype(np.float32)
        i = int(np.argmax(np.abs(xs)))
        if i != info["istar"][g] or np.any(np.abs(xs[:i]) >= abs(xs[i])):
            return False
        if info["s8"][g] != fp.fp8_encode(np.float32([xs[i] * inv_t]))[0]:
            return False
        tot = [sum(int(tables.code_len[info["p"][g], h, s]) for s in info["sym"][g]) for h in range(4)]
        if info["L"][g] != min(tot) or info["h"][g] != tot.index(min(tot)):
            return False
    return True


def test_codebook_is_shortest_and_scale_is_signed_extreme(trained, c1_groups):
    assert check_codebook_and_scale(codec.encode_groups, trained, _t_for(c1_groups), c1_groups[:300])


def _records(block):
    bits = np.unpackbits(np.frombuffer(bytes(block), np.uint8), bitorder="little")
    out = []
    for r in range(16):
        lo = 512 - 15 * (r + 1)
        out.append(int(sum(int(bits[lo + i]) << i for i in range(15))))
    return out


def check_outliers(enc, tables, t, x):
    blocks, info = enc(x, tables, t, return_info=True)
    inv_t = F32(F32(1) / F32(t))
    for g in range(x.shape[0]):
        if info["clipped"][g]:
            if info["n"][g] != 0:
                return False
            continue
        n = min(16, (512 - 16 - int(info["L"][g])) // 15)
        if info["n"][g] != n or n > 16 or 15 * n > 240:
            return False
        xs = x[g].astype(np.float32)
        cand = sorted((j for j in range(128) if j != info["istar"][g]), key=lambda j: (-abs(float(xs[j])), j))
        recs = _records(blocks[g])
        for r in range(n):
            j = cand[r]
            if recs[r] != (j | (int(fp.fp8_encode(np.float32([xs[j] * inv_t]))[0]) << 7)):
                return False
        # bits between the stream end and the records are zero
        bits = np.unpackbits(blocks[g], bitorder="little")
        if np.any(bits[16 + int(info["L"][g]):512 - 15 * n]):
            return False
    return True


def test_outliers_are_the_largest_remaining_values(trained, c1_groups, tabs):
    assert check_outliers(codec.encode_groups, trained, _t_for(c1_groups), c1_groups[:300])
    x = W.random_groups(200, 9, "wide").numpy()
    assert check_outliers(codec.encode_groups, tabs, _t_for(x), x)


# ------------------------------------------------------------- special cases

def test_constant_group_reconstructs_scale_exactly(tabs):
    for v in (0.3, -1.7, 5e-3):
        x = np.full((1, 128), np.float16(v))
        t = _t_for(x)
        blocks, info = codec.encode_groups(x, tabs, t, return_info=True)
        y, dinfo = codec.decode_blocks(blocks, tabs, t, return_info=True)
        S16 = np.float16(info["S"][0])
        assert info["istar"][0] == 0 and y[0, 0] == S16
        n = int(dinfo["n"][0])
        assert np.all(y[0, 1:1 + n] == S16)          # padded values are the remaining largest, j = 1..n


def test_all_zero_group_decodes_to_zero(tabs):
    x = np.zeros((1, 128), np.float16)
    blocks = codec.encode_groups(x, tabs, F32(1.0))
    y = codec.decode_blocks(blocks, tabs, F32(1.0))
    assert np.all(y.astype(np.float32) == 0)


def test_exact_centroid_values_reconstruct_exactly(tabs):
    p = 5
    c = tabs.centroids[p]
    rng = np.random.default_rng(4)
    vals = c[rng.integers(0, 15, 127)]
    vals[:2] = [c[0], c[-1]]
    x = np.concatenate([[1.0], vals]).astype(np.float16)[None]
    blocks, info = codec.encode_groups(x, tabs, F32(1.0), return_info=True)
    assert info["a"][0] == 1.0
    y, dinfo = codec.decode_blocks(blocks, tabs, F32(1.0), return_info=True)
    recs = _records(blocks[0])[: int(dinfo["n"][0])]
    outl = {r & 127 for r in recs}
    k = int(dinfo["k"][0])
    chosen = tabs.centroids[info["p"][0]]
    if chosen[0] == c[0] and chosen[-1] == c[-1] and set(vals.tolist()) <= set(chosen.tolist()):
        for j in range(1, k):
            if j not in outl:
                assert y[0, j] == x[0, j]


def test_forced_clip_at_codeword_boundary_and_inside():
    c = np.tile(np.linspace(-1, 1, 15, dtype=np.float32).astype(np.float16).astype(np.float32), (64, 1))
    L = np.full((64, 4, 16), 8, np.uint8)           # Kraft 1/16: valid, every code 8 bits
    tabs8 = codec.Tables(c, L)
    x = W.random_groups(4, 1).numpy()
    t = _t_for(x)
    blocks, info = codec.encode_groups(x, tabs8, t, return_info=True)
    assert np.all(info["clipped"]) and np.all(info["k"] == 62)      # 16 + 62*8 = 512
    y, dinfo = codec.decode_blocks(blocks, tabs8, t, return_info=True)
    assert np.all(dinfo["k"] == 62)
    assert np.all(y[:, 62:].view(np.uint16) == 0) and np.all(dinfo["n"] == 0)
    # lengths 7 for one symbol class shift the boundary: the last codeword is split
    L2 = L.copy()
    L2[:, :, :8] = 7
    tabs7 = codec.Tables(c, L2)
    blocks, info = codec.encode_groups(x, tabs7, t, return_info=True)
    _, dinfo = codec.decode_blocks(blocks, tabs7, t, return_info=True)
    assert np.array_equal(dinfo["k"], info["k"]) and np.all(info["k"] < 128)
    for g in range(4):
        k = info["k"][g]
        assert np.array_equal(dinfo["sym"][g, :k], info["sym"][g, :k])


# ------------------------------------------------------- two oracles, one spec

def test_literal_matches_vectorised_encode_decode(trained, tabs, c1_groups):
    cases = [(c1_groups[:120], trained), (W.random_groups(60, 3, "wide").numpy(), tabs),
             (W.random_groups(60, 4, "laplace").numpy(), tabs), (W.random_groups(60, 5, "ties").numpy(), tabs)]
    for x, tb in cases:
        t = _t_for(x)
        blocks = codec.encode_groups(x, tb, t)
        y = codec.decode_blocks(blocks, tb, t)
        for g in range(x.shape[0]):
            b = literal.encode_group(x[g], tb.centroids, tb.code_len, t)
            assert b == blocks[g].tobytes()
            d = literal.decode_block(b, tb.centroids, tb.code_len, t)
            assert np.array_equal(d.view(np.uint16), y[g].view(np.uint16))


def test_decoder_total_on_random_blocks(tabs):
    blocks = W.random_blocks(400, 123).numpy()
    for t in (F32(1.0), F32(0.013)):
        y, info = codec.decode_blocks(blocks, tabs, t, return_info=True)
        assert y.shape == (400, 128)
        assert np.all((info["k"] >= 0) & (info["k"] <= 128)) and np.all(info["n"] <= 16)
        for g in range(0, 400, 4):
            d = literal.decode_block(blocks[g].tobytes(), tabs.centroids, tabs.code_len, t)
            a, b = d.view(np.uint16), y[g].view(np.uint16)
            nan = np.isnan(d.astype(np.float32))
            assert np.array_equal(nan, np.isnan(y[g].astype(np.float32)))
            assert np.array_equal(a[~nan], b[~nan])


def test_incomplete_codes_stop_decoding(tabs):
    L = tabs.code_len.copy()
    L[:, :, 0] = 8                                   # drop Kraft below 1 for some books
    tb = codec.Tables(tabs.centroids, L)
    blocks = W.random_blocks(200, 77).numpy()
    y, info = codec.decode_blocks(blocks, tb, F32(1.0), return_info=True)
    for g in range(0, 200, 10):
        d = literal.decode_block(blocks[g].tobytes(), tb.centroids, tb.code_len, F32(1.0))
        nan = np.isnan(d.astype(np.float32))
        assert np.array_equal(d.view(np.uint16)[~nan], y[g].view(np.uint16)[~nan])


# --------------------------------------------------------------- closed forms

def test_compression_ratio_closed_form():
    assert metrics.compression_ratio(10 ** 9, metrics.table_bytes_v1()) == pytest.approx(4.0, rel=1e-5)
    assert metrics.compression_ratio(8192, 0) == 4.0
    r = metrics.compression_ratio(8192, metrics.table_bytes_v1())
    assert 3.9 < r < 4.0


def test_stats_are_consistent(trained, c1_groups):
    _, info = codec.encode_groups(c1_groups, trained, _t_for(c1_groups), return_info=True)
    st = info["stats"]
    assert st["groups"] == c1_groups.shape[0]
    assert st["clipped_groups"] == int(np.sum(info["k"] < 128))
    unc = ~info["clipped"]
    total = 16 * unc.sum() + info["L"][unc].sum() + st["pad_bits"] + st["fill_bits"]
    assert total == 512 * unc.sum()


def test_tables_check_rejects_bad_tables(tabs):
    bad = codec.Tables(tabs.centroids, np.full((64, 4, 16), 1, np.uint8))
    with pytest.raises(ValueError):
        bad.check()
    c = tabs.centroids.copy()
    c[0, 3], c[0, 4] = c[0, 4] + 0.25, c[0, 3]
    with pytest.raises(ValueError):
        codec.Tables(c, tabs.code_len).check()
    tabs.check()


# ------------------------------------------------------------ mutation tests

MUTATIONS = [
    ("gmin includes the scale element", "others[rows, istar] = False", "others[rows, istar] = True"),
    ("wrong end centroid", "c[None, :, N_CENTROIDS - 1]", "c[None, :, N_CENTROIDS - 2]"),
    ("dropped fitness term", "fit = (d1 * d1 + d2 * d2)", "fit = (d1 * d1 + F32(0) * d2)"),
    ("midpoint ties go up", "x32[:, :, None] > thr", "x32[:, :, None] >= thr"),
    ("longest codebook", "h = np.argmin(Lh, axis=1)", "h = np.argmax(Lh, axis=1)"),
    ("unsigned scale", "s8 = fp.fp8_encode((xs * inv_t)", "s8 = fp.fp8_encode((np.abs(xs) * inv_t)"),
    ("smallest outliers", "key = np.where(others, -ax,", "key = np.where(others, ax,"),
    ("one record too many", "free // rec_bits", "free // rec_bits + 1"),
    ("codeword bits reversed", "bit = (cw >> np.maximum(ln - 1 - b, 0)) & 1", "bit = (cw >> b) & 1"),
]


def _mutant(src, old, new):
    assert old in src, old
    mod = types.ModuleType("oracle.codec_mutant")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), "codec_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, old, new, trained, c1_groups):
    src = open(codec.__file__).read()
    mut = _mutant(src, old, new)
    x = c1_groups[:150]
    t = _t_for(x)
    caught = False
    try:
        checks = [
            lambda: check_roundtrip(mut.encode_groups, codec.decode_blocks, x, trained, t) is not None,
            lambda: check_pattern_choice(mut.encode_groups, trained, t, x),
            lambda: check_quantiser(mut.encode_groups, trained, t, x),
            lambda: check_codebook_and_scale(mut.encode_groups, trained, t, x),
            lambda: check_outliers(mut.encode_groups, trained, t, x),
            lambda: check_midpoint_ties(mut.encode_groups),
        ]
        for chk in checks:
            if not chk():
                caught = True
                break
    except (AssertionError, IndexError, ValueError):
        caught = True
    assert caught, name


# ------------------------------------------------- decode pins (hand-built)
#
# The decoder's value rule (c * |S| for centroid symbols, S for the scale
# symbol), its record order (records applied r = 0, 1, ...: a later record
# wins a repeated position) and its stop rule (no records once the stream
# stops early) are pinned here on blocks and groups whose decoded values
# follow from the format alone.

GRID8 = (np.arange(-7, 8) * 0.125).astype(np.float32)     # 15 values exact in FP8 E4M3 and FP16


def grid_tables(code_len_row):
    c = np.tile(GRID8, (64, 1))
    return codec.Tables(c, np.tile(np.asarray(code_len_row, np.uint8), (64, 4, 1)))


# Book with symbol 7 at 2 bits, symbols 6 and 8..15 at 4, symbols 0..5 at 5
# (Kraft 1/4 + 9/16 + 6/32 = 1).  Its canonical codes, by hand: ordered by
# (length, symbol), 7 -> 00; then 4-bit codes from (00 + 1) << 2 = 0100:
# 6 -> 0100, 8 -> 0101, 9 -> 0110, ..., 15 -> 1100; then 5-bit codes from
# (1100 + 1) << 1 = 11010: 0 -> 11010, 1 -> 11011, ..., 5 -> 11111.
BOOK = [5, 5, 5, 5, 5, 5, 4, 2, 4, 4, 4, 4, 4, 4, 4, 4]
BOOK_CODES = {7: "00", 6: "0100", 8: "0101", 9: "0110", 10: "0111", 11: "1000", 12: "1001", 13: "1010",
              14: "1011", 15: "1100", 0: "11010", 1: "11011", 2: "11100", 3: "11101", 4: "11110", 5: "11111"}


class BlockBits:
    """A 512-bit block written bit by bit in the format's order: bit i is bit
    (i & 7) of byte i >> 3; integer fields LSB first, codewords MSB first."""

    def __init__(self):
        self.bits = [0] * 512
        self.pos = 0

    def field(self, value, nbits):
        for b in range(nbits):
            self.bits[self.pos + b] = (value >> b) & 1
        self.pos += nbits

    def code(self, word):
        for ch in word:
            self.bits[self.pos] = int(ch)
            self.pos += 1

    def record(self, r, value, nbits=15):
        lo = 512 - nbits * (r + 1)
        for b in range(nbits):
            self.bits[lo + b] = (value >> b) & 1

    def block(self):
        return np.packbits(np.array(self.bits, np.uint8), bitorder="little")[None]


def test_hand_codes_are_canonical():
    codes = huffman.canonical_codes(BOOK)
    assert {s: format(codes[s], "0%db" % BOOK[s]) for s in range(16)} == BOOK_CODES


def check_negative_scale_group(dec):
    """A group whose largest magnitude is negative: S = -2 (t = 1), a = 2; the
    other 127 values are centroids times a: 100 zeros and 27 values spread
    over the grid.  Every centroid value and every record value is exact, so
    the block decodes to the group itself; writing c * S in place of c * a
    would flip the signs of the centroid values."""
    rng = np.random.default_rng(11)
    others = np.concatenate([np.zeros(100, np.float32), GRID8[rng.integers(0, 15, 27)] * 2])
    x = np.concatenate([[-2.0], rng.permutation(others)]).astype(np.float16)[None]
    tb = grid_tables(BOOK)
    blocks, info = codec.encode_groups(x, tb, F32(1.0), return_info=True)
    assert info["S"][0] == -2.0 and info["a"][0] == 2.0 and not info["clipped"][0]
    y = dec(blocks, tb, F32(1.0))
    assert np.array_equal(y.view(np.uint16), x.view(np.uint16))
    return True


def test_negative_scale_group_decodes_to_itself():
    assert check_negative_scale_group(codec.decode_blocks)


def repeated_record_block():
    """Symbols: 15 at j = 0, then 127 x symbol 7: L = 4 + 254 = 258 bits,
    E = 274, n = min(16, floor(238 / 15)) = 15 records.  Records 0 and 1 both
    name position 5 (FP8 2.0 = 0x40, then 4.0 = 0x48); records 2..14 set
    positions 10..22 to 0.5 (0x30).  Scale byte 0x38 = 1.0, t = 1."""
    bb = BlockBits()
    bb.field(0, 6)
    bb.field(0, 2)
    bb.field(0x38, 8)
    bb.code(BOOK_CODES[15])
    for _ in range(127):
        bb.code(BOOK_CODES[7])
    assert bb.pos == 274
    bb.record(0, 5 | (0x40 << 7))
    bb.record(1, 5 | (0x48 << 7))
    for r in range(2, 15):
        bb.record(r, (8 + r) | (0x30 << 7))
    want = np.zeros(128, np.float16)                      # c[7] * a = 0 * 1 = +0
    want[0] = 1.0
    want[5] = 4.0                                         # the later record wins
    want[10:23] = 0.5
    return bb.block(), want


def stopped_stream_block():
    """A book whose symbol 0 is 8 bits long (Kraft < 1): canonical 8-bit code
    11111000 after the 5-bit codes 11010..11110 of symbols 1..5 (by hand:
    (11110 + 1) << 3), so 11111111 prefixes no codeword.  Stream: symbol 15,
    nine x symbol 7, then 11111111: decoding stops with k = 10 at bit 38.
    The block's last 240 bits hold 16 records naming position 100 (FP8 1.0);
    a stopped stream takes none of them, so values 10..127 are +0."""
    book = list(BOOK)
    book[0] = 8
    codes = dict(BOOK_CODES)
    codes.update({1: "11010", 2: "11011", 3: "11100", 4: "11101", 5: "11110", 0: "11111000"})
    cc = huffman.canonical_codes(book)
    assert {s: format(cc[s], "0%db" % book[s]) for s in range(16)} == codes
    bb = BlockBits()
    bb.field(0, 6)
    bb.field(0, 2)
    bb.field(0x38, 8)
    bb.code(codes[15])
    for _ in range(9):
        bb.code(codes[7])
    bb.code("11111111")
    for r in range(16):
        bb.record(r, 100 | (0x38 << 7))
    want = np.zeros(128, np.float16)
    want[0] = 1.0
    return bb.block(), want, grid_tables(book)


def check_hand_built_blocks(dec):
    blk, want = repeated_record_block()
    y = dec(blk, grid_tables(BOOK), F32(1.0))
    assert np.array_equal(y[0].view(np.uint16), want.view(np.uint16)), y[0]
    blk, want, tb = stopped_stream_block()
    y = dec(blk, tb, F32(1.0))
    assert np.array_equal(y[0].view(np.uint16), want.view(np.uint16)), y[0]
    return True


def test_hand_built_blocks_decode_as_the_format_says():
    assert check_hand_built_blocks(codec.decode_blocks)
    lit = lambda b, tb, t: literal.decode_block(b[0].tobytes(), tb.centroids, tb.code_len, t)[None]
    assert check_hand_built_blocks(lit)
    assert check_negative_scale_group(lit)


DECODE_MUTATIONS = [
    ("centroid times signed scale", "cval = (c[p[:, None], cidx] * a[:, None])", "cval = (c[p[:, None], cidx] * S[:, None])"),
    ("records in reverse order",
     "    for r in range(MAX_OUTLIERS):\n        lo = BLOCK_BITS - rec_bits * (r + 1)\n        rec = (bits",
     "    for r in reversed(range(MAX_OUTLIERS)):\n        lo = BLOCK_BITS - rec_bits * (r + 1)\n        rec = (bits"),
    ("records on a stopped stream", "full = k == group", "full = k >= 0"),
]


@pytest.mark.parametrize("name,old,new", DECODE_MUTATIONS, ids=[m[0] for m in DECODE_MUTATIONS])
def test_decode_pins_catch_planted_mistake(name, old, new):
    mut = _mutant(open(codec.__file__).read(), old, new)
    caught = False
    for chk in (lambda: check_negative_scale_group(mut.decode_blocks),
                lambda: check_hand_built_blocks(mut.decode_blocks)):
        try:
            if not chk():
                caught = True
        except (AssertionError, IndexError, ValueError):
            caught = True
        if caught:
            break
    assert caught, name
