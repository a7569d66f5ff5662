"""Pins for the oracle's table training and quality figures (CPU only).

Training (Ecco review, "Load-bearing premise": patterns and codebooks are
learned offline on calibration data; "Assumptions & free parameters": 64
patterns of 15 centroids, 4 codebooks per pattern; referee report, major
comment 1: code lengths limited to 2..8 bits).  The pages leave the procedure
open; the oracle reads it as k-means patterns plus Lloyd iterations over
codebooks under the encoder's own shortest-code rule.  These tests pin that
reading to answers derived by hand, not to the oracle itself:

  * four clusters of groups with disjoint symbol sets and entropies 0, 1, 2
    and 3 bits: the entropy-quartile start puts each cluster on its own
    codebook and nothing moves after that; each codebook's lengths are the
    optimal 2..8-bit lengths of its cluster's counts plus one, worked out
    by hand below (the optimum of each case is unique as a multiset);
  * a sample of two group shapes, each with 15 distinct FP8-exact values
    and one dominant symbol: the patterns are the two shapes, repeated over
    the 64 slots; the first codebook of each pattern takes the shape's
    lengths, and since the four books tie at the start, every group moves
    to book 0 (lowest id on ties) and the other books fall back to the
    counts of no group plus one, i.e. uniform 4-bit codes;
  * planted mistakes in a copy of the trainer (longest book, no +1
    smoothing, books learned over every pattern's groups, index order in
    place of the entropy order) each break one of these answers.

Quality figures (Fig. 2 caption: index entropy and bit efficiency; Fig. 10
caption: padding and clipping ratios): reconstruction MSE, index entropy,
achieved bits per index and the padding / clipping fractions on two
hand-computed groups.
"""

import types

import numpy as np
import pytest

from oracle import metrics, train

# ---------------------------------------------------------------- codebooks

# Symbol sets of four clusters (disjoint; symbol 15 unused): cluster A codes
# one symbol 128 times (entropy 0), B two symbols 64 times each (1 bit), C
# four symbols 32 times (2 bits), D eight symbols 16 times (3 bits).
CLUSTERS = {"A": [0], "B": [1, 2], "C": [3, 4, 5, 6], "D": list(range(7, 15))}


def cluster_counts(n_each, order="DBAC"):
    rows, labels = [], []
    for _ in range(n_each):
        for name in order:
            r = np.zeros(16, np.int64)
            r[CLUSTERS[name]] = 128 // len(CLUSTERS[name])
            rows.append(r)
            labels.append(name)
    return np.stack(rows), labels


# Optimal lengths of each cluster's summed counts plus one, worked out by
# hand for n_each >= 1 groups per cluster (Kraft capacity in units of 2^-8):
#  A: the common symbol takes 2 bits (64 units); 15 rare symbols share 192
#     units; with x of them at 4 bits (16 units) and the rest at 5 (8 units),
#     16x + 8(15 - x) <= 192 gives x <= 9, so 9 at 4 and 6 at 5 (cost 66 per
#     unit count); a 3-bit common symbol would save at most 4 on the rare
#     ones and cost 128n + 1.
#  B: both common symbols at 2 bits (128 units); 14 rare share 128 units:
#     16x + 8(14 - x) <= 128 gives x <= 2: 2 at 4, 12 at 5.
#  C: commons at (2, 2, 2, 3) (224 units); 12 rare share 32 units: with y at
#     7 bits and z at 8, the best is four at 6 and eight at 7 (4*4 + 8*2 =
#     32); commons at (2, 2, 3, 3) would save 12 on the rare ones and cost
#     32n + 1.
#  D: eight commons can take at most 248 units beside 8 rare symbols: seven
#     at 3 bits and one at 4 (240 units), then 8 rare at 7 bits (16 units).
EXPECTED = {
    "A": ({0: 2}, sorted([4] * 9 + [5] * 6)),
    "B": ({1: 2, 2: 2}, sorted([4] * 2 + [5] * 12)),
    "C": (None, sorted([6] * 4 + [7] * 8)),
    "D": (None, sorted([7] * 8)),
}


def check_cluster_codebooks(learn):
    counts, labels = cluster_counts(3)
    L = np.asarray(learn(counts, 4, 10)).astype(np.int64)
    assert L.shape == (4, 16)
    # the entropy quartiles map A, B, C, D to books 0, 1, 2, 3
    for h, name in enumerate("ABCD"):
        common = CLUSTERS[name]
        rare = [s for s in range(16) if s not in common]
        fixed, rare_lengths = EXPECTED[name]
        if fixed is not None:
            assert {s: int(L[h, s]) for s in fixed} == fixed, (name, L[h])
        if name == "C":
            assert sorted(L[h, common].tolist()) == [2, 2, 2, 3], L[h]
        if name == "D":
            assert sorted(L[h, common].tolist()) == [3] * 7 + [4], L[h]
        assert sorted(L[h, rare].tolist()) == rare_lengths, (name, L[h])
        assert sum(2.0 ** -int(v) for v in L[h]) == 1.0
    # a fixed point: every group is shortest on its own cluster's book
    cost = counts @ L.T
    own = np.array(["ABCD".index(nm) for nm in labels])
    assert np.array_equal(cost.argmin(axis=1), own)
    srt = np.sort(cost, axis=1)
    assert np.all(srt[:, 0] < srt[:, 1])               # strictly, so no tie rule decides it
    return True


def test_codebooks_of_four_clusters_by_hand():
    assert check_cluster_codebooks(train.learn_codebooks)


def test_codebooks_of_no_group_are_uniform():
    L = train.learn_codebooks(np.zeros((0, 16), np.int64), 4, 10)
    assert L.shape == (4, 16) and np.all(L == 4)


# ------------------------------------------------------------ whole trainer

GRID_A = np.arange(-7, 8) * 0.125          # 15 FP8- and FP16-exact values
GRID_B = np.arange(-7, 8) * 0.0625
HEAVY = {"A": 7, "B": 3}                   # the symbol each shape repeats 113 times


def two_shape_sample(n_each=8, seed=0):
    """Groups of 128: the scale element +1.0 first, then the shape's 15
    values once each and its heavy value 112 more times, shuffled."""
    rng = np.random.default_rng(seed)
    rows = []
    for _ in range(n_each):
        for grid, heavy in ((GRID_A, HEAVY["A"]), (GRID_B, HEAVY["B"])):
            vals = np.concatenate([grid, np.full(112, grid[heavy])])
            rows.append(np.concatenate([[1.0], rng.permutation(vals)]))
    return np.stack(rows).astype(np.float16)


def check_two_shape_training(train_tables):
    x = two_shape_sample()
    tb = train_tables(x.ravel(), distinct=2, kmeans_iters=10, huff_iters=10, seed=3)
    c = tb.centroids
    shapes = {tuple(GRID_A.astype(np.float32)), tuple(GRID_B.astype(np.float32))}
    assert {tuple(c[0]), tuple(c[1])} == shapes
    for p in range(64):
        assert np.array_equal(c[p], c[p % 2])
    for p in (0, 1):
        name = "A" if tuple(c[p]) == tuple(GRID_A.astype(np.float32)) else "B"
        heavy = HEAVY[name]
        L = tb.code_len[p].astype(np.int64)
        # book 0: the heavy symbol at 2 bits; the other 14 centroid symbols
        # and the scale symbol (each once per group, 8n + 1 with smoothing)
        # share the rest as 9 at 4 bits and 6 at 5 (case A above)
        assert L[0, heavy] == 2
        assert sorted(np.delete(L[0], heavy).tolist()) == [4] * 9 + [5] * 6
        assert np.all(L[1:] == 4)
    assert np.all(tb.code_len[2:] == 4)          # slots no group selects
    return True


def test_trainer_two_shapes_by_hand():
    assert check_two_shape_training(train.train_tables)


# ------------------------------------------------------------ planted mistakes

TRAIN_MUTATIONS = [
    ("longest codebook", "new = np.argmin(cost, axis=1)", "new = np.argmax(cost, axis=1)"),
    ("no +1 smoothing", "counts[assign == h].sum(axis=0) + 1", "counts[assign == h].sum(axis=0)"),
    ("index order start", "order = np.argsort(_entropy(counts.astype(np.float64)), kind=\"stable\")",
     "order = np.arange(N)"),
    ("books over every pattern's groups", "learn_codebooks(counts[info[\"p\"] == p]",
     "learn_codebooks(counts"),
]


def _train_mutant(old, new):
    src = open(train.__file__).read()
    assert old in src, old
    mod = types.ModuleType("oracle.train_mutant")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), "train_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", TRAIN_MUTATIONS, ids=[m[0] for m in TRAIN_MUTATIONS])
def test_training_pins_catch_planted_mistake(name, old, new):
    mut = _train_mutant(old, new)
    caught = False
    for chk in (lambda: check_cluster_codebooks(mut.learn_codebooks),
                lambda: check_two_shape_training(mut.train_tables)):
        try:
            if not chk():
                caught = True
        except (AssertionError, ValueError, IndexError):
            caught = True
        if caught:
            break
    assert caught, name


# ----------------------------------------------------------------- metrics

def test_reconstruction_by_hand():
    # x = 1, 2, 3, 4 and y = 1, 2, 3, 5: squared errors 0, 0, 0, 1 -> MSE 1/4;
    # var(x) = mean((x - 2.5)^2) = (2.25 + 0.25 + 0.25 + 2.25) / 4 = 1.25
    r = metrics.reconstruction(np.array([[1, 2], [3, 4]], np.float16), np.array([[1, 2], [3, 5]], np.float16))
    assert r["mse"] == 0.25 and r["rel_mse"] == 0.2
    r = metrics.reconstruction(np.ones(4), np.ones(4))
    assert r["mse"] == 0.0 and np.isnan(r["rel_mse"])          # zero variance: no relative figure


def test_index_entropy_by_hand():
    # group 0 codes one symbol 128 times (entropy 0); group 1 two symbols 64
    # times each (entropy 1 bit); unclipped lengths 256 and 384 bits are 2 and
    # 3 bits per index
    sym = np.zeros((2, 128), np.int64)
    sym[1, 64:] = 9
    e = metrics.index_entropy(dict(sym=sym, L=np.array([256, 384])))
    assert e["mean_group_entropy_bits"] == 0.5
    assert e["achieved_bits_per_index"] == 2.5
    # four symbols 32 times each: 2 bits
    sym4 = np.repeat(np.array([[0, 5, 10, 15]]), 32, axis=1)
    assert metrics.index_entropy(dict(sym=sym4, L=np.array([256])))["mean_group_entropy_bits"] == 2.0


def test_padding_figures_by_hand():
    # two groups: one unclipped with 3 records (45 bits), one clipped after 100
    # codewords (28 values lost, no records)
    info = dict(k=np.array([128, 100]), clipped=np.array([False, True]), n=np.array([3, 0]))
    f = metrics.padding_figures(info)
    assert f["clipped_group_frac"] == 0.5
    assert f["clipped_value_frac"] == 28 / 256
    assert f["mean_padded_outliers"] == 1.5
    assert f["pad_bit_frac"] == 45 / 1024


def test_compression_ratio_counts_the_side_data():
    # 512-bit blocks per 2048 FP16 bits: 4x; side data of B bytes adds 8B bits
    assert metrics.compression_ratio(1, 0) == 4.0
    assert metrics.compression_ratio(2, 64) == 4096.0 / (1024.0 + 512.0)
    # side data of the format: 64 x 15 FP16 centroids (1,920 B), 64 x 4 x 16
    # code lengths as bytes (4,096 B) and the FP32 tensor scale (4 B)
    assert metrics.table_bytes_v1() == 1920 + 4096 + 4
