"""Pins of the 2x activation format in the oracle: groups of 64 values in the
same 512-bit block, outlier records of 6 position bits + 8 value bits.

Pinned by: the spec-literal per-group coder (oracle/literal.py, group=64)
against the vectorised one (oracle/codec.py, group=64) on normal, heavy-tailed
and clipping inputs; decoder totality on random blocks; symbol round trips;
the record count closed form; special groups."""

import numpy as np
import pytest

import oracle
from oracle import codec, literal, huffman
import workloads as W

F32 = np.float32
G64 = 64


def random_tables(seed):
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


def clipping_tables(seed):
    """Every pattern the same centroids and symbol 7 coded in 8 bits by every
    book, so a group of values at centroid 7 needs 63 * 8 + len(15) > 496 bits."""
    rng = np.random.default_rng(seed)
    c = np.tile(np.linspace(-1, 1, 15).astype(np.float16).astype(np.float32), (64, 1))
    L = np.zeros((64, 4, 16), np.uint8)
    for p in range(64):
        for h in range(4):
            rank = np.empty(16, np.int64)
            order = [s for s in rng.permutation(16) if s != 7] + [7]
            rank[order] = np.arange(16)
            L[p, h] = huffman.limited_lengths(2.0 ** (15 - rank))
            assert L[p, h, 7] == 8
    return codec.Tables(c, L)


def clipping_groups(n, seed, c7):
    rng = np.random.default_rng(seed)
    amp = rng.uniform(0.5, 2.0, (n, 1))
    x = c7 * amp * (1.0 + rng.uniform(-0.02, 0.02, (n, 64)))
    x[:, 5] = amp[:, 0]                                   # the scale element
    return x.astype(np.float16)


def groups64(n, seed, kind):
    return W.random_groups((n + 1) // 2, seed, kind).numpy().reshape(-1, G64)[:n]


def t_for(x):
    return codec.tensor_scale(float(np.max(np.abs(x.astype(np.float32)))))[0]


@pytest.mark.parametrize("kind,seed", [("normal", 1), ("laplace", 2), ("wide", 3)])
def test_literal_matches_vectorised(kind, seed):
    tb = random_tables(seed)
    x = groups64(80, 10 + seed, kind)
    t = t_for(x)
    blocks = codec.encode_groups(x, tb, t, group=G64)
    y = codec.decode_blocks(blocks, tb, t, group=G64)
    assert y.shape == (80, 64)
    for g in range(x.shape[0]):
        b = literal.encode_group(x[g], tb.centroids, tb.code_len, t, group=G64)
        assert b == blocks[g].tobytes(), g
        d = literal.decode_block(b, tb.centroids, tb.code_len, t, group=G64)
        assert np.array_equal(d.view(np.uint16), y[g].view(np.uint16)), g


def test_clipping_literal_matches_vectorised():
    tb = clipping_tables(7)
    x = np.concatenate([clipping_groups(40, 21, float(tb.centroids[0, 7])), groups64(40, 22, "normal")])
    t = t_for(x)
    blocks, info = codec.encode_groups(x, tb, t, return_info=True, group=G64)
    assert info["clipped"].any()
    y = codec.decode_blocks(blocks, tb, t, group=G64)
    for g in np.nonzero(info["clipped"])[0][:20]:
        assert literal.encode_group(x[g], tb.centroids, tb.code_len, t, group=G64) == blocks[g].tobytes()
        d = literal.decode_block(blocks[g].tobytes(), tb.centroids, tb.code_len, t, group=G64)
        assert np.array_equal(d.view(np.uint16), y[g].view(np.uint16))
        assert np.all(y[g][info["k"][g]:].view(np.uint16) == 0)       # clipped tail decodes to +0


def test_decoder_total_on_random_blocks():
    tb = random_tables(4)
    blocks = W.random_blocks(200, 321).numpy()
    for t in (F32(1.0), F32(0.02)):
        y, info = codec.decode_blocks(blocks, tb, t, return_info=True, group=G64)
        assert y.shape == (200, 64)
        assert np.all((info["k"] >= 0) & (info["k"] <= 64)) and np.all(info["n"] <= 16)
        for g in range(0, 200, 5):
            d = literal.decode_block(blocks[g].tobytes(), tb.centroids, tb.code_len, t, group=G64)
            nan = np.isnan(d.astype(np.float32))
            assert np.array_equal(nan, np.isnan(y[g].astype(np.float32)))
            assert np.array_equal(d.view(np.uint16)[~nan], y[g].view(np.uint16)[~nan])


def test_symbols_round_trip_and_record_count():
    tb = random_tables(5)
    x = groups64(300, 31, "normal")
    t = t_for(x)
    blocks, enc = codec.encode_groups(x, tb, t, return_info=True, group=G64)
    _, dec = codec.decode_blocks(blocks, tb, t, return_info=True, group=G64)
    ok = ~enc["clipped"]
    assert ok.sum() > 100
    assert np.array_equal(dec["sym"][ok], enc["sym"][ok])
    # n = min(16, floor((512 - 16 - L) / 14)) with 14-bit records
    free = 512 - 16 - enc["L"][ok]
    assert np.array_equal(enc["n"][ok], np.minimum(16, free // 14))
    assert np.array_equal(dec["n"][ok], enc["n"][ok])
    # padded positions carry FP8 values of the largest remaining |x|
    y = codec.decode_blocks(blocks, tb, t, group=G64).astype(np.float32)
    inv_t = F32(F32(1.0) / F32(t))
    for g in np.nonzero(ok & (enc["n"] > 0))[0][:50]:
        xs = x[g].astype(np.float32)
        cand = sorted((j for j in range(64) if j != enc["istar"][g]), key=lambda j: (-abs(xs[j]), j))
        for j in cand[:enc["n"][g]]:
            v8 = oracle.fp.fp8_encode(np.array([xs[j] * inv_t], np.float32))
            want = np.float16(F32(oracle.fp.fp8_decode(v8)[0] * F32(t)))
            assert y[g, j] == F32(want)


def test_special_groups():
    tb = random_tables(6)
    zero = np.zeros((1, 64), np.float16)
    t = codec.tensor_scale(0.0)[0]
    y = codec.decode_blocks(codec.encode_groups(zero, tb, t, group=G64), tb, t, group=G64)
    assert np.all(y.astype(np.float32) == 0.0)
    # the scale element comes back as fp16(S), S = f32(FP8(x_i* / t)) * t
    x = groups64(50, 41, "laplace")
    t = t_for(x)
    blocks, info = codec.encode_groups(x, tb, t, return_info=True, group=G64)
    y = codec.decode_blocks(blocks, tb, t, group=G64)
    rows = np.nonzero(~info["clipped"])[0]
    assert rows.size > 20
    assert np.array_equal(y[rows, info["istar"]].view(np.uint16),
                          oracle.fp.fp16_rne(info["S"]).astype(np.float16).view(np.uint16))


def test_trainer_for_64_value_groups():
    sample = W.c1_sample(n_values=256 * 128).numpy()
    tb = oracle.train.train_tables(sample, kmeans_iters=5, huff_iters=3, group=G64)
    tb.check()
    x = W.c1_weight().numpy().reshape(-1, G64)[:400]
    t = t_for(x)
    y = codec.decode_blocks(codec.encode_groups(x, tb, t, group=G64), tb, t, group=G64)
    rel = np.mean((x.astype(np.float64) - y) ** 2) / np.var(x.astype(np.float64))
    assert rel < 0.02
