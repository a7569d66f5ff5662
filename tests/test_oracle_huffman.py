"""Pins for the oracle's prefix codes (CPU only).

Canonical codes: the worked example of RFC 1951 section 3.2.2.  Length
limits: the referee report's 2..8-bit code-length bound.  Optimality: brute
force over every non-decreasing length vector for frequency-sorted symbols
(C(22, 6) = 74,613 candidates), and agreement with textbook Huffman whenever
Huffman's own lengths already fall in [2, 8].
"""

import heapq
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import huffman

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_rfc1951_example():
    g = json.load(open(os.path.join(GOLD, "rfc1951_canonical.json")))
    codes = huffman.canonical_codes(g["lengths"])
    got = [format(c, "0%db" % l) for c, l in zip(codes, g["lengths"])]
    assert got == g["codes_binary"]


@pytest.fixture(scope="module")
def all_sorted_length_vectors():
    vecs = np.array(list(itertools.combinations_with_replacement(range(2, 9), 16)), dtype=np.int64)
    kraft = np.sum(2.0 ** (-vecs), axis=1)
    return vecs[kraft <= 1.0 + 1e-12]


def _huffman_lengths(freqs):
    heap = [(f, i, [i]) for i, f in enumerate(freqs)]
    heapq.heapify(heap)
    depth = [0] * len(freqs)
    uid = len(freqs)
    while len(heap) > 1:
        f1, _, s1 = heapq.heappop(heap)
        f2, _, s2 = heapq.heappop(heap)
        for s in s1 + s2:
            depth[s] += 1
        heapq.heappush(heap, (f1 + f2, uid, s1 + s2))
        uid += 1
    return depth


@pytest.mark.parametrize("seed", range(12))
def test_limited_lengths_optimal_vs_brute_force(seed, all_sorted_length_vectors):
    rng = np.random.default_rng(seed)
    kind = seed % 3
    if kind == 0:
        freqs = rng.integers(1, 50, 16)
    elif kind == 1:
        freqs = (1000 * np.exp(-0.6 * np.arange(16)) + 1).astype(np.int64)   # very skewed
        rng.shuffle(freqs)
    else:
        freqs = rng.geometric(0.05, 16)
    lengths = huffman.limited_lengths(freqs)
    assert all(2 <= l <= 8 for l in lengths)
    assert huffman.kraft_sum(lengths) <= 1
    fs = np.sort(freqs)[::-1]
    brute = int(np.min(all_sorted_length_vectors @ fs))
    assert huffman.code_cost(freqs, lengths) == brute


def test_limited_matches_huffman_when_unconstrained():
    rng = np.random.default_rng(11)
    hits = 0
    for _ in range(200):
        freqs = rng.integers(20, 60, 16)
        hl = _huffman_lengths(list(freqs))
        if min(hl) < 2 or max(hl) > 8:
            continue
        hits += 1
        assert huffman.code_cost(freqs, huffman.limited_lengths(freqs)) == huffman.code_cost(freqs, hl)
    assert hits > 50


def test_positive_frequencies_give_complete_codes():
    rng = np.random.default_rng(5)
    for _ in range(100):
        freqs = rng.integers(1, 10_000, 16) ** rng.integers(1, 3)
        lengths = huffman.limited_lengths(freqs)
        assert huffman.kraft_sum(lengths) == Fraction(1)


def test_canonical_codes_prefix_free_and_ordered():
    rng = np.random.default_rng(9)
    for _ in range(200):
        lengths = huffman.limited_lengths(rng.integers(1, 1000, 16))
        codes = huffman.canonical_codes(lengths)
        assert huffman.is_prefix_free(codes, lengths)
        # canonical order: (length, symbol) order gives increasing left-aligned codes
        order = sorted(range(16), key=lambda s: (lengths[s], s))
        left = [codes[s] << (8 - lengths[s]) for s in order]
        assert left == sorted(left) and len(set(left)) == 16


def test_prefix_check_detects_violation():
    assert not huffman.is_prefix_free([0b01, 0b010], [2, 3])
