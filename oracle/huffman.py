"""Prefix codes for the 16-symbol index alphabet (oracle; test infrastructure only).

The pages: each group's indices are Huffman-coded with one of 4 codebooks per
pattern, the codebook giving the shortest encoding is chosen (Ecco review,
"What carries the argument" and "Core claim"), and the parallel decoder relies
on code lengths being bounded to between 2 and 8 bits (referee report, major
comment 1); the pages give no construction for such lengths.

Readings used here:
  * codes are canonical in the DEFLATE sense (RFC 1951 section 3.2.2):
    symbols ordered by (length, symbol id), each code is the previous one plus
    one, shifted left when the length grows;
  * the lengths of a codebook are the optimal ones for its symbol counts under
    2 <= length <= 8 and the Kraft inequality, found exactly by a knapsack over
    Kraft capacity measured in units of 2**-8.
"""

from fractions import Fraction

import numpy as np

N_SYMBOLS = 16
LEN_MIN = 2
LEN_MAX = 8


def canonical_codes(lengths):
    """Code values (int, MSB-first meaning) for the given code lengths.

    Follows the DEFLATE construction: count codes per length, derive the first
    code of each length, then hand out consecutive values to symbols of that
    length in increasing symbol order.
    """
    lengths = [int(x) for x in lengths]
    max_len = max(lengths)
    bl_count = [0] * (max_len + 1)
    for ln in lengths:
        if ln > 0:
            bl_count[ln] += 1
    next_code = [0] * (max_len + 2)
    code = 0
    for bits in range(1, max_len + 1):
        code = (code + bl_count[bits - 1]) << 1
        next_code[bits] = code
    codes = [0] * len(lengths)
    for sym, ln in enumerate(lengths):
        if ln > 0:
            codes[sym] = next_code[ln]
            next_code[ln] += 1
    return codes


def kraft_sum(lengths):
    return sum(Fraction(1, 2 ** int(ln)) for ln in lengths)


def is_prefix_free(codes, lengths):
    """Pairwise check that no codeword is a prefix of another."""
    words = [format(c, "0%db" % ln) for c, ln in zip(codes, lengths)]
    for i, a in enumerate(words):
        for j, b in enumerate(words):
            if i != j and b.startswith(a):
                return False
    return True


def limited_lengths(freqs, lmin=LEN_MIN, lmax=LEN_MAX):
    """Exact minimum of sum(f_s * len_s) s.t. Kraft <= 1 and lmin <= len <= lmax.

    A 0/1-knapsack over symbols: a code of length l uses 2**(lmax-l) of the
    2**lmax units of Kraft capacity.  dp[i][u] is the least cost of the first i
    symbols using exactly u units.  Ties between optimal length vectors are
    broken towards shorter lengths for lower symbol ids (the first optimal
    choice met when lengths are tried in increasing order).
    """
    freqs = [int(f) for f in freqs]
    n = len(freqs)
    cap = 1 << lmax
    INF = np.iinfo(np.int64).max // 4
    dp = np.full((n + 1, cap + 1), INF, dtype=np.int64)
    choice = np.zeros((n + 1, cap + 1), dtype=np.int64)
    dp[0, 0] = 0
    for i in range(n):
        for ln in range(lmin, lmax + 1):
            w = 1 << (lmax - ln)
            cand = np.full(cap + 1, INF, dtype=np.int64)
            prev = dp[i, : cap + 1 - w]
            cand[w:] = np.where(prev < INF, prev + freqs[i] * ln, INF)
            better = cand < dp[i + 1]
            dp[i + 1] = np.where(better, cand, dp[i + 1])
            choice[i + 1] = np.where(better, ln, choice[i + 1])
    best_u = int(np.argmin(dp[n]))          # first (smallest u) among equal costs
    if dp[n, best_u] >= INF:
        raise ValueError("no feasible length vector")
    lengths = [0] * n
    u = best_u
    for i in range(n, 0, -1):
        ln = int(choice[i, u])
        lengths[i - 1] = ln
        u -= 1 << (lmax - ln)
    return lengths


def code_cost(freqs, lengths):
    return int(sum(int(f) * int(l) for f, l in zip(freqs, lengths)))


def codes_table(code_len):
    """[S,H,16] lengths -> [S,H,16] canonical code values (int64)."""
    code_len = np.asarray(code_len)
    out = np.zeros(code_len.shape, dtype=np.int64)
    for idx in np.ndindex(code_len.shape[:-1]):
        out[idx] = canonical_codes(code_len[idx])
    return out
