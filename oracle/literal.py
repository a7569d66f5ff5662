"""One-group-at-a-time encode / decode in plain Python (oracle; test infrastructure only).

The same rules as `oracle.codec`, written a second time as directly as the
prose reads (Ecco review: "What carries the argument", "Core claim", Fig. 4
caption, referee report major comment 1, "free parameters"), with Python
loops, bit strings and float32 scalars.  It is slow and is used on small
inputs to cross-check the vectorised oracle.
"""

import numpy as np

from . import fp
from .huffman import canonical_codes

F32 = np.float32


def _f8(v):
    return int(fp.fp8_encode(np.array([v], dtype=np.float32))[0])


def _f8val(b):
    return F32(fp.fp8_decode(np.array([b], dtype=np.uint8))[0])


def _h(v):
    return np.float16(F32(v))


def _layout(group):
    # outlier record: log2(group) position bits, then the 8-bit FP8 value
    pos_bits = {128: 7, 64: 6}[group]
    return pos_bits, pos_bits + 8


def encode_group(x, centroids, code_len, t, group=128):
    """x: group (128, or 64 for the activation format) float16 values -> 64-byte block (bytes)."""
    pos_bits, rec_bits = _layout(group)
    t = F32(t)
    inv_t = F32(F32(1.0) / t)
    xs = [F32(v) for v in np.asarray(x, dtype=np.float16)]
    # the scale element: first index of the largest magnitude
    istar = 0
    for j in range(1, group):
        if abs(xs[j]) > abs(xs[istar]):
            istar = j
    s8 = _f8(F32(xs[istar] * inv_t))
    S = F32(_f8val(s8) * t)
    a = F32(abs(S))
    rest = [xs[j] for j in range(group) if j != istar]
    gmin, gmax = min(rest), max(rest)
    # pattern: smallest min/max squared error, first on ties
    best_p, best_f = None, None
    for pp in range(64):
        d1 = F32(gmin - F32(F32(centroids[pp][0]) * a))
        d2 = F32(gmax - F32(F32(centroids[pp][14]) * a))
        f = F32(F32(d1 * d1) + F32(d2 * d2))
        if best_f is None or f < best_f:
            best_p, best_f = pp, f
    pp = best_p
    mids = [F32(F32(F32(centroids[pp][i]) + F32(centroids[pp][i + 1])) * F32(0.5))
            for i in range(14)]
    syms = []
    for j in range(group):
        if j == istar:
            syms.append(15)
            continue
        s = 0
        for mk in mids:
            if xs[j] > F32(mk * a):
                s += 1
        syms.append(s)
    # codebook: shortest total length, first on ties
    best_h, best_L = None, None
    for hh in range(4):
        L = sum(int(code_len[pp][hh][s]) for s in syms)
        if best_L is None or L < best_L:
            best_h, best_L = hh, L
    hh = best_h
    lens = [int(v) for v in code_len[pp][hh]]
    codes = canonical_codes(lens)
    stream = ""
    clipped = False
    for s in syms:
        word = format(codes[s], "0%db" % lens[s])
        room = 512 - 16 - len(stream)
        if len(word) > room:
            stream += word[:room]
            clipped = True
            break
        stream += word
    bits = ["0"] * 512
    head = (pp | (hh << 6)) | (s8 << 8)
    for i in range(16):
        bits[i] = str((head >> i) & 1)
    for i, ch in enumerate(stream):
        bits[16 + i] = ch
    if not clipped:
        free = 512 - 16 - len(stream)
        n = min(16, free // rec_bits)
        cand = sorted((j for j in range(group) if j != istar), key=lambda j: (-abs(xs[j]), j))
        for r in range(n):
            j = cand[r]
            rec = j | (_f8(F32(xs[j] * inv_t)) << pos_bits)
            lo = 512 - rec_bits * (r + 1)
            for i in range(rec_bits):
                bits[lo + i] = str((rec >> i) & 1)
    out = bytearray(64)
    for i in range(512):
        if bits[i] == "1":
            out[i >> 3] |= 1 << (i & 7)
    return bytes(out)


def decode_block(block, centroids, code_len, t, group=128):
    """64-byte block -> group float16 values (numpy array)."""
    pos_bits, rec_bits = _layout(group)
    t = F32(t)
    block = bytes(bytearray(block))
    bits = "".join(str((block[i >> 3] >> (i & 7)) & 1) for i in range(512))
    pp = block[0] & 63
    hh = block[0] >> 6
    s8 = block[1]
    S = F32(_f8val(s8) * t)
    a = F32(abs(S))
    lens = [int(v) for v in code_len[pp][hh]]
    words = {format(c, "0%db" % l): s for s, (c, l) in enumerate(zip(canonical_codes(lens), lens))}
    out = [np.float16(0.0)] * group
    pos = 16
    k = 0
    while k < group:
        hit = None
        for ln in range(2, 9):
            if pos + ln <= 512 and bits[pos:pos + ln] in words and lens[words[bits[pos:pos + ln]]] == ln:
                hit = (words[bits[pos:pos + ln]], ln)
                break
        if hit is None:
            break
        s, ln = hit
        out[k] = _h(S) if s == 15 else _h(F32(F32(centroids[pp][s]) * a))
        pos += ln
        k += 1
    if k == group:
        n = min(16, (512 - pos) // rec_bits)
        for r in range(n):
            lo = 512 - rec_bits * (r + 1)
            rec = sum(int(bits[lo + i]) << i for i in range(rec_bits))
            out[rec & (group - 1)] = _h(F32(_f8val(rec >> pos_bits) * t))
    return np.array(out, dtype=np.float16)
