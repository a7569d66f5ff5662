"""The C ABI on the CPU: the library loads, exports what include/ecco.h
declares, and its host logic (table derivation and validation, argument
checks, training) behaves; no kernel is launched."""

import os
import re

import ctypes

import numpy as np
import pytest

import oracle
from oracle import codec, huffman
import workloads as W

ecco = pytest.importorskip("entropy_coded_group_amd")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLD = os.path.join(ROOT, "tests", "golden", "tables.npz")


def _golden(name="c1"):
    z = np.load(GOLD)
    return codec.Tables(z[name + "_centroids"], z[name + "_code_len"])


def test_library_loads_and_exports_every_declared_symbol():
    L = ecco.lib()
    hdr = open(os.path.join(ROOT, "include", "ecco.h")).read()
    names = sorted(set(re.findall(r"\b(ecco_[a-z0-9_]+)\s*\(", hdr)))
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert "gfx950" in ecco.ecco_version()


def test_strerror_covers_codes():
    for c in range(-6, 1):
        assert ecco.ecco_strerror(c) != "unknown error"


# byte offsets of the blob (ecco_internal.h): header 256, centroids 4096,
# code_len 4096, midpoints 4096, c0c14 512, len4 4096, enc 16384, fp8 1024,
# lut 65536, quantiser bins 8192, their axes 512, their flag 4 (+ padding)
OFF_CENT, OFF_LEN, OFF_MID, OFF_C0, OFF_LEN4, OFF_ENC, OFF_FP8, OFF_LUT = (
    256, 4352, 8448, 12544, 13056, 17152, 33536, 34560)
OFF_QBIN, OFF_QAXIS, OFF_QOK, OFF_PCAND, OFF_PGRID = 100096, 108288, 108800, 108816, 117008
QBINS, QMARGIN = 128, 1e-5
PGRID, PCAND = 32, 8


def test_blob_size_and_layout():
    assert ecco.ecco_tables_size() == 117248        # 117024 rounded up to 256


def _bins(blob):
    qbin = blob[OFF_QBIN:OFF_QBIN + 64 * QBINS].reshape(64, QBINS).astype(np.int64)
    qaxis = np.frombuffer(blob[OFF_QAXIS:OFF_QAXIS + 512].tobytes(), np.float32).reshape(64, 2)
    ok = int(np.frombuffer(blob[OFF_QOK:OFF_QOK + 4].tobytes(), np.uint32)[0])
    return qbin, qaxis, ok


def _bins_meet_rule(mids, qbin, qaxis):
    """Per pattern and bin: the bin's x / a interval from the stored binary32
    B and C, widened by the margin; qbin = the midpoints below it, at most one
    midpoint inside it (the last bin: all 14 below).  Computed here in exact
    rational terms of the stored floats (fractions), not as the library does."""
    from fractions import Fraction as F
    d = F(QMARGIN)
    for p in range(64):
        B, C = F(float(qaxis[p, 0])), F(float(qaxis[p, 1]))
        m = [F(float(v)) for v in mids[p]]
        for j in range(QBINS):
            lo = None if j == 0 else (j - C) / B
            hi = None if j == QBINS - 1 else (j + 1 - C) / B
            below = sum(1 for v in m if lo is not None and v < lo - d)
            inside = sum(1 for v in m if (lo is None or v >= lo - d) and (hi is None or v <= hi + d))
            if qbin[p, j] != below:
                return False
            if (j == QBINS - 1 and below != 14) or inside > 1:
                return False
    return True


def test_quantiser_bins_of_trained_tables():
    """Trained tables get bins (every bin at most one midpoint within the
    margin), and a value's bin then decides all thresholds but one."""
    tb = _golden()
    blob = ecco.ecco_tables_build(tb.centroids, tb.code_len)
    qbin, qaxis, ok = _bins(blob)
    assert ok == 1
    assert _bins_meet_rule(tb.midpoints(), qbin, qaxis)
    # spot check with values: x / a at every midpoint and just beside it
    rng = np.random.default_rng(5)
    for p in rng.choice(64, 8, replace=False):
        mids = tb.midpoints()[p].astype(np.float64)
        for a in (np.float32(1.0), np.float32(0.0173), np.float32(300.0)):
            thr = (tb.midpoints()[p] * a).astype(np.float32)
            xs = np.concatenate([thr, np.nextafter(thr, np.float32(np.inf)), np.nextafter(thr, np.float32(-np.inf)),
                                 (rng.uniform(-1.2, 1.2, 64) * a).astype(np.float32)])
            for x in xs.astype(np.float32):
                pos = np.float32(np.float32(x) * np.float32(qaxis[p, 0] / a) + qaxis[p, 1])
                j = int(min(max(np.floor(min(pos, QBINS - 1)), 0), QBINS - 1))
                s = int(qbin[p, j])
                t = thr[s] if s < 14 else np.float32(3.4028235e38)
                assert s + int(x > t) == int(np.sum(x > thr)), (p, float(a), float(x))


def _pattern_argmin_f32(tb, mn, mx, a):
    """The oracle's pattern choice for one group (binary32 fitness, lowest
    index on ties), written out here."""
    c = tb.centroids
    c0a = (c[:, 0] * np.float32(a)).astype(np.float32)
    c14a = (c[:, 14] * np.float32(a)).astype(np.float32)
    d1 = (np.float32(mn) - c0a).astype(np.float32)
    d2 = (np.float32(mx) - c14a).astype(np.float32)
    return int(np.argmin((d1 * d1 + d2 * d2).astype(np.float32)))


def test_pattern_candidates_hold_the_oracles_choice():
    """For points all over the grid, and on the bisectors of pattern pairs,
    the cell that the encoder computes lists the pattern the oracle picks."""
    rng = np.random.default_rng(31)
    for name, tb in (("c1", _golden()), ("random", codec.Tables(
            np.sort(rng.uniform(-1, 1, (64, 15)), axis=1).astype(np.float16).astype(np.float32), _golden().code_len))):
        blob = ecco.ecco_tables_build(tb.centroids, tb.code_len)
        cand = blob[OFF_PCAND:OFF_PCAND + PGRID * PGRID * PCAND].reshape(PGRID * PGRID, PCAND)
        sx, ox, sy, oy = np.frombuffer(blob[OFF_PGRID:OFF_PGRID + 16].tobytes(), np.float32)
        many = cand[:, 0] == 0xfe
        assert many.mean() < 0.05, (name, many.mean())
        c0, c14 = tb.centroids[:, 0].astype(np.float64), tb.centroids[:, 14].astype(np.float64)
        xr = (-float(ox) / float(sx), (PGRID - float(ox)) / float(sx))
        yr = (-float(oy) / float(sy), (PGRID - float(oy)) / float(sy))
        pts = [np.array([rng.uniform(*xr), rng.uniform(*yr)]) for _ in range(3000)]
        for _ in range(3000):                              # points on the bisector of two patterns
            p, q = rng.choice(64, 2, replace=False)
            mid = np.array([c0[p] + c0[q], c14[p] + c14[q]]) / 2
            dirn = np.array([-(c14[q] - c14[p]), c0[q] - c0[p]])
            pts.append(mid + rng.uniform(-0.3, 0.3) * dirn)
        checked = 0
        for pt in pts:
            for a in (np.float32(1.0), np.float32(0.037), np.float32(211.0)):
                mn, mx = np.float32(pt[0] * a), np.float32(pt[1] * a)
                ra = np.float32(np.float32(1.0) / a)
                gx = int(np.floor(np.float32(mn * np.float32(ra * sx) + ox)))
                gy = int(np.floor(np.float32(mx * np.float32(ra * sy) + oy)))
                if not (0 <= gx < PGRID and 0 <= gy < PGRID):
                    continue
                row = cand[gy * PGRID + gx]
                if row[0] == 0xfe:
                    continue
                best = _pattern_argmin_f32(tb, mn, mx, a)
                assert best in set(int(v) for v in row if v != 0xff), (name, pt, float(a), best, row)
                checked += 1
        assert checked > 10000


def test_quantiser_bins_off_for_crowded_midpoints():
    """Tables with two midpoints closer than a bin get no bins (the encoder
    then walks its threshold tree)."""
    tb = _golden()
    c = tb.centroids.copy()
    c[3, 5] = c[3, 6] = c[3, 7]                         # three equal centroids: two equal midpoints
    blob = ecco.ecco_tables_build(c, tb.code_len)
    assert _bins(blob)[2] == 0


def test_tables_build_roundtrip_and_derived_tables_match_oracle():
    tb = _golden()
    blob = ecco.ecco_tables_build(tb.centroids, tb.code_len)
    assert ecco.ecco_tables_validate(blob) == 0
    c, l = ecco.ecco_tables_get(blob)
    assert np.array_equal(c, tb.centroids) and np.array_equal(l, tb.code_len)
    mids = np.frombuffer(blob[OFF_MID:OFF_MID + 4096].tobytes(), np.float32).reshape(64, 16)
    assert np.array_equal(mids[:, :14].view(np.uint32), tb.midpoints().view(np.uint32))
    assert np.all(np.isinf(mids[:, 14:]))
    enc = np.frombuffer(blob[OFF_ENC:OFF_ENC + 16384].tobytes(), np.uint32).reshape(64, 4, 16)
    lut = blob[OFF_LUT:OFF_LUT + 65536].reshape(64, 4, 256)
    codes = tb.codes()
    for p in range(0, 64, 7):
        for h in range(4):
            for s in range(16):
                ln = int(tb.code_len[p, h, s])
                rev = int(format(int(codes[p, h, s]), "0%db" % ln)[::-1], 2)   # stream order
                # the codeword left-aligned in 32 bits, 32 - len in the low 5 bits
                assert enc[p, h, s] == ((int(codes[p, h, s]) << (32 - ln)) | (32 - ln))
                for w in range(rev, 256, 1 << ln):
                    assert lut[p, h, w] == (s | ((ln - 1) << 5))
    fp8 = np.frombuffer(blob[OFF_FP8:OFF_FP8 + 1024].tobytes(), np.float32)
    ref = oracle.fp.fp8_decode(np.arange(256, dtype=np.uint8))
    ok = ~np.isnan(ref)
    assert np.array_equal(fp8[ok].view(np.uint32), ref[ok].view(np.uint32)) and np.all(np.isnan(fp8[~ok]))


def test_tables_build_rejects_bad_inputs():
    tb = _golden()
    bad_len = tb.code_len.copy()
    bad_len[3, 1, 5] = 1
    with pytest.raises(ecco.EccoError):
        ecco.ecco_tables_build(tb.centroids, bad_len)
    over = tb.code_len.copy()
    over[0, 0, :] = 2                                     # Kraft 4 > 1: no prefix code
    with pytest.raises(ecco.EccoError):
        ecco.ecco_tables_build(tb.centroids, over)
    over = tb.code_len.copy()
    s = int(np.argmax(over[4, 2]))                        # one codeword a bit shorter: Kraft just above 1
    over[4, 2, s] -= 1
    with pytest.raises(ecco.EccoError):
        ecco.ecco_tables_build(tb.centroids, over)
    unsorted = tb.centroids.copy()
    unsorted[2, [4, 5]] = unsorted[2, [5, 4]] + np.float32([0.5, 0])
    with pytest.raises(ecco.EccoError):
        ecco.ecco_tables_build(unsorted, tb.code_len)
    not_half = tb.centroids.copy()
    not_half[1, 7] = np.float32(0.1)                       # not exact in FP16
    with pytest.raises(ecco.EccoError):
        ecco.ecco_tables_build(not_half, tb.code_len)


def test_incomplete_codebooks_get_no_codeword_entries():
    """Codebooks with Kraft sum below 1 are accepted; every window that a
    codeword prefixes holds (symbol, length) as for a complete book, every
    other window the no-codeword entry (symbol 17, length 1: 0x11), and their
    share is 1 - Kraft sum.  The windows are found here by brute force over
    the oracle's canonical codes."""
    tb = _golden()
    L = tb.code_len.copy()
    L[0, 0, :] = 8                                         # Kraft 1/16
    s = int(np.argmin(L[9, 3]))                            # one codeword a bit longer: Kraft just below 1
    L[9, 3, s] += 1
    assert L[20, 1, 3] < 8
    L[20, 1, 3] = 8                                        # one codeword lengthened to 8 bits
    from fractions import Fraction
    blob = ecco.ecco_tables_build(tb.centroids, L)
    assert ecco.ecco_tables_validate(blob) == 0
    lut = blob[OFF_LUT:OFF_LUT + 65536].reshape(64, 4, 256)
    codes = codec.Tables(tb.centroids, L).codes()
    for p, h in ((0, 0), (9, 3), (20, 1), (5, 2)):
        expect = np.full(256, 0x11, np.uint8)
        for sym in range(16):
            ln = int(L[p, h, sym])
            rev = int(format(int(codes[p, h, sym]), "0%db" % ln)[::-1], 2)   # stream order, LSB first
            for w in range(256):
                if w & ((1 << ln) - 1) == rev:
                    assert expect[w] == 0x11, (p, h, w)            # prefix-free: no window twice
                    expect[w] = sym | ((ln - 1) << 5)
        assert np.array_equal(lut[p, h], expect), (p, h)
        share = Fraction(int(np.sum(expect == 0x11)), 256)
        assert share == 1 - huffman.kraft_sum(L[p, h]), (p, h)
    # the header's completeness flag (byte 20): 0 here, 1 for the trained tables;
    # validation recomputes it
    assert int(blob[20]) == 0
    assert int(ecco.ecco_tables_build(tb.centroids, tb.code_len)[20]) == 1
    bad = blob.copy()
    bad[20] = 1
    assert ecco.ecco_tables_validate(bad) == -4


def test_tables_validate_detects_corruption():
    tb = _golden()
    blob = ecco.ecco_tables_build(tb.centroids, tb.code_len)
    bad = blob.copy()
    bad[OFF_LUT + 1000] ^= 1
    assert ecco.ecco_tables_validate(bad) == -4
    bad = blob.copy()
    bad[0] ^= 1
    assert ecco.ecco_tables_validate(bad) == -4
    bad = blob.copy()                                   # a bin changed, checksum recomputed: still caught
    bad[OFF_QBIN + 77] ^= 1
    h = 2166136261
    for v in bad[OFF_CENT:].tobytes():
        h = ((h ^ v) * 16777619) & 0xffffffff
    bad[12:16] = np.frombuffer(np.uint32(h).tobytes(), np.uint8)
    assert ecco.ecco_tables_validate(bad) == -4


def test_tensor_scale_matches_oracle():
    for amax in (0.0, 1e-8, 0.37, 1.0, 448.0, 65504.0, 3.3e-5):
        t_lib = ecco.ecco_tensor_scale_from_amax(amax)
        t_or, _ = codec.tensor_scale(amax)
        assert np.float32(t_lib) == t_or, amax


def test_device_entry_points_check_arguments_before_touching_the_device():
    blob = ecco.ecco_tables_build(*(_golden().centroids, _golden().code_len))
    L = ecco.lib()
    A = 1 << 20                                            # a well-aligned fake address
    assert L.ecco_encode(None, 1, 1, 128, 1, A, 1.0, A, None, None) == -1
    assert L.ecco_encode(A, 1, 1, 128, 1, A, 0.0, A, None, None) == -1          # t must be > 0
    assert L.ecco_encode(A, 0, 1, 128, 1, A, 1.0, A, None, None) == -3
    assert L.ecco_encode(A, 1 << 20, 1 << 12, 1 << 19, 1 << 12, A, 1.0, A, None, None) == -3
    assert L.ecco_encode(A + 2, 1, 1, 128, 1, A, 1.0, A, None, None) == -2
    assert L.ecco_encode(A, 1, 1, 128, 1, A, 1.0, A + 16, None, None) == -2
    assert L.ecco_decode(A, 1, 1, 1, 128, A + 64, 1.0, A, None) == -2
    assert L.ecco_decode(A, 2, 4, 3, 512, A, 1.0, A, None) == -3                 # row stride < groups
    assert L.ecco_decode_speculative(A, 1, 1, 1, 128, A + 64, 1.0, A, None) == -2
    assert L.ecco_decode_speculative(A, 2, 4, 3, 512, A, 1.0, A, None) == -3
    assert L.ecco_decode_speculative(None, 1, 1, 1, 128, A, 1.0, A, None) == -1
    for lanes in (0, 1, 3, 16, 64):
        assert L.ecco_decode_segmented(A, 1, 1, 1, 128, A, 1.0, A, lanes, None) == -1
    assert L.ecco_decode_segmented(A, 1, 1, 1, 128, A + 64, 1.0, A, 4, None) == -2
    assert L.ecco_decode_segmented(A, 2, 4, 3, 512, A, 1.0, A, 4, None) == -3
    assert L.ecco_decode_gemv(A, A, 1.0, 16, 100, A, 1, A, None) == -3          # in % 128
    assert L.ecco_decode_gemv(A, A, 1.0, 16, 128, A, 9, A, None) == -3          # batch > 8
    assert L.ecco_amax(A, 0, A, None) == -3
    # group counts whose 64-bit product wraps (2^33 rows x 2^31 groups = 2^64
    # -> 0, and 2^33 x (2^31 + 1) -> 2^33) are refused, not truncated
    for n_rows, gpr in ((1 << 33, 1 << 31), (1 << 33, (1 << 31) + 1), (1, 1 << 32), (1 << 32, 1)):
        assert L.ecco_encode(A, n_rows, gpr, gpr * 128, gpr, A, 1.0, A, None, None) == -3
        assert L.ecco_encode_act(A, n_rows, gpr, gpr * 64, gpr, A, 1.0, A, None, None) == -3
        assert L.ecco_decode(A, n_rows, gpr, gpr, gpr * 128, A, 1.0, A, None) == -3
        assert L.ecco_decode_act(A, n_rows, gpr, gpr, gpr * 64, A, 1.0, A, None) == -3
        assert L.ecco_decode_speculative(A, n_rows, gpr, gpr, gpr * 128, A, 1.0, A, None) == -3
        assert L.ecco_decode_segmented(A, n_rows, gpr, gpr, gpr * 128, A, 1.0, A, 2, None) == -3
    assert L.ecco_decode_gemv(A, A, 1.0, 1 << 10, 128 << 54, A, 1, A, None) == -3   # 2^10 x 2^54 groups
    # ecco_encode_many: count, reserved field, every job checked
    ej = (ecco.EncodeJob * 2)()
    for j in ej:
        j.x_dev, j.blocks_dev, j.tables_dev = A, A, A
        j.n_rows, j.groups_per_row, j.x_row_stride_elems, j.blk_row_stride_blocks = 2, 4, 512, 4
        j.tensor_scale = 1.0
    ep = ctypes.cast(ej, ctypes.c_void_p)
    assert L.ecco_encode_many(None, 1, None) == -1
    assert L.ecco_encode_many(ep, 0, None) == -3
    assert L.ecco_encode_many(ep, ecco.DECODE_MAX_JOBS + 1, None) == -3
    ej[1].reserved = 3
    assert L.ecco_encode_many(ep, 2, None) == -1
    ej[1].reserved = 0
    ej[1].x_row_stride_elems = 500                                             # < 4 * 128
    assert L.ecco_encode_many(ep, 2, None) == -3
    ej[1].x_row_stride_elems = 512
    ej[0].stats_dev = A + 4
    assert L.ecco_encode_many(ep, 2, None) == -2
    ej[0].stats_dev = None
    ej[1].tensor_scale = 0.0
    assert L.ecco_encode_many(ep, 2, None) == -1
    # ecco_amax_many: count, every job checked
    aj = (ecco.AmaxJob * 3)()
    for j in aj:
        j.x_dev, j.n_values, j.amax_dev = A, 1000, A
    ap = ctypes.cast(aj, ctypes.c_void_p)
    assert L.ecco_amax_many(None, 1, None) == -1
    assert L.ecco_amax_many(ap, 0, None) == -3
    assert L.ecco_amax_many(ap, ecco.AMAX_MAX_JOBS + 1, None) == -3
    aj[2].n_values = 0
    assert L.ecco_amax_many(ap, 3, None) == -3
    aj[2].n_values = 7
    aj[1].x_dev = A + 2
    assert L.ecco_amax_many(ap, 3, None) == -2
    aj[1].x_dev = A
    aj[0].amax_dev = A + 2
    assert L.ecco_amax_many(ap, 3, None) == -2
    aj[0].amax_dev = None
    assert L.ecco_amax_many(ap, 3, None) == -1
    # ecco_decode_gemv_many: count, batch, reserved field, every job checked
    gj = (ecco.GemvJob * 3)()
    for j in gj:
        j.blocks_dev, j.tables_dev, j.x_dev, j.y_dev = A, A, A, A
        j.out_features, j.in_features, j.tensor_scale = 16, 4096, 1.0
    gp = ctypes.cast(gj, ctypes.c_void_p)
    assert L.ecco_decode_gemv_many(None, 1, 1, None) == -1
    assert L.ecco_decode_gemv_many(gp, 0, 1, None) == -3
    assert L.ecco_decode_gemv_many(gp, ecco.GEMV_MAX_JOBS + 1, 1, None) == -3
    assert L.ecco_decode_gemv_many(gp, 3, 0, None) == -3
    assert L.ecco_decode_gemv_many(gp, 3, 9, None) == -3
    gj[2].reserved = 7
    assert L.ecco_decode_gemv_many(gp, 3, 1, None) == -1
    gj[2].reserved = 0
    gj[1].in_features = 4000
    assert L.ecco_decode_gemv_many(gp, 3, 1, None) == -3
    gj[1].in_features = 4096
    gj[2].y_dev = A + 2
    assert L.ecco_decode_gemv_many(gp, 3, 1, None) == -2
    gj[2].y_dev = A
    gj[0].tables_dev = None
    assert L.ecco_decode_gemv_many(gp, 3, 1, None) == -1
    # activation format: the same checks with 64-value groups
    assert L.ecco_encode_act(None, 1, 1, 64, 1, A, 1.0, A, None, None) == -1
    assert L.ecco_encode_act(A, 1, 1, 64, 1, A, float("nan"), A, None, None) == -1
    assert L.ecco_encode_act(A, 0, 1, 64, 1, A, 1.0, A, None, None) == -3
    assert L.ecco_encode_act(A, 2, 4, 200, 4, A, 1.0, A, None, None) == -3       # row stride < 4 * 64
    assert L.ecco_encode_act(A, 1, 1, 64, 1, A + 128, 1.0, A, None, None) == -2  # tables 256-aligned
    assert L.ecco_decode_act(A, 1, 1, 1, 64, A, 1.0, None, None) == -1
    assert L.ecco_decode_act(A, 2, 4, 4, 260, A, 1.0, A, None) == -2             # stride % 8
    assert L.ecco_decode_act(A, 2, 4, 4, 240, A, 1.0, A, None) == -3             # stride < 4 * 64
    assert L.ecco_decode_act(A, 2, 4, 3, 256, A, 1.0, A, None) == -3
    # ecco_decode_many: count, reserved field, and every job checked before launch
    jobs = (ecco.DecodeJob * 3)()
    for j in jobs:
        j.blocks_dev, j.y_dev, j.tables_dev = A, A, A
        j.n_rows, j.groups_per_row, j.blk_row_stride_blocks, j.y_row_stride_elems = 1, 4, 4, 512
        j.tensor_scale = 1.0
    jp = ctypes.cast(jobs, ctypes.c_void_p)
    assert L.ecco_decode_many(None, 1, None) == -1
    assert L.ecco_decode_many(jp, 0, None) == -3
    assert L.ecco_decode_many(jp, ecco.DECODE_MAX_JOBS + 1, None) == -3
    jobs[2].reserved = 1
    assert L.ecco_decode_many(jp, 3, None) == -1
    jobs[2].reserved = 0
    jobs[1].y_dev = A + 2
    assert L.ecco_decode_many(jp, 3, None) == -2
    jobs[1].y_dev = A
    jobs[2].tensor_scale = float("inf")
    assert L.ecco_decode_many(jp, 3, None) == -1
    jobs[2].tensor_scale = 1.0
    jobs[0].n_rows, jobs[0].blk_row_stride_blocks = 2, 3
    assert L.ecco_decode_many(jp, 3, None) == -3
    del blob


def test_binding_refuses_host_memory_for_device_arguments():
    """Host memory passed to a kernel would fault the GPU: the binding refuses
    NumPy arrays and CPU tensors for device arguments before calling the
    library, and non-contiguous tensors where the call fixes the layout."""
    import torch
    host = np.zeros(1024, np.uint16)
    cpu = torch.zeros(1024, dtype=torch.float16)
    with pytest.raises(TypeError):
        ecco.ecco_amax(host, 1024, 1 << 20)
    with pytest.raises(ValueError):
        ecco.ecco_amax(cpu, 1024, 1 << 20)
    with pytest.raises(ValueError):
        ecco.ecco_amax_many([(1 << 20, 1024, 1 << 20), (cpu, 1024, 1 << 20)])
    with pytest.raises(ValueError):
        ecco.ecco_decode(1 << 20, 1, 8, 8, 1024, 1 << 20, 1.0, cpu)
    with pytest.raises(ValueError):
        ecco.ecco_decode_gemv_many([(1 << 20, 1 << 20, 1.0, 4, 128, cpu, 1 << 20)], 1)
    with pytest.raises(ValueError):
        ecco.ecco_attention_decode(1 << 20, 1 << 20, 1.0, 1 << 20, 1 << 20, 1.0, cpu, 1, 1, 1, 8, 8, 0.1,
                                   1 << 20, 1 << 20)


def test_library_training_gives_valid_tables_of_oracle_quality():
    sample = W.c1_sample(n_values=512 * 128).numpy()
    blob = ecco.ecco_train_patterns(sample, kmeans_iters=10, huff_iters=5, threads=4)
    assert ecco.ecco_tables_validate(blob) == 0
    c, l = ecco.ecco_tables_get(blob)
    lib_tabs = codec.Tables(c, l)
    lib_tabs.check()
    for p in range(64):
        for h in range(4):
            assert huffman.kraft_sum(l[p, h]) == 1
    ora_tabs = oracle.train.train_tables(sample, kmeans_iters=10, huff_iters=5)
    x = W.c1_weight().numpy().reshape(-1, 128)[:1024]
    t, _ = codec.tensor_scale(float(np.max(np.abs(x.astype(np.float32)))))
    mse = []
    for tb in (lib_tabs, ora_tabs):
        y = codec.decode_blocks(codec.encode_groups(x, tb, t), tb, t)
        mse.append(oracle.metrics.reconstruction(x, y)["mse"])
    assert mse[0] <= 1.25 * mse[1], mse


def _n_search(blob):
    return int(np.frombuffer(bytes(blob[16:20]), dtype=np.uint32)[0])


def test_tables_record_how_many_patterns_the_encoder_searches():
    tb = _golden()
    assert _n_search(ecco.ecco_tables_build(tb.centroids, tb.code_len)) == 64
    for d in (16, 32):
        blob = ecco.ecco_tables_build(tb.centroids[np.arange(64) % d], tb.code_len)
        assert _n_search(blob) == d and ecco.ecco_tables_validate(blob) == 0
    # only the end centroids decide it (the search compares min and max only)
    c = tb.centroids[np.arange(64) % 16].copy()
    c[40, 7] = c[40, 6]
    assert _n_search(ecco.ecco_tables_build(c, tb.code_len)) == 16
    c[40, 14] = np.float32(np.float16(c[40, 14] * 0.5 + 0.5))
    assert _n_search(ecco.ecco_tables_build(c, tb.code_len)) == 64
    # a blob whose recorded width disagrees with its centroids is rejected
    blob = ecco.ecco_tables_build(tb.centroids, tb.code_len)
    blob[16:20] = np.frombuffer(np.uint32(16).tobytes(), np.uint8)
    assert ecco.ecco_tables_validate(blob) == -4


def test_library_trainer_sixteen_patterns():
    sample = W.c1_sample(n_values=512 * 128).numpy()
    blob = ecco.ecco_train_patterns(sample, kmeans_iters=5, huff_iters=3, threads=4, n_patterns=16)
    assert ecco.ecco_tables_validate(blob) == 0 and _n_search(blob) == 16
    c, _ = ecco.ecco_tables_get(blob)
    assert np.array_equal(c, c[np.arange(64) % 16])
    with pytest.raises(ecco.EccoError):
        ecco.ecco_train_patterns(sample, kmeans_iters=2, huff_iters=2, threads=2, n_patterns=8)


def test_library_trainer_activation_groups():
    """group=64 trains on 64-value groups: valid tables, within the oracle's
    quality on the 2x activation format; other group sizes are rejected."""
    sample = W.act_sample(n_tokens=64).numpy()
    blob = ecco.ecco_train_patterns(sample, kmeans_iters=10, huff_iters=5, threads=4, group=64)
    assert ecco.ecco_tables_validate(blob) == 0
    c, l = ecco.ecco_tables_get(blob)
    lib_tabs = codec.Tables(c, l)
    lib_tabs.check()
    ora_tabs = oracle.train.train_tables(sample, kmeans_iters=10, huff_iters=5, group=64)
    x = W.act_tensor((16, 4096), seed=620).numpy().reshape(-1, 64)
    t, _ = codec.tensor_scale(float(np.max(np.abs(x.astype(np.float32)))))
    mse = []
    for tb in (lib_tabs, ora_tabs):
        y = codec.decode_blocks(codec.encode_groups(x, tb, t, group=64), tb, t, group=64)
        mse.append(oracle.metrics.reconstruction(x, y)["mse"])
    assert mse[0] <= 1.25 * mse[1], mse
    for bad in (32, 96, 256):
        with pytest.raises(ecco.EccoError):
            ecco.ecco_train_patterns(sample, kmeans_iters=2, huff_iters=2, threads=2, group=bad)
    with pytest.raises(ecco.EccoError):                     # not a whole number of groups
        ecco.ecco_train_patterns(sample.ravel()[:100], kmeans_iters=2, huff_iters=2, threads=2, group=64)


def test_attention_checks_arguments_before_touching_the_device():
    L = ecco.lib()
    A = 1 << 20
    args = [A, A, 1.0, A, A, 1.0, A, 2, 3, 4, 100, 128, 0.1, A, A, None]
    def call(**kw):
        a = list(args)
        names = ["k", "kt", "ks", "v", "vt", "vs", "q", "b", "h", "g", "s", "stride", "scale", "ws", "out", "st"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return L.ecco_attention_decode(*a)
    assert call(k=None) == -1
    assert call(ws=None) == -1
    assert call(vs=0.0) == -1
    assert call(g=3) == -3
    assert call(s=0) == -3
    assert call(stride=99) == -3
    assert call(ws=A + 64) == -2
    assert call(q=A + 2) == -2
    assert call(k=A + 32) == -2
    # sizes whose products would wrap: 2^33 x 2^31 sequence-head pairs, a
    # 2^63-token row stride
    assert call(b=1 << 33, h=1 << 31) == -3
    assert call(stride=1 << 63) == -3
    assert ecco.ecco_attention_workspace_size(1 << 33, 1 << 31, 4, 100) == 0
    # the allocation-free variant: the same checks, and a workspace beyond its
    # static scratch (16 x 8 pairs, G = 8, 16,384 tokens: 128 MiB) refused
    # before the device is touched
    args_na = args[:13] + args[14:]
    assert L.ecco_attention_decode_noalloc(*[None] + args_na[1:]) == -1
    big = list(args_na)
    big[7:12] = [16, 8, 8, 16384, 16384]
    assert ecco.ecco_attention_workspace_size(16, 8, 8, 16384) > ecco.ATTENTION_NOALLOC_MAX_WORKSPACE
    assert L.ecco_attention_decode_noalloc(*big) == -3
    fits = list(args_na)
    fits[7:12] = [16, 8, 4, 8192, 8192]
    assert ecco.ecco_attention_workspace_size(16, 8, 4, 8192) <= ecco.ATTENTION_NOALLOC_MAX_WORKSPACE
    assert L.ecco_attention_decode_noalloc(*fits) not in (0, -1, -2, -3)   # a device error here: no GPU
    # workspace: scores [B*H][S][G] floats, partial sums [B*H][ceil(S/128)][G][128] floats, batch maxima
    # [B*H][ceil(S/64)][G] floats and unit (max, weight sum) pairs [B*H][ceil(S/128)][G][2] floats, each
    # 256-aligned
    def up(v):
        return (v + 255) // 256 * 256
    for (b, h, g, s) in [(2, 3, 4, 100), (16, 8, 4, 8192), (1, 1, 1, 1), (1, 2, 8, 129)]:
        units, batches = (s + 127) // 128, (s + 63) // 64
        want = (up(b * h * s * g * 4) + up(b * h * units * g * 128 * 4) + up(b * h * batches * g * 4)
                + up(b * h * units * g * 2 * 4))
        assert ecco.ecco_attention_workspace_size(b, h, g, s) == want
