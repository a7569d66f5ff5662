"""Pins of the pattern-selection study (oracle/study.py) and of the
16-pattern tables (oracle/train.py, distinct=16)."""

import numpy as np

from oracle import codec, fp, study
from oracle.train import train_tables
import workloads as W


def _golden():
    import os
    z = np.load(os.path.join(os.path.dirname(__file__), "golden", "tables.npz"))
    return codec.Tables(z["c1_centroids"], z["c1_code_len"])


def _case(n=300):
    x = W.c1_weight().numpy().reshape(-1, 128)[:n]
    t = codec.tensor_scale(float(np.max(np.abs(W.c1_weight().numpy().astype(np.float32)))))[0]
    return x, t


def test_pattern_errors_brute_force_one_group():
    tb = _golden()
    x, t = _case(3)
    err = study.pattern_errors(x, tb, t)
    t32 = np.float32(t)
    inv_t = np.float32(np.float32(1.0) / t32)
    for g in range(3):
        xs = [float(v) for v in x[g].astype(np.float32)]
        istar = max(range(128), key=lambda j: (abs(xs[j]), -j))
        s8 = fp.fp8_encode(np.array([np.float32(xs[istar]) * inv_t], np.float32))[0]
        a = abs(np.float32(fp.fp8_decode(np.array([s8], np.uint8))[0] * t32))
        for p in range(64):
            c = tb.centroids[p]
            mids = [np.float32(np.float32(c[k] + c[k + 1]) * np.float32(0.5)) for k in range(14)]
            total = 0.0
            for j in range(128):
                if j == istar:
                    continue
                sym = sum(1 for k in range(14) if np.float32(xs[j]) > np.float32(mids[k] * a))
                q = float(np.float16(np.float32(c[sym] * a)))
                total += (xs[j] - q) ** 2
            assert abs(total - err[g, p]) <= 1e-12 * max(1.0, total), (g, p, total, err[g, p])


def test_pattern_error_of_the_chosen_pattern_matches_the_decoder():
    """For blocks that are neither clipped nor padded, the decoder's output is
    exactly the quantised group, so its error must equal the study's."""
    tb = _golden()
    x, t = _case(600)
    blocks, info = codec.encode_groups(x, tb, t, return_info=True)
    y = codec.decode_blocks(blocks, tb, t).astype(np.float64)
    err = study.pattern_errors(x, tb, t)
    plain = np.nonzero((~info["clipped"]) & (info["n"] == 0))[0]
    assert plain.size > 20
    for g in plain:
        d = (x[g].astype(np.float64) - y[g]) ** 2
        d[info["istar"][g]] = 0.0
        assert np.isclose(d.sum(), err[g, info["p"][g]], rtol=1e-12, atol=0), g


def test_selection_study_invariants():
    tb = _golden()
    x, t = _case(400)
    s = study.selection_study(x, tb, t)
    assert 0.0 <= s["frac_differs"] <= 1.0
    assert s["mse_optimal"] <= s["mse_minmax"]
    assert s["gap"] >= 0.0
    # one pattern repeated everywhere: nothing to choose
    one = codec.Tables(np.repeat(tb.centroids[:1], 64, axis=0), tb.code_len)
    s1 = study.selection_study(x, one, t)
    assert s1["frac_differs"] == 0.0 and s1["gap"] == 0.0


def test_sixteen_pattern_tables_repeat_and_never_choose_a_repeat():
    sample = W.c1_sample(n_values=256 * 128).numpy()
    tb = train_tables(sample, distinct=16, kmeans_iters=5, huff_iters=3)
    assert np.array_equal(tb.centroids, tb.centroids[np.arange(64) % 16])
    x, t = _case(500)
    _, info = codec.encode_groups(x, tb, t, return_info=True)
    assert info["p"].max() < 16


def test_design_point_agrees_with_the_codec_at_64_patterns_4_codebooks():
    """At S = 64, H = 4 the sweep's coded length and clip decision are the
    codec's own (header 16 bits)."""
    tb = _golden()
    x, t = _case(800)
    r = study.design_point(x, tb.centroids, tb.code_len, t)
    _, info = codec.encode_groups(x, tb, t, return_info=True)
    assert r["header_bits"] == 16
    assert np.isclose(r["bits_per_group"], np.mean(16 + info["L"]))
    assert np.isclose(r["clipped"], info["clipped"].mean())
    err = study.pattern_errors(x, tb, t)
    assert np.isclose(r["mse"], err[np.arange(len(x)), info["p"]].sum() / (len(x) * 127), rtol=1e-12)


def test_assign_groups_matches_the_codec_choice():
    tb = _golden()
    x, t = _case(500)
    p, sym, _ = study.assign_groups(x, tb.centroids, t)
    _, info = codec.encode_groups(x, tb, t, return_info=True)
    assert np.array_equal(p, info["p"]) and np.array_equal(sym, info["sym"])


def test_design_space_small_sweep():
    """Every configuration yields finite numbers, and the header takes
    log2 S + log2 H + 8 bits."""
    sample = W.c1_sample(n_values=128 * 128).numpy()
    x, t = _case(200)
    ts = codec.tensor_scale(float(np.max(np.abs(sample.astype(np.float32)))))[0]
    res = study.design_space(sample, x, ts, t, S_list=(16, 64), H_list=(1, 4), kmeans_iters=3, huff_iters=3)
    assert set(res) == {(16, 1), (16, 4), (64, 1), (64, 4)}
    assert res[(16, 1)]["header_bits"] == 12 and res[(64, 4)]["header_bits"] == 16
    for r in res.values():
        assert np.isfinite(r["mse"]) and 0 <= r["clipped"] <= 1 and r["bits_per_group"] > 0


def test_v1_tables_hold_every_design_point_the_block_can_carry():
    """Design points with S in {16, 32, 64} and H in {1, 2, 4} written into the
    v1 table slots: the codec uses only p < S and h < H, and its coded length
    of every group is the design point's (the shortest of the H books of the
    min/max pattern), so only the header's fixed 16 bits differ."""
    sample = W.c1_sample(n_values=128 * 128).numpy()
    x, t = _case(300)
    ts = codec.tensor_scale(float(np.max(np.abs(sample.astype(np.float32)))))[0]
    tabs = study.design_tables(sample, ts, S_list=(16, 32, 64), H_list=(1, 2, 4), kmeans_iters=3, huff_iters=3)
    for (S, H), (c, L) in sorted(tabs.items()):
        tb = study.v1_tables(c, L)
        tb.check()
        blocks, info = codec.encode_groups(x, tb, t, return_info=True)
        assert info["p"].max() < S and info["h"].max() < H, (S, H)
        assert np.all((blocks[:, 0] & 63) < S) and np.all((blocks[:, 0] >> 6) < H)
        p, sym, _ = study.assign_groups(x, c, t)
        assert np.array_equal(p, info["p"] % S)
        lens = np.asarray(L, np.int64)[p]
        Lh = np.stack([np.take_along_axis(lens[:, h, :], sym, axis=1).sum(axis=1) for h in range(H)], axis=1)
        assert np.array_equal(Lh.min(axis=1), info["L"]), (S, H)
        r = study.design_point(x, c, L, t)
        assert np.isclose(r["clipped"], np.mean(r["header_bits"] + info["L"] > 512))
    import pytest
    with pytest.raises(ValueError):
        study.v1_tables(tabs[(16, 1)][0][:12], tabs[(16, 1)][1][:12])
