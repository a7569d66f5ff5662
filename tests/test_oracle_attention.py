"""Pins of the attention oracle (oracle/attention.py)."""

import numpy as np

from oracle import attention


def test_matches_row_by_row_definition():
    rng = np.random.default_rng(0)
    K = rng.normal(size=(2, 3, 7, 8))
    V = rng.normal(size=(2, 3, 7, 8))
    q = rng.normal(size=(2, 6, 8))
    out, mag = attention.attention_ref(K, V, q, 0.3)
    for b in range(2):
        for hq in range(6):
            h = hq // 2
            s = np.array([0.3 * sum(q[b, hq, d] * K[b, h, t, d] for d in range(8)) for t in range(7)])
            p = np.exp(s - s.max())
            p /= p.sum()
            o = sum(p[t] * V[b, h, t] for t in range(7))
            m = sum(p[t] * np.abs(V[b, h, t]) for t in range(7))
            assert np.allclose(o, out[b, hq], rtol=1e-13, atol=0)
            assert np.allclose(m, mag[b, hq], rtol=1e-13, atol=0)


def test_closed_forms():
    rng = np.random.default_rng(1)
    K = rng.normal(size=(1, 2, 9, 4))
    V = rng.normal(size=(1, 2, 9, 4))
    # zero query: uniform weights, the mean of the V rows
    out, _ = attention.attention_ref(K, V, np.zeros((1, 4, 4)), 1.0)
    assert np.allclose(out.reshape(1, 2, 2, 4), V.mean(axis=2)[:, :, None, :], rtol=1e-13)
    # one token: its V row
    out, _ = attention.attention_ref(K[:, :, :1], V[:, :, :1], rng.normal(size=(1, 4, 4)), 1.0)
    assert np.allclose(out.reshape(1, 2, 2, 4), V[:, :, :1][:, :, None, 0, :].repeat(2, axis=2), rtol=1e-13)
    # equal V rows: that row whatever the scores
    Vc = np.repeat(V[:, :, :1], 9, axis=2)
    out, _ = attention.attention_ref(K, Vc, rng.normal(size=(1, 4, 4)), 2.0)
    assert np.allclose(out.reshape(1, 2, 2, 4), Vc[:, :, :1][:, :, None, 0, :].repeat(2, axis=2), rtol=1e-13)
    # a dominant score picks its row
    Kd = np.zeros((1, 1, 5, 4)); Kd[0, 0, 3] = [100, 0, 0, 0]
    out, _ = attention.attention_ref(Kd, V[:, :1, :5], np.array([[[1.0, 0, 0, 0]]]), 1.0)
    assert np.allclose(out[0, 0], V[0, 0, 3], rtol=1e-12)


def test_tolerance_check():
    ref = np.array([1.0, -2.0, 0.0])
    mag = np.array([1.0, 2.0, 1.0])
    assert attention.attention_tolerance_ok(ref + 5e-4, ref, mag)[0]
    assert not attention.attention_tolerance_ok(ref + 3e-3, ref, mag)[0]
