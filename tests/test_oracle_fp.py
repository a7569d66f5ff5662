"""Pins for the oracle's number formats (CPU only).

FP8 E4M3FN is checked against the OCP specification's table values and, over
large input sets, against torch's independent float8_e4m3fn cast after the
codec's saturation to +-448; FP16 rounding is checked against torch's cast.
"""

import json
import os

import numpy as np
import torch

from oracle import fp

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _torch_fp8(v32):
    t = torch.from_numpy(np.clip(v32, -448.0, 448.0).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_fp8_spec_table_values():
    g = json.load(open(os.path.join(GOLD, "ocp_fp8_e4m3.json")))
    for code, val in g["pairs"]:
        got = fp.fp8_decode(np.array([code], np.uint8))[0]
        assert got == np.float32(val) and np.signbit(got) == np.signbit(val), (code, val, got)
        assert fp.fp8_encode(np.array([val], np.float32))[0] == code
    for code in g["nan_codes"]:
        assert np.isnan(fp.fp8_decode(np.array([code], np.uint8))[0])


def test_fp8_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = fp.fp8_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_fp8_encode_ties_and_neighbours_vs_torch():
    vals = fp.fp8_decode(np.arange(256, dtype=np.uint8))
    fin = np.sort(np.unique(vals[np.isfinite(vals)]))
    mids = ((fin[:-1].astype(np.float64) + fin[1:]) / 2).astype(np.float32)   # exact ties
    cand = np.concatenate([fin, mids, np.nextafter(mids, np.float32(np.inf)),
                           np.nextafter(mids, np.float32(-np.inf)),
                           np.float32([449, 460, 464, 470, 479.9, 480, 1e6, -1e6, 2 ** -12, -2 ** -12])])
    cand = cand.astype(np.float32)
    assert np.array_equal(fp.fp8_encode(cand), _torch_fp8(cand))


def test_fp8_encode_random_bits_vs_torch():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    assert np.array_equal(fp.fp8_encode(v), _torch_fp8(v))
    # dense sweep of the interesting range
    w = (rng.standard_normal(1_000_000) * np.exp2(rng.integers(-14, 10, 1_000_000))).astype(np.float32)
    assert np.array_equal(fp.fp8_encode(w), _torch_fp8(w))


def test_fp8_encode_all_fp16_inputs_vs_torch():
    h = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float32)
    h = h[np.isfinite(h)]
    for scale in (1.0, 1 / 448.0, 3.7, 1e-3, 250.0):
        v = (h * np.float32(scale)).astype(np.float32)
        assert np.array_equal(fp.fp8_encode(v), _torch_fp8(v)), scale


def test_fp8_roundtrip_is_identity_on_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(fp.fp8_encode(fp.fp8_decode(codes)), codes)


def test_fp8_saturates_and_never_nan():
    v = np.float32([1e30, -1e30, np.inf, -np.inf, 448.0, 500.0])
    out = fp.fp8_encode(v)
    assert list(out) == [0x7E, 0xFE, 0x7E, 0xFE, 0x7E, 0x7E]


def test_fp16_rne_vs_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[~np.isnan(v)]
    ours = fp.fp16_rne(v).view(np.uint16)
    ref = torch.from_numpy(v).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
