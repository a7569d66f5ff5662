"""Decode-phase attention over oracle-decoded K and V caches (oracle; test
infrastructure only).

For every sequence b, kv head h and query head hq = h * G + g (grouped-query
attention, G query heads per kv head), with the caches' decoded FP16 values
K, V [B, H, S, 128] and query q [B, H * G, 128]:
    s_t = scale * q . K_t ;  p = softmax(s) ;  out = sum_t p_t V_t
all in float64.  This is the consumer the pages compress the KV cache for
(Ecco review, "Core claim": KV blocks decompressed on load in the decode
phase).  attention_tolerance_ok bounds the FP32 kernel's error: the scores
are sums of 128 products, the output a convex combination of V rows.
"""

import numpy as np


def attention_ref(K, V, q, scale):
    """K, V [B, H, S, D] (any float), q [B, H * G, D] -> out [B, H * G, D] float64,
    plus mag [B, H * G, D] = sum_t p_t |V_t| (the error scale of each output)."""
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    q = np.asarray(q, np.float64)
    B, H, S, D = K.shape
    G = q.shape[1] // H
    qg = q.reshape(B, H, G, D)
    s = np.einsum("bhgd,bhtd->bhgt", qg, K) * float(scale)
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    p = e / e.sum(axis=-1, keepdims=True)
    out = np.einsum("bhgt,bhtd->bhgd", p, V)
    mag = np.einsum("bhgt,bhtd->bhgd", p, np.abs(V))
    return out.reshape(B, H * G, D), mag.reshape(B, H * G, D)


def attention_tolerance_ok(out, ref, mag, rel=1e-3):
    """|out - ref| <= rel * max(|ref|, mag) elementwise; returns (ok, worst ratio)."""
    out = np.asarray(out, np.float64)
    bound = rel * np.maximum(np.abs(ref), mag) + 1e-30
    ratio = np.abs(out - ref) / bound
    return bool(np.all(ratio <= 1.0)), float(ratio.max())
