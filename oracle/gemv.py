"""Reference GEMV over codec-decoded weights (oracle; test infrastructure only).

The pages' consumer of compressed weights is the decode-phase GEMM of LLM
inference, which is memory-bound at small batch (Ecco review, "If this is
right": speedups concentrate at small batch and long sequences; Fig. 12
caption: normalised memory requests for a GEMM kernel).  The plain definition
is y[b, o] = sum_i W_hat[o, i] * x[b, i] with W_hat the decoded FP16 weights;
it is evaluated here in float64.
"""

import numpy as np

from .codec import decode_blocks, GROUP


def decoded_weight(blocks, tables, t, out_features, in_features):
    w = decode_blocks(blocks.reshape(-1, 64), tables, t)
    return w.reshape(out_features, in_features)


def gemv_ref(w_hat, x):
    """w_hat [out, in] float16, x [batch, in] float16 -> y [batch, out] float64,
    plus the per-element scale sum_i |w x| used by the tolerance rule."""
    w = np.asarray(w_hat, dtype=np.float64)
    xx = np.asarray(x, dtype=np.float64)
    y = xx @ w.T
    mag = np.abs(xx) @ np.abs(w).T
    return y, mag


def gemv_tolerance_ok(y_test, y_ref, mag, in_features, rel=1e-3):
    """|y - y_ref| <= rel * max(|y_ref|, sum_i |w x| / sqrt(in)) elementwise."""
    bound = rel * np.maximum(np.abs(y_ref), mag / np.sqrt(float(in_features)))
    err = np.abs(np.asarray(y_test, dtype=np.float64) - y_ref)
    return bool(np.all(err <= bound)), float(np.max(err / np.maximum(bound, 1e-300)))


__all__ = ["decoded_weight", "gemv_ref", "gemv_tolerance_ok", "GROUP"]
