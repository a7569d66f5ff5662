"""Host-side checks of bench.py's reporting (no GPU): the quality figures the
bench line carries come from the oracle and agree with the format's closed
forms."""

import numpy as np

import bench
import entropy_coded_group_amd as ecco
import workloads as W
from oracle import codec, metrics


def test_quality_figures_follow_the_oracle_and_the_closed_forms():
    x = np.asarray(W.c1_weight()).reshape(-1, 128)
    blob = ecco.ecco_train_patterns(W.c1_sample(n_values=1 << 16), kmeans_iters=5, huff_iters=3)
    t = float(ecco.ecco_tensor_scale_from_amax(float(np.abs(x.astype(np.float32)).max())))
    q = bench.oracle_quality(x, blob, t, 512)
    assert q["groups"] == 512
    # the ratio is that of the whole tensor: 512-bit blocks per 2048 FP16 bits,
    # plus the per-tensor side tables
    n = x.shape[0]
    assert abs(q["compression_ratio"] - 2048.0 * n / (512.0 * n + 8.0 * metrics.table_bytes_v1())) < 1e-12
    assert 3.9 < q["compression_ratio"] < 4.0
    # MSE is that of the oracle's own round trip on the sample
    c, l = ecco.ecco_tables_get(blob)
    tb = codec.Tables(c, l)
    y = codec.decode_blocks(codec.encode_groups(x[:512], tb, t), tb, t)
    mse = float(np.mean((x[:512].astype(np.float64) - y.astype(np.float64)) ** 2))
    assert q["mse"] == mse
    assert 0.0 < q["rel_mse"] < 0.1
    assert 0.0 <= q["clipped_group_frac"] <= 1.0 and 0.0 <= q["mean_padded_outliers"] <= 16.0
    assert 0.0 < q["achieved_bits_per_index"] <= 8.0
