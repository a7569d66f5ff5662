"""Quality figures the pages report for the codec (oracle; test infrastructure only).

  * reconstruction error of the lossy code (the pages judge it through model
    perplexity, which needs trained weights; here MSE and MSE / var(x));
  * memory reduction: blocks of 512 bits per 128 FP16 values give 4x by
    construction, 3.98x once side tables are counted (Ecco review,
    circularity check; Fig. 12 caption);
  * padding and clipping ratios (Fig. 10 caption; "Reading between the lines":
    2-8 % KV padding);
  * index entropy against achieved bits per index (Fig. 2 caption; "most
    weight groups have far lower than 4-bit entropy").
All in float64.
"""

import numpy as np

from .codec import GROUP, BLOCK_BITS, RECORD_BITS


def reconstruction(x, y):
    x = np.asarray(x, dtype=np.float64).ravel()
    y = np.asarray(y, dtype=np.float64).ravel()
    mse = float(np.mean((x - y) ** 2)) if x.size else 0.0
    var = float(np.var(x)) if x.size else 0.0
    return dict(mse=mse, rel_mse=mse / var if var > 0 else float("nan"))


def compression_ratio(n_groups, table_bytes):
    """FP16 bits over stored bits, the side tables included."""
    return (2048.0 * n_groups) / (512.0 * n_groups + 8.0 * table_bytes)


def table_bytes_v1():
    """Bytes of the side data the format needs per tensor: 64x15 FP16 centroids,
    64x4x16 code lengths (4 bits each suffice, counted as bytes), one FP32 t."""
    return 64 * 15 * 2 + 64 * 4 * 16 + 4


def padding_figures(info):
    n_groups = len(info["k"])
    clipped = np.asarray(info["clipped"])
    return dict(
        clipped_group_frac=float(np.mean(clipped)) if n_groups else 0.0,
        clipped_value_frac=float(np.sum(GROUP - np.asarray(info["k"])) / max(1, n_groups * GROUP)),
        mean_padded_outliers=float(np.mean(info["n"])) if n_groups else 0.0,
        pad_bit_frac=float(np.sum(RECORD_BITS * np.asarray(info["n"])) / max(1, n_groups * BLOCK_BITS)),
    )


def index_entropy(info):
    """Entropy (bits) of the centroid-index histogram of each group, averaged,
    against achieved code bits per index (unclipped length / 128)."""
    sym = np.asarray(info["sym"])
    ent = []
    for row in sym:
        cnt = np.bincount(row, minlength=16).astype(np.float64)
        pr = cnt[cnt > 0] / cnt.sum()
        ent.append(float(-(pr * np.log2(pr)).sum()))
    return dict(mean_group_entropy_bits=float(np.mean(ent)) if ent else 0.0,
                achieved_bits_per_index=float(np.mean(np.asarray(info["L"]) / GROUP)) if ent else 0.0)
