"""Pattern-selection study (oracle; test infrastructure only).

The pages choose a group's pattern by comparing only the group's min and max
with each pattern's end centroids, and call a full MSE search too expensive
for the online (KV-cache) compressor; the referee report asks how often the
cheap rule picks a different pattern than the MSE-optimal one and what that
costs, and the free-parameter row on the pattern count sets S = 64 while
the online compressor is described with 16 (Ecco review, "What carries the
argument"; referee report; "Assumptions & free parameters", section 4.3).

pattern_errors(x, tables, t) -> [G, S] quantisation error of every group under
every pattern: the sum over the 127 values other than the scale element of
(x_j - q_j)^2 in float64, where q_j = fp16(c_p[sym_j] * a) and sym_j is the
encoder's midpoint rule (#{k : x_j > m_pk * a}) -- the reconstruction a block
gives before entropy coding (no clipping, no outlier padding).
selection_study(...) compares the encoder's min/max choice with the argmin of
those errors.

    python -m oracle.study     prints the study for the weight and KV
                               workloads with 64 and 16 patterns
    python -m oracle.study design-space
                               the S x H sweep: quantisation MSE, coded
                               bits per group and clipped fraction for
                               S in {16, 32, 64, 128}, H in {1, 2, 4, 8}
                               (header log2 S + log2 H + 8 bits); S = 128
                               and H = 8 do not fit the v1 header and are
                               evaluated without building blocks
"""

import numpy as np

from . import fp
from .codec import encode_groups, decode_blocks, GROUP, Tables

F32 = np.float32


def pattern_errors(x, tables, t, chunk=2048):
    x = np.asarray(x, dtype=np.float16).reshape(-1, GROUP)
    G = x.shape[0]
    out = np.empty((G, tables.centroids.shape[0]), dtype=np.float64)
    m = tables.midpoints()[:, :14]                                   # [S, 14]
    c = tables.centroids                                              # [S, 15]
    t = F32(t)
    inv_t = F32(F32(1.0) / t)
    for g0 in range(0, G, chunk):
        xx = x[g0:g0 + chunk].astype(np.float32)
        n = xx.shape[0]
        rows = np.arange(n)
        istar = np.argmax(np.abs(xx), axis=1)
        s8 = fp.fp8_encode((xx[rows, istar] * inv_t).astype(np.float32))
        a = np.abs((fp.fp8_decode(s8) * t).astype(np.float32))
        thr = (m[None, :, :] * a[:, None, None]).astype(np.float32)          # [n, S, 14]
        sym = np.sum(xx[:, None, :, None] > thr[:, :, None, :], axis=3)       # [n, S, 128]
        rec = (c[None, :, :] * a[:, None, None]).astype(np.float32)          # [n, S, 15]
        q = np.take_along_axis(rec, np.minimum(sym, 14), axis=2)              # [n, S, 128]
        q = fp.fp16_rne(q).astype(np.float64)
        d = (xx[:, None, :].astype(np.float64) - q) ** 2
        d[rows, :, istar] = 0.0
        out[g0:g0 + n] = d.sum(axis=2)
    return out


def selection_study(x, tables, t):
    """Fractions and errors of the min/max choice against the MSE-optimal one."""
    x = np.asarray(x, dtype=np.float16).reshape(-1, GROUP)
    err = pattern_errors(x, tables, t)
    _, info = encode_groups(x, tables, t, return_info=True)
    p_mm = info["p"]
    rows = np.arange(x.shape[0])
    e_mm = err[rows, p_mm]
    e_opt = err.min(axis=1)
    differs = e_mm > e_opt                     # a different, strictly better pattern exists
    n_vals = x.shape[0] * (GROUP - 1)
    return dict(groups=int(x.shape[0]), frac_differs=float(differs.mean()),
                mse_minmax=float(e_mm.sum() / n_vals), mse_optimal=float(e_opt.sum() / n_vals),
                gap=float(e_mm.sum() / max(e_opt.sum(), 1e-300) - 1.0))


def codec_report(x, tables, t):
    """End-to-end numbers of the block codec on x: reconstruction MSE relative
    to the variance, clipped fraction and padded outliers per group."""
    x = np.asarray(x, dtype=np.float16).reshape(-1, GROUP)
    blocks, info = encode_groups(x, tables, t, return_info=True)
    y = decode_blocks(blocks, tables, t).astype(np.float64)
    xf = x.astype(np.float64)
    mse = float(np.mean((xf - y) ** 2))
    return dict(rel_mse=mse / float(np.var(xf)), clipped=float(info["clipped"].mean()),
                outliers_per_group=float(info["n"].mean()))


def assign_groups(x, centroids, t):
    """The encoder's steps 1-4 for an arbitrary number of patterns: pattern p
    (min/max rule, lowest on ties), symbols (scale element = 15) and the
    quantisation error of each group (as pattern_errors, chosen pattern)."""
    x = np.asarray(x, dtype=np.float16).reshape(-1, GROUP)
    c = np.asarray(centroids, np.float32)
    m = ((c[:, :-1] + c[:, 1:]).astype(np.float32) * F32(0.5)).astype(np.float32)       # [S, 14]
    t = F32(t)
    inv_t = F32(F32(1.0) / t)
    xx = x.astype(np.float32)
    n = xx.shape[0]
    rows = np.arange(n)
    istar = np.argmax(np.abs(xx), axis=1)
    s8 = fp.fp8_encode((xx[rows, istar] * inv_t).astype(np.float32))
    a = np.abs((fp.fp8_decode(s8) * t).astype(np.float32))
    others = np.ones_like(xx, dtype=bool)
    others[rows, istar] = False
    gmin = np.min(np.where(others, xx, F32(np.inf)), axis=1).astype(np.float32)
    gmax = np.max(np.where(others, xx, F32(-np.inf)), axis=1).astype(np.float32)
    d1 = (gmin[:, None] - (c[None, :, 0] * a[:, None]).astype(np.float32)).astype(np.float32)
    d2 = (gmax[:, None] - (c[None, :, -1] * a[:, None]).astype(np.float32)).astype(np.float32)
    p = np.argmin((d1 * d1 + d2 * d2).astype(np.float32), axis=1)
    thr = (m[p] * a[:, None]).astype(np.float32)
    sym = np.sum(xx[:, :, None] > thr[:, None, :], axis=2)
    q = fp.fp16_rne((c[p][rows[:, None], sym] * a[:, None]).astype(np.float32)).astype(np.float64)
    err = (xx.astype(np.float64) - q) ** 2
    err[rows, istar] = 0.0
    sym[rows, istar] = 15
    return p, sym, err.sum(axis=1)


def design_point(x, centroids, code_len, t):
    """Bits and error of the block codec with S patterns and H codebooks
    (header log2 S + log2 H + 8 bits, 512-bit blocks): mean quantisation MSE,
    mean coded bits per group (header + shortest codebook), clipped fraction."""
    S, H = np.asarray(code_len).shape[:2]
    p, sym, err = assign_groups(x, centroids, t)
    lens = np.asarray(code_len, np.int64)[p]                                    # [G, H, 16]
    Lh = np.stack([np.take_along_axis(lens[:, h, :], sym, axis=1).sum(axis=1) for h in range(H)], axis=1)
    L = Lh.min(axis=1)
    header = int(np.ceil(np.log2(S))) + int(np.ceil(np.log2(H))) + 8
    return dict(mse=float(err.sum() / (len(p) * (GROUP - 1))), bits_per_group=float(np.mean(header + L)),
                clipped=float(np.mean(header + L > 512)), header_bits=header)


def design_tables(sample, t_sample, S_list=(16, 32, 64, 128), H_list=(1, 2, 4, 8), kmeans_iters=25,
                  huff_iters=10, seed=0):
    """Tables for every (S, H) from one sample (the 1-D k-means runs once):
    {(S, H): (centroids [S, 15], code_len [S, H, 16])}.  Codebooks are
    learned with the trainer's rule (oracle/train.py) on the groups the
    min/max rule gives each pattern."""
    from .kmeans import kmeans_1d_exact, lloyd
    from .train import normalised_groups, learn_codebooks
    xs = np.asarray(sample, np.float16).reshape(-1, GROUP)
    vecs, _ = kmeans_1d_exact(normalised_groups(xs, t_sample), 15)
    out = {}
    for S in S_list:
        cent, _ = lloyd(vecs, min(S, vecs.shape[0]), kmeans_iters, seed)
        cent = np.clip(np.sort(cent.astype(np.float16).astype(np.float32), axis=1), -1.0, 1.0)
        cent = cent.astype(np.float16).astype(np.float32)
        p, sym, _ = assign_groups(xs, cent, t_sample)
        counts = np.zeros((xs.shape[0], 16), dtype=np.int64)
        np.add.at(counts, (np.repeat(np.arange(xs.shape[0]), GROUP), sym.ravel()), 1)
        for H in H_list:
            code_len = np.stack([learn_codebooks(counts[p == k], H, huff_iters) for k in range(cent.shape[0])])
            out[(S, H)] = (cent, code_len)
    return out


def design_space(sample, x, t_sample, t, S_list=(16, 32, 64, 128), H_list=(1, 2, 4, 8), kmeans_iters=25,
                 huff_iters=10, seed=0):
    """Learn tables for every (S, H) from one sample and evaluate each on x."""
    tabs = design_tables(sample, t_sample, S_list, H_list, kmeans_iters, huff_iters, seed)
    return {k: design_point(x, c, l, t) for k, (c, l) in tabs.items()}


def v1_tables(centroids, code_len):
    """A design point with S <= 64 patterns and H <= 4 codebooks written into
    the v1 block's 64 x 4 table slots: slot p holds pattern p mod S and book h
    of a pattern holds book h mod H.  A repeated slot ties in the min/max
    fitness (or in the coded length) with a lower one and loses, so blocks use
    only p < S and h < H and the codec behaves as the design point's own."""
    c = np.asarray(centroids, np.float32)
    L = np.asarray(code_len, np.uint8)
    S, H = L.shape[:2]
    if 64 % S or 4 % H:
        raise ValueError("S must divide 64 and H must divide 4")
    return Tables(c[np.arange(64) % S], L[np.arange(64) % S][:, np.arange(4) % H])


def main_design_space():
    import workloads as W
    from .codec import tensor_scale
    gate = W.c2_layer(0, names=["gate"])["gate"].numpy()
    tw = tensor_scale(float(np.max(np.abs(gate.astype(np.float32)))))[0]
    smp = W.c2_sample("gate").numpy()
    ts = tensor_scale(float(np.max(np.abs(smp.astype(np.float32)))))[0]
    ksmp = W.kv_sample("k").numpy()
    tk = tensor_scale(float(np.max(np.abs(ksmp.astype(np.float32)))))[0]
    kx = W.kv_tensor("k", shape=(1, 8, 1024, 128)).numpy().reshape(-1, GROUP)
    for name, sample, x, t_s, t in (("llama3-8b gate weights", smp, gate.reshape(-1, GROUP)[:8192], ts, tw),
                                    ("kv-cache K", ksmp, kx, tk, tk)):
        res = design_space(sample, x, t_s, t)
        for (S, H), r in sorted(res.items()):
            print("%-24s S=%3d H=%d  header %2d b  MSE %.5g  bits/group %.1f  clipped %.1f %%"
                  % (name, S, H, r["header_bits"], r["mse"], r["bits_per_group"], 100 * r["clipped"]), flush=True)


def main():
    import workloads as W
    from .train import train_tables
    from .codec import tensor_scale
    cases = []
    w = W.c2_layer(0, names=["gate"])["gate"].numpy().reshape(-1, GROUP)[:8192]
    tw = tensor_scale(float(np.max(np.abs(W.c2_layer(0, names=["gate"])["gate"].numpy().astype(np.float32)))))[0]
    cases.append(("llama3-8b gate weights", W.c2_sample("gate").numpy(), w, tw))
    for kind in ("k", "v"):
        smp = W.kv_sample(kind).numpy()
        t = tensor_scale(float(np.max(np.abs(smp.astype(np.float32)))))[0]
        x = W.kv_tensor(kind, shape=(1, 8, 1024, 128)).numpy().reshape(-1, GROUP)
        cases.append(("kv-cache " + kind.upper(), smp, x, t))
    for name, sample, x, t in cases:
        for D in (64, 16):
            tb = train_tables(sample, distinct=D)
            s = selection_study(x, tb, t)
            r = codec_report(x, tb, t)
            print("%-24s S=%2d  groups %d  min/max differs from MSE-optimal in %.1f %%  MSE min/max %.4g  "
                  "optimal %.4g  gap %+.1f %%  | codec rel. MSE %.4g  clipped %.1f %%  outliers/group %.2f"
                  % (name, D, s["groups"], 100 * s["frac_differs"], s["mse_minmax"], s["mse_optimal"],
                     100 * s["gap"], r["rel_mse"], 100 * r["clipped"], r["outliers_per_group"]), flush=True)


if __name__ == "__main__":
    import sys
    if len(sys.argv) > 1 and sys.argv[1] == "design-space":
        main_design_space()
    else:
        main()
