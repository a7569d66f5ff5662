"""Seeded synthetic inputs shaped like the workloads the Ecco pages evaluate on.

The pages measure on LLaMA / LLaMA-2 / LLaMA-3.1 / Mistral weights and KV
caches, calibrated on The Pile and evaluated on WikiText-2 (Ecco review,
"Assumptions & free parameters"; referee report).  Neither trained weights nor
datasets are available, so these generators stand in for them with the shapes
of a LLaMA-3-8B decoder layer, a GQA KV cache and 70B-shaped FFN matrices, and
with heavy-tailed value distributions (per-channel scales, sparse large
outliers, outlier channels in K).

This module holds no arithmetic of the codec: it only draws numbers.  Every
tensor is drawn with a seeded ``torch.Generator`` in float32 and cast to
float16 with round-to-nearest-even, so both the GPU path and the CPU oracle
see identical inputs on any machine.  All are drawn on the CPU except the
32-layer weight set (c4_matrix), which is drawn on the GPU it is encoded on;
the oracle then reads a host copy of the same FP16 tensor.
"""

import numpy as np
import torch

GROUP = 128

# LLaMA-3-8B decoder layer, weights [out, in]
LLAMA3_8B_LAYER = {
    "q": (4096, 4096),
    "k": (1024, 4096),
    "v": (1024, 4096),
    "o": (4096, 4096),
    "gate": (14336, 4096),
    "up": (14336, 4096),
    "down": (4096, 14336),
}
LAYER_ORDER = ["q", "k", "v", "o", "gate", "up", "down"]

# 70B-shaped FFN matrices for the fused decode+GEMV
FFN70B = {"w1": (28672, 8192), "w2": (8192, 28672)}

# KV cache [batch, kv_heads, seq, head_dim]
KV_SHAPE = (16, 8, 8192, 128)
KV_APPEND = 256

# Activations (2x format, groups of 64): LLaMA-3-8B hidden states
# [tokens, hidden] of one 16k-token prefill
ACT_SHAPE = (16384, 4096)
ACT_GROUP = 64


def _gen(seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _laplace(n, scale, g):
    u = torch.rand(n, generator=g, dtype=torch.float64) - 0.5
    return (-scale * torch.sign(u) * torch.log1p(-2.0 * u.abs())).to(torch.float32)


def _outlier_index(n, frac, g):
    m = int(round(frac * n))
    return torch.randperm(n, generator=g)[:m]


def c1_weight(seed=0, shape=(1024, 1024), std=0.02, frac=0.001, lap_scale=0.2):
    """Single weight matrix: N(0, std) with a fraction of entries replaced by
    Laplace(0, lap_scale) draws."""
    g = _gen(seed)
    n = shape[0] * shape[1]
    w = torch.randn(n, generator=g, dtype=torch.float32) * std
    idx = _outlier_index(n, frac, g)
    w[idx] = _laplace(idx.numel(), lap_scale, g)
    return w.reshape(shape).to(torch.float16)


def c1_sample(seed=1, n_values=1 << 20):
    """Calibration sample for c1_weight (same recipe, separate seed)."""
    return c1_weight(seed=seed, shape=(n_values // 1024, 1024))


def llama_matrix(shape, seed, sigma=0.5, frac=0.0005, boost=20.0):
    """W = s_o * z with per-output-row s_o ~ LogNormal(0, sigma), z ~ N(0, 1),
    then a fraction of entries multiplied by `boost`."""
    g = _gen(seed)
    out_f, in_f = shape
    s = torch.exp(sigma * torch.randn(out_f, 1, generator=g, dtype=torch.float32))
    z = torch.randn(out_f, in_f, generator=g, dtype=torch.float32)
    w = (s * z).reshape(-1)
    idx = _outlier_index(w.numel(), frac, g)
    w[idx] = w[idx] * boost
    return w.reshape(shape).to(torch.float16)


def llama_sample(in_features, seed, n_values=1 << 20):
    """Calibration sample of the llama_matrix recipe with the given input width."""
    rows = max(1, n_values // in_features)
    return llama_matrix((rows, in_features), seed)


def c2_layer(layer=0, names=None):
    """One LLaMA-3-8B-shaped decoder layer; matrix m of layer l uses seed 100 + 10 l + m."""
    names = names or LAYER_ORDER
    return {nm: llama_matrix(LLAMA3_8B_LAYER[nm], 100 + 10 * layer + LAYER_ORDER.index(nm))
            for nm in names}


N_LAYERS = 32


def c4_matrix(layer, name, device="cuda"):
    """Matrix `name` of layer `layer` of the 32-layer LLaMA-3-8B-shaped weight
    set, drawn on `device` by torch's generator for that device (seed
    100 + 10 layer + m, m the matrix's place in LAYER_ORDER): the layer
    recipe of llama_matrix -- per-output-row LogNormal(0, 0.5) scales times
    N(0, 1) entries, then 0.05 % of the entries (a randperm prefix) x20 --
    drawn where the weights will live, so that 7e9 values take seconds to
    make.  The same call gives the same tensor on any MI355X; a host copy of
    it is what the oracle sees."""
    m = LAYER_ORDER.index(name)
    out_f, in_f = LLAMA3_8B_LAYER[name]
    g = torch.Generator(device=device)
    g.manual_seed(100 + 10 * int(layer) + m)
    s = torch.exp(0.5 * torch.randn(out_f, 1, generator=g, device=device, dtype=torch.float32))
    w = (s * torch.randn(out_f, in_f, generator=g, device=device, dtype=torch.float32)).reshape(-1)
    idx = torch.randperm(w.numel(), generator=g, device=device)[:int(round(0.0005 * w.numel()))]
    w[idx] = w[idx] * 20.0
    return w.to(torch.float16).reshape(out_f, in_f)


def c2_sample(name):
    """Calibration sample for matrix type `name` (seed 900 + m)."""
    m = LAYER_ORDER.index(name)
    return llama_sample(LLAMA3_8B_LAYER[name][1], 900 + m)


def kv_tensor(kind, shape=KV_SHAPE, seed=None, outlier_seed=2, n_outlier_ch=4, boost=10.0):
    """K or V cache [B, H, S, D]: N(0, 1); K gets n_outlier_ch fixed channels per
    kv-head scaled by `boost`."""
    if seed is None:
        seed = 0 if kind == "k" else 1
    g = _gen(seed)
    B, H, S, D = shape
    x = torch.randn(shape, generator=g, dtype=torch.float32)
    if kind == "k":
        go = _gen(outlier_seed)
        for hh in range(H):
            ch = torch.randperm(D, generator=go)[:n_outlier_ch]
            x[:, hh, :, ch] *= boost
    return x.to(torch.float16)


def kv_sample(kind, n_vectors=8192):
    """Calibration sample for the KV codec: n_vectors head vectors of the same
    recipe (seed 3 for K, 4 for V), with the same outlier channels."""
    seed = 3 if kind == "k" else 4
    B, H, S, D = KV_SHAPE
    s = max(1, n_vectors // H)
    return kv_tensor(kind, shape=(1, H, s, D), seed=seed)


def act_tensor(shape=ACT_SHAPE, seed=600, n_outlier_ch=6, boost=30.0):
    """Hidden states [tokens, hidden]: Laplace(0, 1) values times a per-token
    scale exp(N(0, 0.25)), with n_outlier_ch fixed channels (the same for every
    token) scaled by `boost` -- the few very large activation channels of
    LLM hidden states."""
    g = _gen(seed)
    T, D = shape
    x = _laplace(T * D, 1.0, g).reshape(T, D)
    x *= torch.exp(0.5 * torch.randn(T, 1, generator=g, dtype=torch.float32))
    ch = torch.randperm(D, generator=_gen(610))[:n_outlier_ch]
    x[:, ch] *= boost
    return x.to(torch.float16)


def act_sample(n_tokens=256):
    """Calibration sample for the activation codec: n_tokens hidden-state rows
    of the same recipe (seed 601), with the same outlier channels."""
    return act_tensor(shape=(n_tokens, ACT_SHAPE[1]), seed=601)


def c5_matrix(name):
    return llama_matrix(FFN70B[name], 500 if name == "w1" else 501)


def c5_sample(name):
    return llama_sample(FFN70B[name][1], 510 if name == "w1" else 511)


def c5_x(batch, in_features, seed=502):
    g = _gen(seed)
    return torch.randn(batch, in_features, generator=g, dtype=torch.float32).to(torch.float16)


def random_blocks(n_blocks, seed):
    """Uniformly random 512-bit blocks (decoder totality checks)."""
    g = _gen(seed)
    return torch.randint(0, 256, (n_blocks, 64), generator=g, dtype=torch.int64).to(torch.uint8)


def random_groups(n_groups, seed, kind="normal"):
    """Small assorted groups for parity sweeps: normal, heavy-tailed, wide-range
    or tie-heavy."""
    g = _gen(seed)
    if kind == "normal":
        x = torch.randn(n_groups, GROUP, generator=g, dtype=torch.float32)
    elif kind == "laplace":
        x = _laplace(n_groups * GROUP, 1.0, g).reshape(n_groups, GROUP)
    elif kind == "wide":
        e = torch.randint(-20, 12, (n_groups, GROUP), generator=g).to(torch.float32)
        x = torch.randn(n_groups, GROUP, generator=g, dtype=torch.float32) * torch.exp2(e)
    elif kind == "ties":
        # values from {0, +-1, +-2, +-4} times a per-group power of two: many
        # equal magnitudes (largest-|x| ties, equal min / max, equal outlier
        # candidates) and values on exact binary fractions
        levels = torch.tensor([0.0, 1.0, -1.0, 2.0, -2.0, 4.0, -4.0])
        idx = torch.randint(0, len(levels), (n_groups, GROUP), generator=g)
        e = torch.randint(-12, 8, (n_groups, 1), generator=g).to(torch.float32)
        x = levels[idx] * torch.exp2(e)
    else:
        raise ValueError(kind)
    return x.to(torch.float16)


def as_numpy(t):
    return t.contiguous().numpy()


__all__ = [n for n in dir() if not n.startswith("_")]
