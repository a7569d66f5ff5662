"""Benchmark of the Ecco block codec on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload model|layer|weight|kv|ffn|attn|act|design|copy] [--gpus 1]

Default workload ("model"): the 32-layer LLaMA-3-8B-shaped weight set in
FP16, 6.98e9 parameters (13.96 GB) resident in HBM.  Each layer has q, o
[4096, 4096], k, v [1024, 4096], gate, up [14336, 4096] and down
[4096, 14336], drawn on the GPU (workloads.c4_matrix) with per-output-row
LogNormal(0, 0.5) scales times N(0, 1) entries and 0.05 % of entries x20;
groups of 128 along the input dimension (1,703,936 groups per layer,
54,525,952 in all, 3.49 GB of blocks).  Tables for each matrix type are
learned by ecco_train_patterns from a separate seeded 2**20-value sample of
the same recipe (offline, outside the timed region) and serve all 32 layers.

One step runs every row of the hot path over all 32 layers: per layer one
ecco_amax_many call over the seven matrices; then per layer one
ecco_encode_many launch; then per layer one ecco_decode_many launch into one
reused FP16 buffer of a layer's size (a layer's blocks were written 31
layers -- 3.4 GB of other traffic -- earlier, so they come from HBM, not the
256 MB last-level cache); then per layer the fused decode+GEMV at batch 1 as
a decode step issues it: ecco_decode_gemv_many over q, k, v (same x), then
o, then gate and up (same x), then down.  Each phase of a step (its 32 or
128 launches, back to back) is bracketed by one pair of HIP events on the
stream it runs on.  The reported value is decode throughput -- (64 B
compressed in + 256 B FP16 out) per group over the summed decode phase time
of the timed steps; encode (256 B in + 64 B out per group), amax and the
fused GEMV are reported beside it.

Other workloads (run separately, same JSON line shape):
  layer  one layer of the set above, drawn on the CPU: the same step on one
         layer, plus diagnostics (each matrix decoded by a launch of its own
         and by ecco_decode_speculative, the pages' segment-parallel decode,
         and by ecco_decode_segmented with 2, 4 and 8 lanes per block;
         each amax, encode and GEMV by a call of its own; the step captured
         into a HIP graph and replayed)
  weight one 1024x1024 weight (8,192 groups; launch-bound): amax, encode
         and decode, one call each, device time per call and the
         host-inclusive time of a step
  kv     K and V caches [16, 8, 8192, 128]: append-encode of the last 256
         tokens per row (strided) and decode of the whole cache
  ffn    70B-shaped FFN matrices [28672, 8192], [8192, 28672]: fused
         decode+GEMV at batch 1, 4, 8 against decode followed by a dense GEMV
  attn   decode-phase attention over the compressed K and V caches
         [16, 8, 8192, 128] with 4 query heads per kv head: the fused
         ecco_attention_decode against decode followed by torch's SDPA
  act    the 2x activation format (groups of 64) on LLaMA-3-8B hidden
         states [16384, 4096]: amax, encode and decode
  design the S x H design points the v1 block holds (S in {16, 32, 64}
         patterns, H in {1, 2, 4} codebooks): encode and decode time and the
         codec's quality per point on the gate projection, K, V and the
         1024x1024 weight
  copy   a plain 1 GiB device-to-device copy (the achievable-bandwidth
         reference, and the known-size kernel that calibrates the HBM
         traffic counters FETCH_SIZE / WRITE_SIZE)

The CPU baseline is the oracle (NumPy) timed on a bounded sample of the same
workload on this host -- the first 65,536 groups of layer 0's q: split over
up to 16 worker processes (the reported value), and on one core in-process;
beside it, the one-group-at-a-time oracle (plain Python) on the first 1,024
groups of that sample, on one core.  The codec's quality figures
(reconstruction MSE, compression ratio, clipping and padding) come from the
oracle on the first 8,192 groups of the same q ("quality").
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BYTES_PER_GROUP = 64 + 256


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="model",
                    choices=["model", "layer", "weight", "kv", "ffn", "attn", "act", "design", "copy"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-groups", type=int, default=65536)
    return ap.parse_args()


class Timer:
    """Per-launch HIP event pairs on the given stream, summed per phase."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream
        self.pending = {}

    def run(self, phase, fn):
        ev0 = self.torch.cuda.Event(enable_timing=True)
        ev1 = self.torch.cuda.Event(enable_timing=True)
        ev0.record(self.stream)
        fn()
        ev1.record(self.stream)
        self.pending.setdefault(phase, []).append((ev0, ev1))

    def collect(self):
        out = {k: [a.elapsed_time(b) * 1e-3 for a, b in v] for k, v in self.pending.items()}
        self.pending = {}
        return out


def d2d_copy_gbps(torch, nbytes=1 << 30, reps=20):
    a = torch.empty(nbytes // 2, dtype=torch.float16, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    return 2 * nbytes / sec / 1e9


TRAFFIC_RECORDS = {
    "model": os.path.join(ROOT, "profiles", "decode_kernel__llama3-8b-32-layers__traffic.json"),
    "layer": os.path.join(ROOT, "profiles", "decode_kernel__llama3-8b-layer__traffic.json"),
}
DECODE_SOURCES = ["entropy_coded_group_amd/csrc/ecco_device.h", "entropy_coded_group_amd/csrc/ecco_kernels.hip",
                  "entropy_coded_group_amd/csrc/ecco_internal.h"]


def decode_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per decode launch from the calibrated FETCH_SIZE / WRITE_SIZE
    counters of a profiled run of the workload, or None when the decode
    sources have changed since those counters were taken."""
    try:
        with open(TRAFFIC_RECORDS[workload]) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != decode_sources_sha256():
        return None
    return round(rec["bytes_per_launch"], 0)


def _oracle_chunk(job):
    """One worker's share of the CPU baseline: oracle encode, then decode."""
    from oracle import codec
    x, c, l, t = job
    tb = codec.Tables(c, l)
    t0 = time.perf_counter()
    blocks = codec.encode_groups(x, tb, t)
    t1 = time.perf_counter()
    codec.decode_blocks(blocks, tb, t)
    return t1 - t0, time.perf_counter() - t1


def literal_baseline(x_groups, tables_blob, t, n_groups):
    """The one-group-at-a-time oracle (plain Python loops) on the first
    n_groups groups, one core, in this process."""
    from oracle import literal
    import entropy_coded_group_amd as ecco
    c, l = ecco.ecco_tables_get(tables_blob)
    x = x_groups[:n_groups]
    t0 = time.perf_counter()
    blocks = [literal.encode_group(g, c, l, t) for g in x]
    t1 = time.perf_counter()
    for b in blocks:
        literal.decode_block(b, c, l, t)
    t2 = time.perf_counter()
    n = len(blocks)
    return dict(groups=n, encode_GBps_1core=n * BYTES_PER_GROUP / (t1 - t0) / 1e9,
                decode_GBps_1core=n * BYTES_PER_GROUP / (t2 - t1) / 1e9, seconds=t2 - t0)


def oracle_quality(x_groups, tables_blob, t, n_groups):
    """The codec's quality figures by the oracle on the first n_groups groups
    (untimed): reconstruction MSE, the compression ratio with the side tables
    counted, clipping, padding and index entropy."""
    from oracle import codec, metrics
    import entropy_coded_group_amd as ecco
    c, l = ecco.ecco_tables_get(tables_blob)
    x = x_groups[:n_groups]
    tb = codec.Tables(c, l)
    blocks, info = codec.encode_groups(x, tb, t, return_info=True)
    y = codec.decode_blocks(blocks, tb, t)
    rec = metrics.reconstruction(x.astype(np.float64), y.astype(np.float64))
    # the ratio of the whole tensor over FP16, counting the side data the
    # format needs (centroids, code lengths, t: 6,020 B) and, beside it, the
    # library's whole table blob (which adds the derived midpoints, codes and
    # decode look-up tables)
    out = dict(groups=int(x.shape[0]), mse=rec["mse"], rel_mse=rec["rel_mse"],
               compression_ratio=metrics.compression_ratio(x_groups.shape[0], metrics.table_bytes_v1()),
               compression_ratio_library_blob=metrics.compression_ratio(x_groups.shape[0],
                                                                        ecco.ecco_tables_size() + 4))
    out.update(metrics.padding_figures(info))
    out.update(metrics.index_entropy(info))
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x_groups, tables_blob, t, n_groups, workers):
    """The oracle (vectorised NumPy) on the first n_groups groups: in this
    process on one core, then split over `workers` processes (started fresh,
    warmed up before the timed map)."""
    import multiprocessing as mp
    import entropy_coded_group_amd as ecco
    c, l = ecco.ecco_tables_get(tables_blob)
    x = x_groups[:n_groups]
    n = x.shape[0]
    enc1, dec1 = _oracle_chunk((x, c, l, t))
    out = dict(decode_GBps_1core=n * BYTES_PER_GROUP / dec1 / 1e9, encode_GBps_1core=n * BYTES_PER_GROUP / enc1 / 1e9,
               seconds_1core=enc1 + dec1, groups=n)
    out.update(decode_GBps=out["decode_GBps_1core"], encode_GBps=out["encode_GBps_1core"], seconds=enc1 + dec1,
               workers=1)
    if workers < 2:
        return out
    chunks = [(part, c, l, t) for part in np.array_split(x, workers)]
    try:
        with mp.get_context("spawn").Pool(workers) as pool:
            # imports and warm-up; a worker that cannot start fails the timed
            # leg instead of hanging it
            pool.map_async(_oracle_chunk, [(part[:64], c, l, t) for part, _, _, _ in chunks]).get(timeout=180)
            t0 = time.perf_counter()
            res = pool.map_async(_oracle_chunk, chunks).get(timeout=300)
            wall = time.perf_counter() - t0
    except Exception as e:                                     # report the one-core figures only
        print("bench.py: multi-process CPU baseline skipped: %r" % (e,), file=sys.stderr)
        return out
    # encode and decode run back to back in each worker; the wall time of the
    # map is split between them in proportion to the workers' own timings
    enc_s, dec_s = sum(r[0] for r in res), sum(r[1] for r in res)
    out.update(decode_GBps=n * BYTES_PER_GROUP / (wall * dec_s / (enc_s + dec_s)) / 1e9,
               encode_GBps=n * BYTES_PER_GROUP / (wall * enc_s / (enc_s + dec_s)) / 1e9,
               seconds=wall, workers=workers)
    return out


def train_tables(ecco, sample):
    threads = min(16, os.cpu_count() or 1)
    return ecco.ecco_train_patterns(sample, threads=threads)


def graph_step_us(torch, stream, amax_jobs, encode_jobs, decode_jobs, gemv_jobs, ecco, reps):
    """The step's calls captured once into a HIP graph (torch.cuda.graph) and
    replayed: the library allocates and synchronizes nothing, so the whole
    step captures, and a replay has no per-call host work between kernels
    (replays are checked bit for bit against the eager step in the tests).
    Returns microseconds per replay."""
    def plain_step():
        ecco.ecco_amax_many(amax_jobs)
        ecco.ecco_encode_many(encode_jobs)
        ecco.ecco_decode_many(decode_jobs)
        for jobs in gemv_jobs:
            ecco.ecco_decode_gemv_many(jobs, 1)
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        plain_step()                       # warm-up on a side stream before capture
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plain_step()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def bench_model(args, torch, ecco, W):
    """The 32-layer weight set (see the module docstring).  Returns the timing
    results and layer 0's q (host copy), its tables and scale for the CPU
    baseline and the quality figures."""
    stream = torch.cuda.current_stream()
    t_setup = time.perf_counter()
    blobs = {nm: train_tables(ecco, W.c2_sample(nm)) for nm in W.LAYER_ORDER}
    tdev = {nm: ecco.tables_to_device(b) for nm, b in blobs.items()}
    amax = torch.zeros((W.N_LAYERS, len(W.LAYER_ORDER)), dtype=torch.float32, device="cuda")
    layers = []
    for layer in range(W.N_LAYERS):
        mats = {}
        for nm in W.LAYER_ORDER:
            w = W.c4_matrix(layer, nm)
            out_f, in_f = w.shape
            mats[nm] = dict(w=w, out_f=out_f, in_f=in_f, gpr=in_f // 128, groups=out_f * in_f // 128,
                            blocks=torch.empty((out_f, in_f // 128, 64), dtype=torch.uint8, device="cuda"))
        layers.append(mats)
    # per-tensor scales: the step recomputes amax on the device; the scale is a
    # host argument of the encode / decode calls, so it is fixed here from the
    # same kernel's result
    for layer, mats in enumerate(layers):
        ecco.ecco_amax_many([(m["w"], m["w"].numel(), amax[layer, i:i + 1]) for i, m in enumerate(mats.values())])
    torch.cuda.synchronize()
    amax_host = amax.cpu().numpy()
    for layer, mats in enumerate(layers):
        for i, m in enumerate(mats.values()):
            m["t"] = ecco.ecco_tensor_scale_from_amax(float(amax_host[layer, i]))
    # one reused FP16 buffer of a layer's size; matrix m decodes into its slice
    offs, o = {}, 0
    for nm, m in layers[0].items():
        offs[nm] = o
        o += m["out_f"] * m["in_f"]
    ybuf = torch.empty(o, dtype=torch.float16, device="cuda")
    xin = {f: W.c5_x(1, f).cuda() for f in (4096, 14336)}
    gy = {nm: torch.empty((1, m["out_f"]), dtype=torch.float32, device="cuda") for nm, m in layers[0].items()}
    amax_jobs, encode_jobs, decode_jobs, gemv_jobs = [], [], [], []
    for layer, mats in enumerate(layers):
        amax_jobs.append([(m["w"], m["w"].numel(), amax[layer, i:i + 1]) for i, m in enumerate(mats.values())])
        encode_jobs.append([(m["w"], m["out_f"], m["gpr"], m["in_f"], m["gpr"], tdev[nm], m["t"], m["blocks"], None)
                            for nm, m in mats.items()])
        decode_jobs.append([(m["blocks"], m["out_f"], m["gpr"], m["gpr"], m["in_f"], tdev[nm], m["t"], ybuf[offs[nm]:])
                            for nm, m in mats.items()])
        gemv_jobs.append([[(mats[nm]["blocks"], tdev[nm], mats[nm]["t"], mats[nm]["out_f"], mats[nm]["in_f"],
                            xin[mats[nm]["in_f"]], gy[nm]) for nm in grp]
                          for grp in (["q", "k", "v"], ["o"], ["gate", "up"], ["down"])])
    setup = time.perf_counter() - t_setup
    timer = Timer(torch, stream)

    # each phase's 32 launches run back to back between one pair of events
    # (an event pair around every launch added its own few microseconds to
    # each launch); a launch's time is the phase's over 32
    def amax_phase():
        for jobs in amax_jobs:
            ecco.ecco_amax_many(jobs)

    def encode_phase():
        for jobs in encode_jobs:
            ecco.ecco_encode_many(jobs)

    def decode_phase():
        for jobs in decode_jobs:
            ecco.ecco_decode_many(jobs)

    def gemv_phase():
        for layer_jobs in gemv_jobs:
            for jobs in layer_jobs:
                ecco.ecco_decode_gemv_many(jobs, 1)

    def step():
        timer.run("amax", amax_phase)
        timer.run("encode", encode_phase)
        timer.run("decode", decode_phase)
        timer.run("gemv", gemv_phase)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timer.collect()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ph = timer.collect()
    groups = sum(m["groups"] for mats in layers for m in mats.values())
    dec_t, enc_t = sum(ph["decode"]), sum(ph["encode"])
    n_dec = len(ph["decode"]) * W.N_LAYERS
    res = dict(
        wall=wall, groups=groups, setup_s=setup,
        decode_GBps=groups * args.steps * BYTES_PER_GROUP / dec_t / 1e9,
        encode_GBps=groups * args.steps * BYTES_PER_GROUP / enc_t / 1e9,
        amax_GBps=groups * args.steps * 256 / sum(ph["amax"]) / 1e9,
        decode_launch_us=dec_t / n_dec * 1e6, decode_launches=n_dec,
        decode_launch_us_min=min(ph["decode"]) / W.N_LAYERS * 1e6,
        decode_launch_us_max=max(ph["decode"]) / W.N_LAYERS * 1e6,
        decode_bytes_per_launch=groups // W.N_LAYERS * BYTES_PER_GROUP,
        encode_us_per_layer=enc_t / args.steps / W.N_LAYERS * 1e6,
        decode_us_per_layer=dec_t / args.steps / W.N_LAYERS * 1e6,
        amax_us_per_layer=sum(ph["amax"]) / args.steps / W.N_LAYERS * 1e6,
        gemv_b1_us_per_layer=sum(ph["gemv"]) / args.steps / W.N_LAYERS * 1e6,
        step_device_ms=(dec_t + enc_t + sum(ph["amax"]) + sum(ph["gemv"])) / args.steps * 1e3,
    )
    q0 = layers[0]["q"]
    x0 = q0["w"].cpu().numpy().reshape(-1, 128)
    return res, (x0, blobs["q"], q0["t"])


def bench_layer(args, torch, ecco, W):
    stream = torch.cuda.current_stream()
    mats = {}
    for nm in W.LAYER_ORDER:
        w = W.llama_matrix(W.LLAMA3_8B_LAYER[nm], 100 + W.LAYER_ORDER.index(nm))
        blob = train_tables(ecco, W.c2_sample(nm))
        out_f, in_f = w.shape
        mats[nm] = dict(
            w=w.cuda(), out_f=out_f, in_f=in_f, gpr=in_f // 128, groups=out_f * in_f // 128,
            tdev=ecco.tables_to_device(blob), blob=blob,
            blocks=torch.empty((out_f, in_f // 128, 64), dtype=torch.uint8, device="cuda"),
            y=torch.empty((out_f, in_f), dtype=torch.float16, device="cuda"),
            amax=torch.zeros(1, dtype=torch.float32, device="cuda"),
            gy=torch.empty((1, out_f), dtype=torch.float32, device="cuda"))
    xin = {f: W.c5_x(1, f).cuda() for f in (4096, 14336)}
    # per-tensor scales (the step recomputes amax on the device; the scale is a
    # host argument of the encode/decode calls, so it is fixed here from the
    # same kernel's result)
    for m in mats.values():
        ecco.ecco_amax(m["w"], m["w"].numel(), m["amax"])
    torch.cuda.synchronize()
    for m in mats.values():
        m["t"] = ecco.ecco_tensor_scale_from_amax(m["amax"].item())
    decode_jobs = [(m["blocks"], m["out_f"], m["gpr"], m["gpr"], m["in_f"], m["tdev"], m["t"], m["y"])
                   for m in mats.values()]
    # the GEMVs of a decode step: q, k, v read the same x, and so do gate and
    # up; o and down each wait for their own input
    gemv_groups = [[mats[nm] for nm in grp] for grp in (["q", "k", "v"], ["o"], ["gate", "up"], ["down"])]
    gemv_jobs = [[(m["blocks"], m["tdev"], m["t"], m["out_f"], m["in_f"], xin[m["in_f"]], m["gy"]) for m in grp]
                 for grp in gemv_groups]
    timer = Timer(torch, stream)

    amax_jobs = [(m["w"], m["w"].numel(), m["amax"]) for m in mats.values()]

    encode_jobs = [(m["w"], m["out_f"], m["gpr"], m["in_f"], m["gpr"], m["tdev"], m["t"], m["blocks"], None)
                   for m in mats.values()]

    def step():
        timer.run("amax", lambda: ecco.ecco_amax_many(amax_jobs))
        timer.run("encode", lambda: ecco.ecco_encode_many(encode_jobs))
        timer.run("decode", lambda: ecco.ecco_decode_many(decode_jobs))
        for jobs in gemv_jobs:
            timer.run("gemv", lambda: ecco.ecco_decode_gemv_many(jobs, 1))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timer.collect()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ph = timer.collect()
    groups = sum(m["groups"] for m in mats.values())
    dec_t, enc_t = sum(ph["decode"]), sum(ph["encode"])
    n_dec = len(ph["decode"])
    # diagnostic, outside the timed steps: each matrix decoded by a launch of its own
    for _ in range(3):
        for m in mats.values():
            timer.run("decode_single", lambda: ecco.ecco_decode(m["blocks"], m["out_f"], m["gpr"], m["gpr"],
                                                                m["in_f"], m["tdev"], m["t"], m["y"]))
    # the same matrices by the speculative segment decoder (the pages' method)
    for _ in range(3):
        for m in mats.values():
            timer.run("decode_spec", lambda: ecco.ecco_decode_speculative(m["blocks"], m["out_f"], m["gpr"], m["gpr"],
                                                                          m["in_f"], m["tdev"], m["t"], m["y"]))
    # and by the segment decoder with 2, 4 and 8 lanes per block
    for lanes in (2, 4, 8):
        for _ in range(3):
            for m in mats.values():
                timer.run("decode_seg%d" % lanes,
                          lambda: ecco.ecco_decode_segmented(m["blocks"], m["out_f"], m["gpr"], m["gpr"], m["in_f"],
                                                             m["tdev"], m["t"], m["y"], lanes))
    # each encode by a call of its own
    for _ in range(3):
        for m in mats.values():
            timer.run("encode_single", lambda: ecco.ecco_encode(m["w"], m["out_f"], m["gpr"], m["in_f"], m["gpr"],
                                                                m["tdev"], m["t"], m["blocks"]))
    # each amax by a call of its own
    for _ in range(3):
        for m in mats.values():
            timer.run("amax_single", lambda: ecco.ecco_amax(m["w"], m["w"].numel(), m["amax"]))
    # and each GEMV by a launch of its own
    for _ in range(3):
        for m in mats.values():
            timer.run("gemv_single", lambda: ecco.ecco_decode_gemv(m["blocks"], m["tdev"], m["t"], m["out_f"],
                                                                   m["in_f"], xin[m["in_f"]], 1, m["gy"]))
    torch.cuda.synchronize()
    diag = timer.collect()
    single = diag["decode_single"]
    try:
        graph_us = graph_step_us(torch, stream, amax_jobs, encode_jobs, decode_jobs, gemv_jobs, ecco, args.steps)
    except Exception as e:                     # a diagnostic: the bench line stands without it
        print("bench.py: HIP graph replay not measured: %r" % (e,), file=sys.stderr)
        graph_us = None
    res = dict(
        wall=wall, groups=groups,
        decode_GBps=groups * args.steps * BYTES_PER_GROUP / dec_t / 1e9,
        encode_GBps=groups * args.steps * BYTES_PER_GROUP / enc_t / 1e9,
        decode_launch_us=dec_t / n_dec * 1e6, decode_launches=n_dec,
        decode_bytes_per_launch=groups * BYTES_PER_GROUP,
        encode_us_per_layer=enc_t / args.steps * 1e6,
        decode_us_per_layer=dec_t / args.steps * 1e6,
        gemv_b1_us_per_layer=sum(ph["gemv"]) / args.steps * 1e6,
        amax_us_per_layer=sum(ph["amax"]) / args.steps * 1e6,
        amax_separate_us_per_layer=sum(diag["amax_single"]) / 3 * 1e6,
        encode_separate_us_per_layer=sum(diag["encode_single"]) / 3 * 1e6,
        per_matrix_decode_us={nm: float(np.mean(single[i::len(mats)]) * 1e6) for i, nm in enumerate(mats)},
        gemv_separate_us_per_layer=sum(diag["gemv_single"]) / 3 * 1e6,
        spec_decode_us_per_layer=sum(diag["decode_spec"]) / 3 * 1e6,
        seg_decode_us_per_layer={L: sum(diag["decode_seg%d" % L]) / 3 * 1e6 for L in (2, 4, 8)},
        graph_step_us=graph_us,
    )
    x0 = mats["q"]["w"].cpu().numpy().reshape(-1, 128)
    return res, (x0, mats["q"]["blob"], mats["q"]["t"])


METRIC = "decode GB/s (compressed in + fp16 out) and encode GB/s; % of HBM peak, 1 GPU"


def common_line(args, res, workload, config):
    return {
        "metric": METRIC,
        "value": round(res["decode_GBps"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["wall"] / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 tensors, fp32 arithmetic, u8 blocks",
        "data": "synthetic",
        "config": config,
        "encode_GBps": round(res["encode_GBps"], 1),
        "decode_frac_of_hbm_peak": round(res["decode_GBps"] / HBM_PEAK_GBPS, 4),
        "encode_frac_of_hbm_peak": round(res["encode_GBps"] / HBM_PEAK_GBPS, 4),
        "decode_us_per_layer": round(res["decode_us_per_layer"], 2),
        "encode_us_per_layer": round(res["encode_us_per_layer"], 2),
        "amax_us_per_layer": round(res["amax_us_per_layer"], 2),
        "gemv_b1_us_per_layer": round(res["gemv_b1_us_per_layer"], 2),
        "roofline": {"bound": "hbm", "kernel": "decode_kernel",
                     "achieved": round(res["decode_GBps"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(res["decode_GBps"] / HBM_PEAK_GBPS, 4),
                     "bytes_per_launch": res["decode_bytes_per_launch"],
                     "avg_launch_us": round(res["decode_launch_us"], 3),
                     "traffic": measured_traffic(workload)},
    }


def model_line(args, res):
    line = common_line(args, res, "model", {
        "workload": "llama3-8b 32-layer weight set (224 matrices, 6.98e9 fp16 params, 54,525,952 groups)",
        "groups": res["groups"], "layers": 32,
        "step": "per layer: the 7 matrices' amax in one call; then per layer one encode launch; then per layer "
                "one decode launch into a reused fp16 buffer (blocks written 31 layers earlier); then per layer "
                "the fused decode+GEMV at b=1 in four calls (q+k+v, o, gate+up, down)",
        "tables": "ecco_train_patterns on seeded 2^20-value samples, one set per matrix type"})
    line.update({
        "amax_GBps": round(res["amax_GBps"], 1),
        "decode_launch_us_min_max_over_steps": [round(res["decode_launch_us_min"], 2),
                                                round(res["decode_launch_us_max"], 2)],
        "step_device_ms": round(res["step_device_ms"], 3),
        "setup_s": round(res["setup_s"], 1),
    })
    return line


def layer_line(args, res):
    line = common_line(args, res, "layer", {
        "workload": "llama3-8b-layer (q,k,v,o,gate,up,down; 1,703,936 groups)",
        "groups": res["groups"],
        "step": "the 7 matrices' amax in one call, encoded in one launch and decoded in one "
                "launch; fused decode+GEMV at b=1 in four calls (q+k+v, o, gate+up, down)",
        "tables": "ecco_train_patterns on seeded 2^20-value samples"})
    line.update({
        "encode_us_per_layer_one_call_per_matrix": round(res["encode_separate_us_per_layer"], 2),
        "gemv_b1_us_per_layer_one_call_per_matrix": round(res["gemv_separate_us_per_layer"], 2),
        "step_us_hip_graph_replay": None if res["graph_step_us"] is None else round(res["graph_step_us"], 2),
        "amax_us_per_layer_one_call_per_matrix": round(res["amax_separate_us_per_layer"], 2),
        "amax_GBps": round(res["groups"] * 256 / (res["amax_us_per_layer"] * 1e-6) / 1e9, 1),
        "decode_us_per_matrix_separate_launches": {k: round(v, 2) for k, v in res["per_matrix_decode_us"].items()},
        "speculative_decode_us_per_layer": round(res["spec_decode_us_per_layer"], 2),
        "speculative_decode_GBps": round(res["groups"] * BYTES_PER_GROUP / (res["spec_decode_us_per_layer"] * 1e-6)
                                         / 1e9, 1),
        "segmented_decode_us_per_layer": {"%d_lanes_per_block" % L: round(v, 2)
                                          for L, v in res["seg_decode_us_per_layer"].items()},
    })
    return line


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this codec benchmark runs on exactly one GPU (one process); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import entropy_coded_group_amd as ecco
    import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ecco.lib()
    if args.workload not in ("model", "layer"):
        from bench_workloads import run_workload          # noqa: E402
        line = run_workload(args, torch, ecco, W)
        print(json.dumps(line))
        return
    if args.workload == "model":
        res, (x0, blob0, t0) = bench_model(args, torch, ecco, W)
        line = model_line(args, res)
        sample_of = "layer 0's q matrix"
    else:
        res, (x0, blob0, t0) = bench_layer(args, torch, ecco, W)
        line = layer_line(args, res)
        sample_of = "the q matrix"
    line["d2d_copy_GBps"] = round(d2d_copy_gbps(torch), 1)
    if not args.no_cpu_baseline:
        workers = max(1, min(16, os.cpu_count() or 1))
        cb = cpu_baseline(x0, blob0, t0, args.cpu_groups, workers)
        line["cpu_baseline"] = {"value": round(cb["decode_GBps"], 5), "unit": "GB/s", "cores": cb["workers"],
                                "kind": "oracle",
                                "sample": "first %d groups of %s: oracle encode then decode (NumPy), "
                                          "split over %d process(es), %.2f s; one core in-process %.1f s" % (
                                              cb["groups"], sample_of, cb["workers"], cb["seconds"],
                                              cb["seconds_1core"]),
                                "encode_GBps": round(cb["encode_GBps"], 5),
                                "decode_GBps_1core": round(cb["decode_GBps_1core"], 5),
                                "encode_GBps_1core": round(cb["encode_GBps_1core"], 5),
                                "cpu": cpu_model(), "host_cpus": os.cpu_count()}
        lit = literal_baseline(x0, blob0, t0, 1024)
        line["cpu_baseline"]["literal_oracle_1core"] = {
            "sample": "first %d groups of %s, one group at a time in plain Python, %.1f s" % (
                lit["groups"], sample_of, lit["seconds"]),
            "decode_GBps": round(lit["decode_GBps_1core"], 6), "encode_GBps": round(lit["encode_GBps_1core"], 6)}
        q = oracle_quality(x0, blob0, t0, 8192)
        line["quality"] = dict(
            {k: (round(v, 6) if isinstance(v, float) else v) for k, v in q.items()},
            source="oracle encode + decode of the first %d groups of %s; compression ratios of the whole matrix "
                   "over FP16, counting the format's side data (6,020 B) or the library's table blob" % (
                       q["groups"], sample_of))
    print(json.dumps(line))


if __name__ == "__main__":
    main()
