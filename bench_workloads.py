"""Secondary workloads of bench.py (see its docstring): weight, kv, ffn, attn, act, design, copy."""

import os
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
BYTES_PER_GROUP = 64 + 256


def _events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


_SLEEP_CYCLES_PER_US = []


def _hold_stream(torch, us):
    """Enqueue a spin kernel (torch.cuda._sleep) that keeps the stream busy for
    about `us` microseconds, calibrated once."""
    if not _SLEEP_CYCLES_PER_US:
        a, b = _events(torch, 2)
        torch.cuda.synchronize()
        a.record()
        torch.cuda._sleep(1 << 20)
        b.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_US.append((1 << 20) / max(a.elapsed_time(b) * 1e3, 1.0))
    torch.cuda._sleep(int(us * _SLEEP_CYCLES_PER_US[0]))


def _timed(torch, fn, steps, warmup):
    """Run fn() warmup + steps times; per-call HIP event durations (seconds).
    A spin kernel holds the stream while the host enqueues the timed calls
    (allowing 200 us of host work per call), so each event pair brackets the
    call's device work, not the Python binding's argument marshalling, which
    for calls of a few tens of microseconds would otherwise leave the GPU
    idle in between."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    _hold_stream(torch, 200.0 * steps)
    evs = []
    for _ in range(steps):
        a, b = _events(torch, 2)
        a.record()
        fn()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e-3 for a, b in evs]


def _line(metric, value, unit, args, ms_per_step, config, **extra):
    d = {"metric": metric, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": args.steps,
         "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
         "scaling": "weak", "vs_baseline": None, "dtype": "fp16 tensors, fp32 arithmetic, u8 blocks",
         "data": "synthetic", "config": config}
    d.update(extra)
    return d


def bench_weight(args, torch, ecco, W):
    """One 1024x1024 weight (8,192 groups): small enough that each call is
    bound by launch latency, not by HBM.  Per step: amax, encode, decode,
    each a call of its own.  Device time per call comes from HIP events
    around calls enqueued behind a spin kernel; the host-inclusive time per
    step is the wall clock of `steps` back-to-back steps (amax, scale
    read-back, encode, decode) with one synchronisation per step, as a caller
    that needs the scale on the host sees it."""
    x = W.c1_weight().cuda()
    n_rows, n_cols = x.shape
    gpr = n_cols // 128
    blob = ecco.ecco_train_patterns(W.c1_sample(), threads=min(16, os.cpu_count() or 1))
    tdev = ecco.tables_to_device(blob)
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    ecco.ecco_amax(x, x.numel(), amax)
    torch.cuda.synchronize()
    t = ecco.ecco_tensor_scale_from_amax(amax.item())
    blocks = torch.empty((n_rows, gpr, 64), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)

    def f_amax():
        ecco.ecco_amax(x, x.numel(), amax)

    def f_enc():
        ecco.ecco_encode(x, n_rows, gpr, n_cols, gpr, tdev, t, blocks)

    def f_dec():
        ecco.ecco_decode(blocks, n_rows, gpr, gpr, n_cols, tdev, t, y)

    t_amax = _timed(torch, f_amax, args.steps, args.warmup)
    t_enc = _timed(torch, f_enc, args.steps, args.warmup)
    t_dec = _timed(torch, f_dec, args.steps, args.warmup)
    for _ in range(args.warmup):
        f_amax(); f_enc(); f_dec()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for _ in range(args.steps):
        ecco.ecco_amax(x, x.numel(), amax)
        tt = ecco.ecco_tensor_scale_from_amax(amax.item())
        ecco.ecco_encode(x, n_rows, gpr, n_cols, gpr, tdev, tt, blocks)
        ecco.ecco_decode(blocks, n_rows, gpr, gpr, n_cols, tdev, tt, y)
        torch.cuda.synchronize()
    wall = (time.perf_counter() - w0) / args.steps
    groups = n_rows * gpr
    dev = np.mean(t_amax) + np.mean(t_enc) + np.mean(t_dec)
    dec = groups * BYTES_PER_GROUP / np.mean(t_dec) / 1e9
    return _line("decode GB/s (compressed in + fp16 out), 1 GPU", dec, "GB/s", args, wall * 1e3,
                 {"workload": "one 1024x1024 weight (8,192 groups): amax, encode, decode, one call each",
                  "groups": groups},
                 decode_us=round(np.mean(t_dec) * 1e6, 2), encode_us=round(np.mean(t_enc) * 1e6, 2),
                 amax_us=round(np.mean(t_amax) * 1e6, 2), device_us_per_step=round(dev * 1e6, 2),
                 host_inclusive_us_per_step=round(wall * 1e6, 1),
                 encode_GBps=round(groups * BYTES_PER_GROUP / np.mean(t_enc) / 1e9, 1))


def bench_kv(args, torch, ecco, W):
    B, H, S, D = W.KV_SHAPE
    T = W.KV_APPEND
    caches = {}
    for kind in ("k", "v"):
        sample = W.kv_sample(kind)
        blob = ecco.ecco_train_patterns(sample, threads=min(16, os.cpu_count() or 1))
        amax = float(np.max(np.abs(sample.numpy().astype(np.float32))))
        t = ecco.ecco_tensor_scale_from_amax(amax)          # fixed ahead of time (online codec)
        # the online compressor's 16-pattern variant (16 distinct patterns in the 64 slots)
        blob16 = ecco.ecco_train_patterns(sample, threads=min(16, os.cpu_count() or 1), n_patterns=16)
        x = W.kv_tensor(kind).cuda()
        tdev = ecco.tables_to_device(blob)
        blocks = torch.empty((B, H, S, 64), dtype=torch.uint8, device="cuda")
        ecco.ecco_encode(x, B * H, S - T, S * D, S, tdev, t, blocks)
        caches[kind] = dict(x=x, t=t, tdev=tdev, tdev16=ecco.tables_to_device(blob16), blocks=blocks,
                            y=torch.empty_like(x))
    torch.cuda.synchronize()

    # K and V rows of the step appended by one call
    append_jobs = [(c["x"][:, :, S - T:], B * H, T, S * D, S, c["tdev"], c["t"], c["blocks"][:, :, S - T:], None)
                   for c in caches.values()]

    def append():
        ecco.ecco_encode_many(append_jobs)

    def append_separate():
        for c in caches.values():
            ecco.ecco_encode(c["x"][:, :, S - T:], B * H, T, S * D, S, c["tdev"], c["t"], c["blocks"][:, :, S - T:])

    jobs = [(c["blocks"], 1, B * H * S, B * H * S, B * H * S * D, c["tdev"], c["t"], c["y"]) for c in caches.values()]

    append16_jobs = [(c["x"][:, :, S - T:], B * H, T, S * D, S, c["tdev16"], c["t"], c["blocks"][:, :, S - T:], None)
                     for c in caches.values()]

    def append16():
        ecco.ecco_encode_many(append16_jobs)

    def decode():
        ecco.ecco_decode_many(jobs)

    t_app = _timed(torch, append, args.steps, args.warmup)
    t_app_sep = _timed(torch, append_separate, args.steps, args.warmup)
    t_app16 = _timed(torch, append16, args.steps, args.warmup)
    t_dec = _timed(torch, decode, args.steps, args.warmup)
    g_dec = 2 * B * H * S
    g_app = 2 * B * H * T
    dec = g_dec * BYTES_PER_GROUP / np.mean(t_dec) / 1e9
    app = g_app * BYTES_PER_GROUP / np.mean(t_app) / 1e9
    return _line("decode GB/s (compressed in + fp16 out), 1 GPU", dec, "GB/s", args,
                 (np.mean(t_dec) + np.mean(t_app)) * 1e3,
                 {"workload": "kv-cache K,V [16,8,8192,128]: append-encode 256 tokens (K and V in one launch), decode whole cache (K and V in one launch)",
                  "decode_groups": g_dec, "append_groups": g_app},
                 decode_frac_of_hbm_peak=round(dec / HBM_PEAK_GBPS, 4),
                 append_encode_GBps=round(app, 1), append_encode_us=round(np.mean(t_app) * 1e6, 2),
                 append_encode_us_16_patterns=round(np.mean(t_app16) * 1e6, 2),
                 append_encode_us_one_call_per_tensor=round(np.mean(t_app_sep) * 1e6, 2),
                 decode_us=round(np.mean(t_dec) * 1e6, 2))


def bench_ffn(args, torch, ecco, W):
    out = {}
    for name in ("w1", "w2"):
        w = W.c5_matrix(name)
        out_f, in_f = w.shape
        blob = ecco.ecco_train_patterns(W.c5_sample(name), threads=min(16, os.cpu_count() or 1))
        tdev = ecco.tables_to_device(blob)
        wd = w.cuda()
        amax = torch.zeros(1, dtype=torch.float32, device="cuda")
        ecco.ecco_amax(wd, wd.numel(), amax)
        torch.cuda.synchronize()
        t = ecco.ecco_tensor_scale_from_amax(amax.item())
        blocks = torch.empty((out_f, in_f // 128, 64), dtype=torch.uint8, device="cuda")
        ecco.ecco_encode(wd, out_f, in_f // 128, in_f, in_f // 128, tdev, t, blocks)
        del wd
        wbuf = torch.empty((out_f, in_f), dtype=torch.float16, device="cuda")
        for b in (1, 4, 8):
            x = W.c5_x(b, in_f).cuda()
            y = torch.empty((b, out_f), dtype=torch.float32, device="cuda")
            tf = _timed(torch, lambda: ecco.ecco_decode_gemv(blocks, tdev, t, out_f, in_f, x, b, y),
                        args.steps, args.warmup)

            def unfused():
                ecco.ecco_decode(blocks, out_f, in_f // 128, in_f // 128, in_f, tdev, t, wbuf)
                torch.matmul(x, wbuf.t())

            tu = _timed(torch, unfused, args.steps, args.warmup)
            # the uncompressed reference: the dense GEMV alone on FP16 weights
            # already in HBM (reads 4x the bytes of the fused path)
            td = _timed(torch, lambda: torch.matmul(x, wbuf.t()), args.steps, args.warmup)
            out["%s_b%d" % (name, b)] = dict(fused_us=round(np.mean(tf) * 1e6, 2),
                                             decode_then_gemv_us=round(np.mean(tu) * 1e6, 2),
                                             fp16_dense_gemv_us=round(np.mean(td) * 1e6, 2),
                                             compressed_GBps=round(out_f * in_f / 2 / np.mean(tf) / 1e9, 1),
                                             fp16_equivalent_GBps=round(out_f * in_f * 2 / np.mean(tf) / 1e9, 1))
        del wbuf
    tot_f = sum(v["fused_us"] for v in out.values())
    tot_u = sum(v["decode_then_gemv_us"] for v in out.values())
    return _line("fused decode+GEMV speedup over decode then dense GEMV", tot_u / tot_f, "x", args,
                 tot_f / 1e3, {"workload": "70B FFN [28672,8192] and [8192,28672], batch 1/4/8"},
                 per_case=out)


def bench_attn(args, torch, ecco, W):
    """Decode-phase attention over the compressed [16, 8, 8192, 128] K and V
    caches, 4 query heads per kv head (LLaMA-3-8B GQA): ecco_attention_decode
    against decoding both caches (ecco_decode_many) then torch's fused
    scaled-dot-product attention on the FP16 caches."""
    import torch.nn.functional as F
    B, H, S, D = W.KV_SHAPE
    G = 4
    c = {}
    for kind in ("k", "v"):
        sample = W.kv_sample(kind)
        blob = ecco.ecco_train_patterns(sample, threads=min(16, os.cpu_count() or 1))
        amax = float(np.max(np.abs(sample.numpy().astype(np.float32))))
        t = ecco.ecco_tensor_scale_from_amax(amax)
        x = W.kv_tensor(kind).cuda()
        tdev = ecco.tables_to_device(blob)
        blocks = torch.empty((B, H, S, 64), dtype=torch.uint8, device="cuda")
        ecco.ecco_encode(x, 1, B * H * S, B * H * S * D, B * H * S, tdev, t, blocks)
        c[kind] = dict(t=t, tdev=tdev, blocks=blocks, y=torch.empty_like(x))
        del x
    q = W.c5_x(B * H * G, D, seed=77).cuda().reshape(B, H * G, D)
    ws = torch.empty(ecco.ecco_attention_workspace_size(B, H, G, S), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, H * G, D), dtype=torch.float32, device="cuda")
    scale = 1.0 / np.sqrt(D)

    def fused():
        ecco.ecco_attention_decode(c["k"]["blocks"], c["k"]["tdev"], c["k"]["t"], c["v"]["blocks"], c["v"]["tdev"],
                                   c["v"]["t"], q, B, H, G, S, S, scale, ws, out)

    jobs = [(c[k]["blocks"], 1, B * H * S, B * H * S, B * H * S * D, c[k]["tdev"], c[k]["t"], c[k]["y"])
            for k in ("k", "v")]
    q4 = q.reshape(B, H * G, 1, D)

    def unfused():
        ecco.ecco_decode_many(jobs)
        F.scaled_dot_product_attention(q4, c["k"]["y"], c["v"]["y"], scale=scale, enable_gqa=True)

    tf = _timed(torch, fused, args.steps, args.warmup)
    tu = _timed(torch, unfused, args.steps, args.warmup)
    comp = 2 * B * H * S * 64
    fused_us, unfused_us = np.mean(tf) * 1e6, np.mean(tu) * 1e6
    return _line("fused decode+attention speedup over decode then SDPA", unfused_us / fused_us, "x", args,
                 fused_us / 1e3, {"workload": "decode-phase attention, K,V caches [16,8,8192,128], 4 query heads "
                                              "per kv head, one query token per sequence"},
                 fused_us=round(fused_us, 2), decode_then_sdpa_us=round(unfused_us, 2),
                 compressed_GBps=round(comp / (fused_us * 1e-6) / 1e9, 1),
                 compressed_bytes=comp)


def bench_act(args, torch, ecco, W):
    """2x activation format on LLaMA-3-8B hidden states [16384, 4096] (1,048,576
    groups of 64): per-tensor scale from the tensor's own amax, encode, decode.
    A step is amax + encode + decode; each is also timed on its own."""
    T, D = W.ACT_SHAPE
    G = T * D // W.ACT_GROUP
    blob = ecco.ecco_train_patterns(W.act_sample(), threads=min(16, os.cpu_count() or 1), group=W.ACT_GROUP)
    tdev = ecco.tables_to_device(blob)
    x = W.act_tensor().cuda()
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    ecco.ecco_amax(x, x.numel(), amax)
    torch.cuda.synchronize()
    t = ecco.ecco_tensor_scale_from_amax(amax.item())
    blocks = torch.empty((G, 64), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    stats = torch.zeros(7, dtype=torch.int64, device="cuda")
    ecco.ecco_encode_act(x, 1, G, G * 64, G, tdev, t, blocks, stats)
    torch.cuda.synchronize()
    st = dict(zip(ecco.STATS_FIELDS, stats.cpu().tolist()))

    def do_amax():
        ecco.ecco_amax(x, x.numel(), amax)

    def encode():
        ecco.ecco_encode_act(x, 1, G, G * 64, G, tdev, t, blocks)

    def decode():
        ecco.ecco_decode_act(blocks, 1, G, G, G * 64, tdev, t, y)

    def step():
        # the scale of this step's tensor is the one computed on the host once:
        # the amax pass is timed as the work it is, without a host round trip
        do_amax()
        encode()
        decode()

    t_step = _timed(torch, step, args.steps, args.warmup)
    t_amax = _timed(torch, do_amax, args.steps, args.warmup)
    t_enc = _timed(torch, encode, args.steps, args.warmup)
    t_dec = _timed(torch, decode, args.steps, args.warmup)
    bpg = 64 + 2 * W.ACT_GROUP                              # compressed block + fp16 group
    dec = G * bpg / np.mean(t_dec) / 1e9
    enc = G * bpg / np.mean(t_enc) / 1e9
    xf = x.float()
    err = float(torch.sqrt(((y.float() - xf) ** 2).mean() / (xf ** 2).mean()))
    return _line("activation decode GB/s (compressed in + fp16 out), 1 GPU", dec, "GB/s", args,
                 np.mean(t_step) * 1e3,
                 {"workload": "2x activation format, LLaMA-3-8B hidden states [16384, 4096] fp16 "
                              "(groups of 64): amax + encode + decode per step", "groups": G},
                 decode_frac_of_hbm_peak=round(dec / HBM_PEAK_GBPS, 4), decode_us=round(np.mean(t_dec) * 1e6, 2),
                 encode_GBps=round(enc, 1), encode_us=round(np.mean(t_enc) * 1e6, 2),
                 amax_us=round(np.mean(t_amax) * 1e6, 2), relative_rms_error=round(err, 5),
                 clipped_groups=st["clipped_groups"], mean_outliers_per_group=round(st["padded_outliers"] / G, 3))


def bench_design(args, torch, ecco, W):
    """The S x H design points the v1 block can hold (S in {16, 32, 64}
    patterns, H in {1, 2, 4} codebooks; tables from
    tests/golden/design_tables.npz written into the block's 64 x 4 slots by
    repetition) on full-size tensors: the LLaMA-3-8B gate projection
    [14336, 4096], the KV cache's K and V [16, 8, 8192, 128] and the
    1024x1024 weight.  Per point: encode and decode time, and the codec's
    quality from the GPU's own output (relative MSE of the round trip,
    clipped groups, mean coded bits per group including the 16-bit header)."""
    z = np.load(os.path.join(os.path.dirname(os.path.abspath(__file__)), "tests", "golden", "design_tables.npz"))
    cases = []
    x = W.c1_weight().cuda()
    cases.append(("c1", "1024x1024 weight", x, None))
    x = W.llama_matrix(W.LLAMA3_8B_LAYER["gate"], 104).cuda()
    cases.append(("gate", "llama3-8b gate [14336, 4096]", x, None))
    for kind in ("k", "v"):
        smp = W.kv_sample(kind).numpy()
        t = ecco.ecco_tensor_scale_from_amax(float(np.max(np.abs(smp.astype(np.float32)))))
        cases.append((kind, "kv-cache %s [16, 8, 8192, 128]" % kind.upper(), W.kv_tensor(kind).cuda(), t))
    out = {}
    for name, label, x, t in cases:
        G = x.numel() // 128
        if t is None:
            amax = torch.zeros(1, dtype=torch.float32, device="cuda")
            ecco.ecco_amax(x, x.numel(), amax)
            torch.cuda.synchronize()
            t = ecco.ecco_tensor_scale_from_amax(amax.item())
        blocks = torch.empty((G, 64), dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        st = torch.zeros(7, dtype=torch.int64, device="cuda")
        xf = x.float()
        var = float(((xf - xf.mean()) ** 2).mean())
        rows = {}
        for S in (16, 32, 64):
            for H in (1, 2, 4):
                key = "%s_S%d_H%d" % (name, S, H)
                # slot p holds pattern p mod S, book h of a pattern book h mod H
                c, L = z[key + "_centroids"], z[key + "_code_len"]
                c64 = np.ascontiguousarray(c[np.arange(64) % S], np.float32)
                L64 = np.ascontiguousarray(L[np.arange(64) % S][:, np.arange(4) % H], np.uint8)
                tdev = ecco.tables_to_device(ecco.ecco_tables_build(c64, L64))
                st.zero_()
                ecco.ecco_encode(x, 1, G, G * 128, G, tdev, t, blocks, st)
                ecco.ecco_decode(blocks, 1, G, G, G * 128, tdev, t, y)
                torch.cuda.synchronize()
                s = dict(zip(ecco.STATS_FIELDS, st.cpu().tolist()))
                unclipped = G - s["clipped_groups"]
                # stream bits of the unclipped groups: 496 - pad - fill each; clipped ones fill the block
                bits = 512.0 * s["clipped_groups"] + 16.0 * unclipped + (496.0 * unclipped - s["pad_bits"] -
                                                                          s["fill_bits"])
                mse = float(((y.float() - xf) ** 2).mean())
                te = _timed(torch, lambda: ecco.ecco_encode(x, 1, G, G * 128, G, tdev, t, blocks), args.steps,
                            args.warmup)
                td = _timed(torch, lambda: ecco.ecco_decode(blocks, 1, G, G, G * 128, tdev, t, y), args.steps,
                            args.warmup)
                rows["S%d_H%d" % (S, H)] = dict(
                    rel_mse=round(mse / var, 6), clipped_frac=round(s["clipped_groups"] / G, 4),
                    coded_bits_per_group=round(bits / G, 1),
                    outliers_per_group=round(s["padded_outliers"] / G, 3),
                    encode_us=round(np.mean(te) * 1e6, 2), decode_us=round(np.mean(td) * 1e6, 2),
                    encode_GBps=round(G * BYTES_PER_GROUP / np.mean(te) / 1e9, 1),
                    decode_GBps=round(G * BYTES_PER_GROUP / np.mean(td) / 1e9, 1))
        out[name] = dict(workload=label, groups=G, points=rows)
        del x, y, xf, blocks
        torch.cuda.empty_cache()
    g = out["gate"]["points"]["S64_H4"]
    return _line("decode GB/s at S=64, H=4, gate projection", g["decode_GBps"], "GB/s", args,
                 (g["encode_us"] + g["decode_us"]) / 1e3,
                 {"workload": "S x H design points held by the v1 block: S in {16, 32, 64}, H in {1, 2, 4}"},
                 design_points=out)


def bench_copy(args, torch, ecco, W):
    nbytes = 1 << 30
    a = torch.ones(nbytes // 2, dtype=torch.float16, device="cuda")
    b = torch.empty_like(a)
    ts = _timed(torch, lambda: b.copy_(a), args.steps, args.warmup)
    gbps = 2 * nbytes / np.mean(ts) / 1e9
    return _line("device-to-device copy GB/s (read + write)", gbps, "GB/s", args, np.mean(ts) * 1e3,
                 {"workload": "copy 1 GiB fp16 buffer (torch copy_)", "bytes_read": nbytes,
                  "bytes_written": nbytes}, frac_of_hbm_peak=round(gbps / HBM_PEAK_GBPS, 4))


def run_workload(args, torch, ecco, W):
    return {"weight": bench_weight, "kv": bench_kv, "ffn": bench_ffn, "attn": bench_attn, "design": bench_design,
            "act": bench_act, "copy": bench_copy}[args.workload](args, torch, ecco, W)
