#!/usr/bin/env python3
"""Benchmark of the AWQ per-layer search path on one MI355X.

A step is one pass of the whole path over every searched layer of the
workload, stage after stage on one stream: saliency (awq_act_stats), the
alpha-grid search (awq_search_layer in its three stages: prepare, grid,
select) and packing at the chosen alpha (awq_pack).  Inputs are seeded
synthetic tensors (synth/), resident in HBM before timing starts.  The line
printed on stdout:

  value        search flops of the step (20 grid points x 2 N in out, summed
               over layers) / step time, TFLOP/s; the step time is the wall
               clock of --steps steps run back to back, synchronized on both
               sides, after --warmup steps
  roofline     the dominant kernel (the grid stage: the contraction of the
               produced weight error on layers of many token tiles, else the
               fused kernels): algorithmic flops per search / the time of the
               search's grid stage, from HIP events recorded around each stage
               on its launch stream inside the timed steps, against the fp16
               dense MFMA peak; traffic is HBM bytes per launch from the
               committed rocprofv3 counter summary; stats and pack against the
               HBM peak and a cold plain read of the same input
  kernels      per-stage times, TFLOP/s and GB/s, and stats and pack timed cold
               (last-level cache cleared first) beside the fastest plain read
               measured here (one shot per block, nontemporal loads) of X and
               of W
  measured_peaks  an MFMA-only loop (libawq_calib.so), for comparison with the
               published peak
  cpu_baseline the CPU oracle on a bounded sample of the same workload

`python bench.py --gpus N` with N > 1 exits: the path runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_F16_PEAK_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 fp16 flop/clk (dense)
HBM_PEAK_GBS = 8000.0
METRIC = "AWQ α-grid search TFLOP/s + MFMA util; quant/pack HBM GB/s (1 GPU)"
DEFAULT_CONFIG = 5   # the largest configuration: the 13B-style block, four searches


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def search_flops(spec, n_grid=20):
    return 2.0 * n_grid * spec.n_tokens * spec.in_features * spec.out_features


def stats_bytes(spec):
    return 2.0 * spec.n_tokens * spec.in_features + 4.0 * spec.in_features


def pack_bytes(spec, group=128):
    w = spec.out_features * spec.in_features
    return 2.0 * w + 0.5 * w + 4.0 * w / group + 4.0 * spec.in_features


def weight_error_bytes(spec, n_grid=20):
    """HBM bytes of the contraction path's preparation stage: W read once, the
    fp16 weight error of every grid point written (the scale table and the
    saliency are a few KB)."""
    w = spec.out_features * spec.in_features
    return 2.0 * w + 2.0 * n_grid * w


def source_digest():
    """Digest of the grid kernels' code (search_grid.hip, search_gemm.hip,
    grid_index.h and awq_device.h with comments and blank lines removed and
    lines stripped), so that a counter summary stays valid across edits of
    comments only."""
    h = hashlib.sha256()
    for f in ("search_grid.hip", "search_gemm.hip", "grid_index.h", "awq_device.h"):
        src = open(os.path.join(ROOT, "post_bit_weight_awq_amd", "csrc", f)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        h.update("\n".join(ln.strip() for ln in src.splitlines() if ln.strip()).encode())
    return h.hexdigest()[:16]


def uses_contraction(spec, cfg):
    """Whether the search of this layer produces the weight error in its
    preparation stage and contracts it (256 x 256 tiles)."""
    import post_bit_weight_awq_amd as P
    return P.awq_search_plan(spec.n_tokens, spec.in_features, spec.out_features,
                             cfg).tile_out == 256


def grid_kernel_names(layers, cfg):
    """Names of the grid-stage kernels the searches launch: the contraction of
    the produced weight error on 256 x 256 tiles (layers of many token tiles),
    else the fused kernels: ping-pong on 512- and 256-token tiles, k_grid on
    128."""
    import post_bit_weight_awq_amd as P
    names = []
    for L in layers:
        sp = L["spec"]
        plan = P.awq_search_plan(sp.n_tokens, sp.in_features, sp.out_features, cfg)
        if uses_contraction(sp, cfg):
            nm = "k_grid_gemm"
        else:
            nm = "k_grid_pp" if plan.tile_tokens in (512, 256) else "k_grid"
        if nm not in names:
            names.append(nm)
    return " + ".join(names)


def traffic_from_profiles(workload):
    """HBM bytes per launch of the grid kernel (the mean over the step's grid
    launches) from the committed PMC summary, or None when there is none or the
    kernel source changed since."""
    import glob
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*traffic*.md"))):
        for line in open(path):
            m = re.match(r"\s*traffic:\s*workload=(\S+)\s+source=(\S+)\s+bytes_per_launch=(\S+)",
                         line)
            if m and m.group(1) == workload and m.group(2) == source_digest():
                return float(m.group(3))
    return None


def cpu_baseline(cfg_key, target_s):
    """The oracle, as it stands, on a bounded sample of the workload: for every
    layer of the configuration, stats over all its tokens, then the full
    20-point search and pack on a leading cut of its output rows, the cuts
    sized so that the whole sample takes about target_s seconds.  Reported in
    the metric's unit: search flops of the sampled rows over the sample's
    stats + search + pack time."""
    import numpy as np
    import synth
    from oracle import awq_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    layers = synth.CONFIGS[cfg_key].layers
    per_layer_s = target_s / len(layers)
    t_stats = t_search = t_pack = 0.0
    flops = 0.0
    parts = []
    per_layer = []
    for li, spec in enumerate(layers):
        _, X, W = synth.make_layer(cfg_key, li)
        t0 = time.perf_counter()
        sal = O.act_stats(X)
        ts = time.perf_counter() - t0
        t_stats += ts
        # size the row cut from a probe of one grid point on 512 rows (smaller
        # probes are dominated by per-call costs and undersize the cut)
        rows = min(512, spec.out_features)
        s, inv_s = O.scale_table(sal)
        t0 = time.perf_counter()
        O.tile_sq_error(X, W, s[5], inv_s[5], slice(0, spec.n_tokens), slice(0, rows))
        per_row_alpha = (time.perf_counter() - t0) / rows
        rows = int(max(8, min(spec.out_features, per_layer_s / (20 * per_row_alpha + 1e-12))))
        Wc = np.ascontiguousarray(W[:rows])
        del W
        t0 = time.perf_counter()
        res = O.search_layer(X, Wc, sal)
        tq = time.perf_counter() - t0
        t_search += tq
        t0 = time.perf_counter()
        O.pack(Wc, res.s_best)
        tp = time.perf_counter() - t0
        t_pack += tp
        flops += 2.0 * 20 * spec.n_tokens * spec.in_features * rows
        parts.append(f"{spec.name} {spec.n_tokens}x{spec.in_features}: {rows} of "
                     f"{spec.out_features} rows")
        per_layer.append({"layer": spec.name, "rows": rows, "stats_s": round(ts, 3),
                          "search_s": round(tq, 3), "pack_s": round(tp, 3)})
    return {
        "value": flops / (t_stats + t_search + t_pack) / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"every layer of config {cfg_key} ({synth.CONFIGS[cfg_key].workload}): stats "
                   f"over all tokens, 20-point search and pack on a leading cut of output rows ("
                   + "; ".join(parts) + ")"),
        "seconds": {"stats": t_stats, "search": t_search, "pack": t_pack},
        "per_layer": per_layer,
        "host": {"affinity_cores": len(os.sched_getaffinity(0)), "blas_threads": int(threads)},
    }


def load_calib():
    """The measured-peak reference kernels (libawq_calib.so), or None."""
    import ctypes
    path = os.path.join(ROOT, "post_bit_weight_awq_amd", "libawq_calib.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.awq_calib_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.awq_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                   ctypes.c_void_p]
    lib.awq_calib_read_oneshot.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                           ctypes.c_void_p]
    return lib


def cold_measurements(awq, cfg, layers, calib):
    """Stats and pack with the 256 MB last-level cache (MALL) cleared first by a
    512 MiB streaming read; as plain-read references, the fastest read measured
    here (one shot per block, nontemporal loads) of X and of W after the same
    clear; and an MFMA-only loop as the measured MFMA peak."""
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    flush = torch.zeros(1 << 29, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")

    def do_flush():
        assert calib.awq_calib_read(flush.data_ptr(), flush.numel(), sink.data_ptr(), 2048,
                                    stream) == 0

    def timed(fn, reps=5):
        # median over reps; the flush kernel keeps the GPU busy while the
        # host enqueues fn, so the interval holds GPU time only
        ts = []
        for _ in range(reps):
            do_flush()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return sorted(ts)[reps // 2]

    res = {}
    for L in layers:
        spec = L["spec"]
        xb = L["X"].numel() * 2
        ms_stats = timed(lambda: awq.awq_act_stats(L["X"], out=L["sal"], workspace=L["sws"]))
        ms_pack = timed(lambda: awq.awq_pack(L["W"], L["s_best"], cfg, qweight=L["qw"],
                                             step=L["st"], zero=L["zr"]))
        wb = L["W"].numel() * 2
        ms_read = timed(lambda: calib.awq_calib_read_oneshot(L["X"].data_ptr(), xb,
                                                             sink.data_ptr(), stream))
        ms_read_w = timed(lambda: calib.awq_calib_read_oneshot(L["W"].data_ptr(), wb,
                                                               sink.data_ptr(), stream))
        res[spec.name] = {"stats_gbs_cold": round(stats_bytes(spec) / (ms_stats * 1e-3) / 1e9, 1),
                          "pack_gbs_cold": round(pack_bytes(spec, cfg.group_size) /
                                                 (ms_pack * 1e-3) / 1e9, 1),
                          "plain_read_of_X_gbs_cold": round(xb / (ms_read * 1e-3) / 1e9, 1),
                          "plain_read_of_W_gbs_cold": round(wb / (ms_read_w * 1e-3) / 1e9, 1)}
    # the stage over the whole step, one event pair around its back-to-back
    # calls (every input read once after the MALL clear), so the few
    # microseconds an event adds between stages do not count against a stage
    # of 10-50 us launches
    res["_block"] = {
        "stats_ms": timed(lambda: [awq.awq_act_stats(L["X"], out=L["sal"], workspace=L["sws"])
                                   for L in layers]),
        "pack_ms": timed(lambda: [awq.awq_pack(L["W"], L["s_best"], cfg, qweight=L["qw"],
                                               step=L["st"], zero=L["zr"]) for L in layers]),
        "plain_read_of_X_ms": timed(lambda: [calib.awq_calib_read_oneshot(
            L["X"].data_ptr(), L["X"].numel() * 2, sink.data_ptr(), stream)
            for L in layers]),
        "plain_read_of_W_ms": timed(lambda: [calib.awq_calib_read_oneshot(
            L["W"].data_ptr(), L["W"].numel() * 2, sink.data_ptr(), stream)
            for L in layers]),
    }
    del flush
    out_buf = torch.empty(1024 * 512, dtype=torch.float32, device="cuda")
    n_iter = 1024
    assert calib.awq_calib_mfma(out_buf.data_ptr(), 1024, n_iter, stream) == 0
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    assert calib.awq_calib_mfma(out_buf.data_ptr(), 1024, n_iter, stream) == 0
    b.record()
    b.synchronize()
    flops = 1024 * 8 * n_iter * 32 * 16384.0
    mfma = flops / (a.elapsed_time(b) * 1e-3) / 1e12
    return res, round(mfma, 1)


DECODE_LAYERS = (("qkv", 5120, 15360), ("o_proj", 5120, 5120), ("gate_up", 5120, 27648),
                 ("down", 13824, 5120))


def decode_bench(tokens, reps):
    """W4A16 decode on the 13B block's four linears (packed by awq_pack from the
    seeded synthetic weights): each measurement clears the 256 MB MALL with a
    512 MiB read first, as a decode step over a whole model would find it."""
    import numpy as np
    import torch
    import synth
    import post_bit_weight_awq_amd as awq
    calib = load_calib()
    if calib is None:
        raise RuntimeError("libawq_calib.so is missing: run post_bit_weight_awq_amd/build.py")
    awq.load()
    stream = torch.cuda.current_stream().cuda_stream
    layers = []
    for li, (name, k, o) in enumerate(DECODE_LAYERS):
        _, X, W = synth.make_custom(max(tokens), k, o, seed=1000 + li)
        Wd = torch.from_numpy(W).cuda()
        s = torch.ones(k, dtype=torch.float32, device="cuda")
        qw, st, zr = awq.awq_pack(Wd, s)
        del Wd
        layers.append(dict(name=name, k=k, o=o, X=torch.from_numpy(X).cuda(), qw=qw, st=st, zr=zr))
    torch.cuda.synchronize()
    flush = torch.zeros(1 << 29, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")

    def do_flush():
        assert calib.awq_calib_read(flush.data_ptr(), flush.numel(), sink.data_ptr(), 2048,
                                    stream) == 0

    def median_ms(fn):
        fn()
        ts = []
        for _ in range(reps):
            do_flush()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return sorted(ts)[len(ts) // 2]

    def layer_bytes(L, m):
        return (L["o"] * L["k"] // 2 + 4 * L["o"] * L["k"] // 128 + 2 * m * L["k"]
                + 4 * m * L["o"])

    # folding s of the four searches upstream: the two norm gains, v_proj's rows
    # (feeding o_proj) and up_proj's rows (feeding down), in place
    gen = torch.Generator(device="cuda").manual_seed(7)
    fold_arrays = [("input_norm_gain", (5120,)), ("v_proj_weight", (5120, 5120)),
                   ("post_attention_norm_gain", (5120,)), ("up_proj_weight", (13824, 5120))]
    folds = []
    for name, shape in fold_arrays:
        a = torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.float16)
        sv = torch.rand(shape[0], generator=gen, device="cuda") * 4 + 0.5
        folds.append((name, a, sv))

    def fold_all():
        for _, a, sv in folds:
            awq.awq_fold_inverse_scale(a, sv, out=a)
    fold_ms = median_ms(fold_all)
    fold_bytes = sum(4 * a.numel() + 4 * sv.numel() for _, a, sv in folds)
    res = {"fold": {"arrays": [[n, list(a.shape)] for n, a, _ in folds],
                    "us": round(fold_ms * 1e3, 2),
                    "gbs": round(fold_bytes / (fold_ms * 1e-3) / 1e9, 1)}}
    for m in tokens:
        ys = [torch.empty((m, L["o"]), dtype=torch.float32, device="cuda") for L in layers]
        xs = [L["X"][:m].contiguous() for L in layers]
        per = {}
        for L, x, y in zip(layers, xs, ys):
            ms = median_ms(lambda: awq.awq_w4a16_matmul(x, L["qw"], L["st"], L["zr"], out=y))
            rd = median_ms(lambda: calib.awq_calib_read_oneshot(L["qw"].data_ptr(),
                                                                L["qw"].numel() * 4,
                                                                sink.data_ptr(), stream))
            per[L["name"]] = {"shape": [m, L["k"], L["o"]], "us": round(ms * 1e3, 2),
                              "gbs": round(layer_bytes(L, m) / (ms * 1e-3) / 1e9, 1),
                              "plain_read_of_codes_gbs": round(L["qw"].numel() * 4 /
                                                               (rd * 1e-3) / 1e9, 1)}

        def block():
            for L, x, y in zip(layers, xs, ys):
                awq.awq_w4a16_matmul(x, L["qw"], L["st"], L["zr"], out=y)
        ms = median_ms(block)
        tot = sum(layer_bytes(L, m) for L in layers)
        res[m] = {"block_us": round(ms * 1e3, 2), "block_gbs": round(tot / (ms * 1e-3) / 1e9, 1),
                  "block_bytes": tot, "layers": per,
                  "fp16_weights_us_at_same_rate": round(
                      sum(2 * L["o"] * L["k"] for L in layers) / (tot / (ms * 1e-3)) * 1e6, 2)}
    return res


def ablation_bench(configs):
    """Best search loss with four saliency choices on the same seeded layers:
    activation magnitude (the method), weight magnitude, and each restricted to
    the top 1% of channels (others unscaled); the loss at alpha = 0 is plain
    round-to-nearest.  All on the GPU path."""
    import torch
    import synth
    import post_bit_weight_awq_amd as awq
    awq.load()
    cfg = awq.default_config()
    rows = []
    for c, layer in configs:
        spec, X, W = synth.make_layer(c, layer)
        Xd, Wd = torch.from_numpy(X).cuda(), torch.from_numpy(W).cuda()
        del X, W
        k = spec.in_features
        n1 = max(1, round(0.01 * k))
        sal_a = awq.awq_act_stats(Xd)
        sal_w = awq.awq_weight_saliency(Wd)
        choices = {"activation": sal_a, "weight": sal_w,
                   "activation_top1pct": awq.awq_select_top_channels(sal_a, n1),
                   "weight_top1pct": awq.awq_select_top_channels(sal_w, n1)}
        out = {"config": c, "layer": spec.name, "shape": [spec.n_tokens, k, spec.out_features],
               "top_channels": n1}
        for name, sal in choices.items():
            r = awq.awq_search_layer(Xd, Wd, sal, cfg)
            losses = r.losses.cpu().numpy()
            b = int(r.best_idx.item())
            out[name] = {"best_alpha": b / cfg.n_grid, "best_loss": float(losses[b])}
            out["rtn_loss"] = float(losses[0])
        for name in choices:
            out[name]["vs_rtn"] = round(out[name]["best_loss"] / out["rtn_loss"], 4)
        rows.append(out)
        log(f"ablation {spec.name}: " + ", ".join(f"{n} {out[n]['vs_rtn']}" for n in choices))
        del Xd, Wd
        torch.cuda.empty_cache()
    return rows


def quant_variant_bench(configs):
    """Output MSE of plain round-to-nearest (alpha = 0) and of the searched
    scales for each quantizer variant (group size, bit width, zero point or
    symmetric), with the storage per weight of each format."""
    import torch
    import synth
    import post_bit_weight_awq_amd as awq
    out = []
    for c, layer in configs:
        spec, X, W = synth.make_layer(c, layer)
        Xd, Wd = torch.from_numpy(X).cuda(), torch.from_numpy(W).cuda()
        del X, W
        sal = awq.awq_act_stats(Xd)
        for g in (128, 64, 32):
            for b in (4, 3):
                for zp in (True, False):
                    cfg = awq.default_config(group_size=g, w_bit=b, zero_point=zp)
                    r = awq.awq_search_layer(Xd, Wd, sal, cfg)
                    losses = r.losses.cpu().numpy()
                    best = int(r.best_idx.item())
                    out.append({"config": c, "layer": spec.name, "group": g, "w_bit": b,
                                "zero_point": zp, "rtn_loss": float(losses[0]),
                                "awq_loss": float(losses[best]), "best_alpha": best / cfg.n_grid,
                                "bits_per_weight": 4 + 32.0 / g})
        log(f"quantizer variants done for {spec.name}")
        del Xd, Wd
        torch.cuda.empty_cache()
    return out


def copy_calibration(mib):
    """A plain device-to-device copy of a known size (PMC byte-counter scale)."""
    import torch
    n = mib * (1 << 20)
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 3}))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the shader clock rises over the first ~10 ms of sustained load: 20 warm-up
    # steps of the default layer reach the steady state
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=DEFAULT_CONFIG, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=25.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0)
    ap.add_argument("--group", type=int, default=128, choices=[32, 64, 128],
                    help="quantization group size (ablation variants; the method uses 128)")
    ap.add_argument("--w-bit", type=int, default=4, choices=[3, 4])
    ap.add_argument("--symmetric", action="store_true",
                    help="symmetric round-to-nearest codes instead of a zero point")
    ap.add_argument("--ablation", action="store_true",
                    help="best loss with activation vs weight saliency, all vs top 1% channels")
    ap.add_argument("--decode", action="store_true",
                    help="time the W4A16 product on packed weights (13B block, 1 and 16 tokens)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this path runs on one GPU; multi-GPU runs are not part of it "
              "(each GPU would search its own share of output rows and all-reduce 20 "
              "partial sums)", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return

    if args.ablation:
        import torch
        if not torch.cuda.is_available():
            print("bench.py: no GPU visible", file=sys.stderr)
            sys.exit(1)
        cases = [(1, 0), (2, 0), (3, 0), (4, 0), (4, 1), (5, 0), (5, 1), (5, 2), (5, 3)]
        rows = ablation_bench(cases)
        variants = quant_variant_bench([(2, 0), (5, 3)])
        print(json.dumps({"metric": "best search loss / round-to-nearest loss per saliency choice",
                          "unit": "ratio", "higher_is_better": False, "n_gpus": 1,
                          "data": "synthetic (seeded generators, outlier-channel activations)",
                          "rows": rows, "quantizer_variants": variants}))
        return

    if args.decode:
        import torch
        if not torch.cuda.is_available():
            print("bench.py: no GPU visible", file=sys.stderr)
            sys.exit(1)
        res = decode_bench((1, 16), max(5, args.steps))
        fold = res.pop("fold")
        one = res[1]
        print(json.dumps({
            "metric": "W4A16 decode product on packed AWQ weights, HBM GB/s (1 GPU)",
            "value": one["block_gbs"], "unit": "GB/s", "n_gpus": 1, "steps": max(5, args.steps),
            "warmup": 1, "ms_per_step": round(one["block_us"] / 1e3, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
            "data": "synthetic (seeded N(0,0.02) weights packed by awq_pack; N(0,1) activations)",
            "config": {"workload": "llama13b_block_decode_w4a16_tok1",
                       "layers": [list(x) for x in DECODE_LAYERS], "tokens": 1,
                       "cache": "MALL cleared before each measurement"},
            "roofline": {"bound": "hbm", "kernel": "k_w4a16_gemv", "achieved": one["block_gbs"],
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(one["block_gbs"] / HBM_PEAK_GBS, 4), "traffic": None},
            "by_tokens": res,
            "fold_inverse_scale": dict(fold, bound="hbm", peak_gbs=HBM_PEAK_GBS,
                                       frac=round(fold["gbs"] / HBM_PEAK_GBS, 4))}))
        return

    import numpy as np
    import torch
    import synth
    import post_bit_weight_awq_amd as awq

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    awq.load()
    cfgspec = synth.CONFIGS[args.config]
    cfg = awq.default_config(group_size=args.group, w_bit=args.w_bit,
                             zero_point=not args.symmetric)
    layers = []
    for li, spec in enumerate(cfgspec.layers):
        _, X, W = synth.make_layer(args.config, li)
        Xd = torch.from_numpy(X).cuda()
        Wd = torch.from_numpy(W).cuda()
        del X, W
        n, k, o = spec.n_tokens, spec.in_features, spec.out_features
        L = dict(spec=spec, X=Xd, W=Wd,
                 sal=torch.empty(k, dtype=torch.float32, device="cuda"),
                 sws=torch.empty(awq.awq_act_stats_workspace_size(n, k), dtype=torch.uint8,
                                 device="cuda"),
                 ws=torch.empty(awq.awq_search_workspace_size(n, k, o, cfg), dtype=torch.uint8,
                                device="cuda"),
                 losses=torch.empty(cfg.n_grid, dtype=torch.float64, device="cuda"),
                 best=torch.empty(1, dtype=torch.int32, device="cuda"),
                 s_best=torch.empty(k, dtype=torch.float32, device="cuda"),
                 qw=torch.empty((o, k // 8), dtype=torch.int32, device="cuda"),
                 st=torch.empty((o, k // cfg.group_size), dtype=torch.float16, device="cuda"),
                 zr=torch.empty((o, k // cfg.group_size), dtype=torch.float16, device="cuda"))
        layers.append(L)
        log(f"layer {spec.name}: {n}x{k}->{o}")
    torch.cuda.synchronize()

    names = ("stats", "prepare", "grid", "select", "pack")

    def step(ev=None):
        """One pass of the hot path over every layer: saliency, search (prepare,
        grid, select), pack, with a HIP event before and after each stage on the
        stream the calls launch on (torch's current stream)."""
        for li, L in enumerate(layers):
            e = ev[li] if ev is not None else None

            def mark(j):
                if e is not None:
                    e[j].record()
            mark(0)
            awq.awq_act_stats(L["X"], out=L["sal"], workspace=L["sws"])
            mark(1)
            for j, stg in enumerate((awq.STAGE_PREPARE, awq.STAGE_GRID, awq.STAGE_SELECT)):
                awq.awq_search_layer(L["X"], L["W"], L["sal"], cfg, workspace=L["ws"],
                                     losses=L["losses"], best_idx=L["best"],
                                     s_best=L["s_best"], stages=stg)
                mark(2 + j)
            awq.awq_pack(L["W"], L["s_best"], cfg, qweight=L["qw"], step=L["st"], zero=L["zr"])
            mark(5)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed region: exactly args.steps steps, synchronized on both sides; the
    # per-stage events inside it are the live kernel timings (each event adds a few
    # microseconds of queue time, well under 1 % of a block step)
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in layers]
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    per = {nm: [0.0] * len(layers) for nm in names}
    samples = {nm: [[] for _ in layers] for nm in names}
    for s in range(args.steps):
        for li in range(len(layers)):
            e = evs[s][li]
            for j, nm in enumerate(names):
                dt = e[j].elapsed_time(e[j + 1])
                per[nm][li] += dt / args.steps
                samples[nm][li].append(dt)

    def med(xs):
        return sorted(xs)[len(xs) // 2]

    F = [search_flops(L["spec"], cfg.n_grid) for L in layers]
    total_F = sum(F)
    value = total_F / (ms_per_step * 1e-3) / 1e12
    grid_ms = sum(per["grid"])
    achieved = total_F / (grid_ms * 1e-3) / 1e12
    kernels = {}
    for li, L in enumerate(layers):
        spec = L["spec"]
        kernels[spec.name] = {
            "shape": [spec.n_tokens, spec.in_features, spec.out_features],
            "best_idx": int(L["best"].item()),
            "losses": [float(v) for v in L["losses"].cpu().tolist()],
            "ms": {nm: round(per[nm][li], 5) for nm in names},
            "ms_median": {nm: round(med(samples[nm][li]), 5) for nm in names},
            "ms_min": {nm: round(min(samples[nm][li]), 5) for nm in names},
            "grid_tflops": round(F[li] / (per["grid"][li] * 1e-3) / 1e12, 2),
            "search_tflops": round(F[li] / ((per["prepare"][li] + per["grid"][li] +
                                             per["select"][li]) * 1e-3) / 1e12, 2),
            # the few-microsecond stages from their median: one late sample moves a mean
            "stats_gbs": round(stats_bytes(spec) / (med(samples["stats"][li]) * 1e-3) / 1e9, 1),
            "pack_gbs": round(pack_bytes(spec, cfg.group_size) /
                              (med(samples["pack"][li]) * 1e-3) / 1e9, 1),
        }
    traffic = traffic_from_profiles(cfgspec.workload)
    calib = load_calib()
    measured = None
    block_cold = None
    if calib is not None:
        cold, mfma_peak = cold_measurements(awq, cfg, layers, calib)
        block_cold = cold.pop("_block")
        for name, v in cold.items():
            kernels[name].update(v)
        measured = {"mfma_f16_loop_tflops": mfma_peak,
                    "note": "MFMA-only register loop with the grid kernel's instruction and "
                            "wavefront shape; *_cold: MALL cleared by a 512 MiB read first"}

    def hbm_stage(stage, nbytes, plain_key):
        """Bytes of the stage over all layers / the sum of its median times in
        the timed steps, against the HBM peak and against a plain streaming
        read of the same input (cold, same size) where one was measured; for
        stats and pack also the step's calls timed back to back after a MALL
        clear (one event pair, so no between-stage event time is counted)."""
        b = sum(nbytes(L["spec"]) for L in layers)
        ms = sum(med(samples[stage][li]) for li in range(len(layers)))
        gbs = b / (ms * 1e-3) / 1e9
        r = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_step": b,
             "per_layer": {L["spec"].name: round(nbytes(L["spec"]) / (
                 med(samples[stage][li]) * 1e-3) / 1e9, 1) for li, L in enumerate(layers)}}
        if plain_key and all(plain_key in kernels[L["spec"].name] for L in layers):
            pr = {L["spec"].name: kernels[L["spec"].name][plain_key] for L in layers}
            r["plain_read_gbs_cold"] = pr
            r["frac_of_plain_read"] = {n: round(r["per_layer"][n] / pr[n], 3) for n in pr}
        if block_cold is not None and stage + "_ms" in block_cold:
            # the step's calls back to back after a MALL clear, one event pair
            bg = b / (block_cold[stage + "_ms"] * 1e-3) / 1e9
            src = "X" if stage == "stats" else "W"
            rd = block_cold["plain_read_of_" + src + "_ms"]
            rb = sum(L[src].numel() * 2 for L in layers)
            r["back_to_back_cold"] = {
                "achieved": round(bg, 1), "frac": round(bg / HBM_PEAK_GBS, 4),
                "plain_read_gbs": round(rb / (rd * 1e-3) / 1e9, 1),
                "frac_of_plain_read": round(bg / (rb / (rd * 1e-3) / 1e9), 3)}
        return r

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded generators, outlier-channel activations, N(0,0.02) weights)",
        "config": {"workload": cfgspec.workload, "layers": [
            {"name": L["spec"].name, "n_tokens": L["spec"].n_tokens,
             "in_features": L["spec"].in_features, "out_features": L["spec"].out_features}
            for L in layers], "group_size": cfg.group_size, "w_bit": cfg.w_bit,
            "zero_point": bool(cfg.zero_point), "n_grid": cfg.n_grid},
        "roofline": {"bound": "mfma",
                     "kernel": grid_kernel_names(layers, cfg) + " (the grid stage of each "
                               "search: all 20 grid points' contractions and squared errors; "
                               "the weight-error production is in the prepare stage)",
                     "achieved": round(achieved, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": traffic,
                     "flops_per_search": {L["spec"].name: F[li] for li, L in enumerate(layers)},
                     "grid_ms_per_search": {L["spec"].name: round(per["grid"][li], 5)
                                            for li, L in enumerate(layers)},
                     "frac_per_layer": {L["spec"].name: round(
                         F[li] / (per["grid"][li] * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)
                         for li, L in enumerate(layers)},
                     "stats": hbm_stage("stats", stats_bytes, "plain_read_of_X_gbs_cold"),
                     **({"weight_error": hbm_stage(
                         "prepare", lambda sp: weight_error_bytes(sp, cfg.n_grid), "")}
                        if all(uses_contraction(L["spec"], cfg) for L in layers) else {}),
                     "pack": hbm_stage("pack", lambda sp: pack_bytes(sp, cfg.group_size),
                                       "plain_read_of_W_gbs_cold")},
        "kernels": kernels,
        "measured_peaks": measured,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(args.config, args.cpu_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
