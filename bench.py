"""Benchmark of the fine-grained FP8 hot path on one MI355X.

Default workload: the dense Fprop GEMM shaped like a DeepSeek-V3 MoE
down-projection, M=4096 tokens, K=2048, N=7168, BF16 output.  One step is the
whole path on one batch: online 1x128 quantization of the fp32 activations and
online 128x128 quantization of the fp32 weights (training re-quantizes its
master weights every step), both in one launch (fp8_quant_fprop_operands), and
the block-scaled FP8 GEMM.  Four independent
input sets rotate from step to step so that no step finds its inputs in the
256 MB last-level cache; all inputs are resident in HBM before timing starts.

Prints one JSON line.  `value` = GEMM FLOPs / step time (TFLOPS, whole step).
A step is two launches on one stream with nothing between them; HIP events
bracket only the whole timed region.  `step_three_launches_ms` times the same
step with the two quantizations as separate launches.  `kernels_us` holds each kernel's
duration alone: the mean of back-to-back launches between two HIP events on
the bench stream, right after the timed steps, which is what a kernel trace of
the same command reports per launch.  `roofline` describes the GEMM kernel,
with that duration, as a fraction of the dense FP8 MFMA peak (the metric's
basis); `frac_of_bf16_peak` is the same rate against the BF16 matrix cores
the exact engine runs on.  `masked_decode` holds the masked-layout MoE decode
GEMMs' HBM rates (both shapes, plain and decode-tiled weights).  `fp8mfma_engine`
and `mx_variant` time, on the same shape, the GEMMs with other numeric
contracts (FP8 MFMA on the block-scaled codes; MX operands), not the step.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0        # MI355X dense FP8 MFMA, published
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense BF16 MFMA, published
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E, published
METRIC = "FP8 block-scaled GEMM TFLOPS + % of MI355X FP8 MFMA peak (dense, MoE grouped)"
GEMM_SRC = os.path.join(ROOT, "fp8_fine_grained_amd", "csrc", "gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_dense_4096x7168x2048_traffic.md")


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--sets", type=int, default=4, help="rotating input sets")
    p.add_argument("--cpu-rows", type=int, default=4096, help="rows of the oracle's timed sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--settle-s", type=float, default=0.5,
                   help="seconds of untimed steps before the warmup steps (clock settling)")
    p.add_argument("--profile-kernel", choices=["gemm", "quant_act", "quant_weight", "quant_fprop", "copy", "masked",
                                                "masked_tiled", "masked_down", "masked_down_tiled", "trio_fprop",
                                                "trio_dgrad", "trio_wgrad", "contig", "mx", "fp8mfma"],
                   help="counter-collection driver: launch only this kernel `steps` times (gemm, quant_*: on "
                        "the dense_fprop inputs; copy: a 1 GiB device-to-device copy, the byte-counter "
                        "calibration; masked*: the masked decode GEMM, gate+up or down shape, on plain / "
                        "decode-tiled weights; trio_*: the linear_trio GEMMs; contig: the moe_contig "
                        "gate+up GEMM; mx: the MX GEMM on the dense_fprop shape; fp8mfma: the FP8-MFMA engine on "
                        "the dense_fprop inputs); prints no JSON")
    p.add_argument("--workload", default="dense_fprop",
                   choices=["dense_fprop", "dense_small", "linear_trio", "moe_contig", "moe_masked", "dense_mx"],
                   help="dense_fprop is the headline step; the others print one line per measured kernel")
    return p.parse_args()


def source_hash():
    with open(GEMM_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def stored_traffic():
    """HBM bytes per GEMM launch from the committed counter summary, if it was
    taken on the current kernel source; otherwise None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m_src = re.search(r"kernel source sha256/16:\s*([0-9a-f]+)", text)
    m_b = re.search(r"HBM bytes per launch \(calibrated\):\s*([0-9.eE+]+)", text)
    if not (m_src and m_b) or m_src.group(1) != source_hash():
        return None
    return float(m_b.group(1))


def cpu_baseline(x, w, rows, min_seconds=10.0):
    """The oracle, untouched, on the first `rows` rows of one input set (whole
    passes repeated until `min_seconds` have elapsed): 1x128
    quantization of those rows, 128x128 quantization of the whole weight
    (every output row needs all of it), exact dequantization and the float64
    GEMM plus |A||B| bound term.  Rate reported in the GEMM's FLOP units."""
    from oracle import gemm, quant, e4m3
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = 1
    reps = 0
    t0 = time.perf_counter()
    while True:     # whole passes until about 10 s of CPU work
        qa, sa = quant.quant_act_1x128(x[:rows])
        qb, sb = quant.quant_weight_128x128(w)
        c, s = gemm.gemm_blockscaled_ref(qa, sa, qb, sb)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    flops = 2.0 * rows * w.shape[0] * w.shape[1] * reps
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOPS", "cores": max(blas, e4m3._threads()),
            "kind": "oracle",
            "sample": f"{rows} of 4096 activation rows (1x128 quantization), the full 7168x2048 weight "
                      f"(128x128 quantization), float64 GEMM and |A||B| on those rows, {reps} passes in "
                      f"{dt:.2f} s"}


_SETTLE = {"seconds": 0.5}


_FLUSH = {}


def _flush(stream):
    """Read a 512 MB buffer (twice the 256 MB last-level cache) on the stream,
    so the next launch finds none of its inputs in any cache.  Reading, not
    writing: a write would leave dirty lines whose write-back then competes
    with the timed kernel for HBM."""
    import torch
    if "buf" not in _FLUSH:
        _FLUSH["buf"] = torch.ones(1 << 27, dtype=torch.float32, device="cuda")
        _FLUSH["sum"] = torch.empty((), dtype=torch.float32, device="cuda")
    torch.sum(_FLUSH["buf"], dim=0, out=_FLUSH["sum"])


def time_launches(fn, steps, warmup, stream):
    """Duration (ms) of one fn() with its inputs in HBM, not in a cache: each of
    `steps` launches follows an untimed 512 MB read and is bracketed by its
    own pair of HIP events on the launch stream; the mean over the launches, the
    median of three such runs.  Each call first keeps the GPU busy with fn for
    --settle-s seconds, untimed, so the clock has settled after the set-up
    work between lines."""
    import torch
    t_end = time.perf_counter() + _SETTLE["seconds"]
    n = 0
    while time.perf_counter() < t_end:
        fn(n)
        n += 1
        if n % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    runs = []
    for _ in range(3):
        ev = []
        for i in range(steps):
            _flush(stream)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn(i)
            b.record(stream)
            ev.append((a, b))
        torch.cuda.synchronize()
        runs.append(sum(a.elapsed_time(b) for a, b in ev) / steps)
    return float(np.median(runs))


def rotating_launches(fns, steps, warmup, stream):
    """Duration (ms) of one launch in a stream of back-to-back launches that
    cycle through len(fns) input sets, each larger than the 256 MB last-level
    cache, so that every launch reads its inputs from HBM while the next
    launch's dispatch overlaps the current one (as in a model's decode step).
    `steps` launches between two HIP events on the launch stream; the median
    of three such runs, after --settle-s seconds of untimed launches and
    `warmup` more."""
    import torch
    t_end = time.perf_counter() + _SETTLE["seconds"]
    n = 0
    while time.perf_counter() < t_end:
        fns[n % len(fns)]()
        n += 1
        if n % 64 == 0:
            torch.cuda.synchronize()
    for i in range(warmup):
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    runs = []
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(steps):
            fns[i % len(fns)]()
        b.record(stream)
        torch.cuda.synchronize()
        runs.append(a.elapsed_time(b) / steps)
    return float(np.median(runs))


def extra_line(workload, kernel, ms, flops=None, nbytes=None, args=None, config=None, peak=None):
    line = {"metric": METRIC if flops else "HBM GB/s of " + kernel, "workload": workload, "kernel": kernel,
            "us": round(ms * 1e3, 2), "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "data": "synthetic, seeded (drawn on the GPU)", "config": config or {}}
    if flops:
        tf = flops / (ms * 1e-3) / 1e12
        line.update({"value": round(tf, 2), "unit": "TFLOPS",
                     "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS,
                                  "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4),
                                  "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                                  "matrix_cores": peak or "BF16 (codes widened exactly)"}})
    if nbytes:
        gbs = nbytes / (ms * 1e-3) / 1e9
        line.setdefault("value", round(gbs, 1))
        line.setdefault("unit", "GB/s")
        line["hbm"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                       "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": int(nbytes)}
    print(json.dumps(line), flush=True)


def gpu_acts(gen, rows, K, frac, mult, sigma=1.0):
    """N(0, sigma) activations with whole outlier channels, drawn on the GPU."""
    import torch
    x = torch.randn((rows, K), generator=gen, device="cuda") * sigma
    if frac > 0:
        n = max(1, int(round(frac * K)))
        idx = torch.randperm(K, generator=gen, device="cuda")[:n]
        x[:, idx] *= mult
    return x


def masked_inputs(gen, G, MMAX, N, K):
    """The masked decode workload on the GPU: seeded valid-row counts, 1x128
    quantized activations and 128x128 quantized expert weights."""
    import torch
    import fp8_fine_grained_amd as fp8
    import workloads
    mm, _ = workloads.moe_masked_inputs(N, 128, G, MMAX)
    a = gpu_acts(gen, G * MMAX, K, 0.001, 100.0).reshape(G, MMAX, K).contiguous()
    qa = torch.empty((G, MMAX, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty((G, K // 128, MMAX), dtype=torch.float32, device="cuda")
    for g in range(G):
        fp8.fp8_quant_act_1x128(a[g], q=qa[g], s=sa[g])
    del a
    qb = torch.empty((G, N, K), dtype=torch.uint8, device="cuda")
    sb = torch.empty((G, N // 128, K // 128), dtype=torch.float32, device="cuda")
    for g in range(G):
        wg = torch.randn((N, K), generator=gen, device="cuda") * 0.02
        fp8.fp8_quant_weight_128x128(wg, q=qb[g], s=sb[g])
    mmt = torch.from_numpy(mm.astype(np.int32)).cuda()
    c = torch.empty((G, MMAX, N), dtype=torch.bfloat16, device="cuda")
    return mm, qa, sa, qb, sb, mmt, c


def trio_inputs(gen):
    """The linear_trio tensors on the GPU (8192 tokens, 7168 in, 2048 out):
    activations with outlier channels, weights, upstream gradients."""
    import torch
    TOK, IN, OUT = 8192, 7168, 2048
    x = gpu_acts(gen, TOK, IN, 0.001, 100.0)
    w = torch.randn((OUT, IN), generator=gen, device="cuda") * 0.02
    dy = torch.randn((TOK, OUT), generator=gen, device="cuda") * 1e-3
    return x, w, dy


def contig_inputs(gen):
    """The moe_contig gate+up GEMM's operands on the GPU: 32 experts' rows in
    128-aligned segments (seeded counts), 1x128-quantized, and 32 experts'
    128x128-quantized 4096x7168 weights."""
    import torch
    import fp8_fine_grained_amd as fp8
    import workloads
    G, N, K = 32, 4096, 7168
    counts, off = workloads.moe_contig_layout()
    mt = int(off[-1])
    a = torch.zeros((mt, K), device="cuda")
    xa = gpu_acts(gen, int(counts.sum()), K, 0.001, 100.0)
    pos = 0
    for g in range(G):
        a[int(off[g]):int(off[g]) + int(counts[g])] = xa[pos:pos + int(counts[g])]
        pos += int(counts[g])
    del xa
    qa, sa = fp8.fp8_quant_act_1x128(a)
    qb = torch.empty((G, N, K), dtype=torch.uint8, device="cuda")
    sb = torch.empty((G, N // 128, K // 128), dtype=torch.float32, device="cuda")
    for g in range(G):
        wg = torch.randn((N, K), generator=gen, device="cuda") * 0.02
        fp8.fp8_quant_weight_128x128(wg, q=qb[g], s=sb[g])
    offs = torch.from_numpy(off.astype(np.int32)).cuda()
    return a, qa, sa, qb, sb, offs, counts, mt


def mx_experts(gen, G, N, K):
    """G experts' fresh N(0, 0.02) weights [N][K], MX-quantized one by one on
    the GPU: codes [G][N][K] and E8M0 bytes [G][K/32][N]."""
    import torch
    import fp8_fine_grained_amd as fp8
    qb = torch.empty((G, N, K), dtype=torch.uint8, device="cuda")
    eb = torch.empty((G, K // 32, N), dtype=torch.uint8, device="cuda")
    for g in range(G):
        wg = torch.randn((N, K), generator=gen, device="cuda") * 0.02
        fp8.fp8_quant_mx_1x32(wg, q=qb[g], e=eb[g])
    return qb, eb


def profile_other(args):
    """Counter-collection driver for the masked decode GEMMs (both shapes),
    the linear_trio GEMMs and the contiguous grouped GEMM: build that
    workload's inputs, then launch only the named kernel `steps` times."""
    import torch
    import fp8_fine_grained_amd as fp8
    import workloads
    fp8.load_library()
    k = args.profile_kernel
    if k.startswith("masked"):
        gen = torch.Generator(device="cuda").manual_seed(workloads.SEEDS.get("moe_masked", 105))
        N, K = (7168, 2048) if k.startswith("masked_down") else (4096, 7168)
        mm, qa, sa, qb, sb, mmt, c = masked_inputs(gen, 32, 128, N, K)
        if k.endswith("_tiled"):
            qb = fp8.fp8_tile_weights_decode(qb)
            fn = lambda: fp8.fp8_grouped_gemm_masked_tiled(qa, sa, qb, sb, mmt, out=c)
        else:
            fn = lambda: fp8.fp8_grouped_gemm_masked(qa, sa, qb, sb, mmt, out=c)
        what = f"N={N} K={K}, valid rows {int(mm.sum())}"
    elif k.startswith("trio_"):
        gen = torch.Generator(device="cuda").manual_seed(workloads.SEEDS.get("linear_trio", 1))
        x, w, dy = trio_inputs(gen)
        if k == "trio_fprop":
            qx, sx = fp8.fp8_quant_act_1x128(x)
            qw, sw = fp8.fp8_quant_weight_128x128(w)
            c = torch.empty((x.shape[0], w.shape[0]), dtype=torch.bfloat16, device="cuda")
            fn = lambda: fp8.fp8_gemm_blockscaled(qx, sx, qw, sw, 0, torch.bfloat16, out=c)
        elif k == "trio_dgrad":
            qd, sd = fp8.fp8_quant_act_1x128(dy)
            qwt, swt = fp8.fp8_quant_weight_128x128(w, transpose_out=True)
            c = torch.empty((x.shape[0], x.shape[1]), dtype=torch.bfloat16, device="cuda")
            fn = lambda: fp8.fp8_gemm_blockscaled(qd, sd, qwt, swt, 0, torch.bfloat16, out=c)
        else:
            qdt, sdt = fp8.fp8_quant_act_1x128(dy, transpose_out=True)
            qxt, sxt = fp8.fp8_quant_act_1x128(x, transpose_out=True)
            c = torch.empty((w.shape[0], w.shape[1]), dtype=torch.float32, device="cuda")
            fn = lambda: fp8.fp8_gemm_blockscaled(qdt, sdt, qxt, sxt, 1, torch.float32, out=c)
        del x, w, dy
        what = "8192 tokens, 7168 in, 2048 out"
    elif k == "mx":
        gen = torch.Generator(device="cuda").manual_seed(workloads.SEEDS.get("dense_mx", 1))
        M, N, K = 4096, 7168, 2048
        qa, ea = fp8.fp8_quant_mx_1x32(gpu_acts(gen, M, K, 0.001, 100.0))
        qb, eb = fp8.fp8_quant_mx_1x32(torch.randn((N, K), generator=gen, device="cuda") * 0.02)
        c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        fn = lambda: fp8.fp8_gemm_mx(qa, ea, qb, eb, torch.bfloat16, out=c)
        what = f"{M}x{N}x{K}"
    else:
        gen = torch.Generator(device="cuda").manual_seed(workloads.SEEDS.get("moe_contig", 1))
        a, qa, sa, qb, sb, offs, counts, mt = contig_inputs(gen)
        del a
        c = torch.empty((mt, qb.shape[1]), dtype=torch.bfloat16, device="cuda")
        fn = lambda: fp8.fp8_grouped_gemm_contiguous(qa, sa, qb, sb, offs, out=c)
        what = f"{mt} padded rows, {int(counts.sum())} routed"
    torch.cuda.synchronize()
    for _ in range(args.steps):
        fn()
    torch.cuda.synchronize()
    print(f"profiled {k} x{args.steps} ({what})", flush=True)


MASKED_SETS = 3   # rotating input sets of the masked decode timing (each >= 470 MB of weights)


def masked_sets(gen, G, MMAX, N, K):
    """MASKED_SETS independent masked-decode input sets (same valid-row
    counts, fresh activations and weights), each with its decode-tiled copy."""
    import fp8_fine_grained_amd as fp8
    out = []
    for _ in range(MASKED_SETS):
        mm, qa, sa, qb, sb, mmt, c = masked_inputs(gen, G, MMAX, N, K)
        out.append(dict(mm=mm, qa=qa, sa=sa, qb=qb, sb=sb, mmt=mmt, c=c, qt=fp8.fp8_tile_weights_decode(qb)))
    return out


def masked_times(sets, args, stream):
    """(plain, tiled) per-launch ms of the masked GEMM: back to back over the
    rotating sets (rotating_launches), and single launches after a cache
    flush, each between its own events (time_launches; the events add their
    dispatch gap, about 5 us)."""
    import fp8_fine_grained_amd as fp8
    plain = [lambda s=s: fp8.fp8_grouped_gemm_masked(s["qa"], s["sa"], s["qb"], s["sb"], s["mmt"], out=s["c"])
             for s in sets]
    tiled = [lambda s=s: fp8.fp8_grouped_gemm_masked_tiled(s["qa"], s["sa"], s["qt"], s["sb"], s["mmt"], out=s["c"])
             for s in sets]
    return {"plain": rotating_launches(plain, args.steps, args.warmup, stream),
            "tiled": rotating_launches(tiled, args.steps, args.warmup, stream),
            "plain_single": time_launches(lambda i: plain[0](), args.steps, args.warmup, stream),
            "tiled_single": time_launches(lambda i: tiled[0](), args.steps, args.warmup, stream)}


def masked_decode_rates(args):
    """HBM rate of the masked-layout decode GEMM on both MoE shapes (gate+up
    K=7168 N=4096, down K=2048 N=7168; 32 experts, 128-row buffers, U{1..64}
    valid rows), on plain and on decode-tiled weights.  Bytes: every expert's
    weights and scales, the valid A rows and their scales, the valid C rows."""
    import torch
    import workloads
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device="cuda").manual_seed(workloads.SEEDS.get("moe_masked", 105))
    out = {}
    G, MMAX = 32, 128
    for name, (N, K) in (("gate_up", (4096, 7168)), ("down", (7168, 2048))):
        sets = masked_sets(gen, G, MMAX, N, K)
        valid = int(sets[0]["mm"].sum())
        nbytes = G * N * K + G * (N // 128) * (K // 128) * 4 + valid * K + valid * (K // 128) * 4 + valid * N * 2
        t = masked_times(sets, args, stream)
        gbs = {k: nbytes / (v * 1e-3) / 1e9 for k, v in t.items()}
        out[name] = {"N": N, "K": K, "valid_rows": valid, "algorithmic_bytes": int(nbytes),
                     "plain_us": round(t["plain"] * 1e3, 2), "plain_gbs": round(gbs["plain"], 1),
                     "plain_frac_of_hbm": round(gbs["plain"] / PEAK_HBM_GBS, 4),
                     "tiled_us": round(t["tiled"] * 1e3, 2), "tiled_gbs": round(gbs["tiled"], 1),
                     "tiled_frac_of_hbm": round(gbs["tiled"] / PEAK_HBM_GBS, 4),
                     "single_launch": {"plain_us": round(t["plain_single"] * 1e3, 2),
                                       "plain_frac_of_hbm": round(gbs["plain_single"] / PEAK_HBM_GBS, 4),
                                       "tiled_us": round(t["tiled_single"] * 1e3, 2),
                                       "tiled_frac_of_hbm": round(gbs["tiled_single"] / PEAK_HBM_GBS, 4)}}
        del sets
        torch.cuda.empty_cache()
    out["note"] = (f"back-to-back launches cycling through {MASKED_SETS} input sets (each set's weights exceed "
                   "the 256 MB last-level cache, so every launch streams them from HBM) between two HIP events; "
                   "single_launch: each launch after an untimed 512 MB read, between its own events (which add "
                   "their dispatch gap, about 5 us); tiled = weights in the decode-tiled layout "
                   "(fp8_tile_weights_decode, arranged once at load time); target >= 0.70 of the 8 TB/s HBM peak")
    return out


def run_extra(args):
    """The --workload lines.  Every kernel line is timed back to back over
    rotating input sets whose bytes together exceed the 256 MB last-level
    cache (rotating_launches), with one launch after a cache flush between
    its own events beside it (time_launches: `single_launch_us`)."""
    import torch
    import fp8_fine_grained_amd as fp8
    import workloads
    fp8.load_library()
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device="cuda").manual_seed(workloads.SEEDS.get(args.workload, 1))
    T, W = args.steps, args.warmup

    def line(workload, kernel, fn, sets, config, **kw):
        fns = [lambda s=s: fn(s) for s in sets]
        ms = rotating_launches(fns, T, W, stream)
        ms1 = time_launches(lambda i: fns[0](), T, W, stream)
        extra_line(workload, kernel, ms, args=args, config=dict(
            config, timing=f"back to back over {len(sets)} rotating input sets",
            single_launch_us=round(ms1 * 1e3, 2)), **kw)

    if args.workload == "dense_small":
        # launch-latency bound: one small set, back-to-back launches
        M, N, K = 128, 256, 512
        x = gpu_acts(gen, M, K, 0.005, 50.0)
        w = torch.randn((N, K), generator=gen, device="cuda") * 0.02
        qa, sa = fp8.fp8_quant_act_1x128(x)
        qb, sb = fp8.fp8_quant_weight_128x128(w)
        sets = [dict(qa=qa, sa=sa, qb=qb, sb=sb, c=torch.empty((M, N), dtype=torch.bfloat16, device="cuda"))]
        line("dense_small 128x256x512", "gemm_blockscaled",
             lambda s: fp8.fp8_gemm_blockscaled(s["qa"], s["sa"], s["qb"], s["sb"], 0, torch.bfloat16, out=s["c"]),
             sets, {"M": M, "N": N, "K": K, "note": "launch-latency bound"}, flops=2.0 * M * N * K)
    elif args.workload == "dense_mx":
        # the MX variant on the dense Fprop shapes: 1x32 blocks with E8M0 scales,
        # scales applied inside the FP8 MFMA, so its peak is the FP8 one
        M, N, K = 4096, 7168, 2048
        sets = []
        for _ in range(6):   # ~200 MB each
            x = gpu_acts(gen, M, K, 0.001, 100.0)
            w = torch.randn((N, K), generator=gen, device="cuda") * 0.02
            qa, ea = fp8.fp8_quant_mx_1x32(x)
            qb, eb = fp8.fp8_quant_mx_1x32(w)
            sets.append(dict(x=x, w=w, qa=qa, ea=ea, qb=qb, eb=eb,
                             c=torch.empty((M, N), dtype=torch.bfloat16, device="cuda")))
        cfg = {"M": M, "N": N, "K": K, "scales": "E8M0 per 1x32 block"}
        line("dense_mx", "quant_mx_1x32 X", lambda s: fp8.fp8_quant_mx_1x32(s["x"], q=s["qa"], e=s["ea"]), sets,
             cfg, nbytes=M * K * 5 + M * K // 32)
        line("dense_mx", "quant_mx_1x32 W", lambda s: fp8.fp8_quant_mx_1x32(s["w"], q=s["qb"], e=s["eb"]), sets,
             cfg, nbytes=N * K * 5 + N * K // 32)
        line("dense_mx", "gemm_mx 4096x7168x2048 BF16",
             lambda s: fp8.fp8_gemm_mx(s["qa"], s["ea"], s["qb"], s["eb"], torch.bfloat16, out=s["c"]), sets, cfg,
             flops=2.0 * M * N * K, peak="FP8 (scaled MFMA)")
    elif args.workload == "linear_trio":
        TOK, IN, OUT = 8192, 7168, 2048
        bf = torch.bfloat16
        sets = []
        for _ in range(4):   # ~1.3 GB each
            x, w, dy = trio_inputs(gen)
            s = dict(x=x, w=w, dy=dy, xh=x.to(bf), dyh=dy.to(bf), wh=w.to(bf))
            s["qx"], s["sx"] = fp8.fp8_quant_act_1x128(x)
            s["qxt"], s["sxt"] = fp8.fp8_quant_act_1x128(x, transpose_out=True)
            s["qd"], s["sd"] = fp8.fp8_quant_act_1x128(dy)
            s["qdt"], s["sdt"] = fp8.fp8_quant_act_1x128(dy, transpose_out=True)
            s["qw"], s["sw"] = fp8.fp8_quant_weight_128x128(w)
            s["qwt"], s["swt"] = fp8.fp8_quant_weight_128x128(w, transpose_out=True)
            # outputs of the timed quantizer launches other than the operands' own
            # (those rewrite the same bytes): requantization and the bf16 inputs
            for k in ("qx", "qxt", "qdt", "qw", "qwt"):
                s["o" + k] = torch.empty_like(s[k])
                s["o" + k.replace("q", "s", 1)] = torch.empty_like(s[k.replace("q", "s", 1)])
            s["yb"] = torch.empty((TOK, OUT), dtype=bf, device="cuda")
            s["qy"] = torch.empty((TOK, OUT), dtype=torch.uint8, device="cuda")
            s["sy"] = torch.empty((OUT // 128, TOK), dtype=torch.float32, device="cuda")
            s["dxb"] = torch.empty((TOK, IN), dtype=bf, device="cuda")
            s["dwf"] = torch.empty((OUT, IN), dtype=torch.float32, device="cuda")
            sets.append(s)
        cfg = {"tokens": TOK, "in": IN, "out": OUT}
        q1 = fp8.fp8_quant_act_1x128
        for name, src, tr, q, sc in (("quant_act_1x128 X rowwise", "x", False, "qx", "sx"),
                                     ("quant_act_1x128 X token-wise", "x", True, "qxt", "sxt"),
                                     ("quant_act_1x128 dY rowwise", "dy", False, "qd", "sd"),
                                     ("quant_act_1x128 dY token-wise", "dy", True, "qdt", "sdt")):
            n = sets[0][src].numel()
            line("linear_trio", name, lambda s, src=src, tr=tr, q=q, sc=sc: q1(s[src], transpose_out=tr, q=s[q],
                                                                                s=s[sc]),
                 sets, cfg, nbytes=n * 5 + (n // 128) * 4)
        for name, tr, q, sc in (("quant_weight_128x128 W", False, "qw", "sw"),
                                ("quant_weight_128x128 W transposed", True, "qwt", "swt")):
            line("linear_trio", name, lambda s, tr=tr, q=q, sc=sc: fp8.fp8_quant_weight_128x128(
                s["w"], transpose_out=tr, q=s[q], s=s[sc]), sets, cfg, nbytes=sets[0]["w"].numel() * 5)
        n = sets[0]["x"].numel()
        line("linear_trio", "requant_act_tokenwise X (rowwise FP8 cache -> token-wise)",
             lambda s: fp8.fp8_requant_act_tokenwise(s["qx"], s["sx"], qt=s["oqxt"], st=s["osxt"]), sets, cfg,
             nbytes=n * 2 + (n // 128) * 8)
        qh = fp8.fp8_quant_act_1x128_bf16
        for name, src, tr, q, sc in (("quant_act_1x128_bf16 X rowwise", "xh", False, "oqx", "osx"),
                                     ("quant_act_1x128_bf16 X token-wise", "xh", True, "oqxt", "osxt"),
                                     ("quant_act_1x128_bf16 dY token-wise", "dyh", True, "oqdt", "osdt")):
            n = sets[0][src].numel()
            line("linear_trio", name, lambda s, src=src, tr=tr, q=q, sc=sc: qh(s[src], transpose_out=tr, q=s[q],
                                                                                s=s[sc]),
                 sets, cfg, nbytes=n * 3 + (n // 128) * 4)
        for name, tr, q, sc in (("quant_weight_128x128_bf16 W", False, "oqw", "osw"),
                                ("quant_weight_128x128_bf16 W transposed", True, "oqwt", "oswt")):
            line("linear_trio", name, lambda s, tr=tr, q=q, sc=sc: fp8.fp8_quant_weight_128x128_bf16(
                s["wh"], transpose_out=tr, q=s[q], s=s[sc]), sets, cfg, nbytes=sets[0]["wh"].numel() * 3)
        fl = 2.0 * TOK * IN * OUT
        g = fp8.fp8_gemm_blockscaled
        line("linear_trio", "gemm Fprop 8192x2048x7168 BF16",
             lambda s: g(s["qx"], s["sx"], s["qw"], s["sw"], 0, bf, out=s["yb"]), sets, cfg, flops=fl)
        line("linear_trio", "gemm Fprop 8192x2048x7168, FP8 out (fused 1x128 quantization)",
             lambda s: fp8.fp8_gemm_blockscaled_fp8out(s["qx"], s["sx"], s["qw"], s["sw"], q=s["qy"], s=s["sy"]),
             sets, cfg, flops=fl)
        line("linear_trio", "gemm Dgrad 8192x7168x2048 BF16",
             lambda s: g(s["qd"], s["sd"], s["qwt"], s["swt"], 0, bf, out=s["dxb"]), sets, cfg, flops=fl)
        line("linear_trio", "gemm Wgrad 2048x7168x8192 FP32 (1x128 B)",
             lambda s: g(s["qdt"], s["sdt"], s["qxt"], s["sxt"], 1, torch.float32, out=s["dwf"]), sets, cfg,
             flops=fl)
        # the MX variant of the trio: every operand MX-quantized along its GEMM's contraction
        for s in sets:
            s["mqx"], s["mex"] = fp8.fp8_quant_mx_1x32(s["x"])
            s["mqw"], s["mew"] = fp8.fp8_quant_mx_1x32(s["w"])
            s["mqd"], s["med"] = fp8.fp8_quant_mx_1x32(s["dy"])
            s["mqwt"], s["mewt"] = fp8.fp8_quant_mx_1x32_transposed(s["w"])
            s["mqdt"], s["medt"] = fp8.fp8_quant_mx_1x32_transposed(s["dy"])
            s["mqxt"], s["mext"] = fp8.fp8_quant_mx_1x32_transposed(s["x"])
        n = sets[0]["x"].numel()
        line("linear_trio", "quant_mx_1x32_transposed X (blocks of 32 tokens)",
             lambda s: fp8.fp8_quant_mx_1x32_transposed(s["x"], q=s["mqxt"], e=s["mext"]), sets,
             dict(cfg, scales="E8M0 per 32 tokens"), nbytes=n * 5 + n // 32)
        mcfg = dict(cfg, scales="E8M0 per 1x32 block along each GEMM's contraction")
        gm = fp8.fp8_gemm_mx
        line("linear_trio", "gemm_mx Fprop 8192x2048x7168 BF16 (MX operands)",
             lambda s: gm(s["mqx"], s["mex"], s["mqw"], s["mew"], bf, out=s["yb"]), sets, mcfg, flops=fl,
             peak="FP8 (scaled MFMA)")
        line("linear_trio", "gemm_mx Dgrad 8192x7168x2048 BF16 (MX operands)",
             lambda s: gm(s["mqd"], s["med"], s["mqwt"], s["mewt"], bf, out=s["dxb"]), sets, mcfg, flops=fl,
             peak="FP8 (scaled MFMA)")
        line("linear_trio", "gemm_mx Wgrad 2048x7168x8192 FP32 (MX operands)",
             lambda s: gm(s["mqdt"], s["medt"], s["mqxt"], s["mext"], torch.float32, out=s["dwf"]), sets, mcfg,
             flops=fl, peak="FP8 (scaled MFMA)")
    elif args.workload == "moe_contig":
        G, N, K = 32, 4096, 7168
        sets = []
        for _ in range(2):   # ~2.9 GB each
            a, qa, sa, qb, sb, offs, counts, mt = contig_inputs(gen)
            sets.append(dict(a=a, qa=qa, sa=sa, qb=qb, sb=sb, offs=offs,
                             c=torch.empty((mt, N), dtype=torch.bfloat16, device="cuda"),
                             qy=torch.zeros((mt, N), dtype=torch.uint8, device="cuda"),
                             sy=torch.zeros((N // 128, mt), dtype=torch.float32, device="cuda")))
        cfg = {"experts": G, "routed_rows": int(counts.sum()), "padded_rows": mt, "N": N, "K": K}
        na = sets[0]["a"].numel()
        line("moe_contig", "quant_act_1x128 A rows",
             lambda s: fp8.fp8_quant_act_1x128(s["a"], q=s["qa"], s=s["sa"]), sets, cfg,
             nbytes=na * 5 + (na // 128) * 4)
        fl = 2.0 * int(counts.sum()) * N * K
        line("moe_contig", "grouped_gemm_contiguous gate+up",
             lambda s: fp8.fp8_grouped_gemm_contiguous(s["qa"], s["sa"], s["qb"], s["sb"], s["offs"], out=s["c"]),
             sets, dict(cfg, flops_counted="valid rows only"), flops=fl)
        line("moe_contig", "grouped_gemm_contiguous gate+up, FP8 out (fused 1x128 quantization)",
             lambda s: fp8.fp8_grouped_gemm_contiguous_fp8out(s["qa"], s["sa"], s["qb"], s["sb"], s["offs"],
                                                              q=s["qy"], s=s["sy"]),
             sets, dict(cfg, flops_counted="valid rows only",
                        output="FP8 codes + 1x128 scales along N: the down projection's A operand"), flops=fl)
        # the MX variant on the same rows (1x32 blocks, E8M0 scales applied in the FP8 MFMA)
        for s in sets:
            s["qam"], s["eam"] = fp8.fp8_quant_mx_1x32(s["a"])
            s["qbm"], s["ebm"] = mx_experts(gen, G, N, K)
        line("moe_contig", "grouped_gemm_contiguous_mx gate+up (MX operands)",
             lambda s: fp8.fp8_grouped_gemm_contiguous_mx(s["qam"], s["eam"], s["qbm"], s["ebm"], s["offs"],
                                                          out=s["c"]),
             sets, dict(cfg, flops_counted="valid rows only", scales="E8M0 per 1x32 block"), flops=fl,
             peak="FP8 (scaled MFMA)")
    elif args.workload == "moe_masked":
        G, MMAX = 32, 128
        for (N, K) in ((4096, 7168), (7168, 2048)):
            # the decode-tiled copies are rearranged once, when weights are
            # loaded; the rearrangement is not in the timed loop
            sets = masked_sets(gen, G, MMAX, N, K)
            valid = int(sets[0]["mm"].sum())
            nbytes = G * N * K + G * (N // 128) * (K // 128) * 4 + valid * K + valid * (K // 128) * 4 + valid * N * 2
            cfg = {"experts": G, "M_max": MMAX, "valid_rows": valid, "N": N, "K": K,
                   "bytes": "all expert weights + scales + valid A rows + valid C rows"}
            line("moe_masked", f"grouped_gemm_masked N={N} K={K}",
                 lambda s: fp8.fp8_grouped_gemm_masked(s["qa"], s["sa"], s["qb"], s["sb"], s["mmt"], out=s["c"]),
                 sets, cfg, nbytes=nbytes)
            line("moe_masked", f"grouped_gemm_masked_tiled N={N} K={K}",
                 lambda s: fp8.fp8_grouped_gemm_masked_tiled(s["qa"], s["sa"], s["qt"], s["sb"], s["mmt"],
                                                             out=s["c"]),
                 sets, dict(cfg, weights="decode-tiled layout (fp8_tile_weights_decode)"), nbytes=nbytes)
            # the same GEMM writing the down projection's (or next layer's) FP8 operand
            for s in sets:
                s["qy"] = torch.zeros((G, MMAX, N), dtype=torch.uint8, device="cuda")
                s["sy"] = torch.zeros((G, N // 128, MMAX), dtype=torch.float32, device="cuda")
            nbytes_q = nbytes - valid * N * 2 + valid * N + valid * (N // 128) * 4
            line("moe_masked", f"grouped_gemm_masked_tiled_fp8out N={N} K={K} (fused 1x128 output quantization)",
                 lambda s: fp8.fp8_grouped_gemm_masked_tiled_fp8out(s["qa"], s["sa"], s["qt"], s["sb"], s["mmt"],
                                                                    q=s["qy"], s=s["sy"]),
                 sets, dict(cfg, weights="decode-tiled layout", output="FP8 codes + 1x128 scales along N"),
                 nbytes=nbytes_q)
            # the MX variant: the same valid-row counts, fresh MX operands
            for s in sets:
                a = gpu_acts(gen, G * MMAX, K, 0.001, 100.0).reshape(G, MMAX, K)
                s["qam"] = torch.empty((G, MMAX, K), dtype=torch.uint8, device="cuda")
                s["eam"] = torch.empty((G, K // 32, MMAX), dtype=torch.uint8, device="cuda")
                for g in range(G):
                    fp8.fp8_quant_mx_1x32(a[g], q=s["qam"][g], e=s["eam"][g])
                del a
                s["qbm"], s["ebm"] = mx_experts(gen, G, N, K)
            nbytes_mx = G * N * K + G * (K // 32) * N + valid * K + valid * (K // 32) + valid * N * 2
            line("moe_masked", f"grouped_gemm_masked_mx N={N} K={K} (MX operands)",
                 lambda s: fp8.fp8_grouped_gemm_masked_mx(s["qam"], s["eam"], s["qbm"], s["ebm"], s["mmt"],
                                                          out=s["c"]),
                 sets, dict(cfg, scales="E8M0 per 1x32 block", bytes="all expert weights + E8M0 scales + valid A "
                            "rows + scales + valid C rows"), nbytes=nbytes_mx)
            for s in sets:
                s["qbmt"] = fp8.fp8_tile_weights_decode(s["qbm"])
            line("moe_masked", f"grouped_gemm_masked_tiled_mx N={N} K={K} (MX operands, decode-tiled weights)",
                 lambda s: fp8.fp8_grouped_gemm_masked_tiled_mx(s["qam"], s["eam"], s["qbmt"], s["ebm"], s["mmt"],
                                                                out=s["c"]),
                 sets, dict(cfg, scales="E8M0 per 1x32 block", weights="decode-tiled layout",
                            bytes="all expert weights + E8M0 scales + valid A rows + scales + valid C rows"),
                 nbytes=nbytes_mx)
            del sets


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; use --gpus 1"}))
        sys.exit(2)
    _SETTLE["seconds"] = args.settle_s
    if args.profile_kernel and (args.profile_kernel.startswith(("masked", "trio_")) or
                                args.profile_kernel in ("contig", "mx")):
        profile_other(args)
        return
    if args.workload != "dense_fprop":
        run_extra(args)
        return

    import torch
    import fp8_fine_grained_amd as fp8
    import workloads

    fp8.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    M, N, K = 4096, 7168, 2048
    sets = []
    host0 = None
    for i in range(args.sets):
        x, w = workloads.dense_fprop(seed_offset=i)
        if i == 0:
            host0 = (x, w)
        xs = torch.from_numpy(x).to(dev)
        ws = torch.from_numpy(w).to(dev)
        sets.append(dict(
            x=xs, w=ws,
            qa=torch.empty((M, K), dtype=torch.uint8, device=dev),
            sa=torch.empty((K // 128, M), dtype=torch.float32, device=dev),
            qb=torch.empty((N, K), dtype=torch.uint8, device=dev),
            sb=torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev),
            c=torch.empty((M, N), dtype=torch.bfloat16, device=dev)))
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()

    if args.profile_kernel:
        s = sets[0]
        fp8.fp8_quant_act_1x128(s["x"], q=s["qa"], s=s["sa"])
        fp8.fp8_quant_weight_128x128(s["w"], q=s["qb"], s=s["sb"])
        if args.profile_kernel == "copy":
            src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
            dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            if args.profile_kernel == "gemm":
                fp8.fp8_gemm_blockscaled(s["qa"], s["sa"], s["qb"], s["sb"], fp8.BSCALE_128x128, torch.bfloat16,
                                         out=s["c"])
            elif args.profile_kernel == "fp8mfma":
                fp8.fp8_gemm_blockscaled_fp8mfma(s["qa"], s["sa"], s["qb"], s["sb"], fp8.BSCALE_128x128,
                                                 torch.bfloat16, out=s["c"])
            elif args.profile_kernel == "quant_act":
                fp8.fp8_quant_act_1x128(s["x"], q=s["qa"], s=s["sa"])
            elif args.profile_kernel == "quant_weight":
                fp8.fp8_quant_weight_128x128(s["w"], q=s["qb"], s=s["sb"])
            elif args.profile_kernel == "quant_fprop":
                fp8.fp8_quant_fprop_operands(s["x"], s["w"], s["qa"], s["sa"], s["qb"], s["sb"])
            else:
                dst.copy_(src)
        torch.cuda.synchronize()
        print(f"profiled {args.profile_kernel} x{args.steps}", flush=True)
        return

    # One stream, launches back to back and nothing between them: an event or
    # a cross-stream wait costs this stack 5-10 us of idle GPU per use (seen in
    # the kernel trace).  The two quantizations share one launch, so their small
    # grids overlap instead of each ramping up and draining on its own.
    def step(i):
        s = sets[i % len(sets)]
        fp8.fp8_quant_fprop_operands(s["x"], s["w"], s["qa"], s["sa"], s["qb"], s["sb"])
        fp8.fp8_gemm_blockscaled(s["qa"], s["sa"], s["qb"], s["sb"], fp8.BSCALE_128x128, torch.bfloat16, out=s["c"])

    def step_three_launches(i):
        s = sets[i % len(sets)]
        fp8.fp8_quant_act_1x128(s["x"], q=s["qa"], s=s["sa"])
        fp8.fp8_quant_weight_128x128(s["w"], q=s["qb"], s=s["sb"])
        fp8.fp8_gemm_blockscaled(s["qa"], s["sa"], s["qb"], s["sb"], fp8.BSCALE_128x128, torch.bfloat16, out=s["c"])

    def timed_steps(fn):
        for i in range(args.warmup):
            fn(i)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(args.steps):
            fn(i)
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / args.steps

    # Untimed settling before the warmup steps: the GPU clock takes a few
    # hundred milliseconds of load to reach its steady level, and a timed loop
    # started sooner runs 10-20% slow (seen as a slow first repetition of
    # otherwise identical loops).
    t_end = time.perf_counter() + args.settle_s
    i = 0
    while time.perf_counter() < t_end:
        step(i)
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ms_step = timed_steps(step)
    ms_step3 = timed_steps(step_three_launches)

    def back_to_back(launch):
        # one kernel alone, `steps` launches between two events on the bench
        # stream, right after the timed steps
        for i in range(3):
            launch(sets[i % len(sets)])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            launch(sets[i % len(sets)])
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    def gemm_back_to_back():
        return back_to_back(lambda s: fp8.fp8_gemm_blockscaled(s["qa"], s["sa"], s["qb"], s["sb"], fp8.BSCALE_128x128,
                                                               torch.bfloat16, out=s["c"]))

    t_fprop = back_to_back(lambda s: fp8.fp8_quant_fprop_operands(s["x"], s["w"], s["qa"], s["sa"], s["qb"], s["sb"]))
    t_act = back_to_back(lambda s: fp8.fp8_quant_act_1x128(s["x"], q=s["qa"], s=s["sa"]))
    t_w = back_to_back(lambda s: fp8.fp8_quant_weight_128x128(s["w"], q=s["qb"], s=s["sb"]))
    t_gemm = gemm_back_to_back()
    # the same GEMM with the next layer's 1x128 quantization fused into its epilogue
    qy = torch.empty((M, N), dtype=torch.uint8, device=dev)
    sy = torch.empty((N // 128, M), dtype=torch.float32, device=dev)
    t_fp8out = back_to_back(lambda s: fp8.fp8_gemm_blockscaled_fp8out(s["qa"], s["sa"], s["qb"], s["sb"], q=qy, s=sy))
    # the FP8-MFMA engine (its own entry point, looser error bound), GEMM alone
    t_fp8mfma = back_to_back(lambda s: fp8.fp8_gemm_blockscaled_fp8mfma(s["qa"], s["sa"], s["qb"], s["sb"],
                                                                        fp8.BSCALE_128x128, torch.bfloat16,
                                                                        out=s["c"]))
    # the MX variant on the same shape: the step's fp32 inputs MX-quantized
    # (1x32 blocks, E8M0 scales applied inside the scaled FP8 MFMA), GEMM alone
    for s in sets:
        s["mqa"], s["mea"] = fp8.fp8_quant_mx_1x32(s["x"])
        s["mqb"], s["meb"] = fp8.fp8_quant_mx_1x32(s["w"])
    t_mx = back_to_back(lambda s: fp8.fp8_gemm_mx(s["mqa"], s["mea"], s["mqb"], s["meb"], torch.bfloat16, out=s["c"]))
    # the masked-layout decode GEMMs (32 experts, 128-row buffers, U{1..64}
    # valid rows): HBM-bound, so their figure is GB/s against 8 TB/s
    masked = masked_decode_rates(args)

    # Measured references on this machine, the same way: the platform's own BF16
    # GEMM (torch.matmul, no block scales) on the same M x N x K, and a device
    # copy (read + write bytes).  They put the exact engine's rate next to what
    # the vendor library reaches with the same matrix cores, and the quantizers'
    # bytes next to an achievable stream.
    ab = torch.randn((M, K), device=dev, dtype=torch.bfloat16)
    bb = torch.randn((K, N), device=dev, dtype=torch.bfloat16)   # contiguous [K][N]: a plain 2-D product
    cb = torch.empty((M, N), device=dev, dtype=torch.bfloat16)
    t_bf16_lib = back_to_back(lambda s: torch.matmul(ab, bb, out=cb))
    # the platform's FP8 GEMM with one scale per row of A and per column of B
    # (torch._scaled_mm, row-wise): no 1x128 / 128x128 blocks, so not this
    # method, but the FP8 matrix cores as the vendor library drives them
    t_fp8_lib = None
    try:
        af = torch.randn((M, K), device=dev).to(torch.float8_e4m3fn)
        wf = torch.randn((N, K), device=dev).to(torch.float8_e4m3fn)
        ra, rb = torch.ones((M, 1), device=dev), torch.ones((1, N), device=dev)
        t_fp8_lib = back_to_back(lambda s: torch._scaled_mm(af, wf.t(), scale_a=ra, scale_b=rb,
                                                             out_dtype=torch.bfloat16))
        del af, wf, ra, rb
    except (RuntimeError, AttributeError, TypeError):
        t_fp8_lib = None
    src = torch.empty(1 << 28, device=dev, dtype=torch.float32)
    dst = torch.empty_like(src)
    t_copy = back_to_back(lambda s: dst.copy_(src))
    copy_gbs = 2.0 * src.numel() * 4 / (t_copy * 1e-3) / 1e9
    del ab, bb, cb, src, dst

    flops = 2.0 * M * N * K
    value = flops / (ms_step * 1e-3) / 1e12
    gemm_tflops = flops / (t_gemm * 1e-3) / 1e12
    act_bytes = M * K * 5 + (K // 128) * M * 4
    w_bytes = N * K * 5 + (N // 128) * (K // 128) * 4
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic (seeded: activations N(0,1) with 0.1% outlier channels x100, weights N(0,0.02))",
        "config": {"workload": "dense_fprop: M=4096 N=7168 K=2048, 1x128 activation / 128x128 weight scales, "
                               "BF16 out; step = quant_fprop_operands (1x128 activation + 128x128 weight "
                               "quantization, one launch) + gemm_blockscaled",
                   "M": M, "N": N, "K": K, "rotating_input_sets": args.sets},
        "pct_of_fp8_peak_step": round(100 * value / PEAK_FP8_TFLOPS, 2),
        "step_three_launches_ms": round(ms_step3, 5),
        "kernels_us": {"quant_fprop_operands": round(t_fprop * 1e3, 2),
                       "quant_act_1x128": round(t_act * 1e3, 2), "quant_weight_128x128": round(t_w * 1e3, 2),
                       "gemm_blockscaled": round(t_gemm * 1e3, 2)},
        "quant_gbs": {"fprop_operands": round((act_bytes + w_bytes) / (t_fprop * 1e-3) / 1e9, 1),
                      "act": round(act_bytes / (t_act * 1e-3) / 1e9, 1),
                      "weight": round(w_bytes / (t_w * 1e-3) / 1e9, 1)},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
                     "traffic": stored_traffic(),
                     "kernel": "gemm_wide_o0_dense (dense, 128x128 B scales, BF16 out, 448 tiles of 256x256): "
                               "FP8 operands widened exactly to BF16 in registers and multiplied on the BF16 "
                               "matrix cores (gfx950's FP8 MFMA keeps ~14 bits per group of 8 products, outside "
                               "the 2^-14 contract), so this engine's own ceiling is the BF16 peak, half the FP8 "
                               "one: frac_of_bf16_peak",
                     "frac_of_bf16_peak": round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
                     "pct_of_fp8_peak": round(100 * gemm_tflops / PEAK_FP8_TFLOPS, 2),
                     "kernel_us": round(t_gemm * 1e3, 2),
                     "duration_source": "mean of `steps` back-to-back launches on the bench stream between two "
                                        "HIP events, right after the timed steps",
                     "kernel_source": source_hash()},
        "fp8_out_fused": {"gemm_us": round(t_fp8out * 1e3, 2),
                          "tflops": round(flops / (t_fp8out * 1e-3) / 1e12, 2),
                          "note": "same GEMM writing FP8 codes + 1x128 scales along N (the next layer's A "
                                  "operand) instead of BF16; not the timed step"},
        "measured_reference": {
            "torch_bf16_matmul_us": round(t_bf16_lib * 1e3, 2),
            "torch_bf16_matmul_tflops": round(flops / (t_bf16_lib * 1e-3) / 1e12, 2),
            "gemm_frac_of_torch_bf16_matmul": round(t_bf16_lib / t_gemm, 4),
            "torch_fp8_scaled_mm_rowwise_tflops": (round(flops / (t_fp8_lib * 1e-3) / 1e12, 2)
                                                   if t_fp8_lib else None),
            "device_copy_gbs": round(copy_gbs, 1),
            "quant_fprop_frac_of_copy": round((act_bytes + w_bytes) / (t_fprop * 1e-3) / 1e9 / copy_gbs, 4),
            "note": "same box, same run: torch.matmul on BF16 operands of the same shape (no block scales), "
                    "torch._scaled_mm on FP8 operands with row/column scales (no 1x128 / 128x128 blocks), and a "
                    "1 GiB device-to-device copy (read + write bytes), each as back-to-back launches between two "
                    "HIP events"},
        "fp8mfma_engine": {"gemm_us": round(t_fp8mfma * 1e3, 2),
                           "tflops": round(flops / (t_fp8mfma * 1e-3) / 1e12, 2),
                           "pct_of_fp8_peak": round(100 * flops / (t_fp8mfma * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 2),
                           "note": "fp8_gemm_blockscaled_fp8mfma: FP8 matrix cores, error bound 2^-9 * sum|ab| "
                                   "(gfx950 FP8 MFMA accumulates 8-product groups with ~14 bits); not the timed "
                                   "step"},
        "mx_variant": {"gemm_us": round(t_mx * 1e3, 2),
                       "tflops": round(flops / (t_mx * 1e-3) / 1e12, 2),
                       "pct_of_fp8_peak": round(100 * flops / (t_mx * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 2),
                       "note": "fp8_gemm_mx on the same inputs MX-quantized (1x32 blocks, E8M0 scales applied inside "
                               "the scaled FP8 MFMA): another numeric contract (power-of-two scales, error bound "
                               "2^-9 * sum|ab|); not the timed step"},
        "masked_decode": masked,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(host0[0], host0[1], args.cpu_rows)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
