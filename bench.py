"""Throughput of the H-BitLinear forward on one MI355X.

Default workload: the seven linear layers of one 7B-shaped BitNet v2 block
at M = 65536 tokens (64 sequences x 1024): Q, K, V (4096 -> 4096) and up,
gate (4096 -> 16384) as plain BitLinear, Wo (4096 -> 4096) and Wdown
(16384 -> 4096) as H-BitLinear with the rotation.  Activations bf16
Student-t(3) with 1 % of channels x20, weights N(0, 0.02^2) ternarised.  One
step = the block's 4 quantisations (Q/K/V and up/gate share theirs) and 7
matmuls, inputs resident in HBM.  The headline is INT4 activations on the
FP6 x FP4 matrix cores; INT8 activations are timed beside it.

Prints one JSON line.  ``roofline`` is for the dominant kernel (the
matrix-core matmul): algorithmic ops per launch over its average duration,
from HIP events around every launch of the timed steps on the stream the
library launches on.  ``cpu_baseline`` is the CPU oracle timed on a bounded
sample of rows of the same workload, at all cores and at one thread.

Other workloads (--workload): tiny, wo_7b, wdown_7b (single layers), decode,
msweep (layer time over token counts 1-4096 for BitLinear INT8 against
H-BitLinear INT8/INT4, and the break-even batch where the rotated INT4 layer
catches up), kvcache (the post-RoPE K/V quantiser on one 7B layer's cache
states), and copy (a plain device copy of known size, to calibrate the
HBM traffic counters).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "H-BitLinear tokens/sec & effective TOPS at 7B shapes; % HBM BW / % i8 MFMA peak"
HBM_PEAK_GBS = 8000.0
I8_PEAK_TOPS = 5000.0
MX_PEAK_TOPS = 10100.0  # dense FP6/FP4 matrix cores, vendor figure
MEASURED = os.path.join(ROOT, "profiles", "measured.json")


def measured():
    """Measured peaks and per-launch HBM counters of this repository's
    profiles (profiles/measured.json), or {} if absent."""
    try:
        with open(MEASURED) as f:
            return json.load(f)
    except (OSError, ValueError):
        return {}


def _sha256(rel):
    import hashlib
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def counter_traffic(workload, which):
    """HBM bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE) of the
    matmul ("gemm") or rotation/quantisation ("quant") kernel of a layer
    workload, from the committed counter runs, if the kernel's source is
    still the one they were taken on; else None."""
    c = measured().get("counters", {}).get(workload)
    if not c:
        return None
    src = {"gemm": "bit_quantization_amd/csrc/k_gemm.hip", "quant": "bit_quantization_amd/csrc/k_quant.hip",
           "gemm_mx": "bit_quantization_amd/csrc/k_gemm_mx.hip", "quant_mx": "bit_quantization_amd/csrc/k_quant.hip"}[which]
    if _sha256(src) != c.get(f"{which}_source_sha256"):
        return None
    return c[f"{which}_hbm_read_bytes"] + c[f"{which}_hbm_write_bytes"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 300 warm-up passes let the clocks settle (the first few hundred launches
    # of a process run 3-5 % slower)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="block_7b",
                    choices=["tiny", "wo_7b", "wdown_7b", "decode", "block_7b", "msweep", "kvcache", "copy"])
    ap.add_argument("--copy-mib", type=int, default=1024,
                    help="copy: bytes moved per launch (calibrates the HBM traffic counters)")
    ap.add_argument("--decode-m", type=int, default=1)
    ap.add_argument("--decode-k", type=int, default=16384)
    ap.add_argument("--decode-mats", type=int, default=0,
                    help="distinct weight matrices cycled (0: enough for >= 512 MiB)")
    ap.add_argument("--bits", type=int, default=0, help="block_7b: 8 or 4 (0: both); kvcache: 3 or 4 (0: 4)")
    ap.add_argument("--path", default="auto", choices=["auto", "int8", "mx"],
                    help="INT4 layers: int8 matrix cores, or FP6 x FP4 (mx); auto takes mx where it applies "
                         "(INT4, K a power of two >= 1024, M K >= 2^19; smaller M K stream the weights)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=20)
    return ap.parse_args()


def dev_x(x_np):
    import torch
    if x_np.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x_np).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x_np)).cuda()


def time_stream(fn, reps):
    """Average GPU duration (s) of ``fn`` (one or more library launches).

    The ``reps`` calls are captured once into a HIP graph and the graph is
    replayed, so that host launch overhead does not leak into the figure;
    HIP events on the current stream (where the library enqueues) bracket the
    replays.  Falls back to back-to-back eager launches if capture fails."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        g.replay()
        torch.cuda.synchronize()
        n = 5
        a.record()
        for _ in range(n):
            g.replay()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) / 1e3 / (n * reps)
    except Exception:  # capture unsupported: eager launches
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) / 1e3 / reps


def graph_of(fn):
    """One call of ``fn`` captured as a HIP graph (None if capture fails)."""
    import torch
    fn()
    torch.cuda.synchronize()
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        g.replay()
        torch.cuda.synchronize()
        return g
    except Exception:
        torch.cuda.synchronize()
        return None


def cpu_baseline(x_np, w_np, bits, had, min_seconds=10.0, chunk=64):
    """The CPU oracle (whole layer: fp64 rotation, quantiser, triple-loop
    integer matmul) over consecutive chunks of the workload's token rows,
    until at least ``min_seconds`` of work; tokens/s over the rows done."""
    import oracle
    packed, alpha, _ = oracle.ternarize(w_np)
    M = x_np.shape[0]
    chunk = min(chunk, M)
    rows = 0
    t0 = time.perf_counter()
    while True:
        a = rows % M
        b = min(a + chunk, M)
        oracle.forward(np.ascontiguousarray(x_np[a:b]), packed, alpha, bits, hadamard=had)
        rows += b - a
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": rows / dt, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{rows} token rows (chunks of {chunk}, cycling over the workload's {M}), whole layer "
                      f"(fp64 rotation, quantiser, triple-loop integer matmul), {dt:.1f} s"}


def cold_inputs(x):
    """Distinct copies of the layer input, together more than twice the 256
    MiB Infinity Cache, so that a quantiser reading them in turn streams its
    input from HBM; just ``x`` when it is under 4 MiB (launch-bound)."""
    nb = x.numel() * x.element_size()
    if nb < (4 << 20):
        return [x]
    n = min(64, -(-(512 << 20) // nb))
    return [x] + [x.clone() for _ in range(n - 1)]


def time_cycled(fn_of_x, xs, reps):
    """time_stream over calls that take the inputs xs in turn."""
    i = [0]

    def call():
        fn_of_x(xs[i[0] % len(xs)])
        i[0] += 1
    return time_stream(call, max(reps, 2 * len(xs)))


def layer_roofline(hbl, x, packed, alpha, bits, had, M, N, K, reps):
    """Per-kernel timing of one layer: rotation+quantisation, then matmul.
    The quantiser is timed on the one input (cache-resident when it fits)
    and over inputs cycled beyond the Infinity Cache (from HBM)."""
    q, s, rs = hbl.hadamard_quant(x, bits, hadamard=had)
    out = hbl.ternary_gemm(q, bits, s, rs, packed, alpha, K)
    t_q = time_stream(lambda: hbl.hadamard_quant(x, bits, hadamard=had), reps)
    xs = cold_inputs(x)
    t_q_hbm = time_cycled(lambda xx: hbl.hadamard_quant(xx, bits, hadamard=had), xs, reps)
    del xs
    t_g = time_stream(lambda: hbl.ternary_gemm(q, bits, s, rs, packed, alpha, K, out=out), reps)
    x_bytes = M * K * x.element_size()
    code_bytes = M * K // (2 if bits == 4 else 1)
    q_bytes = x_bytes + code_bytes + 8 * M
    return t_q, t_q_hbm, t_g, q_bytes, code_bytes


def layer_roofline_mx(hbl, x, wq, alpha, had, M, N, K, reps):
    """Per-kernel timing of one layer on the FP6 x FP4 path (the quantiser
    also over inputs cycled beyond the Infinity Cache, as layer_roofline)."""
    c, s = hbl.hadamard_quant_mx(x, hadamard=had)
    out = hbl.ternary_gemm_mx(c, s, wq, alpha, K, N=N)
    t_q = time_stream(lambda: hbl.hadamard_quant_mx(x, hadamard=had), reps)
    xs = cold_inputs(x)
    t_q_hbm = time_cycled(lambda xx: hbl.hadamard_quant_mx(xx, hadamard=had), xs, reps)
    del xs
    t_g = time_stream(lambda: hbl.ternary_gemm_mx(c, s, wq, alpha, K, out=out), reps)
    code_bytes = M * K * 3 // 4
    q_bytes = M * K * x.element_size() + code_bytes + 4 * M
    return t_q, t_q_hbm, t_g, q_bytes, code_bytes


def use_mx(args, bits, M, K):
    if args.path == "int8" or bits != 4:
        return False
    ok = K >= 1024 and (K & (K - 1)) == 0 and K % 512 == 0
    # the FP6 x FP4 layer (K split over the partial sums below 256 tiles)
    # beats weight streaming from M K >= 2^19 (M >= 128 at K = 4096, M >= 32
    # at K = 16384)
    return ok and (args.path == "mx" or M * K >= 1 << 19)


def time_passes(args, torch, layer):
    """Seconds per whole-layer pass: a HIP graph holds `per` passes back to
    back, as a serving loop replays them (per divides the step count, so
    exactly `steps` passes are timed)."""
    per = max(d for d in range(1, 11) if args.steps % d == 0)

    def passes():
        for _ in range(per):
            layer()

    g = graph_of(passes)
    run = g.replay if g is not None else passes
    for _ in range(-(-args.warmup // per)):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps // per):
        run()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / args.steps, (f"hip graph of {per} passes" if g is not None else "eager")


def run_layer(args, hbl, torch, x_np, w_np, bits, had, label):
    M, K = x_np.shape
    N = w_np.shape[0]
    x = dev_x(x_np)
    packed, alpha = hbl.ternarize_weights(torch.from_numpy(w_np).cuda())
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mx = use_mx(args, bits, M, K)
    ws = hbl.forward_workspace(M, N, K, bits, "cuda")

    def layer_int8():
        hbl.forward(x, packed, alpha, bits, hadamard=had, out=out, workspace=ws)

    # A step is one whole-layer pass (both kernels) of the product path.
    if mx:
        wq = hbl.prepare_weights_mx(packed, K)
        ws_mx = hbl.forward_mx_workspace(M, N, K, "cuda")

        def layer():
            hbl.forward_mx(x, wq, alpha, hadamard=had, out=out, workspace=ws_mx)
    else:
        layer = layer_int8
    dt, launch = time_passes(args, torch, layer)

    if mx:
        t_q, t_q_hbm, t_g, q_bytes, code_bytes = layer_roofline_mx(hbl, x, wq, alpha, had, M, N, K, args.kernel_reps)
        # the same layer on the int8 matrix cores, timed the same way, for comparison
        dt_int8, _ = time_passes(args, torch, layer_int8)
    else:
        t_q, t_q_hbm, t_g, q_bytes, code_bytes = layer_roofline(hbl, x, packed, alpha, bits, had, M, N, K,
                                                                 args.kernel_reps)
    ops = 2.0 * M * N * K
    gemm_tops = ops / t_g / 1e12
    w_bytes = N * K // 4
    peaks = measured().get("peaks", {})
    best = peaks.get("i8_mfma_tops_best")
    int4_like = peaks.get("i8_mfma_tops_int4_like") if bits == 4 else peaks.get("i8_mfma_tops_int8_like")
    hbm_meas = peaks.get("hbm_read_gbs")
    wl = args.workload
    if mx:
        mx_best = peaks.get("fp6fp4_mfma_tops_best")
        mx_like = peaks.get("fp6fp4_mfma_tops_int4_like")
        roofline = {"bound": "mfma", "kernel": "k_gemm_mx (FP6 x FP4 ternary matmul)", "achieved": gemm_tops,
                    "peak": MX_PEAK_TOPS, "unit": "TOP/s", "frac": gemm_tops / MX_PEAK_TOPS,
                    "traffic": counter_traffic(wl, "gemm_mx"), "avg_kernel_us": t_g * 1e6,
                    "algorithmic_ops_per_launch": ops,
                    "measured_peak": {"fp6fp4_mfma_tops": mx_best, "frac": gemm_tops / mx_best if mx_best else None,
                                      "fp6fp4_mfma_tops_same_operand_bits": mx_like,
                                      "frac_same_operand_bits": gemm_tops / mx_like if mx_like else None,
                                      "i8_mfma_tops": best, "frac_of_i8": gemm_tops / best if best else None,
                                      "source": "profiles/peaks.md"}}
    else:
        roofline = {"bound": "mfma", "kernel": "k_gemm_pt (ternary matmul)", "achieved": gemm_tops,
                    "peak": I8_PEAK_TOPS, "unit": "TOP/s", "frac": gemm_tops / I8_PEAK_TOPS,
                    "traffic": counter_traffic(wl, "gemm"), "avg_kernel_us": t_g * 1e6,
                    "algorithmic_ops_per_launch": ops,
                    "measured_peak": {"i8_mfma_tops": best, "frac": gemm_tops / best if best else None,
                                      "i8_mfma_tops_same_operand_bits": int4_like,
                                      "frac_same_operand_bits": gemm_tops / int4_like if int4_like else None,
                                      "source": "profiles/peaks.md"}}
    res = {
        "metric": METRIC,
        "value": M / dt,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dt * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp6xfp4" if mx else "i8",
        "data": "synthetic",
        "config": {"workload": label, "M": M, "K": K, "N": N, "bits": bits, "hadamard": had,
                   "x_dtype": "bf16" if x_np.dtype == np.uint16 else "f32",
                   "path": "FP6 x FP4 matrix cores (exact)" if mx else "int8 matrix cores"},
        "effective_tops": ops / dt / 1e12,
        "roofline": roofline,
        "fused": {"effective_tops": ops / dt / 1e12,
                  "frac_of_measured_i8_peak": ops / dt / 1e12 / best if best else None,
                  "frac_of_published_i8_peak": ops / dt / 1e12 / I8_PEAK_TOPS},
        # the quantiser against HBM: inputs cycled beyond the Infinity Cache;
        # the one input replayed (cache-resident when it fits) beside it
        "quant_kernel": {"bound": "hbm", "avg_kernel_us": t_q_hbm * 1e6,
                         "algorithmic_bytes_per_launch": q_bytes,
                         "achieved_gbs": q_bytes / t_q_hbm / 1e9,
                         "frac": q_bytes / t_q_hbm / 1e9 / HBM_PEAK_GBS,
                         "frac_of_measured_read_peak": q_bytes / t_q_hbm / 1e9 / hbm_meas if hbm_meas else None,
                         "input": "distinct copies of the input read in turn, more than twice the 256 MiB "
                                  "Infinity Cache in all (one input below 4 MiB)",
                         "one_input_replayed": {"avg_kernel_us": t_q * 1e6, "achieved_gbs": q_bytes / t_q / 1e9},
                         "traffic": counter_traffic(wl, "quant_mx" if mx else "quant")},
        "gemm_bytes_min": code_bytes + w_bytes + 2 * M * N,
        "launch": launch,
    }
    if mx:
        res["int8_path"] = {"ms_per_step": dt_int8 * 1e3, "tokens_per_s": M / dt_int8,
                            "effective_tops": ops / dt_int8 / 1e12}
    return res


def run_decode(args, hbl, torch):
    import workloads
    M, K, N = args.decode_m, args.decode_k, 4096
    w_bytes = N * K // 4
    n_mats = args.decode_mats or max(10, -(-(512 << 20) // w_bytes))
    x = dev_x(workloads.decode_inputs(K, M))
    # distinct matrices: the 10 seeded ones, repeated at distinct addresses
    base = [hbl.ternarize_weights(torch.from_numpy(workloads.decode_weights(K, N, i)).cuda()) for i in range(10)]
    mats = [(base[i % 10][0].clone(), base[i % 10][1].clone()) for i in range(n_mats)]
    del base
    bits = 8
    q, s, rs = hbl.hadamard_quant(x, bits)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = hbl.forward_workspace(M, N, K, bits, "cuda")

    # one graph holds one decode call per matrix (cycling the matrices);
    # a step is one call
    def all_mats():
        for p, a in mats:
            hbl.forward(x, p, a, bits, out=out, workspace=ws)

    g = graph_of(all_mats)
    run = g.replay if g is not None else all_mats
    reps = max(1, -(-args.steps // n_mats))
    for _ in range(max(1, args.warmup // n_mats)):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        run()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / (reps * n_mats)
    # matmul kernel alone, cycling the matrices
    ctr = [0]

    def gem():
        p, a = mats[ctr[0] % n_mats]
        ctr[0] += 1
        hbl.ternary_gemm(q, bits, s, rs, p, a, K, out=out)

    t_g = time_stream(gem, n_mats)
    t_q = time_stream(lambda: hbl.hadamard_quant(x, bits), args.kernel_reps)
    g_bytes = w_bytes + M * K + 8 * M + 2 * M * N
    if M <= (1 if K > 4096 else 2):
        # one or two tokens: the layer is one launch (rotation, quantisation
        # and weight streaming in k_decode_token), so the step is that kernel;
        # algorithmic bytes: weights, the bf16 token rows, the bf16 outputs
        kern, t_k, k_bytes = "k_decode_token (the layer in one launch)", dt, w_bytes + 2 * M * K + 2 * M * N
    else:
        kern, t_k, k_bytes = "k_gemv_dot / k_gemv (weight streaming)", t_g, g_bytes
    bw = k_bytes / t_k / 1e9
    return {
        "metric": METRIC, "value": M / dt, "unit": "tokens/s", "n_gpus": 1, "steps": reps * n_mats,
        "warmup": args.warmup, "ms_per_step": dt * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "i8", "data": "synthetic",
        "config": {"workload": f"decode M={M} K={K} N={N} INT8, {n_mats} matrices cycled", "M": M, "K": K,
                   "N": N, "bits": 8, "hadamard": True, "matrices": n_mats},
        "launch": "hip graph" if g is not None else "eager",
        "roofline": {"bound": "hbm", "kernel": kern, "achieved": bw,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": bw / HBM_PEAK_GBS, "traffic": None,
                     "avg_kernel_us": t_k * 1e6, "algorithmic_bytes_per_launch": k_bytes,
                     "measured_peak": {"hbm_read_gbs": measured().get("peaks", {}).get("hbm_read_gbs"),
                                       "frac": (bw / measured()["peaks"]["hbm_read_gbs"]
                                                if measured().get("peaks", {}).get("hbm_read_gbs") else None),
                                       "source": "profiles/peaks.md"}},
        "quant_kernel": {"avg_kernel_us": t_q * 1e6, "note": "hbl_hadamard_quant alone"},
        "gemv_kernel": {"avg_kernel_us": t_g * 1e6, "achieved_gbs": g_bytes / t_g / 1e9,
                        "note": "hbl_ternary_gemm alone on the same codes"},
    }


def run_msweep(args, hbl, torch):
    """Layer time against the token count M = 1 ... 4096 at the two 7B input
    widths (K = 4096 and 16384, N = 4096), for four layer kinds:
      bitlinear_a8   plain BitLinear, INT8 codes, no rotation (the b1.58 layer)
      hbitlinear_a8  H-BitLinear, INT8 codes
      hbitlinear_a4  H-BitLinear, INT4 codes, on the path the library takes
                     for that M (weight streaming up to 128 tokens, then the
                     FP6 x FP4 matmul)
      norm_hbitlinear_a4  H-BitLinear INT4 with the RMSNorm layer in front
                     (int8 matrix cores)
    Each time is one whole layer call (quantisation kernel + matmul kernel),
    averaged over HIP-graph replays that cycle enough distinct weight
    matrices (>= 512 MiB) that the weights stream from HBM.  The break-even
    batch is the smallest M from which on the rotated INT4 layer is no slower
    than the plain INT8 one."""
    import workloads
    Ms = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096]
    kinds = [("bitlinear_a8", 8, False, False), ("hbitlinear_a8", 8, True, False),
             ("hbitlinear_a4", 4, True, False), ("norm_hbitlinear_a4", 4, True, True)]
    table, breakeven = [], {}
    for K in (4096, 16384):
        N = 4096
        n_mats = max(10, -(-(512 << 20) // (N * K // 4)))
        base = [hbl.ternarize_weights(torch.from_numpy(workloads.decode_weights(K, N, i)).cuda()) for i in range(10)]
        mats = [(base[i % 10][0].clone(), base[i % 10][1].clone()) for i in range(n_mats)]
        del base
        mats_mx = [hbl.prepare_weights_mx(p, K) for p, _ in mats]
        gain = torch.from_numpy(np.random.default_rng(K).uniform(0.5, 1.5, K).astype(np.float32)).cuda()
        rows = []
        for M in Ms:
            x = dev_x(workloads.student_t_rows(workloads.SEEDS["decode"], 7000 + M, M, K, None, 1.0))
            out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            row = {"K": K, "N": N, "M": M}
            for name, bits, had, norm in kinds:
                mx = not norm and use_mx(args, bits, M, K)
                ws = hbl.forward_mx_workspace(M, N, K, "cuda") if mx else hbl.forward_workspace(M, N, K, bits, "cuda")

                def all_mats():
                    for (p, a), q in zip(mats, mats_mx):
                        if mx:
                            hbl.forward_mx(x, q, a, hadamard=had, out=out, workspace=ws)
                        elif norm:
                            hbl.norm_forward(x, p, a, bits, gain=gain, hadamard=had, out=out, workspace=ws)
                        else:
                            hbl.forward(x, p, a, bits, hadamard=had, out=out, workspace=ws)

                t = time_stream(all_mats, 2) / n_mats
                row[f"{name}_us"] = t * 1e6
                if name == "hbitlinear_a4":
                    row["a4_path"] = "FP6 x FP4" if mx else ("weight streaming" if M <= 128 else "int8 matrix cores")
            row["rotation_overhead_a8"] = row["hbitlinear_a8_us"] / row["bitlinear_a8_us"] - 1.0
            row["a4_vs_bitlinear_a8"] = row["hbitlinear_a4_us"] / row["bitlinear_a8_us"]
            rows.append(row)
            print(json.dumps({"progress": row}), file=sys.stderr, flush=True)
            del x, out
        breakeven[K] = None
        for i in range(len(rows)):
            if all(r["hbitlinear_a4_us"] <= r["bitlinear_a8_us"] for r in rows[i:]):
                breakeven[K] = rows[i]["M"]
                break
        table += rows
        del mats, mats_mx
        torch.cuda.empty_cache()
    return {
        "metric": "H-BitLinear vs BitLinear layer time over the token count (break-even batch)",
        "value": breakeven[16384], "unit": "tokens (smallest M from which H-BitLinear INT4 <= BitLinear INT8, K=16384)",
        "n_gpus": 1, "higher_is_better": False, "dtype": "i8", "data": "synthetic",
        "config": {"workload": "msweep: M = 1..4096, K in {4096, 16384}, N = 4096, weights cycled from HBM"},
        "breakeven_m": {str(k): v for k, v in breakeven.items()}, "sweep": table,
    }


def run_kvcache(args, hbl, torch):
    """The post-RoPE QKV / KV-cache quantiser on one 7B layer's K and V
    states: 64 sequences x 1024 positions x 32 heads x 128 (bf16), b-bit
    codes with the [BOS] position kept at 8 bits.  A step quantises K and V."""
    import workloads
    B, S, H, D = 64, 1024, 32, 128
    bits = args.bits if args.bits in (3, 4) else 4
    rows = B * S * H
    kv = []
    for i in range(2):
        x_np = workloads.student_t_rows(workloads.SEEDS["decode"], 9000 + i, rows, D, None, 1.0)
        kv.append(dev_x(x_np).view(B, S, H, D))
    outs = [(torch.empty((B, S, H, D * bits // 8), dtype=torch.uint8, device="cuda"),
             torch.empty((B, S, H), dtype=torch.float32, device="cuda"),
             torch.empty((B, H, D), dtype=torch.uint8, device="cuda"),
             torch.empty((B, H), dtype=torch.float32, device="cuda")) for _ in range(2)]

    def quant(i):
        c, s_, bc, bs = outs[i]
        x = kv[i]
        hbl._check(hbl.lib().hbl_kv_quant(x.data_ptr(), hbl.DTYPE_BF16, B, S, H, D, bits, 1, c.data_ptr(),
                                          s_.data_ptr(), bc.data_ptr(), bs.data_ptr(), hbl._stream()),
                   "hbl_kv_quant")

    dt, launch = time_passes(args, torch, lambda: (quant(0), quant(1)))
    t_k = time_stream(lambda: quant(0), args.kernel_reps)
    elems = B * S * H * D
    k_bytes = elems * 2 + elems * bits // 8 + 4 * B * S * H + B * H * (D + 4)
    gbs = k_bytes / t_k / 1e9
    hbm = measured().get("peaks", {}).get("hbm_read_gbs")
    return {"metric": "post-RoPE K/V cache quantiser throughput", "value": B * S / dt, "unit": "tokens/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": dt * 1e3,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": f"kvcache: K and V of one 7B layer, {B} x {S} positions x {H} heads x {D}, "
                                   f"{bits}-bit codes, BOS at 8 bits", "B": B, "S": S, "H": H, "D": D, "bits": bits},
            "roofline": {"bound": "hbm", "kernel": "k_kv_quant", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": None, "avg_kernel_us": t_k * 1e6,
                         "algorithmic_bytes_per_launch": k_bytes,
                         "measured_peak": {"hbm_read_gbs": hbm, "frac": gbs / hbm if hbm else None}},
            "launch": launch}


BLOCK_GROUPS = [("attn_in", False, ["q", "k", "v"]), ("o_in", True, ["o"]),
                ("ffn_in", False, ["up", "gate"]), ("down_in", True, ["down"])]


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def block_cpu_baseline(bits, rows_all_cores=256, rows_one_core=16):
    """The CPU oracle on the 7B block, as it stands: per activation input the
    quantiser (fp64 rotation for Wo and Wdown), then for each linear its
    triple-loop integer matmul and the rescale, on the first R token rows of
    each input; tokens/s = R / (time of the whole block on those rows).  The
    oracle's work is linear in the token count, so the rate applies to M
    (extrapolated).  Timed at all cores and at one thread."""
    import oracle
    import workloads
    ws = {}
    for name, K, N, had in workloads.BLOCK_7B_LAYERS:
        packed, alpha, _ = oracle.ternarize(workloads.block_weights(name))
        ws[name] = (packed, alpha, K)
    R = max(rows_all_cores, rows_one_core)
    xs = {name: workloads.block_input(name, M=R) for name, _ in workloads.BLOCK_7B_INPUTS}

    def run(rows):
        t = 0.0
        for inp, had, layers in BLOCK_GROUPS:
            x = np.ascontiguousarray(xs[inp][:rows])
            t0 = time.perf_counter()
            codes, scales, _ = oracle.quantize(x, bits, hadamard=had)
            for layer in layers:
                packed, alpha, K = ws[layer]
                acc = oracle.gemm_i32(codes, bits, packed, K)
                oracle.dequant_output(acc, scales, alpha)
            t += time.perf_counter() - t0
        return rows / t, t

    all_cores = oracle.num_threads()
    v_all, t_all = run(rows_all_cores)
    oracle.set_num_threads(1)
    try:
        v_one, t_one = run(rows_one_core)
    finally:
        oracle.set_num_threads(all_cores)
    what = ("the 7 linears of the block (4 quantisations with the fp64 rotation on Wo/Wdown inputs, 7 triple-loop "
            f"integer matmuls and rescales), INT{bits}")
    return {"value": v_all, "unit": "tokens/s", "cores": all_cores, "kind": "oracle",
            "sample": f"first {rows_all_cores} token rows of each of the 4 block inputs, {what}; {t_all:.1f} s; "
                      f"rate extrapolated to M = 65536 (the work is linear in M)",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "single_thread": {"value": v_one, "unit": "tokens/s", "cores": 1,
                              "sample": f"first {rows_one_core} token rows of each input, same work; {t_one:.1f} s; "
                                        "extrapolated"}}


def run_block(args, hbl, torch):
    """The seven linears of one 7B block at M = 65536 tokens, the pages'
    largest shape (hidden 4096, FFN 16384).  Q/K/V share one quantisation of
    their input, up/gate another (plain BitLinear); Wo and Wdown rotate
    their inputs (H-BitLinear).  One step = the block's 4 quantisations and 7
    matmuls, inputs resident in HBM.  The headline mode is INT4 on the FP6 x
    FP4 matrix cores (--path int8: the int8 matrix cores); INT8 activations
    are timed beside it.  Every launch of the timed steps is bracketed by HIP
    events on the stream the library launches on (torch's current stream),
    which gives the per-kernel averages of the roofline."""
    import workloads
    M = workloads.CONFIGS["block_7b"]["M"]
    print(f"[bench] block_7b: drawing inputs (M = {M})", file=sys.stderr, flush=True)
    xs = {name: dev_x(workloads.block_input(name)) for name, _ in workloads.BLOCK_7B_INPUTS}
    dims = {name: (K, N, had) for name, K, N, had in workloads.BLOCK_7B_LAYERS}
    ws = {name: hbl.ternarize_weights(torch.from_numpy(workloads.block_weights(name)).cuda())
          for name, *_ in workloads.BLOCK_7B_LAYERS}
    out = {name: torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for name, K, N, _ in workloads.BLOCK_7B_LAYERS}
    in_k = dict(workloads.BLOCK_7B_INPUTS)
    peaks = measured().get("peaks", {})

    def mode(bits):
        mx = use_mx(args, bits, M, 4096)  # both input widths (4096, 16384) qualify
        qbuf = {}
        for inp, had, layers in BLOCK_GROUPS:
            K = in_k[inp]
            shape, dt = (((M + 255) // 256 * 256, K // 4 * 3), torch.uint8) if mx else hbl.codes_shape(M, K, bits)
            qbuf[inp] = (torch.empty(shape, dtype=dt, device="cuda"), torch.empty(M, dtype=torch.float32, device="cuda"),
                         torch.empty(M, dtype=torch.int32, device="cuda"))
        wmx = {name: hbl.prepare_weights_mx(ws[name][0], dims[name][0]) for name in dims} if mx else {}

        def quant(inp, had):
            q, sc, rs = qbuf[inp]
            x = xs[inp]
            if mx:
                hbl._check(hbl.lib().hbl_hadamard_quant_mx(x.data_ptr(), hbl.DTYPE_BF16, M, x.shape[1], x.shape[1],
                                                           hbl.HADAMARD if had else 0, q.data_ptr(), sc.data_ptr(),
                                                           hbl._stream()), "hbl_hadamard_quant_mx")
            else:
                hbl._check(hbl.lib().hbl_hadamard_quant(x.data_ptr(), hbl.DTYPE_BF16, M, x.shape[1], x.shape[1],
                                                        hbl.HADAMARD if had else 0, bits, q.data_ptr(), sc.data_ptr(),
                                                        rs.data_ptr(), hbl._stream()), "hbl_hadamard_quant")

        def gemm(inp, layer):
            q, sc, rs = qbuf[inp]
            p, a = ws[layer]
            if mx:
                hbl.ternary_gemm_mx(q, sc, wmx[layer], a, in_k[inp], out=out[layer])
            else:
                hbl.ternary_gemm(q, bits, sc, rs, p, a, in_k[inp], out=out[layer])

        def step(ev=None):
            for inp, had, layers in BLOCK_GROUPS:
                if ev is not None:
                    ev.append(("quant", inp, torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)))
                    ev[-1][2].record()
                quant(inp, had)
                if ev is not None:
                    ev[-1][3].record()
                for layer in layers:
                    if ev is not None:
                        ev.append(("gemm", layer, torch.cuda.Event(enable_timing=True),
                                   torch.cuda.Event(enable_timing=True)))
                        ev[-1][2].record()
                    gemm(inp, layer)
                    if ev is not None:
                        ev[-1][3].record()

        print(f"[bench] block_7b INT{bits}: {args.warmup} warm-up and {args.steps} timed steps",
              file=sys.stderr, flush=True)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        ev = []
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step(ev)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        kern = {}
        for kind, name, a, b in ev:
            kern.setdefault((kind, name), []).append(a.elapsed_time(b) * 1e-3)
        k_us = {f"{kind} {name}": float(np.mean(v)) * 1e6 for (kind, name), v in kern.items()}
        gemm_s = sum(float(np.mean(v)) for (kind, _), v in kern.items() if kind == "gemm")
        quant_s = sum(float(np.mean(v)) for (kind, _), v in kern.items() if kind == "quant")
        ops = sum(2.0 * M * K * N for K, N, _ in dims.values())
        code_b = {inp: (M * in_k[inp] * 3 // 4 if mx else M * in_k[inp] // (2 if bits == 4 else 1))
                  for inp, _, _ in BLOCK_GROUPS}
        q_bytes = sum(M * in_k[inp] * 2 + code_b[inp] + (4 if mx else 8) * M for inp, _, _ in BLOCK_GROUPS)
        g_min = sum(code_b[inp] + dims[l][1] * dims[l][0] // 4 + 2 * M * dims[l][1]
                    for inp, _, layers in BLOCK_GROUPS for l in layers)
        return {"bits": bits, "mx": mx, "dt": dt, "k_us": k_us, "gemm_s": gemm_s, "quant_s": quant_s, "ops": ops,
                "q_bytes": q_bytes, "gemm_bytes_min": g_min, "n_gemm": len(dims), "n_quant": len(BLOCK_GROUPS)}

    modes = [4, 8] if args.bits == 0 else [args.bits]
    res_modes = {b: mode(b) for b in modes}
    head = res_modes[modes[0]]
    bits, mx, dt = head["bits"], head["mx"], head["dt"]
    ops = head["ops"]
    n_g, n_q = head["n_gemm"], head["n_quant"]
    gemm_tops = ops / head["gemm_s"] / 1e12
    best = peaks.get("i8_mfma_tops_best")
    if mx:
        peak, kernel = MX_PEAK_TOPS, "k_gemm_mx (FP6 x FP4 ternary matmul)"
        meas = peaks.get("fp6fp4_mfma_tops_best")
    else:
        peak, kernel = I8_PEAK_TOPS, "k_gemm_pt (int8 ternary matmul)"
        meas = best
    hbm_meas = peaks.get("hbm_read_gbs")
    roofline = {"bound": "mfma", "kernel": kernel, "achieved": gemm_tops, "peak": peak, "unit": "TOP/s",
                "frac": gemm_tops / peak, "traffic": counter_traffic("block_7b", "gemm_mx" if mx else "gemm"),
                "avg_kernel_us": head["gemm_s"] / n_g * 1e6, "algorithmic_ops_per_launch": ops / n_g,
                "launches_per_step": n_g,
                "measured_peak": {"tops": meas, "frac": gemm_tops / meas if meas else None,
                                  "i8_mfma_tops": best, "frac_of_i8": gemm_tops / best if best else None,
                                  "source": "profiles/peaks.md"}}
    q_gbs = head["q_bytes"] / head["quant_s"] / 1e9
    res = {
        "metric": METRIC, "value": M / dt, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": dt * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp6xfp4" if mx else "i8", "data": "synthetic",
        "config": {"workload": "block_7b: the 7 linears of one 7B block (Q/K/V 4096->4096 and up/gate "
                               "4096->16384 plain BitLinear; Wo 4096->4096 and Wdown 16384->4096 H-BitLinear), "
                               f"M = {M} tokens (64 x 1024), INT{bits} activations",
                   "M": M, "bits": bits, "x_dtype": "bf16",
                   "path": "FP6 x FP4 matrix cores (exact)" if mx else "int8 matrix cores"},
        "effective_tops": ops / dt / 1e12,
        "roofline": roofline,
        "fused": {"effective_tops": ops / dt / 1e12,
                  "frac_of_measured_i8_peak": ops / dt / 1e12 / best if best else None,
                  "frac_of_published_i8_peak": ops / dt / 1e12 / I8_PEAK_TOPS},
        "quant_kernel": {"bound": "hbm", "kernel": "k_fwht_quant64 (rotation + quantisation)",
                         "avg_kernel_us": head["quant_s"] / n_q * 1e6,
                         "algorithmic_bytes_per_launch": head["q_bytes"] / n_q, "achieved_gbs": q_gbs,
                         "frac": q_gbs / HBM_PEAK_GBS,
                         "frac_of_measured_read_peak": q_gbs / hbm_meas if hbm_meas else None,
                         "traffic": counter_traffic("block_7b", "quant_mx" if mx else "quant")},
        "gemm_bytes_min_per_step": head["gemm_bytes_min"],
        "kernel_us": head["k_us"],
        "launch": "eager launches on one stream, HIP events around each launch",
    }
    for b, r in res_modes.items():
        if r is head:
            continue
        res[f"int{b}_mode"] = {"tokens_per_s": M / r["dt"], "ms_per_step": r["dt"] * 1e3,
                               "effective_tops": r["ops"] / r["dt"] / 1e12,
                               "frac_of_measured_i8_peak": r["ops"] / r["dt"] / 1e12 / best if best else None,
                               "path": "FP6 x FP4 matrix cores" if r["mx"] else "int8 matrix cores",
                               "gemm_tops": r["ops"] / r["gemm_s"] / 1e12, "kernel_us": r["k_us"]}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import bit_quantization_amd as hbl
    import workloads
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.workload == "copy":
        # a plain device-to-device copy of known size, for counter calibration
        n = args.copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        t = time_stream(lambda: dst.copy_(src), max(3, args.steps))
        print(json.dumps({"workload": "copy", "bytes_read": n, "bytes_written": n, "avg_kernel_us": t * 1e6,
                          "achieved_gbs": 2 * n / t / 1e9}), flush=True)
        return

    if args.workload == "decode":
        res = run_decode(args, hbl, torch)
        if not args.no_cpu_baseline:
            x_np = workloads.decode_inputs(args.decode_k, args.decode_m)
            w_np = workloads.decode_weights(args.decode_k, 4096, 0)
            res["cpu_baseline"] = cpu_baseline(x_np, w_np, 8, True)
        print(json.dumps(res), flush=True)
        return

    if args.workload == "block_7b":
        res = run_block(args, hbl, torch)
        if not args.no_cpu_baseline:
            print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
            res["cpu_baseline"] = block_cpu_baseline(res["config"]["bits"])
        print(json.dumps(res), flush=True)
        return

    if args.workload == "msweep":
        print(json.dumps(run_msweep(args, hbl, torch)), flush=True)
        return

    if args.workload == "kvcache":
        print(json.dumps(run_kvcache(args, hbl, torch)), flush=True)
        return

    c = {"tiny": workloads.tiny, "wo_7b": workloads.wo_7b, "wdown_7b": workloads.wdown_7b}[args.workload]()
    label = {"tiny": "tiny: M=8 K=N=256 INT4 H-BitLinear",
             "wo_7b": "wo_7b: 7B attention output projection, M=2048 K=N=4096 INT4 H-BitLinear",
             "wdown_7b": "wdown_7b: 7B FFN down projection, M=4096 K=16384 N=4096 INT4 H-BitLinear"}[args.workload]
    res = run_layer(args, hbl, torch, c["x"], c["w"], c["bits"], True, label)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(c["x"], c["w"], c["bits"], True)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
