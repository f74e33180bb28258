"""Benchmark of the BitLinear hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch of synthetic input:
RMSNorm + per-token int8 activation quantization, absmean ternary weight
quantization + packing (both quantizers in one bitnet_quant_operands call),
the ternary x int8 forward with dequantization, and the STE backward
(grad_x and grad_W).  Inputs are generated once on the
host (seeded, see workloads.py), copied to HBM before timing, and every
output buffer is preallocated, so the timed region is device work only.

Default workload: small_llama (M=8192 tokens, K=512, N=1376: the MLP
up-projection of the ~15M-parameter LLaMA-shaped model), the forward plus
STE backward configuration.  Other workloads (--workload) are for
profiling: tiny, prefill_7b (forward only), decode_7b (packed GEMV only,
pre-quantized operands, weight copies rotated so every launch streams its
weights from HBM), qat_70b_mlp (full step) and copy (a 1 GiB device copy,
the calibration kernel for the HBM byte counters).

Prints ONE JSON line.  `value` is the step's algorithmic operation rate:
(2MNK int8 forward + 2MNK bf16 grad_x + 2MNK bf16 grad_W) / step time,
in TOPS (forward-only workloads count 2MNK; decode reports GB/s of the
bytes the GEMV must move).  `roofline` is the longest single product of
the step (the backward call counts as its grad_x and grad_W products), its
algorithmic work per launch over its per-launch time from HIP events on the
stream it runs on; its `traffic` is the HBM bytes per launch from rocprofv3
FETCH_SIZE + WRITE_SIZE recorded under profiles/ (null once the kernel
sources differ from the profiled ones).  `kernels` breaks the step down per
call; `cpu_baseline` is the CPU oracle timed on this host (a bounded sample
of the same workload).
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import bit_ternary_quantized_amd as bt  # noqa: E402
import workloads  # noqa: E402

METRIC = "BitLinear fwd int8 TOPS & packed-GEMV GB/s (fraction of MI355X roofline)"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0    # dense int8 MFMA
BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="small_llama",
                    choices=["small_llama", "tiny", "prefill_7b", "decode_7b", "qat_70b_mlp", "copy"])
    ap.add_argument("--decode-m", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--two-streams", action="store_true",
                    help="run the two quantizers as two calls (act_quant, weight_quant) on two streams "
                         "inside the step graph (default: one bitnet_quant_operands call; every call in "
                         "order on one stream)")
    ap.add_argument("--step-only", action="store_true",
                    help="time only the step's calls and its two backward products (no variant calls)")
    return ap.parse_args()


class Timer:
    """HIP events around each ABI call of a step, on the call's stream."""

    def __init__(self, names, steps):
        self.names = names
        self.ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
                   for _ in range(steps)]

    def mark(self, step, i):
        self.ev[step][i].record(torch.cuda.current_stream())

    def mean_ms(self):
        out = {}
        for i, n in enumerate(self.names):
            out[n] = statistics.fmean(e[i].elapsed_time(e[i + 1]) for e in self.ev)
        return out


# --------------------------------------------------------------- workloads

def setup_layer(name):
    d = workloads.workload(name)
    M, N, K = d["M"], d["N"], d["K"]
    dev = "cuda:0"
    x, w = d["x"].to(dev), d["w"].to(dev)
    gy = d["gy"].to(dev) if "gy" in d else None
    buf = {
        "Xq": torch.empty(M, K, dtype=torch.int8, device=dev),
        "scale_x": torch.empty(M, dtype=torch.float32, device=dev),
        "W_packed": torch.empty(N, K // 4, dtype=torch.uint8, device=dev),
        "gamma": torch.empty(1, dtype=torch.float32, device=dev),
        "ws_wq": torch.empty(bt.bitnet_workspace_bytes(bt.BITNET_OP_WEIGHT_QUANT, M, N, K),
                             dtype=torch.uint8, device=dev),
        "Y": torch.empty(M, N, dtype=torch.float32, device=dev),
        "counts": torch.empty(4, dtype=torch.int64, device=dev),
        "ws_cc": torch.empty(bt.bitnet_workspace_bytes(bt.BITNET_OP_CODE_COUNTS, 0, N, K), dtype=torch.uint8,
                             device=dev),
        "W_packed_rows": torch.empty(N, K // 4, dtype=torch.uint8, device=dev),
        "gamma_rows": torch.empty(N, dtype=torch.float32, device=dev),
        "ws_wqr": torch.empty(bt.bitnet_workspace_bytes(bt.BITNET_OP_WEIGHT_QUANT_ROWS, 0, N, K), dtype=torch.uint8,
                              device=dev),
    }
    if gy is not None:
        buf["grad_x"] = torch.empty(M, K, dtype=torch.float32, device=dev)
        buf["grad_W"] = torch.empty(N, K, dtype=torch.float32, device=dev)
        buf["ws_bwd"] = torch.empty(bt.bitnet_workspace_bytes(bt.BITNET_OP_LINEAR_BWD_STE, M, N, K),
                                    dtype=torch.uint8, device=dev)
        buf["grad_X"] = torch.empty(M, K, dtype=torch.float32, device=dev)
        buf["w_clamp"] = w.clone()  # the clamp runs in place on a copy
    return d, x, w, gy, buf


def layer_counts(M, N, K, x_bytes, w_bytes, gy):
    """Algorithmic work of each call (bytes moved once, or ops)."""
    c = {
        "act_quant": {"bytes": M * K * x_bytes + M * K + 4 * M, "bound": "hbm"},
        # two reads of W: gamma needs the full reduction before any code exists
        "weight_quant": {"bytes": 2 * N * K * w_bytes + N * K // 4 + 4, "bound": "hbm"},
        "linear_fwd": {"ops": 2 * M * N * K, "bytes": M * K + N * K // 4 + 4 * M + 4 * M * N,
                       "peak_ops": INT8_PEAK_TOPS},
        # both quantizers in one call: act_quant's bytes plus weight_quant's
        "quant_operands": {"bytes": M * K * x_bytes + M * K + 4 * M + 2 * N * K * w_bytes + N * K // 4 + 4,
                           "bound": "hbm"},
        # zero / +1 / -1 counts of the packed codes (monitoring): the codes read once
        "code_counts": {"bytes": N * K // 4 + 32, "bound": "hbm"},
        # per-output-channel variants: per-row weight quant (two reads of W),
        # the forward with a scale per output channel
        "weight_quant_rows": {"bytes": 2 * N * K * w_bytes + N * K // 4 + 4 * N, "bound": "hbm"},
        "linear_fwd_channel": {"ops": 2 * M * N * K, "bytes": M * K + N * K // 4 + 4 * M + 4 * N + 4 * M * N,
                               "peak_ops": INT8_PEAK_TOPS},
    }
    if gy:
        c["linear_bwd_ste"] = {"ops": 4 * M * N * K,
                               "bytes": 2 * M * N + M * K + N * K // 4 + 4 * M + 4 * M * K + 4 * N * K,
                               "peak_ops": BF16_PEAK_TFLOPS}
        c["bwd_grad_x"] = {"ops": 2 * M * N * K, "bytes": 2 * M * N + N * K // 4 + 4 + 4 * M * K,
                           "peak_ops": BF16_PEAK_TFLOPS}
        c["bwd_grad_x_channel"] = {"ops": 2 * M * N * K, "bytes": 2 * M * N + N * K // 4 + 4 * N + 4 * M * K,
                                   "peak_ops": BF16_PEAK_TFLOPS}
        c["bwd_grad_W"] = {"ops": 2 * M * N * K, "bytes": 2 * M * N + M * K + 4 * M + 4 * N * K,
                           "peak_ops": BF16_PEAK_TFLOPS}
        # RMSNorm backward (after the STE backward): x and fp32 grad_x read, fp32 grad_X written
        c["rmsnorm_bwd"] = {"bytes": M * K * x_bytes + 4 * M * K + 4 * M * K, "bound": "hbm"}
        # grad_W with the master-weight range gate: the master weights read as well
        c["bwd_grad_W_gated"] = {"ops": 2 * M * N * K,
                                 "bytes": 2 * M * N + M * K + 4 * M + 4 * N * K + w_bytes * N * K,
                                 "peak_ops": BF16_PEAK_TFLOPS}
        # the master-weight clamp: read and written in place
        c["weight_clamp"] = {"bytes": 2 * N * K * w_bytes, "bound": "hbm"}
    for v in c.values():
        if "ops" in v:
            ridge = v["peak_ops"] * 1e12 / (HBM_PEAK_GBS * 1e9)
            v["bound"] = "mfma" if v["ops"] / v["bytes"] > ridge else "hbm"
    return c


KERNEL_OF = {
    "act_quant": "act_quant_rows_kernel (rows of whole 16-byte blocks), else act_quant_kernel",
    "weight_quant": "wq_row_abs_sum_kernel + wq_gamma_kernel + wq_pack_kernel",
    "linear_fwd": "gemm_i8t2_kernel",
    "bwd_grad_x": "bwd_kernel<grad_x>",
    "bwd_grad_W": "bwd_kernel<grad_W> (+ split_reduce_kernel when split)",
    "rmsnorm_bwd": "rmsnorm_bwd_kernel",
    "bwd_grad_W_gated": "bwd_kernel<grad_W> with the range gate (+ split_reduce_kernel when split)",
    "weight_clamp": "weight_clamp_kernel",
    "code_counts": "code_counts_kernel + code_counts_final_kernel",
    "quant_operands": "quant_operands_kernel + wq_pack_kernel (+ wq_gamma_kernel)",
    "weight_quant_rows": "wq_row_abs_sum_kernel + wq_rows_gamma_kernel + wq_pack_rows_kernel",
    "linear_fwd_channel": "gemm_i8t2_kernel (per-channel epilogue) or gemv_t2_kernel",
    "bwd_grad_x_channel": "bwd_kernel<grad_x> (per-channel code scales)",
}
# sources each call's kernels are built from: the HBM traffic recorded under
# profiles/ is used only while these files are unchanged
SOURCES_OF = {
    "act_quant": ["bit_ternary_quantized_amd/csrc/quant.hip"],
    "weight_quant": ["bit_ternary_quantized_amd/csrc/quant.hip"],
    "linear_fwd": ["bit_ternary_quantized_amd/csrc/gemm_i8.hip", "bit_ternary_quantized_amd/csrc/gemv.hip"],
    "bwd_grad_x": ["bit_ternary_quantized_amd/csrc/bwd.hip"],
    "bwd_grad_W": ["bit_ternary_quantized_amd/csrc/bwd.hip"],
    "rmsnorm_bwd": ["bit_ternary_quantized_amd/csrc/norm_bwd.hip"],
    "bwd_grad_W_gated": ["bit_ternary_quantized_amd/csrc/bwd.hip"],
    "weight_clamp": ["bit_ternary_quantized_amd/csrc/quant.hip"],
    "code_counts": ["bit_ternary_quantized_amd/csrc/quant.hip"],
    "quant_operands": ["bit_ternary_quantized_amd/csrc/quant.hip"],
    "weight_quant_rows": ["bit_ternary_quantized_amd/csrc/quant.hip"],
    "linear_fwd_channel": ["bit_ternary_quantized_amd/csrc/gemm_i8.hip", "bit_ternary_quantized_amd/csrc/gemv.hip"],
    "bwd_grad_x_channel": ["bit_ternary_quantized_amd/csrc/bwd.hip"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def source_digest(call):
    import hashlib
    h = hashlib.sha256()
    for rel in SOURCES_OF.get(call, []) + ["bit_ternary_quantized_amd/csrc/common.h"]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(call, workload):
    """HBM bytes per launch of `call` from rocprofv3 FETCH_SIZE + WRITE_SIZE
    (scaled by the copy calibration), as recorded under profiles/; None when
    absent or when the kernel sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(f"{call}@{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != source_digest(call):
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def rate(entry, ms):
    s = ms * 1e-3
    if entry["bound"] == "hbm":
        a = entry["bytes"] / s / 1e9
        return {"bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": a / HBM_PEAK_GBS}
    a = entry["ops"] / s / 1e12
    return {"bound": "mfma", "achieved": a, "peak": entry["peak_ops"], "unit": "TFLOP/s",
            "frac": a / entry["peak_ops"]}


def cpu_baseline_layer(d, gy_present, budget_s=12.0):
    """The oracle on this host, on the first S tokens of the same layer: act
    quant of those S rows, weight quant of the whole W (a step needs it
    whatever the token count), forward and STE backward over the S tokens.
    S is sized from a short calibration run so that one sample takes about
    half the budget; the sample repeats until the budget is spent (at most
    three times) and the median counts.  Rate = the GPU's algorithmic ops
    for S tokens / seconds."""
    import oracle
    M, N, K = d["M"], d["N"], d["K"]
    xh = workloads.host_array(d["x"])
    wh = workloads.host_array(d["w"])
    gyh = workloads.host_array(d["gy"]) if gy_present else None

    def run(S):
        t0 = time.perf_counter()
        q, s = oracle.act_quant(xh[:S])
        c, g = oracle.weight_quant(wh)
        oracle.gemm_i32(q, c)
        if gyh is not None:
            oracle.ste_grad_x(gyh[:S], c, g)
            oracle.ste_grad_w(gyh[:S], q, s)
        return time.perf_counter() - t0

    S = min(M, 64)
    t = run(S)
    S = int(max(1, min(M, S * (budget_s / 2) / max(t, 1e-9))))
    times = []
    t_start = time.perf_counter()
    while not times or (time.perf_counter() - t_start < budget_s and len(times) < 3):
        times.append(run(S))
    ops = (2 + (4 if gy_present else 0)) * S * N * K
    sec = statistics.median(times)
    return {"value": ops / sec / 1e12, "unit": "TOPS", "cores": oracle.get_threads(), "kind": "oracle",
            "sample": f"first {S} of {M} tokens: act quant of those rows, weight quant of all of W, "
                      f"forward{' and STE backward' if gy_present else ''}; median of {len(times)} run(s) "
                      f"of {sec:.2f} s",
            "seconds": sec}


def capture(fn):
    """Capture the kernels one call enqueues into a HIP graph (torch stream
    capture; the library launches on the current stream and allocates
    nothing when every buffer is passed in)."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # one eager run on the capture stream before capturing
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


SLEEP_CYCLES = 50_000_000  # bounded spin that lets the host enqueue ahead
REPS = 8                   # launches of one call per timed graph


def bench_layer(args, name):
    d, x, w, gy, b = setup_layer(name)
    M, N, K = d["M"], d["N"], d["K"]
    calls = {
        "act_quant": lambda: bt.bitnet_act_quant(x, 1e-5, Xq=b["Xq"], scale_x=b["scale_x"]),
        "weight_quant": lambda: bt.bitnet_weight_quant(w, W_packed=b["W_packed"], gamma=b["gamma"],
                                                       workspace=b["ws_wq"]),
        "linear_fwd": lambda: bt.bitnet_linear_fwd(b["Xq"], b["scale_x"], b["W_packed"], b["gamma"], Y=b["Y"]),
    }
    if gy is not None:
        calls["linear_bwd_ste"] = lambda: bt.bitnet_linear_bwd_ste(
            gy, b["Xq"], b["scale_x"], b["W_packed"], b["gamma"], grad_x=b["grad_x"], grad_W=b["grad_W"],
            workspace=b["ws_bwd"])
    names = list(calls)
    # the backward call's two products, each timed on its own (not part of
    # the step): grad_x is one kernel, grad_W one kernel plus the ordered
    # split reduction when its token range is split
    parts = {
        "code_counts": lambda: bt.bitnet_code_counts(b["W_packed"], K, counts=b["counts"], workspace=b["ws_cc"]),
        # both quantizers in one call (one launch fewer; same outputs)
        "quant_operands": lambda: bt.bitnet_quant_operands(x, w, 1e-5, Xq=b["Xq"], scale_x=b["scale_x"],
                                                           W_packed=b["W_packed"], gamma=b["gamma"],
                                                           workspace=b["ws_wq"]),
        # per-output-channel variants (own buffers; not part of the step)
        "weight_quant_rows": lambda: bt.bitnet_weight_quant_rows(w, W_packed=b["W_packed_rows"], gamma=b["gamma_rows"],
                                                                 workspace=b["ws_wqr"]),
        "linear_fwd_channel": lambda: bt.bitnet_linear_fwd_channel(b["Xq"], b["scale_x"], b["W_packed_rows"],
                                                                   b["gamma_rows"], Y=b["Y"]),
    }
    if gy is not None:
        parts["bwd_grad_x"] = lambda: bt.bitnet_linear_bwd_ste(
            gy, b["Xq"], b["scale_x"], b["W_packed"], b["gamma"], want_grad_W=False, grad_x=b["grad_x"])
        parts["bwd_grad_x_channel"] = lambda: bt.bitnet_linear_bwd_ste_channel(
            gy, b["Xq"], b["scale_x"], b["W_packed_rows"], b["gamma_rows"], want_grad_W=False, grad_x=b["grad_x"])
        parts["bwd_grad_W"] = lambda: bt.bitnet_linear_bwd_ste(
            gy, b["Xq"], b["scale_x"], b["W_packed"], b["gamma"], want_grad_x=False, grad_W=b["grad_W"],
            workspace=b["ws_bwd"])
        # the gradient through the RMSNorm in front of the quantizer, from the
        # step's grad_x (timed on its own; not part of the step)
        parts["rmsnorm_bwd"] = lambda: bt.bitnet_rmsnorm_bwd(x, b["grad_x"], 1e-5, grad_X=b["grad_X"])
        # the STE variants: grad_W gated by the master weights in [-1, 1], and
        # the clamp of the master weights after an update
        parts["bwd_grad_W_gated"] = lambda: bt.bitnet_linear_bwd_ste_gated(
            gy, b["Xq"], b["scale_x"], b["W_packed"], b["gamma"], w, -1.0, 1.0, want_grad_x=False,
            grad_W=b["grad_W"], workspace=b["ws_bwd"])
        parts["weight_clamp"] = lambda: bt.bitnet_weight_clamp(b["w_clamp"], -1.0, 1.0)

    # --two-streams: the two quantizers (X and W), which are independent, run
    # on two streams (default priority) forked and joined with events, so the
    # graph holds parallel branches; then the forward GEMM and the backward
    # call.  Measured: 1-2.5% faster at the 7B and 70B shapes, 7% slower at
    # small_llama (the join between the branches costs more than the overlap
    # of two short kernels saves), so the default runs every call in order on
    # one stream.  The backward's two products on two streams measured slower
    # still: their workgroups, one per CU each, then compete for the CUs.
    side = torch.cuda.Stream()

    def fork_join(main_fn, side_fn):
        main = torch.cuda.current_stream()
        e0 = torch.cuda.Event()
        e0.record(main)
        side.wait_event(e0)
        with torch.cuda.stream(side):
            side_fn()
        e1 = torch.cuda.Event()
        e1.record(side)
        main_fn()
        main.wait_event(e1)

    # The step: both quantizers in one call (bitnet_quant_operands: the same
    # outputs as act_quant + weight_quant with one launch fewer), the forward,
    # the backward.
    step_calls = dict(calls)
    step_calls["quant_operands"] = parts["quant_operands"]
    step_names = ["quant_operands", "linear_fwd"] + (["linear_bwd_ste"] if gy is not None else [])

    def step():
        if not args.two_streams:
            for n in step_names:
                step_calls[n]()
            return
        fork_join(calls["act_quant"], calls["weight_quant"])
        calls["linear_fwd"]()
        if gy is not None:
            calls["linear_bwd_ste"]()

    g_step = capture(step)
    for _ in range(args.warmup):
        g_step.replay()
    torch.cuda.synchronize()

    # timed region: K whole steps, one graph launch each
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        g_step.replay()
    end.record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    dev_ms = start.elapsed_time(end) / args.steps

    # per-call device time: each call captured REPS times back to back in
    # one graph; K replays of each, bracketed by HIP events on the stream
    # they run on.  A bounded spin first lets the host enqueue the whole loop,
    # so no host gap sits between two events.
    if args.step_only:
        parts = {n: f for n, f in parts.items() if n in ("bwd_grad_x", "bwd_grad_W", "quant_operands")}
    allc = dict(calls, **parts)
    timed = list(allc)
    g_rep = {n: capture(lambda n=n: [allc[n]() for _ in range(REPS)]) for n in timed}
    timer = Timer(timed, args.steps)
    torch.cuda.synchronize()
    torch.cuda._sleep(SLEEP_CYCLES)
    for i in range(args.steps):
        for j, n in enumerate(timed):
            timer.mark(i, j)
            g_rep[n].replay()
        timer.mark(i, len(timed))
    torch.cuda.synchronize()
    per = {n: v / REPS for n, v in timer.mean_ms().items()}

    counts = layer_counts(M, N, K, d["x"].element_size(), d["w"].element_size(), gy is not None)
    kernels = {n: {"ms": per[n], **rate(counts[n], per[n])} for n in timed}
    fwd_bwd = 2 + (4 if gy is not None else 0)
    value = fwd_bwd * M * N * K / (ms * 1e-3) / 1e12
    # roofline: the longest single product of the step (the backward call
    # counts as its two products)
    # the step's own products only (the other timed calls are variants)
    cands = [n for n in timed if n in ("act_quant", "weight_quant", "linear_fwd", "bwd_grad_x", "bwd_grad_W")]
    dom = max(cands, key=lambda n: per[n])
    roof = dict(rate(counts[dom], per[dom]))
    roof["kernel"] = KERNEL_OF[dom] + f" ({dom})"
    roof["traffic"] = measured_traffic(dom, name)
    out = {
        "metric": METRIC, "value": value, "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "device_ms_per_step": dev_ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "i8+bf16" if gy is not None else "i8",
        "data": "synthetic",
        "config": {"workload": name, "M": M, "N": N, "K": K, "x_dtype": str(d["x"].dtype).split(".")[-1],
                   "w_dtype": str(d["w"].dtype).split(".")[-1],
                   "step": "act_quant+weight_quant (two streams)+" + "+".join(step_names[1:]) if args.two_streams
                   else "+".join(step_names), "launch": "one HIP graph per step",
                   "schedule": "two streams: act_quant || weight_quant, then linear_fwd, then linear_bwd_ste"
                   if args.two_streams else "every call in order on one stream"},
        "roofline": roof,
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_layer(d, gy is not None)
    return out


def bench_decode(args):
    """Packed GEMV at decode shape; weights rotated over enough copies that
    every launch reads its 2-bit weights from HBM, not the 256 MB cache."""
    M = args.decode_m
    d = workloads.workload("decode_7b", M=M)
    N, K = d["N"], d["K"]
    dev = "cuda:0"
    q, s, gm = d["q"].to(dev), d["scale_x"].to(dev), d["gamma"].to(dev)
    wp0 = bt.bitnet_pack_ternary(d["codes"].to(dev))
    copies = max(2, (512 << 20) // wp0.numel() + 1)  # > 2x the Infinity Cache
    wps = [wp0] + [wp0.clone() for _ in range(copies - 1)]
    Y = torch.empty(M, N, dtype=torch.float32, device=dev)
    # one graph = one launch per weight copy, back to back; each replay
    # streams every copy once
    g = capture(lambda: [bt.bitnet_linear_fwd(q, s, wp, gm, Y=Y) for wp in wps])
    for _ in range(max(1, args.warmup // copies)):
        g.replay()
    torch.cuda.synchronize()
    reps = max(1, args.steps // copies)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda._sleep(SLEEP_CYCLES)
    t0 = time.perf_counter()
    for i in range(reps):
        ev[i].record()
        g.replay()
    ev[-1].record()
    torch.cuda.synchronize()
    ms = statistics.fmean(ev[i].elapsed_time(ev[i + 1]) for i in range(reps)) / copies
    nbytes = N * K // 4 + M * K + 4 * M + 4 + 4 * M * N
    gbs = nbytes / (ms * 1e-3) / 1e9

    # a whole decode step from the unquantized activations, per weight copy:
    # act_quant then the GEMV (two launches), and the fused call (one launch)
    x = d["x"].to(dev)
    q2, s2 = torch.empty_like(q), torch.empty_like(s)

    def per_launch_ms(fn, weights=wps):
        gr = capture(lambda: [fn(wp) for wp in weights])
        for _ in range(max(1, args.warmup // copies)):
            gr.replay()
        torch.cuda.synchronize()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        torch.cuda._sleep(SLEEP_CYCLES)
        for i in range(reps):
            e[i].record()
            gr.replay()
        e[-1].record()
        torch.cuda.synchronize()
        return statistics.fmean(e[i].elapsed_time(e[i + 1]) for i in range(reps)) / copies

    # algorithmic bytes of a decode step: x (bf16) and the packed weights in, Y out
    step_bytes = N * K // 4 + 2 * M * K + 4 + 4 * M * N

    def entry(t_ms, nb):
        a = nb / (t_ms * 1e-3) / 1e9
        return {"ms": t_ms, "bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": a / HBM_PEAK_GBS}

    kernels = {"linear_fwd": entry(ms, nbytes)}
    kernels["act_quant+linear_fwd"] = entry(per_launch_ms(lambda wp: (
        bt.bitnet_act_quant(x, 1e-5, Xq=q2, scale_x=s2), bt.bitnet_linear_fwd(q2, s2, wp, gm, Y=Y))), step_bytes)
    kernels["linear_fwd_decode"] = entry(
        per_launch_ms(lambda wp: bt.bitnet_linear_fwd_decode(x, wp, gm, 1e-5, Y=Y)), step_bytes)
    if K == 4096:  # the same call on the weights in the decode layout (repacked once, untimed)
        wds = [bt.bitnet_pack_decode(wp) for wp in wps]
        kernels["linear_fwd_decode@decode_layout"] = entry(
            per_launch_ms(lambda wd: bt.bitnet_linear_fwd_decode(x, wd, gm, 1e-5, Y=Y, N=N), wds), step_bytes)
    out = {
        "metric": METRIC, "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "i8", "data": "synthetic",
        "config": {"workload": "decode_7b", "M": M, "N": N, "K": K, "weight_copies": copies,
                   "launches_timed": reps * copies},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "gemv_row_kernel" if M == 1 and K % 64 == 0 and K <= 8192 else "gemv_t2_kernel"},
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        import oracle
        qh, ch = d["q"].numpy(), d["codes"].numpy()
        t = time.perf_counter()
        oracle.gemm_i32(qh, ch)
        sec = time.perf_counter() - t
        out["cpu_baseline"] = {"value": nbytes / sec / 1e9, "unit": "GB/s", "cores": oracle.get_threads(),
                               "kind": "oracle", "sample": f"whole GEMV (M={M}) once, {sec:.2f} s"}
    return out


def bench_copy(args):
    """Device-to-device copy of a known size (1 GiB, four times the Infinity
    Cache): the calibration kernel for the HBM byte counters."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    for _ in range(max(1, args.warmup)):
        b.copy_(a)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        b.copy_(a)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    gbs = 2 * n / (ms * 1e-3) / 1e9
    return {"metric": "HBM copy GB/s (counter calibration)", "value": gbs, "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
            "config": {"workload": "copy", "bytes_read": n, "bytes_written": n},
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": None, "kernel": "device copy"}}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    bt.load_library()
    if args.workload == "decode_7b":
        out = bench_decode(args)
    elif args.workload == "copy":
        out = bench_copy(args)
    else:
        out = bench_layer(args, args.workload)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
