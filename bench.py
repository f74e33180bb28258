"""Benchmark of the BitLinear hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload: prefill_7b, the 7B-shaped prefill forward (M = 8192 tokens,
K = 4096, N = 4096; bf16 X with 0.1% outlier columns, bf16 master weights).
A step is one forward pass of the layer over that batch: RMSNorm + per-token
int8 activation quantization and absmean ternary weight quantization with
2-bit packing (both in one bitnet_quant_operands call), then the ternary x
int8 product with its dequantization (bitnet_linear_fwd).  Inputs are drawn
once on the host (seeded, workloads.py), copied to HBM before timing, and
every output buffer is preallocated, so the timed region is device work
only; each step is one HIP graph replay.

The JSON line carries:
  value       forward int8 TOPS: 2*M*N*K over the step time;
  roofline    the step's dominant kernel, the int8 GEMM (gemm_i8t2_kernel):
              2*M*N*K over its mean launch time from HIP events on its
              stream, against the 5.0 POPS dense int8 peak and against the
              measured ceiling (back-to-back int8 MFMAs on this device), with
              the clock the device held; traffic = HBM bytes per launch from
              rocprofv3 FETCH_SIZE + WRITE_SIZE recorded under profiles/;
  decode      the packed GEMV at the 7B decode shape (N = 11008, K = 4096) at
              M = 1 and M = 16, weights rotated over enough copies that every
              launch streams them from HBM: GB/s against 8 TB/s and against a
              one-launch streaming read of the same byte count;
  ceilings    the measured ceilings (streaming reads of 11.3 MB, 12.0 MB and
              67 MB, int8 and bf16 MFMA loops with their clocks);
  kernels     every call of the step, and the variants, timed on its own (8
              launches back to back; warm_cache marks the calls whose bytes
              fit in the 256 MB Infinity Cache, which then serves them);
  cpu_baseline  the CPU oracle on this host's cores, on a bounded sample of
              the same workload (threads and CPU model stated);
  inputs      sha256 of every input tensor;
  configs     the other layer configurations of the job, compactly: tiny
              (32x256->256 fp32), small_llama (8192x512->1376, forward and
              STE backward) and qat_70b_mlp (4096x8192->28672, forward and
              STE backward): forward and backward times and rates, and each
              call of their steps.

Other workloads (--workload): small_llama and qat_70b_mlp add the STE backward
(value stays the forward int8 rate; the backward's bf16 rate is reported on
its own), tiny, decode_7b (the GEMV and the fused decode calls in detail) and
copy (the 1 GiB device copy that calibrates the HBM byte counters).
"""
import argparse
import hashlib
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
INFINITY_CACHE = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="prefill_7b",
                    choices=["prefill_7b", "small_llama", "qat_70b_mlp", "tiny", "decode_7b", "copy"])
    ap.add_argument("--decode-m", type=int, default=16, help="tokens of --workload decode_7b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="leave the decode GEMV out of a layer run")
    ap.add_argument("--no-ceilings", action="store_true", help="leave the calibration kernels out")
    ap.add_argument("--no-configs", action="store_true",
                    help="prefill_7b: leave out the compact timings of tiny, small_llama and qat_70b_mlp")
    ap.add_argument("--two-streams", action="store_true",
                    help="run the two quantizers as two calls (act_quant, weight_quant) on two streams "
                         "inside the step graph (default: one bitnet_quant_operands call; every call in "
                         "order on one stream)")
    ap.add_argument("--step-only", action="store_true",
                    help="time only the step's calls (and the backward's two products), no variant calls")
    return ap.parse_args()


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def sha256(t):
    h = hashlib.sha256()
    h.update(t.detach().cpu().contiguous().view(torch.uint8).numpy().tobytes())
    return h.hexdigest()


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
# Untimed warm-up: the W steps asked for, continued until at least this much
# device time has passed.  Measured at the 7B prefill step: the first 48 steps
# after idle took 184.5 us each, the same graph 167 us after 10 ms more work
# and 160 us after 30 ms (clocks and power state settling), so a few steps of
# warm-up time the GPU coming out of idle, not the kernels.
WARMUP_MIN_MS = 100.0


def warm_up(g, steps):
    """Replay `g` (one step) `steps` times, then until WARMUP_MIN_MS of device
    time has passed; returns the number of steps run."""
    n = 0
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        g.replay()
        n += 1
    end.record()
    torch.cuda.synchronize()
    while start.elapsed_time(end) < WARMUP_MIN_MS:
        for _ in range(max(1, steps)):
            g.replay()
            n += 1
        end.record()
        torch.cuda.synchronize()
    return n
REPS = 8                   # launches of one call per timed graph


def time_graph(g, reps, warmup, per_replay):
    """Mean device time of one unit of a graph: `reps` replays bracketed by
    HIP events on the current stream (the stream the graph runs on), after
    `warmup` untimed replays; each replay holds `per_replay` units."""
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda._sleep(SLEEP_CYCLES)
    for i in range(reps):
        ev[i].record()
        g.replay()
    ev[-1].record()
    torch.cuda.synchronize()
    return statistics.fmean(ev[i].elapsed_time(ev[i + 1]) for i in range(reps)) / per_replay


def hbm_entry(ms, nbytes, ceiling_gbs=None):
    a = nbytes / (ms * 1e-3) / 1e9
    e = {"ms": ms, "bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": a / HBM_PEAK_GBS,
         "bytes": nbytes}
    if ceiling_gbs:
        e["ceiling"] = ceiling_gbs
        e["frac_of_ceiling"] = a / ceiling_gbs
    return e


def mfma_entry(ms, ops, peak):
    a = ops / (ms * 1e-3) / 1e12
    return {"ms": ms, "bound": "mfma", "achieved": a, "peak": peak, "unit": "TFLOP/s", "frac": a / peak, "ops": ops}


# ---------------------------------------------------------------- ceilings

def cold_buffers(nbytes, min_total=2 * INFINITY_CACHE, dev="cuda:0"):
    """Enough distinct buffers of `nbytes` that reading them in turn streams
    from HBM, not from the 256 MB Infinity Cache."""
    copies = max(2, -(-min_total // nbytes))
    return [torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(i & 0xff) for i in range(copies)]


def stream_ceiling(nbytes, args, bufs=None):
    """Best one-launch cold read of `nbytes` over a few launch shapes: ms and
    GB/s, with the per-shape times."""
    nbytes -= nbytes % 16
    if bufs is None:
        bufs = cold_buffers(nbytes)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    reps = max(8, args.steps // len(bufs))
    per = {}
    for wg in (256, 512, 1024, 2048, 4096, 8192):
        g = capture(lambda wg=wg: [bt.bitnet_calib_stream_read(b, nbytes, wg, sink=sink) for b in bufs])
        per[wg] = time_graph(g, reps, 1, len(bufs))
    best = min(per, key=per.get)
    return {"bytes": nbytes, "ms": per[best], "achieved": nbytes / (per[best] * 1e-3) / 1e9, "unit": "GB/s",
            "workgroups": best, "ms_by_workgroups": {str(k): v for k, v in per.items()},
            "copies_rotated": len(bufs), "kernel": "stream_read_kernel (bitnet_calib_stream_read)"}


def mfma_ceiling(kind, args):
    """Back-to-back MFMAs on random operands over the whole device; rate and
    the clock each workgroup measured (cycles / 100 MHz ticks)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs, iters = 4 * cus, 2048  # four 4-wave workgroups per CU: 4 waves per SIMD
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    clocks = torch.zeros(wgs, 2, dtype=torch.int64, device="cuda:0")
    ops = [0.0]

    def launch():
        _, ops[0] = bt.bitnet_calib_mfma(kind, wgs, iters, sink=sink, clocks=clocks)
    g = capture(launch)
    ms = time_graph(g, max(3, args.steps // 10), 2, 1)
    c = clocks.cpu().double()
    ghz = float((c[:, 0] / c[:, 1]).median()) * 0.1
    i8 = kind in (bt.BITNET_CALIB_MFMA_I8, bt.BITNET_CALIB_MFMA_I8_TERNARY)
    peak = INT8_PEAK_TOPS if i8 else BF16_PEAK_TFLOPS
    a = ops[0] / (ms * 1e-3) / 1e12
    operands = "random x ternary codes" if kind in (bt.BITNET_CALIB_MFMA_I8_TERNARY,
                                                   bt.BITNET_CALIB_MFMA_BF16_TERNARY) else "random x random"
    return {"kind": ("int8 v_mfma_i32_32x32x32_i8" if i8 else "bf16 v_mfma_f32_32x32x16_bf16") + ", " + operands,
            "ms": ms, "achieved": a, "unit": "TFLOP/s", "peak": peak, "frac": a / peak, "clock_ghz": ghz,
            "workgroups": wgs, "iters": iters}


def ceilings(args, sizes):
    out = {"stream_read": {}, "clock_note": "shader clock = cycle counter / 100 MHz real-time counter, "
                                            "median over the workgroups of the MFMA loop"}
    for label, nbytes in sizes.items():
        out["stream_read"][label] = stream_ceiling(nbytes, args)
    out["mfma_int8"] = mfma_ceiling(bt.BITNET_CALIB_MFMA_I8, args)
    out["mfma_int8_ternary"] = mfma_ceiling(bt.BITNET_CALIB_MFMA_I8_TERNARY, args)
    out["mfma_bf16"] = mfma_ceiling(bt.BITNET_CALIB_MFMA_BF16, args)
    out["mfma_bf16_ternary"] = mfma_ceiling(bt.BITNET_CALIB_MFMA_BF16_TERNARY, args)
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
        "ws_wq": torch.empty(max(16, bt.bitnet_workspace_bytes(bt.BITNET_OP_WEIGHT_QUANT, M, N, K)),
                             dtype=torch.uint8, device=dev),
        "Y": torch.empty(M, N, dtype=torch.float32, device=dev),
        "counts": torch.empty(4, dtype=torch.int64, device=dev),
        "ws_cc": torch.empty(bt.bitnet_workspace_bytes(bt.BITNET_OP_CODE_COUNTS, 0, N, K), dtype=torch.uint8,
                             device=dev),
        "W_packed_rows": torch.empty(N, K // 4, dtype=torch.uint8, device=dev),
        "gamma_rows": torch.empty(N, dtype=torch.float32, device=dev),
        "grad_s": torch.empty(N, dtype=torch.float32, device=dev),
        "ws_wqc": torch.empty(bt.bitnet_workspace_bytes(bt.BITNET_OP_WEIGHT_QUANT_COUNTED, 0, N, K),
                              dtype=torch.uint8, device=dev),
        "ws_wqr": torch.empty(bt.bitnet_workspace_bytes(bt.BITNET_OP_WEIGHT_QUANT_ROWS, 0, N, K), dtype=torch.uint8,
                              device=dev),
    }
    if gy is not None:
        buf["grad_x"] = torch.empty(M, K, dtype=torch.float32, device=dev)
        buf["grad_W"] = torch.empty(N, K, dtype=torch.float32, device=dev)
        buf["ws_bwd"] = torch.empty(max(16, bt.bitnet_workspace_bytes(bt.BITNET_OP_LINEAR_BWD_STE, M, N, K)),
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
        # weight quant counting its codes as it writes them: weight_quant's bytes plus the counts
        "weight_quant_counted": {"bytes": 2 * N * K * w_bytes + N * K // 4 + 4 + 32, "bound": "hbm"},
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
        # gradient of a learned per-channel scale: grad_W and the codes read once
        c["channel_scale_grad"] = {"bytes": 4 * N * K + N * K // 4 + 4 * N, "bound": "hbm"}
    for v in c.values():
        if "ops" in v:
            ridge = v["peak_ops"] * 1e12 / (HBM_PEAK_GBS * 1e9)
            v["bound"] = "mfma" if v["ops"] / v["bytes"] > ridge else "hbm"
    return c


KERNEL_OF = {
    "act_quant": "act_quant_rows_kernel (rows of whole 16-byte blocks), else act_quant_kernel",
    "weight_quant": "wq_row_abs_sum_kernel + wq_pack_kernel / wq_pack_pub_kernel (gamma in the pack launch)",
    "linear_fwd": "gemm_i8t2_kernel",
    "bwd_grad_x": "bwd_kernel<grad_x>",
    "bwd_grad_W": "bwd_kernel<grad_W> (+ split_reduce_kernel when split; xdeq_t_kernel first for a tall output)",
    "rmsnorm_bwd": "rmsnorm_bwd_kernel",
    "bwd_grad_W_gated": "bwd_kernel<grad_W> with the range gate (+ split_reduce_kernel when split; xdeq_t_kernel first for a tall output)",
    "weight_clamp": "weight_clamp_kernel",
    "code_counts": "code_counts_kernel + code_counts_final_kernel",
    "weight_quant_counted": "wq_row_abs_sum_kernel + the counting pack + counted_sum_kernel",
    "quant_operands": "wq_row_abs_sum_kernel + act_pack_kernel (more activation than weight bytes), "
                      "else quant_operands_kernel + wq_pack_kernel / wq_pack_pub_kernel",
    "weight_quant_rows": "wq_row_abs_sum_kernel (with the row gammas) + wq_pack_rows_kernel",
    "linear_fwd_channel": "gemm_i8t2_kernel (per-channel epilogue) or gemv_t2_kernel",
    "bwd_grad_x_channel": "bwd_kernel<grad_x> (per-channel code scales)",
    "channel_scale_grad": "channel_scale_grad_kernel",
}
# sources each call's kernels are built from: the HBM traffic recorded under
# profiles/ is used only while these files are unchanged
SOURCES_OF = {
    "act_quant": ["bit_ternary_quantized_amd/csrc/quant.hip"],
    "weight_quant": ["bit_ternary_quantized_amd/csrc/quant.hip"],
    "linear_fwd": ["bit_ternary_quantized_amd/csrc/gemm_i8.hip", "bit_ternary_quantized_amd/csrc/gemv.hip"],
    "bwd_grad_x": ["bit_ternary_quantized_amd/csrc/bwd.hip"],
    "bwd_grad_W": ["bit_ternary_quantized_amd/csrc/bwd.hip"],
    "linear_bwd_ste": ["bit_ternary_quantized_amd/csrc/bwd.hip"],
    "rmsnorm_bwd": ["bit_ternary_quantized_amd/csrc/norm_bwd.hip"],
    "bwd_grad_W_gated": ["bit_ternary_quantized_amd/csrc/bwd.hip"],
    "weight_clamp": ["bit_ternary_quantized_amd/csrc/quant.hip"],
    "code_counts": ["bit_ternary_quantized_amd/csrc/quant.hip"],
    "weight_quant_counted": ["bit_ternary_quantized_amd/csrc/quant.hip"],
    "quant_operands": ["bit_ternary_quantized_amd/csrc/quant.hip"],
    "weight_quant_rows": ["bit_ternary_quantized_amd/csrc/quant.hip"],
    "linear_fwd_channel": ["bit_ternary_quantized_amd/csrc/gemm_i8.hip", "bit_ternary_quantized_amd/csrc/gemv.hip"],
    "bwd_grad_x_channel": ["bit_ternary_quantized_amd/csrc/bwd.hip"],
    "decode_gemv": ["bit_ternary_quantized_amd/csrc/gemv.hip"],
    "channel_scale_grad": ["bit_ternary_quantized_amd/csrc/scale_grad.hip"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def source_digest(call):
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
    if entry["bound"] == "hbm":
        return hbm_entry(ms, entry["bytes"])
    return mfma_entry(ms, entry["ops"], entry["peak_ops"])


def cpu_baseline_layer(d, gy_present, budget_s=12.0):
    """The oracle on this host, on the first S tokens of the same layer: act
    quant of those S rows, weight quant of the whole W (a step needs it
    whatever the token count), the forward (and, for a training workload,
    the STE backward) over the S tokens.  S is sized from a short calibration
    run so that one sample takes about half the budget; the sample repeats
    until the budget is spent (at most three times) and the median counts.
    Rate = the GPU's algorithmic ops for S tokens / seconds."""
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

    S = min(M, 16)
    t = run(S)
    S = int(max(1, min(M, S * (budget_s / 2) / max(t, 1e-9))))
    times = []
    t_start = time.perf_counter()
    while not times or (time.perf_counter() - t_start < budget_s and len(times) < 3):
        times.append(run(S))
    ops = (2 + (4 if gy_present else 0)) * S * N * K
    sec = statistics.median(times)
    return {"value": ops / sec / 1e12, "unit": "TOPS", "cores": oracle.get_threads(), "cpu": cpu_model(),
            "kind": "oracle",
            "sample": f"first {S} of {M} tokens: act quant of those rows, weight quant of all of W, "
                      f"forward{' and STE backward' if gy_present else ''}; median of {len(times)} run(s) "
                      f"of {sec:.2f} s; ops counted as the GPU's ({'6' if gy_present else '2'}*S*N*K)",
            "seconds": sec}


def bench_layer(args, name):
    d, x, w, gy, b = setup_layer(name)
    M, N, K = d["M"], d["N"], d["K"]
    inputs = {"x": sha256(d["x"]), "w": sha256(d["w"])}
    if gy is not None:
        inputs["grad_y"] = sha256(d["gy"])
    calls = {
        "act_quant": lambda: bt.bitnet_act_quant(x, 1e-5, Xq=b["Xq"], scale_x=b["scale_x"]),
        "weight_quant": lambda: bt.bitnet_weight_quant(w, W_packed=b["W_packed"], gamma=b["gamma"],
                                                       workspace=b["ws_wq"]),
        # both quantizers in one call (one launch fewer; same outputs)
        "quant_operands": lambda: bt.bitnet_quant_operands(x, w, 1e-5, Xq=b["Xq"], scale_x=b["scale_x"],
                                                           W_packed=b["W_packed"], gamma=b["gamma"],
                                                           workspace=b["ws_wq"]),
        "linear_fwd": lambda: bt.bitnet_linear_fwd(b["Xq"], b["scale_x"], b["W_packed"], b["gamma"], Y=b["Y"]),
    }
    if gy is not None:
        calls["linear_bwd_ste"] = lambda: bt.bitnet_linear_bwd_ste(
            gy, b["Xq"], b["scale_x"], b["W_packed"], b["gamma"], grad_x=b["grad_x"], grad_W=b["grad_W"],
            workspace=b["ws_bwd"])
        # the backward call's two products, each timed on its own: grad_x is
        # one kernel, grad_W one kernel plus the ordered split reduction when
        # its token range is split
        calls["bwd_grad_x"] = lambda: bt.bitnet_linear_bwd_ste(
            gy, b["Xq"], b["scale_x"], b["W_packed"], b["gamma"], want_grad_W=False, grad_x=b["grad_x"])
        calls["bwd_grad_W"] = lambda: bt.bitnet_linear_bwd_ste(
            gy, b["Xq"], b["scale_x"], b["W_packed"], b["gamma"], want_grad_x=False, grad_W=b["grad_W"],
            workspace=b["ws_bwd"])
    variants = {
        "code_counts": lambda: bt.bitnet_code_counts(b["W_packed"], K, counts=b["counts"], workspace=b["ws_cc"]),
        # the weight quantizer with the counts made on the way (one pass fewer over the codes)
        "weight_quant_counted": lambda: bt.bitnet_weight_quant_counted(w, W_packed=b["W_packed"], gamma=b["gamma"],
                                                                       counts=b["counts"], workspace=b["ws_wqc"]),
        # per-output-channel variants (own buffers; not part of the step)
        "weight_quant_rows": lambda: bt.bitnet_weight_quant_rows(w, W_packed=b["W_packed_rows"], gamma=b["gamma_rows"],
                                                                 workspace=b["ws_wqr"]),
        "linear_fwd_channel": lambda: bt.bitnet_linear_fwd_channel(b["Xq"], b["scale_x"], b["W_packed_rows"],
                                                                   b["gamma_rows"], Y=b["Y"]),
    }
    if gy is not None:
        variants["bwd_grad_x_channel"] = lambda: bt.bitnet_linear_bwd_ste_channel(
            gy, b["Xq"], b["scale_x"], b["W_packed_rows"], b["gamma_rows"], want_grad_W=False, grad_x=b["grad_x"])
        # the gradient through the RMSNorm in front of the quantizer, from the
        # step's grad_x (timed on its own; not part of the step)
        variants["rmsnorm_bwd"] = lambda: bt.bitnet_rmsnorm_bwd(x, b["grad_x"], 1e-5, grad_X=b["grad_X"])
        # the STE variants: grad_W gated by the master weights in [-1, 1], and
        # the clamp of the master weights after an update
        variants["bwd_grad_W_gated"] = lambda: bt.bitnet_linear_bwd_ste_gated(
            gy, b["Xq"], b["scale_x"], b["W_packed"], b["gamma"], w, -1.0, 1.0, want_grad_x=False,
            grad_W=b["grad_W"], workspace=b["ws_bwd"])
        variants["weight_clamp"] = lambda: bt.bitnet_weight_clamp(b["w_clamp"], -1.0, 1.0)
        # the gradient of a learned per-channel scale from the step's grad_W
        variants["channel_scale_grad"] = lambda: bt.bitnet_channel_scale_grad(b["grad_W"], b["W_packed_rows"],
                                                                               grad_s=b["grad_s"])

    # --two-streams: the two quantizers (X and W), which are independent, run
    # on two streams (default priority) forked and joined with events, so the
    # graph holds parallel branches.  Measured faster at the 7B and 70B shapes
    # by 1-2.5% against the two calls in order, but not against the one
    # bitnet_quant_operands call the default step makes.
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

    def forward():
        if args.two_streams:
            fork_join(calls["act_quant"], calls["weight_quant"])
        else:
            calls["quant_operands"]()
        calls["linear_fwd"]()

    # the step: the forward (both quantizers in one call, then the product);
    # a training workload adds the backward call, timed as its own graph so
    # the forward's rate stays the forward's
    g_fwd = capture(forward)
    warmup_run = warm_up(g_fwd, args.warmup)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        g_fwd.replay()
    end.record()
    torch.cuda.synchronize()
    fwd_wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    fwd_ms = start.elapsed_time(end) / args.steps
    bwd_ms = None
    if gy is not None:
        g_bwd = capture(calls["linear_bwd_ste"])
        warm_up(g_bwd, args.warmup)
        bwd_ms = time_graph(g_bwd, args.steps, 0, 1)

    # per-call device time: each call captured REPS times back to back in
    # one graph; K replays of each, bracketed by HIP events on the stream
    # they run on.  A bounded spin first lets the host enqueue the whole loop,
    # so no host gap sits between two events.
    allc = dict(calls) if args.step_only else dict(calls, **variants)
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
    del g_rep

    counts = layer_counts(M, N, K, d["x"].element_size(), d["w"].element_size(), gy is not None)
    kernels = {n: rate(counts[n], per[n]) for n in timed}
    for n in kernels:
        kernels[n]["kernel"] = KERNEL_OF.get(n, n)
        # each call is replayed back to back: operands that fit in the 256 MB
        # Infinity Cache are then read from it, not from HBM
        kernels[n]["warm_cache"] = counts[n]["bytes"] < INFINITY_CACHE

    ceil = None
    if not args.no_ceilings:
        sizes = {"act_quant_x": M * K * d["x"].element_size()}
        ceil = ceilings(args, sizes)
        # the activation quantizer against a one-launch read of its input
        kernels["act_quant"]["ceiling_read_gbs"] = ceil["stream_read"]["act_quant_x"]["achieved"]
        # the products against back-to-back MFMAs on operands of their kind:
        # the forward and grad_x multiply by ternary codes, grad_W by
        # dequantized activations
        for n, c in (("linear_fwd", "mfma_int8_ternary"), ("bwd_grad_x", "mfma_bf16_ternary"),
                     ("bwd_grad_W", "mfma_bf16")):
            if n in kernels and kernels[n]["bound"] == "mfma":
                kernels[n]["ceiling"] = ceil[c]["achieved"]
                kernels[n]["frac_of_ceiling"] = kernels[n]["achieved"] / ceil[c]["achieved"]

    value = 2 * M * N * K / (fwd_ms * 1e-3) / 1e12
    # roofline: the forward's dominant kernel (the int8 GEMM at the
    # prefill and training shapes)
    roof = dict(kernels["linear_fwd"])
    roof["kernel"] = KERNEL_OF["linear_fwd"] + " (bitnet_linear_fwd)"
    roof["traffic"] = measured_traffic("linear_fwd", name)
    roof["per_launch"] = f"{M}x{N}x{K} int8 product, 2*M*N*K = {2 * M * N * K} ops per launch"
    if ceil is not None and roof["bound"] == "mfma":
        # the forward's operands are int8 activations and ternary codes
        c = ceil["mfma_int8_ternary"]
        roof["ceiling"] = c["achieved"]
        roof["frac_of_ceiling"] = roof["achieved"] / c["achieved"]
        roof["ceiling_clock_ghz"] = c["clock_ghz"]
    out = {
        "metric": METRIC, "value": value, "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "warmup_steps_run": warmup_run, "ms_per_step": fwd_ms,
        "host_ms_per_step": fwd_wall_ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8", "data": "synthetic",
        "config": {"workload": name, "M": M, "N": N, "K": K, "x_dtype": str(d["x"].dtype).split(".")[-1],
                   "w_dtype": str(d["w"].dtype).split(".")[-1],
                   "step": ("act_quant || weight_quant (two streams)" if args.two_streams else "quant_operands")
                   + " + linear_fwd (the forward)",
                   "value": "2*M*N*K int8 ops per forward step / step time",
                   "launch": "one HIP graph per step"},
        "roofline": roof,
    }
    if bwd_ms is not None:
        out["backward"] = {"ms": bwd_ms, "call": "linear_bwd_ste (grad_x and grad_W)",
                           **{k: v for k, v in mfma_entry(bwd_ms, 4 * M * N * K, BF16_PEAK_TFLOPS).items()
                              if k != "ms"}}
        out["config"]["backward"] = "linear_bwd_ste timed as its own graph; not in value"
        dom = max(("bwd_grad_x", "bwd_grad_W"), key=lambda n: per[n])
        out["backward"]["dominant"] = dom
        out["backward"]["dominant_traffic"] = measured_traffic(dom, name)
    if not args.no_decode and name == "prefill_7b":
        out["decode"] = {}
        for m in (1, 16):
            e = decode_gemv(args, m)[0]
            e.pop("inputs_sha256")
            out["decode"][f"M={m}"] = e
    out["kernels"] = kernels
    if ceil is not None:
        out["ceilings"] = ceil
    out["inputs"] = {"generator": "workloads.py (torch CPU generators; X seed 0, W 1, grad_y 2)", "sha256": inputs}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_layer(d, gy is not None)
    return out


# ------------------------------------------------------------------ decode

def decode_gemv(args, M):
    """The packed GEMV (bitnet_linear_fwd from q) at the 7B decode shape, with
    the weights rotated over enough copies that every launch reads them from
    HBM; and a one-launch cold streaming read of the same byte count."""
    d = workloads.workload("decode_7b", M=M)
    N, K = d["N"], d["K"]
    dev = "cuda:0"
    q, s, gm = d["q"].to(dev), d["scale_x"].to(dev), d["gamma"].to(dev)
    wp0 = bt.bitnet_pack_ternary(d["codes"].to(dev))
    copies = max(2, (2 * INFINITY_CACHE) // wp0.numel() + 1)
    wps = [wp0] + [wp0.clone() for _ in range(copies - 1)]
    Y = torch.empty(M, N, dtype=torch.float32, device=dev)
    g = capture(lambda: [bt.bitnet_linear_fwd(q, s, wp, gm, Y=Y) for wp in wps])
    reps = max(8, args.steps // copies * 4)
    ms = time_graph(g, reps, max(1, args.warmup // copies), copies)
    del g
    nbytes = N * K // 4 + M * K + 4 * M + 4 + 4 * M * N
    ceiling = None
    if not args.no_ceilings:
        ceiling = stream_ceiling(nbytes, args)
    e = hbm_entry(ms, nbytes, ceiling["achieved"] if ceiling else None)
    e["kernel"] = "gemv_row_kernel" if M == 1 and K % 64 == 0 and K <= 8192 else "gemv_t2_kernel"
    e["traffic"] = measured_traffic("decode_gemv", f"decode_7b_m{M}")
    e["config"] = {"M": M, "N": N, "K": K, "weight_copies": copies, "launches_timed": reps * copies,
                   "bytes": "N*K/4 packed weights + M*K q + 4*M scale_x + 4 gamma + 4*M*N Y"}
    if ceiling:
        e["ceiling_read"] = ceiling
    e["inputs_sha256"] = {"q": sha256(d["q"]), "codes": sha256(d["codes"]), "scale_x": sha256(d["scale_x"])}
    return e, (q, s, gm, wps, Y, d)


def bench_decode(args):
    """Packed GEMV at decode shape and the whole decode step from bf16 X (two
    calls, the fused call, the fused call on the decode layout)."""
    M = args.decode_m
    e, (q, s, gm, wps, Y, d) = decode_gemv(args, M)
    N, K = d["N"], d["K"]
    dev = "cuda:0"
    copies = len(wps)
    reps = max(8, args.steps // copies * 4)
    x = d["x"].to(dev)
    q2, s2 = torch.empty_like(q), torch.empty_like(s)

    def per_launch_ms(fn, weights=wps):
        gr = capture(lambda: [fn(wp) for wp in weights])
        return time_graph(gr, reps, max(1, args.warmup // copies), copies)

    # algorithmic bytes of a decode step: x (bf16) and the packed weights in, Y out
    step_bytes = N * K // 4 + 2 * M * K + 4 + 4 * M * N
    kernels = {"linear_fwd": {k: v for k, v in e.items() if k not in ("ceiling_read", "inputs_sha256")}}
    kernels["act_quant+linear_fwd"] = hbm_entry(per_launch_ms(lambda wp: (
        bt.bitnet_act_quant(x, 1e-5, Xq=q2, scale_x=s2), bt.bitnet_linear_fwd(q2, s2, wp, gm, Y=Y))), step_bytes)
    kernels["linear_fwd_decode"] = hbm_entry(
        per_launch_ms(lambda wp: bt.bitnet_linear_fwd_decode(x, wp, gm, 1e-5, Y=Y)), step_bytes)
    if K == 4096:  # the same call on the weights in the decode layout (repacked once, untimed)
        wds = [bt.bitnet_pack_decode(wp) for wp in wps]
        kernels["linear_fwd_decode@decode_layout"] = hbm_entry(
            per_launch_ms(lambda wd: bt.bitnet_linear_fwd_decode(x, wd, gm, 1e-5, Y=Y, N=N), wds), step_bytes)
    out = {
        "metric": METRIC, "value": e["achieved"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": e["ms"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "i8", "data": "synthetic",
        "config": {"workload": "decode_7b", **e["config"]},
        "roofline": {k: e[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic", "kernel")},
        "kernels": kernels,
        "inputs": {"sha256": e["inputs_sha256"]},
    }
    if "ceiling_read" in e:
        out["roofline"]["ceiling"] = e["ceiling"]
        out["roofline"]["frac_of_ceiling"] = e["frac_of_ceiling"]
        out["ceilings"] = {"stream_read": {"decode_bytes": e["ceiling_read"]}}
    if not args.no_cpu_baseline:
        import oracle
        qh, ch = d["q"].numpy(), d["codes"].numpy()
        t = time.perf_counter()
        oracle.gemm_i32(qh, ch)
        sec = time.perf_counter() - t
        nbytes = e["bytes"]
        out["cpu_baseline"] = {"value": nbytes / sec / 1e9, "unit": "GB/s", "cores": oracle.get_threads(),
                               "cpu": cpu_model(), "kind": "oracle",
                               "sample": f"whole GEMV (M={M}) once, {sec:.2f} s"}
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


def config_summary(args, name):
    """The step of another configuration, compactly: the forward (both
    quantizers in one call, then the product) and, for a training
    configuration, the STE backward, each as its own graph, and the step's
    calls one by one."""
    sub = argparse.Namespace(**vars(args))
    sub.step_only, sub.no_ceilings, sub.no_cpu_baseline, sub.no_decode, sub.two_streams = True, True, True, True, False
    sub.steps, sub.warmup = max(5, args.steps // 5), max(2, args.warmup // 5)
    r = bench_layer(sub, name)
    c = r["config"]
    out = {"M": c["M"], "N": c["N"], "K": c["K"], "x_dtype": c["x_dtype"], "w_dtype": c["w_dtype"],
           "forward_us": r["ms_per_step"] * 1e3, "forward_int8_tops": r["value"],
           "gemm": {k: r["roofline"][k] for k in ("ms", "bound", "achieved", "unit", "frac")}}
    if "backward" in r:
        b = r["backward"]
        out["backward_us"] = b["ms"] * 1e3
        out["backward_bf16_tflops"] = b["achieved"]
        out["backward_frac"] = b["frac"]
        out["step_us"] = (r["ms_per_step"] + b["ms"]) * 1e3
    out["calls_us"] = {n: e["ms"] * 1e3 for n, e in r["kernels"].items()}
    out["inputs_sha256"] = r["inputs"]["sha256"]
    return out


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
        if args.workload == "prefill_7b" and not args.no_configs:
            # the other layer configurations of the same job, compactly (their
            # parity is in the tests; these are their timings on this device)
            out["configs"] = {}
            for name in ("tiny", "small_llama", "qat_70b_mlp"):
                out["configs"][name] = config_summary(args, name)
                torch.cuda.empty_cache()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
