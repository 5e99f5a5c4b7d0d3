"""Benchmark of the W8A8 FP8 block-scaled linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_qkv]
                    [--no-cpu-baseline] [--no-others] [--traffic-file PATH]

A step is one pass of the hot path over one batch: dynamic per-token group-128
activation quantization of the BF16 input, then the block-scaled FP8 GEMM
(weights were block-quantized once, untimed, as the offline step they are).
The headline workload is the decode fused-QKV projection (M=1, K=7168, N=9216),
whose metric is achieved GB/s: its weight stream is 99.9% of its bytes.  Inputs
are resident in HBM before timing; weight copies are rotated so that the weights
touched between two uses of one copy exceed twice the 256 MB Infinity Cache.

Timing: W untimed warm-up steps, then K steps bracketed by device synchronization,
run as one replay of a HIP graph holding the K steps (the host's launch cost stays
out of the device timeline).  The dominant kernel (the GEMM) is also captured
alone, K launches, and replayed between HIP events on the stream it runs on,
giving its average duration for the roofline.

Printed: ONE JSON line.  Besides the contract fields it carries the other
workloads' numbers ("workloads"), measured the same way, and those of the NVFP4
weight-only linear ("w4a16": one nvfp4_w4a16_linear launch per step, graph-timed,
weights rotated over copies like the FP8 weights).  ``--workload w4a16_...`` times
one NVFP4 workload alone.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA
MALL_BYTES = 256 << 20         # Infinity Cache
METRIC = "FP8 block-GEMM TFLOP/s (prefill) and GB/s (decode M=1..8), % of roofline"
# Sources each GEMM kernel's HBM traffic depends on: a committed counter reading is
# used only while these files are unchanged.
KERNEL_SOURCES = {
    "decode": ["gemm_decode.hip", "launch.h", "device_common.h", "api.hip"],
    "mid": ["gemm_mid.hip", "launch.h", "device_common.h", "api.hip"],
    "prefill": ["gemm_prefill.hip", "splitk.hip", "launch.h", "device_common.h", "api.hip"],
    "w4a16": ["w4a16.hip", "splitk.hip", "launch.h", "device_common.h", "api.hip"],
}
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense BF16 MFMA
W4_METRIC = "NVFP4 W4A16 linear: GB/s (decode, M<=64) and TFLOP/s (M>64), % of roofline"
DECODE_MAX_M = 16               # block_linear takes the decode kernel for M <= 16,
MID_MAX_M = 64                  # the mid-size kernel for M <= 64, else the prefill tiles


def gemm_kind(M):
    return "decode" if M <= DECODE_MAX_M else ("mid" if M <= MID_MAX_M else "prefill")


def kernel_kind(wl):
    """Source set of the kernel that runs workload ``wl``."""
    from synth import W4A16_WORKLOADS
    return "w4a16" if wl.name in W4A16_WORKLOADS else gemm_kind(wl.M)


def kernel_source_hash(kind):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "fp8_block_scaled_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode_qkv")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-others", action="store_true", help="skip the other workloads")
    p.add_argument("--no-ceilings", action="store_true", help="skip the measured stream-read and MFMA ceilings")
    p.add_argument("--traffic-file", default=os.path.join(ROOT, "profiles", "traffic.json"))
    p.add_argument("--make-traffic", metavar="DIR",
                   help="write --traffic-file from rocprofv3 FETCH_SIZE/WRITE_SIZE runs under DIR "
                        "(DIR/<workload>/{fetch,write}, DIR/copy/{fetch,write})")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain 512 MiB device copy, 10 times (reference for HBM byte counters)")
    p.add_argument("--summarize", metavar="DIR",
                   help="print a per-kernel summary of the rocprofv3 CSV output under DIR and exit")
    return p.parse_args()


def dev_bf16(bits):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


class Case:
    """Device-resident inputs and preallocated outputs of one linear workload."""

    def __init__(self, wl, x_bits=None, gu_dev=None):
        import torch
        import fp8_block_scaled_amd as fb
        import synth
        self.wl = wl
        M, K, N = wl.M, wl.K, wl.N
        wbytes = N * K
        self.copies = max(1, min(16, -(-2 * MALL_BYTES // wbytes)))
        w = synth.make_weight(wl)
        wd = dev_bf16(w)
        qw, ws = fb.quant_weight(wd)
        del wd
        self.qw = [qw] + [qw.clone() for _ in range(self.copies - 1)]
        self.ws = [ws] + [ws.clone() for _ in range(self.copies - 1)]
        if gu_dev is not None:        # down projection: its input is SiLU(gate)*up of the gate/up output
            self.gu = gu_dev
            self.x = None
        else:
            self.x = dev_bf16(x_bits if x_bits is not None else synth.make_activation(wl))
            self.gu = None
        self.q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
        self.s = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
        self.y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        need = fb.workspace_size(M, N, K)
        self.workspace = fb.get_workspace("cuda", need) if need else None
        torch.cuda.synchronize()

    def quant(self):
        import fp8_block_scaled_amd as fb
        if self.gu is not None:
            fb.silu_mul_quant(self.gu, self.q, self.s)
        else:
            fb.quant_act(self.x, self.q, self.s)

    def gemm(self, i):
        import fp8_block_scaled_amd as fb
        c = i % self.copies
        fb.block_linear(self.q, self.s, self.qw[c], self.ws[c], out=self.y, workspace=self.workspace)


def gate_up_output():
    """The gate/up projection's output on the GPU, BF16 [8, 16384]: the spec_mlp_gu
    workload's activations quantized and multiplied by its block-quantized weights.
    The down projection's input is SiLU(gate)*up of this tensor, as in the model."""
    import torch
    import fp8_block_scaled_amd as fb
    import synth
    from synth import WORKLOADS
    gw = WORKLOADS["spec_mlp_gu"]
    q, s = fb.quant_act(dev_bf16(synth.make_activation(gw)))
    wd = dev_bf16(synth.make_weight(gw))
    qw, ws = fb.quant_weight(wd)
    del wd
    gu = fb.block_linear(q, s, qw, ws)
    torch.cuda.synchronize()
    del q, s, qw, ws
    return gu


def make_case(wl):
    """A Case for workload ``wl``; the down projection takes SiLU(gate)*up of the
    gate/up projection's GPU output."""
    if wl.x_kind == "silu":
        return Case(wl, gu_dev=gate_up_output())
    return Case(wl)


def _replay_ms(graph):
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def time_case(case, steps, warmup):
    """W eager warm-up steps, then K steps timed as one replay of a HIP graph that
    holds them (so host launch cost is not in the measurement).  The GEMM and the
    quantizer are also captured alone, K launches each, for their average duration
    on the stream they run on.  Returns (ms per step, GEMM us, quant us)."""
    import torch
    for i in range(warmup):
        case.quant()
        case.gemm(i)
    torch.cuda.synchronize()
    g_step, g_gemm, g_quant = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_step):
        for i in range(steps):
            case.quant()
            case.gemm(i)
    with torch.cuda.graph(g_gemm):
        for i in range(steps):
            case.gemm(i)
    with torch.cuda.graph(g_quant):
        for i in range(steps):
            case.quant()
    for g in (g_step, g_gemm, g_quant):     # untimed replay: first-replay costs
        g.replay()
    torch.cuda.synchronize()
    ms_step = _replay_ms(g_step) / steps
    gemm_us = _replay_ms(g_gemm) * 1e3 / steps
    quant_us = _replay_ms(g_quant) * 1e3 / steps
    del g_step, g_gemm, g_quant
    return ms_step, gemm_us, quant_us


def time_rmsnorm_quant(wl, steps):
    """Average duration of fp8_rmsnorm_quant on the workload's activations (graph-timed)
    and its HBM roofline: read x and gamma, write codes and scales."""
    import numpy as np
    import torch
    import fp8_block_scaled_amd as fb
    import synth
    from synth.gen import f32_to_bf16_bits
    M, K = wl.M, wl.K
    x = torch.from_numpy(synth.make_activation(wl).view(np.int16)).cuda()
    g = synth.bf16_normal(1, K, 0.1, wl.seed, synth.TID_GAMMA)[0]
    g = f32_to_bf16_bits(((g.astype(np.uint32) << 16).view(np.float32) + 1.0).astype(np.float32))
    g = torch.from_numpy(g.view(np.int16)).cuda()
    q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    s = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
    for _ in range(3):
        fb.rmsnorm_quant(x, g, 1e-5, q, s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(steps):
            fb.rmsnorm_quant(x, g, 1e-5, q, s)
    graph.replay()
    us = _replay_ms(graph) * 1e3 / steps
    nbytes = 2 * M * K + 2 * K + M * K + 4 * M * (K // 128)
    achieved = nbytes / (us * 1e-6) / 1e9
    return {"M": M, "K": K, "us": round(us, 2),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4)}}


def time_silu_mul_quant(M, I, steps):
    """Average duration of fp8_silu_mul_quant on [gate | up] BF16 [M, 2I] ~ N(0, 1.7^2)
    (the gate/up GEMM's output scale) and its HBM roofline: read gate and up, write
    codes and scales."""
    import numpy as np
    import torch
    import fp8_block_scaled_amd as fb
    import synth
    gu = torch.from_numpy(synth.bf16_normal(M, 2 * I, 1.7, 0, synth.TID_GU).view(np.int16)).cuda()
    q = torch.empty((M, I), dtype=torch.uint8, device="cuda")
    s = torch.empty((M, I // 128), dtype=torch.float32, device="cuda")
    gu = gu.view(torch.bfloat16)
    for _ in range(3):
        fb.silu_mul_quant(gu, q, s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(steps):
            fb.silu_mul_quant(gu, q, s)
    graph.replay()
    us = _replay_ms(graph) * 1e3 / steps
    nbytes = 4 * M * I + M * I + 4 * M * (I // 128)
    achieved = nbytes / (us * 1e-6) / 1e9
    return {"M": M, "I": I, "us": round(us, 2),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4)}}


def time_m_sweep(Ms=(32, 64, 128, 512, 2048), N=7168, K=7168, copies=8, steps=40):
    """block_linear on the o_proj shape (N = K = 7168) for row counts between the
    decode and the prefill workloads: batched decode and chunked prefill.  Weights
    from the prefill_oproj generator, rotated over `copies` copies."""
    import numpy as np
    import torch
    import fp8_block_scaled_amd as fb
    import synth
    wl = synth.WORKLOADS["prefill_oproj"]
    w = torch.from_numpy(synth.make_weight(wl).view(np.int16)).cuda()
    qw, ws = fb.quant_weight(w)
    del w
    sets = [(qw, ws)] + [(qw.clone(), ws.clone()) for _ in range(copies - 1)]
    out = {}
    for M in Ms:
        x = torch.from_numpy(synth.activation_rows(wl, np.arange(M)).view(np.int16)).cuda()
        q, s = fb.quant_act(x)
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        for i in range(3):
            fb.block_linear(q, s, *sets[i % copies], out=y)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(steps):
                fb.block_linear(q, s, *sets[i % copies], out=y)
        graph.replay()
        us = _replay_ms(graph) * 1e3 / steps
        nbytes = N * K + 4 * (N // 128) * (K // 128) + M * K + 4 * M * (K // 128) + 2 * M * N
        # the binding passes a workspace when the size query asks for one: then the
        # call runs split-K prefill tiles whatever M is
        kind = "prefill split-K" if fb.workspace_size(M, N, K) > 0 else gemm_kind(M)
        out[str(M)] = {"kernel": kind, "us": round(us, 2),
                       "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                       "TFLOP/s": round(2 * M * N * K / (us * 1e-6) / 1e12, 1)}
        del graph, x, q, s, y
    return out


class W4Case:
    """Device-resident inputs of one NVFP4 W4A16 workload: packed codes and group scales
    (rotated over copies so that the weights touched between two uses of one copy exceed
    twice the Infinity Cache), BF16 activations, a preallocated output."""

    def __init__(self, wl):
        import numpy as np
        import torch
        import synth
        self.wl = wl
        w4, bs, g = synth.w4a16_weight(wl)
        wbytes = w4.nbytes + bs.nbytes
        self.copies = max(1, min(16, -(-2 * MALL_BYTES // wbytes)))
        self.w4 = [torch.from_numpy(w4).cuda()]
        self.bs = [torch.from_numpy(bs).cuda()]
        for _ in range(self.copies - 1):
            self.w4.append(self.w4[0].clone())
            self.bs.append(self.bs[0].clone())
        self.g = float(g)
        self.x = dev_bf16(synth.w4a16_activation_rows(wl, np.arange(wl.M)))
        self.y = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()

    def gemm(self, i):
        import fp8_block_scaled_amd as fb
        c = i % self.copies
        fb.nvfp4_linear(self.x, self.w4[c], self.bs[c], self.g, out=self.y)


def time_w4(case, steps, warmup):
    """Average duration of nvfp4_w4a16_linear: K launches captured in a HIP graph and
    replayed between events on the stream they run on."""
    import torch
    for i in range(warmup):
        case.gemm(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            case.gemm(i)
    graph.replay()
    torch.cuda.synchronize()
    us = _replay_ms(graph) * 1e3 / steps
    del graph
    return us


def w4_roofline(wl, us, traffic):
    """Weight streaming (M <= 64) against HBM, larger M against the dense BF16 MFMA peak."""
    if wl.M <= 64:
        achieved = wl.gemm_bytes() / (us * 1e-6) / 1e9
        r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = wl.gemm_flops() / (us * 1e-6) / 1e12
        r = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
    r["traffic"] = traffic
    return r


def time_w4_all(steps, traffic_file, names=None):
    """Every NVFP4 W4A16 workload (or the named ones): duration, rates and roofline."""
    import torch
    from synth import W4A16_WORKLOADS
    out = {}
    for name in names or W4A16_WORKLOADS:
        wl = W4A16_WORKLOADS[name]
        print(f"[bench] {name}: setup", file=sys.stderr, flush=True)
        case = W4Case(wl)
        us = time_w4(case, max(5, min(steps, 50 if wl.M > 64 else steps)), 3)
        out[name] = {"M": wl.M, "K": wl.K, "N": wl.N, "us": round(us, 2),
                     "GB/s": round(wl.gemm_bytes() / (us * 1e-6) / 1e9, 1),
                     "TFLOP/s": round(wl.gemm_flops() / (us * 1e-6) / 1e12, 1),
                     "roofline": w4_roofline(wl, us, load_traffic(traffic_file, wl)),
                     "weight_copies_rotated": case.copies}
        del case
        torch.cuda.empty_cache()
    return out


def roofline_for(wl, gemm_us, traffic):
    if wl.M <= 16:
        achieved = wl.gemm_bytes() / (gemm_us * 1e-6) / 1e9
        r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = wl.gemm_flops() / (gemm_us * 1e-6) / 1e12
        r = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": round(achieved / FP8_PEAK_TFLOPS, 4)}
    r["traffic"] = traffic
    return r


def load_traffic(path, wl):
    """HBM bytes per GEMM dispatch from committed rocprofv3 counter runs, or None when
    absent or taken on different kernel sources."""
    try:
        with open(path) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    ent = t.get("workloads", {}).get(wl.name)
    if not ent or ent.get("kernel_source_hash") != kernel_source_hash(kernel_kind(wl)):
        return None
    return ent.get("bytes_per_dispatch")


def _counter_means(directory, name_filter):
    """{(kernel name, grid): {counter: mean value}} over rocprofv3 counter CSVs, for the
    kernels whose names contain one of the substrings ``name_filter``."""
    if isinstance(name_filter, str):
        name_filter = (name_filter,)
    import csv
    import glob
    from collections import defaultdict
    acc = defaultdict(lambda: defaultdict(list))
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if any(f in r["Kernel_Name"] for f in name_filter):
                    acc[(r["Kernel_Name"], r["Grid_Size"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    # Setup work (e.g. the gate/up GEMM whose output feeds the down projection) runs once;
    # the timed call's kernels run at every step: keep the kernels dispatched at least
    # half as often as the most frequent one.
    counts = {k: max(len(v) for v in d.values()) for k, d in acc.items()}
    top = max(counts.values(), default=0)
    return {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in acc.items() if counts[k] * 2 >= top}


def make_traffic(directory, out_path):
    """HBM bytes per GEMM call = FETCH_SIZE and WRITE_SIZE (KiB per dispatch, summed over
    the kernels of one call), each scaled by what that counter reads for a plain device
    copy of known size."""
    from synth import WORKLOADS

    def one(d, what, counter):
        m = _counter_means(d, what)
        if len(m) != 1:
            raise SystemExit(f"{d}: expected one {what!r} kernel/grid, found {sorted(m)}")
        (key, vals), = m.items()
        return key, vals[counter]

    copy_bytes = 512 << 20
    _, copy_fetch = one(os.path.join(directory, "copy", "fetch"), "copyBuffer", "FETCH_SIZE")
    _, copy_write = one(os.path.join(directory, "copy", "write"), "copyBuffer", "WRITE_SIZE")
    f_fac, w_fac = copy_bytes / (copy_fetch * 1024), copy_bytes / (copy_write * 1024)
    doc = {"method": ("rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE, on bench.py --workload W "
                      "--no-others, kernels matching gemm_ (w4a16_ for the NVFP4 workloads) or splitk_reduce; KiB per "
                      "dispatch x 1024 x the factor that maps the same counter onto a 512 MiB device "
                      "copy's bytes"),
           "copy_factor": {"FETCH_SIZE": round(f_fac, 4), "WRITE_SIZE": round(w_fac, 4)},
           "workloads": {}}
    from synth import W4A16_WORKLOADS
    for name, wl in list(WORKLOADS.items()) + list(W4A16_WORKLOADS.items()):
        d = os.path.join(directory, name)
        if not os.path.isdir(d):
            continue
        filt = ("w4a16_" if name in W4A16_WORKLOADS else "gemm_", "splitk_reduce")
        # One call may launch several kernels (a split-K tile and its reduce):
        # the call's bytes are the sum over them, the dominant one names the entry.
        fm = _counter_means(os.path.join(d, "fetch"), filt)
        wm = _counter_means(os.path.join(d, "write"), filt)
        if not fm or set(fm) != set(wm):
            raise SystemExit(f"{d}: fetch/write kernels differ: {sorted(fm)} vs {sorted(wm)}")
        fetch = sum(v["FETCH_SIZE"] for v in fm.values())
        write = sum(v["WRITE_SIZE"] for v in wm.values())
        kf = max(fm, key=lambda k: fm[k]["FETCH_SIZE"])
        total = fetch * 1024 * f_fac + write * 1024 * w_fac
        doc["workloads"][name] = {
            "kernel": kf[0], "grid": int(kf[1]), "kernel_source_hash": kernel_source_hash(kernel_kind(wl)),
            "fetch_kib": round(fetch, 1), "write_kib": round(write, 1),
            "bytes_per_dispatch": int(round(total)), "algorithmic_bytes": wl.gemm_bytes(),
            "ratio_to_algorithmic": round(total / wl.gemm_bytes(), 3)}
        if len(fm) > 1:
            doc["workloads"][name]["kernels_per_call"] = sorted(k[0] for k in fm)
    # Workloads not measured in this run keep their earlier entries (each entry's bytes
    # are already scaled by the copy factor of its own run).
    try:
        with open(out_path) as fh:
            old = json.load(fh).get("workloads", {})
    except (OSError, ValueError):
        old = {}
    for name, ent in old.items():
        doc["workloads"].setdefault(name, ent)
    with open(out_path, "w") as fh:
        json.dump(doc, fh, indent=1)
        fh.write("\n")
    print(json.dumps(doc, indent=1))


_CEIL = None


def ceil_lib():
    """libfp8bs_ceilings.so: the measurement kernels (stream read, MFMA loop, clock)."""
    global _CEIL
    if _CEIL is None:
        import ctypes
        path = os.path.join(ROOT, "fp8_block_scaled_amd", "libfp8bs_ceilings.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m fp8_block_scaled_amd.build`")
        lib = ctypes.CDLL(path)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.fp8bs_ceil_stream_read.argtypes = [P, I64, P, I, I, I, I, P]
        lib.fp8bs_ceil_stream_read.restype = I
        lib.fp8bs_ceil_mfma.argtypes = [I, I, I, P, P, P]
        lib.fp8bs_ceil_mfma.restype = I
        lib.fp8bs_ceil_wallclock_khz.argtypes = []
        lib.fp8bs_ceil_wallclock_khz.restype = I
        _CEIL = lib
    return _CEIL


STREAM_CONFIGS = [(wgs, threads, unroll, nt) for wgs in (256, 512, 1024, 2048) for threads in (256, 512, 1024)
                  for unroll in (4, 8) for nt in (0, 1)]


def stream_ceiling(nbytes, copies, steps=100):
    """The best rate of a plain streaming read of ``nbytes`` (each launch reads one of
    ``copies`` buffers in turn, so the Infinity Cache cannot serve them), over the
    launch shapes of STREAM_CONFIGS, graph-timed like the GEMMs.  The read kernel
    moves exactly ``nbytes`` per launch."""
    import torch
    lib = ceil_lib()
    n = (nbytes + 15) // 16 * 16
    bufs = [torch.ones(n, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    sink = torch.empty(2048 * 1024, dtype=torch.int32, device="cuda")
    best = None
    for cfg in STREAM_CONFIGS:
        def launch(i):
            rc = lib.fp8bs_ceil_stream_read(bufs[i % copies].data_ptr(), n, sink.data_ptr(), *cfg,
                                            torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise RuntimeError(f"stream read launch failed ({rc})")
        for i in range(3):
            launch(i)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(steps):
                launch(i)
        graph.replay()
        us = _replay_ms(graph) * 1e3 / steps
        del graph
        if best is None or us < best[0]:
            best = (us, cfg)
    del bufs, sink
    torch.cuda.empty_cache()
    us, (wgs, threads, unroll, nt) = best
    return {"bytes": n, "us": round(us, 2), "GB/s": round(n / (us * 1e-6) / 1e9, 1), "copies_rotated": copies,
            "launch": {"workgroups": wgs, "threads": threads, "loads_in_flight_per_lane": unroll,
                       "nontemporal": bool(nt)}}


def mfma_ceiling(promote, wgs=512, iters=2000):
    """FP8 MFMA rate of a register-only loop (8 chains of v_mfma_f32_16x16x128_f8f6f4
    per wave, 2 waves per SIMD), and the shader clock it ran at (s_memtime over
    s_memrealtime).  With ``promote`` every MFMA starts from zero and is folded into
    FP32 accumulators by four FMAs, the GEMM's promotion per K block."""
    import torch
    lib = ceil_lib()
    out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    clk = torch.zeros(2, dtype=torch.int64, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    for _ in range(2):
        if lib.fp8bs_ceil_mfma(wgs, iters, int(promote), out.data_ptr(), clk.data_ptr(), st) != 0:
            raise RuntimeError("MFMA loop launch failed")
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        lib.fp8bs_ceil_mfma(wgs, iters, int(promote), out.data_ptr(), clk.data_ptr(), st)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    flops = wgs * 4 * iters * 8 * 65536
    ticks, real = (int(v) for v in clk.cpu().tolist())
    khz = lib.fp8bs_ceil_wallclock_khz()
    clock_ghz = ticks / (real / (khz * 1e3)) / 1e9 if real > 0 and khz > 0 else None
    tflops = flops / (us * 1e-6) / 1e12
    r = {"TFLOP/s": round(tflops, 1), "us": round(us, 1), "flop": flops,
         "shader_clock_GHz": round(clock_ghz, 3) if clock_ghz else None,
         "frac_of_5000": round(tflops / FP8_PEAK_TFLOPS, 4)}
    if clock_ghz:
        # Dense FP8 peak at the clock observed: 256 CUs x 8192 flop per clock.
        r["peak_at_observed_clock_TFLOP/s"] = round(256 * 8192 * clock_ghz * 1e9 / 1e12, 1)
    return r


def smi_snapshot():
    """amd-smi's clock and power readings for GPU 0 at this moment (None if unavailable)."""
    import subprocess
    try:
        p = subprocess.run(["amd-smi", "metric", "-g", "0", "--clock", "--power", "--json"],
                           capture_output=True, text=True, timeout=30)
        if p.returncode != 0:
            return None
        d = json.loads(p.stdout)
    except Exception:
        return None
    d = d[0] if isinstance(d, list) and d else d
    if isinstance(d, dict) and "gpu_data" in d:
        d = d["gpu_data"][0] if d["gpu_data"] else d
    out = {}
    pw = d.get("power", {}) if isinstance(d, dict) else {}
    for k in ("socket_power", "current_socket_power", "average_socket_power"):
        if isinstance(pw.get(k), dict) and "value" in pw[k]:
            out["power_W"] = pw[k]["value"]
            break
    ck = d.get("clock", {}) if isinstance(d, dict) else {}
    for k in ("gfx_0", "GFX_0", "gfx"):
        if isinstance(ck.get(k), dict):
            c = ck[k].get("clk", ck[k])
            out["gfx_clock_MHz"] = c.get("value") if isinstance(c, dict) else c
            break
    mem = ck.get("mem_0") if isinstance(ck, dict) else None
    if isinstance(mem, dict):
        c = mem.get("clk", mem)
        out["mem_clock_MHz"] = c.get("value") if isinstance(c, dict) else c
    return out or None


def cpu_env():
    """Host cores this process may use, the CPU model, and the BLAS thread count the
    oracle's float64 matmul is given: the cores, capped at 16 (one GPU's share of the
    host), set explicitly through threadpoolctl and recorded."""
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    blas = max(1, min(16, cores))
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cores": cores, "blas_threads": blas, "cpu_model": model}


def _timing_weights(wl):
    """Weight codes and block scales of ``wl``'s shape for timing the oracle: codes drawn
    uniformly over the finite E4M3 bytes, scales over [1e-4, 1e-3).  The weights'
    block quantization is the offline step (untimed on both sides), and the oracle's
    dequantize-and-matmul costs the same for any values."""
    import numpy as np
    rng = np.random.default_rng(wl.seed)
    qw = rng.integers(0, 256, (wl.N, wl.K), dtype=np.uint8)
    qw[(qw & 0x7F) == 0x7F] ^= 1                  # no NaN codes
    ws = rng.uniform(1e-4, 1e-3, (wl.N // 128, wl.K // 128)).astype(np.float32)
    return qw, ws


def _oracle_step(wl, rows, qw, ws):
    """One pass of the oracle over ``rows`` of workload ``wl``: quantize the rows'
    activations (the down projection: SiLU(gate)*up of a gate/up tensor of N(0, 1.7^2),
    then quantize) and dequantize-and-multiply in float64.  Returns seconds."""
    import oracle
    import synth
    from synth import WORKLOADS
    if wl.x_kind == "silu":
        gw = WORKLOADS["spec_mlp_gu"]
        gu = synth.bf16_normal(len(rows), gw.N, 1.7, gw.seed, synth.TID_GU)
        x = None
    else:
        x = synth.activation_rows(wl, rows)
    t0 = time.perf_counter()
    q, s = oracle.silu_mul_quant(gu) if x is None else oracle.quant_act(x)
    oracle.linear_ref(q, s, qw, ws)
    return time.perf_counter() - t0


def cpu_baseline_per_config(env):
    """The oracle on every workload: in full for the decode shapes, on a few hundred
    rows for the prefill shapes, with a labelled linear extrapolation t(M) = a + b M
    fitted from two row counts (256 and 1024) (the weights are dequantized once per call, a fixed
    cost; quantization and the matmul grow with the rows)."""
    import numpy as np
    from synth import WORKLOADS
    out = {}
    for name in ("tiny", "decode_qkv", "spec_mlp_gu", "spec_mlp_down", "prefill_oproj", "fusion_fc"):
        wl = WORKLOADS[name]
        print(f"[bench] cpu baseline (oracle): {name}", file=sys.stderr, flush=True)
        qw, ws = _timing_weights(wl)
        if wl.M <= 16:
            reps = 3 if wl.M * wl.N * wl.K < 1e9 else 1
            t = min(_oracle_step(wl, np.arange(wl.M), qw, ws) for _ in range(reps))
            out[name] = {"rows": wl.M, "s": round(t, 4), "GB/s": round((wl.quant_bytes() + wl.gemm_bytes()) / t / 1e9, 4),
                         "GFLOP/s": round(wl.gemm_flops() / t / 1e9, 2), "timed": "full call"}
        else:
            # Row counts far enough apart that the matmul's growth stands well above the
            # run-to-run spread of the fixed weight dequantization (at 64 and 256 rows the
            # two times of prefill_oproj came out equal); best of two calls each.
            r1, r2 = 256, 1024
            _oracle_step(wl, np.arange(16), qw, ws)          # untimed: first-touch costs
            t1 = min(_oracle_step(wl, np.arange(r1), qw, ws) for _ in range(2))
            t2 = min(_oracle_step(wl, np.arange(r2), qw, ws) for _ in range(2))
            b = max((t2 - t1) / (r2 - r1), 1e-12)
            a = max(t1 - b * r1, 0.0)
            full = a + b * wl.M
            out[name] = {"rows": [r1, r2], "s": [round(t1, 4), round(t2, 4)],
                         "s_per_row": round(b, 6), "fixed_s": round(a, 4),
                         "extrapolated_full_M_s": round(full, 2),
                         "extrapolated_GFLOP/s": round(wl.gemm_flops() / full / 1e9, 2),
                         "timed": f"rows 0..{r1 - 1} and 0..{r2 - 1}; full M={wl.M} is a linear extrapolation"}
        del qw, ws
    out["weights"] = "E4M3 codes drawn uniformly (finite codes), scales uniform: the offline quantization is untimed"
    return out


def cpu_baseline(wl, env, budget_s=12.0):
    """The oracle, as it stands, on the same workload: quantize the activation row(s)
    and dequantize-and-matmul in float64, repeated for about budget_s seconds."""
    import synth
    import oracle
    x = synth.make_activation(wl)
    w = synth.make_weight(wl)
    qw, ws = oracle.quant_weight(w)            # offline step, untimed as on the GPU
    reps, t0 = 0, time.perf_counter()
    while True:
        q, s = oracle.quant_act(x)
        oracle.linear_ref(q, s, qw, ws)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 1000:
            break
    per_step = el / reps
    bytes_step = wl.quant_bytes() + wl.gemm_bytes()
    return {"value": round(bytes_step / per_step / 1e9, 4), "unit": "GB/s", "cores": env["blas_threads"],
            "kind": "oracle", "cpu_model": env["cpu_model"], "cores_available": env["cores"],
            "sample": (f"{reps} full steps of {wl.name} (M={wl.M}, K={wl.K}, N={wl.N}): numpy quantizer "
                       f"(1 thread) + float64 dequantize-and-matmul (BLAS, {env['blas_threads']} threads set "
                       f"through threadpoolctl), {el:.1f} s, {per_step * 1e3:.1f} ms/step")}


def summarize_rocprof(directory):
    """Per-kernel, per-grid summary of rocprofv3 CSV output (kernel trace and/or
    counter collection) found under ``directory``: dispatch count, mean and min
    duration, and the mean of every collected counter."""
    import csv
    import glob
    from collections import defaultdict
    rows_t = defaultdict(list)
    rows_c = defaultdict(lambda: defaultdict(list))
    for f in glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                key = (r["Kernel_Name"], r.get("Grid_Size_X", r.get("Grid_Size", "")))
                rows_t[key].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                key = (r["Kernel_Name"], r.get("Grid_Size", ""))
                rows_c[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
    for key in sorted(set(rows_t) | set(rows_c)):
        name, grid = key
        print(f"kernel {name}  grid {grid}")
        if key in rows_t:
            d = rows_t[key]
            print(f"  dispatches {len(d)}  mean {sum(d) / len(d) / 1e3:.2f} us  min {min(d) / 1e3:.2f} us")
        for cname, vals in sorted(rows_c.get(key, {}).items()):
            print(f"  {cname} mean {sum(vals) / len(vals):.6g} over {len(vals)} dispatches")


def main():
    args = parse()
    if args.summarize:
        summarize_rocprof(args.summarize)
        return 0
    if args.make_traffic:
        make_traffic(args.make_traffic, args.traffic_file)
        return 0
    if args.copy_calibration:
        import torch
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 512 << 20, "copy_bytes_written": 512 << 20, "copies": 10}))
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        return 2
    import numpy as np
    import torch
    import synth
    from synth import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    from synth import W4A16_WORKLOADS
    if args.workload in W4A16_WORKLOADS:
        # One NVFP4 workload alone (used for its kernel profiles).
        w4 = time_w4_all(args.steps, args.traffic_file, [args.workload])[args.workload]
        print(json.dumps({"metric": W4_METRIC, "value": w4["roofline"]["achieved"],
                          "unit": w4["roofline"]["unit"], "n_gpus": 1, "steps": args.steps,
                          "warmup": 3, "ms_per_step": round(w4["us"] * 1e-3, 5), "higher_is_better": True,
                          "scaling": "weak", "vs_baseline": None, "dtype": "bf16 x nvfp4 (fp32 accumulate)",
                          "data": "synthetic (seeded; Philox per-row streams)",
                          "config": {"workload": args.workload, "M": w4["M"], "K": w4["K"], "N": w4["N"]},
                          "roofline": w4["roofline"], "cpu_baseline": None}), flush=True)
        return 0
    wl = WORKLOADS[args.workload]
    print(f"[bench] {wl.name}: setup", file=sys.stderr, flush=True)
    case = make_case(wl)
    ms, gemm_us, quant_us = time_case(case, args.steps, args.warmup)
    step_bytes = wl.quant_bytes() + wl.gemm_bytes()
    value = step_bytes / (ms * 1e-3) / 1e9
    traffic = load_traffic(args.traffic_file, wl)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate, bf16 in/out)",
        "data": "synthetic (seeded; Philox per-row streams)",
        "config": {"workload": wl.name, "M": wl.M, "K": wl.K, "N": wl.N,
                   "step": "quant_act + block_linear", "weight_copies_rotated": case.copies,
                   "step_bytes": step_bytes},
        "roofline": roofline_for(wl, gemm_us, traffic),
        "kernels_us": {"block_linear": round(gemm_us, 2), "quant_act": round(quant_us, 2)},
    }
    out["smi_after_headline"] = smi_snapshot()
    del case
    torch.cuda.empty_cache()

    if not args.no_ceilings:
        # Measured ceilings next to the published peaks: a plain streaming read at each
        # decode workload's byte count (same rotation as its weights), and the FP8 MFMA
        # loop alone and with the promotion FMAs.
        print("[bench] ceilings", file=sys.stderr, flush=True)
        ceil = {"stream_read": {}}
        for name in ("decode_qkv", "spec_mlp_gu", "spec_mlp_down"):
            w2 = WORKLOADS[name]
            copies = max(1, min(16, -(-2 * MALL_BYTES // (w2.N * w2.K))))
            ceil["stream_read"][name] = stream_ceiling(w2.gemm_bytes(), copies)
        ceil["mfma_fp8"] = mfma_ceiling(False)
        ceil["mfma_fp8_with_promotion"] = mfma_ceiling(True)
        ceil["smi"] = smi_snapshot()
        out["ceilings"] = ceil
        sr = ceil["stream_read"].get(wl.name)
        if sr and out["roofline"]["bound"] == "hbm":
            out["roofline"]["measured_stream_ceiling_GB/s"] = sr["GB/s"]
            out["roofline"]["frac_of_measured_ceiling"] = round(out["roofline"]["achieved"] / sr["GB/s"], 4)

    if not args.no_others:
        others = {}
        order = ["tiny", "spec_mlp_gu", "spec_mlp_down", "prefill_oproj", "fusion_fc"]
        for name in order:
            if name == wl.name:
                continue
            w2 = WORKLOADS[name]
            print(f"[bench] {name}: setup", file=sys.stderr, flush=True)
            c2 = make_case(w2)
            steps = max(5, min(args.steps, 50 if w2.M > 16 else args.steps))
            ms2, g2, q2 = time_case(c2, steps, max(2, min(args.warmup, 5)))
            rl = roofline_for(w2, g2, load_traffic(args.traffic_file, w2))
            others[name] = {"M": w2.M, "K": w2.K, "N": w2.N, "ms_per_step": round(ms2, 5),
                            "block_linear_us": round(g2, 2), "quant_us": round(q2, 2),
                            "gemm_roofline": rl, "weight_copies_rotated": c2.copies}
            if w2.x_kind == "silu":
                others[name]["input"] = "SiLU(gate)*up of the gate/up projection's GPU output, re-quantized"
            if w2.M > 16:
                others[name]["smi_after"] = smi_snapshot()
            del c2
            torch.cuda.empty_cache()
        out["workloads"] = others
        ceil = out.get("ceilings")
        if ceil:
            for name, ent in others.items():
                rl = ent["gemm_roofline"]
                sr = ceil["stream_read"].get(name)
                if rl["bound"] == "hbm" and sr:
                    rl["measured_stream_ceiling_GB/s"] = sr["GB/s"]
                    rl["frac_of_measured_ceiling"] = round(rl["achieved"] / sr["GB/s"], 4)
                elif rl["bound"] == "mfma":
                    for key in ("mfma_fp8", "mfma_fp8_with_promotion"):
                        rl[f"frac_of_{key}_loop"] = round(rl["achieved"] / ceil[key]["TFLOP/s"], 4)
        print("[bench] M sweep", file=sys.stderr, flush=True)
        out["m_sweep"] = time_m_sweep()
        out["w4a16"] = time_w4_all(args.steps, args.traffic_file)
        print("[bench] rmsnorm_quant", file=sys.stderr, flush=True)
        out["rmsnorm_quant"] = {name: time_rmsnorm_quant(WORKLOADS[name], 50 if name == "prefill_oproj" else 200)
                                for name in ("decode_qkv", "prefill_oproj")}
        print("[bench] silu_mul_quant", file=sys.stderr, flush=True)
        out["silu_mul_quant"] = {"spec_mlp (M=8, I=8192)": time_silu_mul_quant(8, 8192, 200),
                                 "prefill chunk (M=2048, I=8192)": time_silu_mul_quant(2048, 8192, 50)}

    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        env = cpu_env()
        try:
            from threadpoolctl import threadpool_limits
            limiter = threadpool_limits(limits=env["blas_threads"])
        except Exception:  # pragma: no cover
            limiter = None
        out["cpu_baseline"] = cpu_baseline(wl, env)
        if not args.no_others:
            out["cpu_baseline_per_config"] = cpu_baseline_per_config(env)
        del limiter
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
