"""Benchmark: one step = the whole FP8 linear-layer path, forward and backward.

Default workload `ffn_dense`, the dense FFN's two linears (synthetic, seeded;
inputs resident in HBM): up X [8192, 7168] (Student-t(3)), W_up [7168, 18432],
dY_up [8192, 18432]; down H [8192, 18432] (Student-t(3)), W_down [18432, 7168],
dY_down [8192, 7168].  Per linear, in order:

  quantize X 1x128 -> quantize W 128x128 (both layouts) -> Fprop Y = X W (bf16)
  -> quantize dY 1x128 and 128x1 (one fused read) -> Dgrad dX = dY W^T (bf16)
  -> requant X 128x1 -> Wgrad dW = X^T dY (fp32)

six GEMMs of 2*8192*7168*18432 FLOP each; the down projection's Fprop and the
up projection's Dgrad contract over 18432 = 144 blocks.
`--workload linear_dsv3_attn` runs the same step once at the DeepSeek-V3
attention-projection shape X [4096, 7168], W [7168, 7168], dY [4096, 7168].

Prints one JSON line (and keeps a copy as results/<workload>[_ue8m0][_sr].json;
`--results DIR` moves it, `--results ''` drops it).  `value` is the step's GEMM throughput (GEMM FLOP over
the whole step time, quantization included) in TFLOP/s.  Per-kernel durations
come from HIP events recorded around every launch on the stream the kernels
run on, over the timed steps (warm: the steps run back to back); `roofline`
prices the dominant kernel against MI355X's dense FP8 MFMA peak (5.0 PFLOP/s
at 2.4 GHz) and, with the shader clock measured while that kernel runs back to
back (`clock_mhz`; the chip lowers it under this load), against the peak at
that clock (`frac_at_clock`); `clock_mhz_mfma_only` is the clock under a probe
that runs FP8 MFMAs and nothing else, and `staging_probe` the cycles that the
GEMM's per-block staging traffic (fragment reads, direct-to-LDS operand loads,
both) takes on one compute unit beside the 2048 its MFMAs need.
Per GEMM, `hipblaslt_plain_fp8` times hipBLASLt's plain FP8 GEMM (one tensor-wide
scale, no per-block rescale) on the same operands, as a reference (ffn_dense by
default, `--no-blas-reference` skips it; `--blas-reference` for linear_dsv3_attn).
`kernels` lists every kernel's rate against its own roofline (HBM for the
quantizers).  The default line also carries `quant_stress`: the five
quantizers alone on the stress tensor X [16384, 7168], each launch cold (the
`--workload quant_stress` measurement condensed; `--no-quant-stress` skips it).  `cold` is the median of 50 steps after 10 warm-ups, each after a
1 GiB read scrub outside its events, labelled as such.  `cpu_baseline` times
the CPU oracle on a bounded, seeded sample of the same work (for ffn_dense and
moe_grouped 1/8 of the 128x128 output tiles, first and last tiles included;
the fraction is printed), with the host's CPU model, thread count and the
oracle's one-thread quantizer rate.

`--recipe ue8m0` runs the same step with power-of-two (UE8M0) scales, which the
matrix core applies itself (no vector-ALU rescale).  Its weight cast has two
stages by default, as in the pages' conventions: the FP8 cast with fp32 tile
scales, then the decoded weight requantized to power-of-two tiles
(`--ue8m0-weights direct` casts the bf16 weight straight to power-of-two tiles).

`--rounding sr` quantizes X, W and dY with stochastic rounding (one Philox
word per element); the requant of the saved X stays round-to-nearest.

`--schedule overlap` runs the casts that no GEMM waits for on a second HIP
stream beside the GEMMs (quantize X beside quantize W; the dY casts and the X
requant beside Fprop; in the MoE step the down weights' cast, the dY casts and
both requants).  Every GEMM waits for the casts it reads, and a step's second
stream waits for the previous step's GEMMs, so steps never overlap.  The
default, `serial`, runs every kernel on one stream in the order above: beside
a GEMM's blocks the casts get few CUs, and the cross-stream waits cost more
than the overlap saves in the linear step.

`--workload moe_grouped` times one GPU's MoE expert share as a SwiGLU FFN
instead (32 experts, 8192 tokens routed top-8; gate/up and down projections,
forward and backward, with the SwiGLU casts fused into the SwiGLU kernels);
`value` then counts the routed rows' GEMM FLOP.

`--workload quant_stress` times the quantizers alone on the stress tensor
X [16384, 7168] (per-row scales 10^U(-6,3), signed zeros, zero tiles, tiny and
subnormal negatives): 1x128, 128x1, 128x128 (both layouts), the fused dual
cast and the 128x1 requant of the 1x128 codes.  Every launch runs cold: a
1 GiB read scrub before it (outside its events) evicts L2 and the Infinity
Cache.  Per kernel the median over the timed steps; `value` is the summed
algorithmic bytes over the summed medians in GB/s, and `roofline` prices the
slowest kernel against 8 TB/s.  `copy_reference` times a plain streaming
kernel with the 1x128 cast's traffic (2 bytes read, 1 written per element)
the same way, and `copy_reference_1to1` a byte copy with the requant's (1
read, 1 written); each kernel's `frac_of_copy` compares its rate with the
reference of its own mix.
`us_warm` / `GB/s_warm` are the same launches back to back without the scrub
(warm cache), labelled as such; `value` uses the cold medians.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload W] [--no-cpu-baseline]
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

HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
FP8_PEAK = 5.0e15          # FLOP/s, MI355X dense FP8 MFMA
T = 128
COPY_BYTES = 1 << 30       # the calibration copy reads and writes this many bytes
CSRC = os.path.join(ROOT, "fine_grained_block_amd", "csrc")


def kernel_source_hash():
    """First 16 hex digits of sha256 over the kernel sources (csrc/*.hip, *.hpp, by
    name): a traffic record is valid only for the sources it was measured on."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".hpp")):
            h.update(f.encode())
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_record(kernel):
    """HBM bytes per launch of `kernel` from a committed rocprofv3 summary
    (profiles/*_traffic.md, line 'traffic-record: kernel=... bytes=... source=...'),
    or None when there is none or the kernel sources changed since."""
    d = os.path.join(ROOT, "profiles")
    if not os.path.isdir(d):
        return None
    want = kernel_source_hash()
    for f in sorted(os.listdir(d)):
        if not f.endswith("_traffic.md"):
            continue
        for line in open(os.path.join(d, f)):
            if line.strip().startswith("traffic-record:"):
                kv = dict(t.split("=", 1) for t in line.split(":", 1)[1].split())
                if kv.get("kernel") == kernel and kv.get("source") == want:
                    return int(kv["bytes"])
    return None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", choices=["ffn_dense", "linear_dsv3_attn", "moe_grouped", "quant_stress"],
                   default="ffn_dense",
                   help="ffn_dense (default): the dense FFN's up and down linears, fwd+bwd (the largest "
                        "single-GPU workload, contraction up to 18432); linear_dsv3_attn: the DeepSeek-V3 "
                        "attention projection's linear; moe_grouped: one GPU's MoE expert share as a SwiGLU "
                        "FFN, fwd+bwd; quant_stress: the quantizers alone on X [16384,7168], cold cache")
    p.add_argument("--recipe", choices=["fp32", "ue8m0"], default="fp32",
                   help="fp32: scales absmax/448 (default); ue8m0: power-of-two scales, applied by the matrix core")
    p.add_argument("--ue8m0-weights", choices=["two-stage", "direct"], default="two-stage",
                   help="with --recipe ue8m0: two-stage (default) = FP8 cast with fp32 tile scales, then "
                        "requant of the decoded weight to power-of-two tiles; direct = one power-of-two cast")
    p.add_argument("--rounding", choices=["rn", "sr"], default="rn",
                   help="rn: round-to-nearest casts (default); sr: stochastic rounding of the X, W and dY "
                        "casts (Philox words; the requant of X stays round-to-nearest)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--separate-dy-casts", action="store_true",
                   help="quantize dY with two kernels (1x128, then 128x1) instead of the fused one")
    p.add_argument("--copy-calibration", action="store_true",
                   help="after the timed region, run a plain streaming kernel (1 GiB read, 1 GiB "
                        "written) three times: it scales rocprofv3's FETCH_SIZE/WRITE_SIZE to bytes")
    p.add_argument("--schedule", choices=["serial", "overlap"], default="serial",
                   help="serial (default): every kernel on one stream, in step order; "
                        "overlap: casts that no GEMM waits for run on a second stream")
    p.add_argument("--blas-reference", action="store_true",
                   help="linear_dsv3_attn: also time hipBLASLt's plain FP8 GEMM (torch._scaled_mm, one "
                        "tensor-wide scale, no per-block rescale) on each step GEMM's operands; reported per "
                        "GEMM as `hipblaslt_plain_fp8` (ffn_dense does this by default)")
    p.add_argument("--no-blas-reference", action="store_true",
                   help="ffn_dense: skip the hipBLASLt plain-FP8 reference timings")
    p.add_argument("--no-quant-stress", action="store_true",
                   help="ffn_dense: skip the quant_stress summary (the five quantizers cold on the stress "
                        "tensor) that the line carries as `quant_stress`")
    p.add_argument("--cold-iters", type=int, default=50,
                   help="cold-cache step timings after the timed region: median of this many steps, each "
                        "after a 1 GiB scrub (0 = skip)")
    p.add_argument("--cpu-tile-frac", type=float, default=0.125,
                   help="ffn_dense / moe_grouped CPU baseline: fraction of the 128x128 output tiles the oracle "
                        "computes (seeded; first and last tiles included)")
    p.add_argument("--cpu-rows", type=int, default=0,
                   help="Fprop/Dgrad output rows in the CPU-baseline sample (0 = auto, ~15 s of GEMM work)")
    p.add_argument("--results", default="results",
                   help="directory that receives the printed JSON line as <workload>[_ue8m0][_sr].json "
                        "(empty: write nothing)")
    return p.parse_args()


def emit(args, out):
    """Print the JSON line and keep a copy under --results, named for the workload and recipe."""
    line = json.dumps(out)
    print(line, flush=True)
    if args.results:
        name = args.workload + ("_ue8m0" if args.recipe == "ue8m0" else "") + ("_sr" if args.rounding == "sr" else "")
        os.makedirs(args.results, exist_ok=True)
        with open(os.path.join(args.results, name + ".json"), "w") as f:
            f.write(line + "\n")


def algorithmic_bytes(M, K, N):
    """Bytes each kernel must move: every input read once, every output written once."""
    nbK, nbN, nbM = K // T, N // T, -(-M // T)
    Mp = nbM * T
    return {
        "quantize_1x128_x": M * K * 2 + M * K + nbK * M * 4,
        "quantize_128x128_w": K * N * 2 + 2 * K * N + nbK * nbN * 4,
        "quantize_1x128_dy": M * N * 2 + M * N + nbN * M * 4,
        "quantize_128x1_dy": M * N * 2 + N * Mp + nbM * N * 4,
        "requant_128x1_x": M * K + nbK * M * 4 + K * Mp + nbM * K * 4,
        "quantize_dual_dy": M * N * 2 + M * N + nbN * M * 4 + N * Mp + nbM * N * 4,
        # two-stage weight cast: the first stage writes the row-major codes only
        "quantize_128x128_w_stage1": K * N * 2 + K * N + nbK * nbN * 4,
        "requant_128x128_w": K * N + nbK * nbN * 4 + 2 * K * N + nbK * nbN * 4,
    }


def linear_step(fgb, torch, dev, d, separate_dy=False, ue8m0=False, sr=False, bufs=None, two_stage=False):
    """The linear layer's step at X [M,K], W [K,N], dY [M,N]: (name, launch, work,
    lane, deps) per kernel in issue order, work = {"flop": ...} or {"bytes": ...}
    (algorithmic); lane 1 = the second stream, deps = kernels it reads the
    output of (only waits across streams matter)."""
    import numpy as np
    M, K, N = d["M"], d["K"], d["N"]

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    x, w, dy = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["dy"])
    u8 = dict(dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    Mp = -(-M // T) * T
    b = {
        "qx": torch.empty((M, K), **u8), "sx": torch.empty((K // T, M), **f32),
        "qw": torch.empty((K, N), **u8), "qwT": torch.empty((N, K), **u8), "sw": torch.empty((K // T, N // T), **f32),
        "y": torch.empty((M, N), dtype=torch.bfloat16, device=dev),
        "qdy": torch.empty((M, N), **u8), "sdy": torch.empty((N // T, M), **f32),
        "dx": torch.empty((M, K), dtype=torch.bfloat16, device=dev),
        "qdyT": torch.empty((N, Mp), **u8), "sdyT": torch.empty((Mp // T, N), **f32),
        "qxT": torch.empty((K, Mp), **u8), "sxT": torch.empty((Mp // T, K), **f32),
        "dw": torch.empty((K, N), **f32),
    }
    two_stage = two_stage and ue8m0
    if two_stage:
        b["qw1"] = torch.empty((K, N), **u8)
        b["sw1"] = torch.empty((K // T, N // T), **f32)
    if bufs is not None:
        bufs.update(b)
    ab = algorithmic_bytes(M, K, N)
    flop = {"flop": 2.0 * M * N * K}
    # stochastic rounding: one (seed, salt) per step, a salt per tensor
    srk = (lambda salt: (0x5EED, salt)) if sr else (lambda salt: None)
    if separate_dy:
        dy_casts = [
            ("quantize_1x128_dy", lambda: fgb.quantize_1x128(dy, q=b["qdy"], s=b["sdy"], ue8m0=ue8m0, sr=srk(3)),
             {"bytes": ab["quantize_1x128_dy"]}),
            ("quantize_128x1_dy", lambda: fgb.quantize_128x1(dy, qT=b["qdyT"], sT=b["sdyT"], ue8m0=ue8m0, sr=srk(3)),
             {"bytes": ab["quantize_128x1_dy"]}),
        ]
    else:
        dy_casts = [
            ("quantize_dual_dy", lambda: fgb.quantize_dual(dy, q=b["qdy"], s=b["sdy"], qT=b["qdyT"], sT=b["sdyT"],
                                                          ue8m0=ue8m0, sr=srk(3)),
             {"bytes": ab["quantize_dual_dy"]}),
        ]
    if two_stage:
        w_casts = [
            # first stage with the pages' weight amax floor 1e-4 (conventions row "Weight floors")
            ("quantize_128x128_w_stage1", lambda: fgb.quantize_128x128(w, 1e-4, q=b["qw1"], s=b["sw1"],
                                                                       want_qT=False),
             {"bytes": ab["quantize_128x128_w_stage1"]}),
            ("requant_128x128_w", lambda: fgb.requant_128x128_ue8m0(b["qw1"], b["sw1"], q2=b["qw"], q2T=b["qwT"],
                                                                    s2=b["sw"]),
             {"bytes": ab["requant_128x128_w"]}),
        ]
    else:
        w_casts = [
            ("quantize_128x128_w", lambda: fgb.quantize_128x128(w, q=b["qw"], qT=b["qwT"], s=b["sw"], ue8m0=ue8m0,
                                                                sr=srk(2)),
             {"bytes": ab["quantize_128x128_w"]}),
        ]
    steps = [
        ("quantize_1x128_x", lambda: fgb.quantize_1x128(x, q=b["qx"], s=b["sx"], ue8m0=ue8m0, sr=srk(1)),
         {"bytes": ab["quantize_1x128_x"]}),
    ] + w_casts + [
        ("gemm_fprop", lambda: fgb.gemm_fprop(b["qx"], b["sx"], b["qwT"], b["sw"], y=b["y"], ue8m0=ue8m0), flop),
    ] + dy_casts + [
        ("gemm_dgrad", lambda: fgb.gemm_dgrad(b["qdy"], b["sdy"], b["qw"], b["sw"], dx=b["dx"], ue8m0=ue8m0), flop),
        ("requant_128x1_x", lambda: fgb.requant_128x1(b["qx"], b["sx"], qT=b["qxT"], sT=b["sxT"], ue8m0=ue8m0),
         {"bytes": ab["requant_128x1_x"]}),
        ("gemm_wgrad", lambda: fgb.gemm_wgrad(b["qxT"], b["sxT"], b["qdyT"], b["sdyT"], M, dw=b["dw"], ue8m0=ue8m0),
         flop),
    ]
    dy_names = [n for n, _, _ in dy_casts]
    w_names = [n for n, _, _ in w_casts]
    lanes = {"quantize_1x128_x": (1, []),
             "gemm_fprop": (0, ["quantize_1x128_x", w_names[-1]]),
             "gemm_dgrad": (0, dy_names + [w_names[-1]]),
             "requant_128x1_x": (1, ["quantize_1x128_x"]),
             "gemm_wgrad": (0, dy_names + ["requant_128x1_x"])}
    for n in dy_names:
        lanes[n] = (1, [])
    for n in w_names:
        lanes[n] = (0, [])
    order = ["quantize_1x128_x"] + w_names + ["gemm_fprop"] + dy_names + \
            ["gemm_dgrad", "requant_128x1_x", "gemm_wgrad"]
    by = {name: (name, fn, work) for name, fn, work in steps}
    steps = [by[n] + lanes[n] for n in order]

    def rename(n):
        if n == "quantize_128x128_w_stage1":
            return n
        n = n + "_ue8m0" if ue8m0 else n
        return n + "_sr" if sr and n.startswith("quantize") else n
    return [(rename(n), fn, work, lane, [rename(x) for x in deps]) for n, fn, work, lane, deps in steps]


def moe_step(fgb, torch, dev, d, bufs=None):
    """One GPU's MoE expert share as a full SwiGLU FFN step, forward and backward:
    quantize X and the expert weights, gate/up Fprop -> [G | U], SwiGLU forward
    (emits the E4M3 stash of [G | U] and H's 1x128 codes), down Fprop; quantize dY
    both ways, down Dgrad -> dH, requant H, down Wgrad, SwiGLU backward (emits
    [dG | dU] in both tile orientations), gate/up Dgrad, requant X, gate/up Wgrad.
    GEMM work counts the routed rows only (padding rows are computed, not counted);
    each projection's expert weights are quantized in one launch."""
    import numpy as np
    E, R = d["E"], d["R_pad"]
    rows = int(np.sum(d["loads"]))
    Dm, F2, F = d["d_model"], d["d_ff2"], d["d_ff"]
    od = torch.from_numpy(np.asarray(d["offsets"], np.int32)).to(dev)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    u8 = dict(dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    bf = dict(dtype=torch.bfloat16, device=dev)
    x, dy = to_dev(d["x"]), to_dev(d["dy_down"])
    w_up, w_down = to_dev(d["w_up"]), to_dev(d["w_down"])
    Rt = R // T
    b = {
        "qx": torch.empty((R, Dm), **u8), "sx": torch.empty((Dm // T, R), **f32),
        "qxT": torch.empty((Dm, R), **u8), "sxT": torch.empty((Rt, Dm), **f32),
        "qwu": torch.empty((E, Dm, F2), **u8), "qwuT": torch.empty((E, F2, Dm), **u8),
        "swu": torch.empty((E, Dm // T, F2 // T), **f32),
        "qwd": torch.empty((E, F, Dm), **u8), "qwdT": torch.empty((E, Dm, F), **u8),
        "swd": torch.empty((E, F // T, Dm // T), **f32),
        # padding rows of a GEMM output stay zero (the grouped GEMMs compute them as 0)
        "gu": torch.zeros((R, F2), **bf),
        "q_gu": torch.empty((R, F2), **u8), "s_gu": torch.empty((F2 // T, R), **f32),
        "q_h": torch.empty((R, F), **u8), "s_h": torch.empty((F // T, R), **f32),
        "q_hT": torch.empty((F, R), **u8), "s_hT": torch.empty((Rt, F), **f32),
        "y": torch.empty((R, Dm), **bf),
        "qdy": torch.empty((R, Dm), **u8), "sdy": torch.empty((Dm // T, R), **f32),
        "qdyT": torch.empty((Dm, R), **u8), "sdyT": torch.empty((Rt, Dm), **f32),
        "dh": torch.zeros((R, F), **bf),
        "q_dgu": torch.empty((R, F2), **u8), "s_dgu": torch.empty((F2 // T, R), **f32),
        "q_dguT": torch.empty((F2, R), **u8), "s_dguT": torch.empty((Rt, F2), **f32),
        "dx": torch.empty((R, Dm), **bf),
        "dw_up": torch.empty((E, Dm, F2), **f32), "dw_down": torch.empty((E, F, Dm), **f32),
    }
    if bufs is not None:
        bufs.update(b)

    def quant_w(w, q, qT, s):                 # all experts' weights in one launch
        fgb.quantize_128x128_batched(w, q=q, qT=qT, s=s)

    loads = [int(n) for n in d["loads"]]

    def grouped_roofline(kind, K, N):
        """Sum over experts of max(FLOP / FP8 peak, bytes / HBM peak) in
        microseconds for one grouped call (routed rows only): Fprop/Dgrad read
        the expert's [rows, K] codes, its [N, K] weight codes and their fp32
        scales and write [rows, N] bf16; Wgrad reads both transposed operands
        (K and N codes per row) and their scales and writes the expert's fp32
        [K, N] dW, also for an empty expert (zeros).  Returns (us, number of
        experts below the ridge)."""
        tot, mem_bound = 0.0, 0
        for n in loads:
            fl = 2.0 * n * K * N
            if kind == "rows":
                by = n * K + 4 * n * (K // T) + N * K + 4 * (K // T) * (N // T) + 2 * n * N
            else:
                by = n * (K + N) + 4 * (n // T + (n % T > 0)) * (K + N) + 4 * K * N
            tc, tm = fl / FP8_PEAK, by / HBM_PEAK
            mem_bound += tm > tc
            tot += max(tc, tm)
        return tot * 1e6, mem_bound

    def gwork(flop, kind, K, N):
        us, mb = grouped_roofline(kind, K, N)
        return {"flop": flop, "roofline_us": us, "experts_memory_bound": mb}

    up = {"flop": 2.0 * rows * Dm * F2}
    down = {"flop": 2.0 * rows * F * Dm}
    fup, fdown = gwork(up["flop"], "rows", Dm, F2), gwork(down["flop"], "rows", F, Dm)
    dup, ddown = gwork(up["flop"], "rows", F2, Dm), gwork(down["flop"], "rows", Dm, F)
    wup, wdown = gwork(up["flop"], "k", Dm, F2), gwork(down["flop"], "k", F, Dm)
    nb2, nb1 = F2 // T, F // T
    swf_bytes = R * F2 * 2 + R * F2 + 4 * R * nb2 + R * F + 4 * R * nb1
    swb_bytes = R * F2 + 4 * R * nb2 + R * F * 2 + R * F2 + 4 * R * nb2 + F2 * R + 4 * Rt * F2
    ab_x = algorithmic_bytes(R, Dm, F2)
    ab_h = algorithmic_bytes(R, F, Dm)
    steps = [
        ("quantize_1x128_x", lambda: fgb.quantize_1x128(x, q=b["qx"], s=b["sx"]), {"bytes": ab_x["quantize_1x128_x"]}),
        ("quantize_128x128_w_up", lambda: quant_w(w_up, b["qwu"], b["qwuT"], b["swu"]),
         {"bytes": E * algorithmic_bytes(R, Dm, F2)["quantize_128x128_w"]}),
        ("gemm_fprop_grouped_up", lambda: fgb.gemm_fprop_grouped(od, b["qx"], b["sx"], b["qwuT"], b["swu"], y=b["gu"]),
         fup),
        ("swiglu_fwd_quant", lambda: fgb.swiglu_fwd_quant(b["gu"], q_gu=b["q_gu"], s_gu=b["s_gu"], q_h=b["q_h"],
                                                          s_h=b["s_h"]), {"bytes": swf_bytes}),
        ("quantize_128x128_w_down", lambda: quant_w(w_down, b["qwd"], b["qwdT"], b["swd"]),
         {"bytes": E * algorithmic_bytes(R, F, Dm)["quantize_128x128_w"]}),
        ("gemm_fprop_grouped_down", lambda: fgb.gemm_fprop_grouped(od, b["q_h"], b["s_h"], b["qwdT"], b["swd"],
                                                                   y=b["y"]), fdown),
        ("quantize_dual_dy", lambda: fgb.quantize_dual(dy, q=b["qdy"], s=b["sdy"], qT=b["qdyT"], sT=b["sdyT"]),
         {"bytes": ab_h["quantize_dual_dy"]}),
        ("gemm_dgrad_grouped_down", lambda: fgb.gemm_dgrad_grouped(od, b["qdy"], b["sdy"], b["qwd"], b["swd"],
                                                                   dx=b["dh"]), ddown),
        ("requant_128x1_h", lambda: fgb.requant_128x1(b["q_h"], b["s_h"], qT=b["q_hT"], sT=b["s_hT"]),
         {"bytes": algorithmic_bytes(R, F, Dm)["requant_128x1_x"]}),
        ("gemm_wgrad_grouped_down", lambda: fgb.gemm_wgrad_grouped(od, b["q_hT"], b["s_hT"], b["qdyT"], b["sdyT"],
                                                                   dw=b["dw_down"]), wdown),
        ("swiglu_bwd_quant", lambda: fgb.swiglu_bwd_quant(b["q_gu"], b["s_gu"], b["dh"], q=b["q_dgu"], s=b["s_dgu"],
                                                          qT=b["q_dguT"], sT=b["s_dguT"]), {"bytes": swb_bytes}),
        ("gemm_dgrad_grouped_up", lambda: fgb.gemm_dgrad_grouped(od, b["q_dgu"], b["s_dgu"], b["qwu"], b["swu"],
                                                                 dx=b["dx"]), dup),
        ("requant_128x1_x", lambda: fgb.requant_128x1(b["qx"], b["sx"], qT=b["qxT"], sT=b["sxT"]),
         {"bytes": ab_x["requant_128x1_x"]}),
        ("gemm_wgrad_grouped_up", lambda: fgb.gemm_wgrad_grouped(od, b["qxT"], b["sxT"], b["q_dguT"], b["s_dguT"],
                                                                 dw=b["dw_up"]), wup),
    ]
    # second stream: the down weights' cast, the dY casts and the two requants
    lanes = {"quantize_128x128_w_down": (1, []), "quantize_dual_dy": (1, []),
             "requant_128x1_x": (1, ["quantize_1x128_x"]), "requant_128x1_h": (1, ["swiglu_fwd_quant"]),
             "gemm_fprop_grouped_down": (0, ["quantize_128x128_w_down"]),
             "gemm_dgrad_grouped_down": (0, ["quantize_dual_dy", "quantize_128x128_w_down"]),
             "gemm_wgrad_grouped_down": (0, ["requant_128x1_h", "quantize_dual_dy"]),
             "gemm_wgrad_grouped_up": (0, ["requant_128x1_x"])}
    order = ["quantize_1x128_x", "quantize_128x128_w_up", "quantize_128x128_w_down", "gemm_fprop_grouped_up",
             "swiglu_fwd_quant", "quantize_dual_dy", "requant_128x1_h", "requant_128x1_x",
             "gemm_fprop_grouped_down", "gemm_dgrad_grouped_down", "gemm_wgrad_grouped_down", "swiglu_bwd_quant",
             "gemm_dgrad_grouped_up", "gemm_wgrad_grouped_up"]
    by = {name: (name, fn, work) for name, fn, work in steps}
    assert sorted(order) == sorted(by)
    return [by[n] + lanes.get(n, (0, [])) for n in order]


def quant_stress_bytes(R, C):
    """Algorithmic bytes of each quantizer on X [R, C] (bf16 in; codes, scales out)."""
    nbR, nbC = -(-R // T), -(-C // T)
    Rp = nbR * T
    return {
        "quantize_1x128": R * C * 2 + R * C + nbC * R * 4,
        "quantize_128x1": R * C * 2 + C * Rp + nbR * C * 4,
        "quantize_128x128": R * C * 2 + 2 * R * C + nbR * nbC * 4,
        "quantize_dual": R * C * 2 + R * C + nbC * R * 4 + C * Rp + nbR * C * 4,
        "requant_128x1": R * C + nbC * R * 4 + C * Rp + nbR * C * 4,
    }


def quant_stress_main(args, np, torch, fgb, wl, emit_line=True):
    """--workload quant_stress: each quantizer cold, median over the timed steps.
    Prints the JSON line (emit) and returns it as a dict."""
    dev = torch.device("cuda:0")
    d = wl.quant_stress()
    R, C = d["R"], d["C"]
    x = torch.from_numpy(np.ascontiguousarray(d["x"]).view(np.int16)).to(dev).view(torch.bfloat16)
    u8 = dict(dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    nbR, nbC = -(-R // T), -(-C // T)
    Rp = nbR * T
    b = {"q": torch.empty((R, C), **u8), "s": torch.empty((nbC, R), **f32),
         "qT": torch.empty((C, Rp), **u8), "sT": torch.empty((nbR, C), **f32),
         "qw": torch.empty((R, C), **u8), "qwT": torch.empty((C, R), **u8), "sw": torch.empty((nbR, nbC), **f32),
         "q2": torch.empty((R, C), **u8), "s2": torch.empty((nbC, R), **f32),
         "qT2": torch.empty((C, Rp), **u8), "sT2": torch.empty((nbR, C), **f32),
         "rqT": torch.empty((C, Rp), **u8), "rsT": torch.empty((nbR, C), **f32)}
    ab = quant_stress_bytes(R, C)
    kernels = [
        ("quantize_1x128", lambda: fgb.quantize_1x128(x, q=b["q"], s=b["s"])),
        ("quantize_128x1", lambda: fgb.quantize_128x1(x, qT=b["qT"], sT=b["sT"])),
        ("quantize_128x128", lambda: fgb.quantize_128x128(x, q=b["qw"], qT=b["qwT"], s=b["sw"])),
        ("quantize_dual", lambda: fgb.quantize_dual(x, q=b["q2"], s=b["s2"], qT=b["qT2"], sT=b["sT2"])),
        ("requant_128x1", lambda: fgb.requant_128x1(b["q"], b["s"], qT=b["rqT"], sT=b["rsT"])),
    ]
    # reference: a plain streaming kernel that reads 2 bytes and writes 1 per element of X,
    # the 1x128 cast's traffic without its arithmetic
    n_ref = R * C // 4
    ref_in = torch.ones(2 * n_ref, dtype=torch.float32, device=dev)
    ref_out = torch.empty(n_ref, dtype=torch.float32, device=dev)
    kernels.append(("copy_reference", lambda: torch.add(ref_in[:n_ref], ref_in[n_ref:], out=ref_out)))
    ab["copy_reference"] = 3 * n_ref * 4
    # and one with the requant's traffic: 1 byte read and 1 written per element
    ref8_in = torch.ones(R * C, dtype=torch.uint8, device=dev)
    ref8_out = torch.empty(R * C, dtype=torch.uint8, device=dev)
    kernels.append(("copy_reference_1to1", lambda: ref8_out.copy_(ref8_in)))
    ab["copy_reference_1to1"] = 2 * R * C
    scrub = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        for _, fn in kernels:
            fn()
    torch.cuda.synchronize()
    times = {name: [] for name, _ in kernels}
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for name, fn in kernels:
            torch.sum(scrub, dim=(0,), out=sink)      # 1 GiB read: L2 and Infinity Cache cold
            a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            e.record()
            torch.cuda.synchronize()
            times[name].append(a.elapsed_time(e))
    wall = time.perf_counter() - t0
    # warm-cache medians, labelled as such: the same launches back to back, no scrub
    warm = {name: [] for name, _ in kernels}
    for _ in range(args.steps):
        for name, fn in kernels:
            a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            e.record()
            torch.cuda.synchronize()
            warm[name].append(a.elapsed_time(e))
    med_warm = {n: float(np.median(v)) for n, v in warm.items()}
    med = {n: float(np.median(v)) for n, v in times.items()}
    ref_ms = med.pop("copy_reference")
    ref_b = ab.pop("copy_reference")
    ref_rate = ref_b / (ref_ms * 1e-3)
    ref1_ms = med.pop("copy_reference_1to1")
    ref1_b = ab.pop("copy_reference_1to1")
    ref1_rate = ref1_b / (ref1_ms * 1e-3)
    kinfo = {}
    for n, ms in med.items():
        rate = ab[n] / (ms * 1e-3)
        # each kernel against the copy with its own mix of reads and writes
        rr = ref1_rate if n.startswith("requant") else ref_rate
        kinfo[n] = {"us": round(ms * 1e3, 2), "GB/s": round(rate / 1e9, 1),
                    "frac_hbm_peak": round(rate / HBM_PEAK, 4), "frac_of_copy": round(rate / rr, 3),
                    "bytes": ab[n], "us_warm": round(med_warm[n] * 1e3, 2),
                    "GB/s_warm": round(ab[n] / (med_warm[n] * 1e-3) / 1e9, 1)}
    total_ms = sum(med.values())
    total_b = sum(ab.values())
    dom = max(med, key=med.get)
    dom_rate = ab[dom] / (med[dom] * 1e-3)
    out = {
        "metric": "block-scaled FP8 GEMM TFLOP/s (% FP8 MFMA peak) + quant GB/s (% HBM) at 1 GPU",
        "value": round(total_b / (total_ms * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 -> e4m3 codes (u8) + fp32 scales",
        "data": "synthetic quantization stress tensor (seeded; per-row scales 10^U(-6,3), signed zeros, "
                "zero tiles, tiny and subnormal negatives; bf16)",
        "config": {"workload": "quant_stress: X[16384,7168] bf16 through the five quantizers, each launch cold "
                               "(1 GiB read scrub before it, outside its events); per-kernel median",
                   "R": R, "C": C, "quant_bytes_per_step": total_b,
                   "wall_s_incl_scrubs": round(wall, 2)},
        "quant_frac_hbm_peak": round(total_b / (total_ms * 1e-3) / HBM_PEAK, 4),
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(dom_rate / 1e9, 1),
                     "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": round(dom_rate / HBM_PEAK, 4),
                     "traffic": traffic_record("stress_" + dom)},
        "kernels": kinfo,
        "copy_reference": {"us": round(ref_ms * 1e3, 2), "GB/s": round(ref_rate / 1e9, 1),
                           "frac_hbm_peak": round(ref_rate / HBM_PEAK, 4), "bytes": ref_b,
                           "what": "torch add of two fp32 halves into a third: reads 2 and writes 1 byte per "
                                   "byte of X's elements, cold like the casts"},
        "copy_reference_1to1": {"us": round(ref1_ms * 1e3, 2), "GB/s": round(ref1_rate / 1e9, 1),
                                "frac_hbm_peak": round(ref1_rate / HBM_PEAK, 4), "bytes": ref1_b,
                                "what": "torch copy of R*C bytes: the requant's mix (1 byte read, 1 written "
                                        "per element), cold like the casts; the requant's frac_of_copy uses it"},
    }
    if args.copy_calibration:
        a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        c = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=c)
        torch.cuda.synchronize()
        del a, c
    if not args.no_cpu_baseline:
        import oracle
        t1 = time.perf_counter()
        oq, os_ = oracle.quantize_1x128(d["x"])
        oracle.quantize_128x1(d["x"])
        oracle.quantize_128x128(d["x"])
        oracle.quantize_1x128(d["x"])          # the dual cast's two outputs, as two oracle calls
        oracle.quantize_128x1(d["x"])
        oracle.requant_128x1(oq, os_)
        tq = time.perf_counter() - t1
        out["cpu_baseline"] = {"value": round(total_b / tq / 1e9, 3), "unit": "GB/s", "cores": oracle.max_threads(),
                               "kind": "oracle",
                               "sample": f"the whole workload: the five quantizers on the full tensor ({tq:.1f} s; "
                                         "the dual cast as the 1x128 and 128x1 oracle calls)"}
    if emit_line:
        emit(args, out)
    return out


def quant_stress_summary(args, np, torch, fgb, wl):
    """The quant_stress measurement (20 cold launches of each quantizer after 5
    warm-ups, no CPU baseline), condensed for another workload's line."""
    sub = argparse.Namespace(**vars(args))
    sub.steps, sub.warmup, sub.no_cpu_baseline, sub.copy_calibration = 20, 5, True, False
    q = quant_stress_main(sub, np, torch, fgb, wl, emit_line=False)
    return {"what": q["config"]["workload"] + " (20 cold launches per kernel after 5 warm-ups)",
            "GB/s": q["value"], "frac_hbm_peak": q["quant_frac_hbm_peak"],
            "kernels": {k: {"us": v["us"], "GB/s": v["GB/s"], "frac_hbm_peak": v["frac_hbm_peak"],
                            "frac_of_copy": v["frac_of_copy"]} for k, v in q["kernels"].items()},
            "copy_reference_frac_hbm_peak": q["copy_reference"]["frac_hbm_peak"],
            "copy_reference_1to1_frac_hbm_peak": q["copy_reference_1to1"]["frac_hbm_peak"]}


def make_runner(torch, dev, kernels, overlap):
    """step(events=None) launching `kernels` (name, fn, work, lane, deps) once.
    overlap: lane-1 kernels go to a second stream (default priority); a kernel
    waits for the events of its deps on the other stream; the second stream
    first waits for everything the main stream has queued (the previous step),
    and the main stream finally waits for the second.  events[i] = (start, end)
    timing events recorded on kernel i's stream."""
    main_s = torch.cuda.current_stream(dev)
    side_s = torch.cuda.Stream(dev) if overlap else main_s
    lane_of = {name: lane for name, _, _, lane, _ in kernels}
    done = {name: torch.cuda.Event() for name, _, _, _, _ in kernels}

    def step(events=None):
        if overlap:
            side_s.wait_stream(main_s)
        for i, (name, fn, _, lane, deps) in enumerate(kernels):
            s = side_s if overlap and lane == 1 else main_s
            with torch.cuda.stream(s):
                if overlap:
                    for dname in deps:
                        if lane_of[dname] != lane:
                            s.wait_event(done[dname])
                if events is not None:
                    events[i][0].record(s)
                fn()
                if events is not None:
                    events[i][1].record(s)
                if overlap:
                    done[name].record(s)
        if overlap:
            main_s.wait_stream(side_s)
    return step


def prefixed(kernels, p):
    """The same kernel list with every name (and dependency) prefixed by p."""
    return [(p + n, fn, work, lane, [p + x for x in deps]) for n, fn, work, lane, deps in kernels]


def cpu_model():
    """(model name, logical CPUs) of the host, from /proc/cpuinfo."""
    name, n = "unknown", 0
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name") and name == "unknown":
                    name = line.split(":", 1)[1].strip()
                if line.startswith("processor"):
                    n += 1
    except OSError:
        pass
    return name, n or os.cpu_count()


def _probe_lib():
    import ctypes
    path = os.path.join(ROOT, "fine_grained_block_amd", "libfgb_probe.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    L.fgb_probe_clock.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    L.fgb_probe_clock.restype = ctypes.c_int
    L.fgb_probe_clock_begin.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_void_p]
    L.fgb_probe_clock_begin.restype = ctypes.c_int
    L.fgb_probe_clock_end.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    L.fgb_probe_clock_end.restype = ctypes.c_int
    L.fgb_probe_staging.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    L.fgb_probe_staging.restype = ctypes.c_int
    return L


def probe_staging(torch, dev, iters=20000):
    """Per-compute-unit cycles per 128-deep block of the GEMM's staging traffic
    (libfgb_probe.so: the 256x256 tile's fragment reads, its direct-to-LDS
    operand loads, both), beside the 2048 cycles its MFMAs take at the peak
    rate; None if the probe is missing."""
    import ctypes
    L = _probe_lib()
    if L is None:
        return None
    cyc = (ctypes.c_double * 3)()
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    if L.fgb_probe_staging(iters, cyc, st) != 0:
        return None
    reads, dma, both = cyc[0], cyc[1], cyc[2]
    return {"what": "one 256x256 tile per CU, per 128-deep block: cycles of the fragment reads alone (192 KB "
                    "ds_read_b128), of the direct-to-LDS operand loads alone (64 KB global_load_lds_dwordx4 "
                    "from L2), of both; the block's 64 FP8 MFMAs per SIMD take 2048 cycles at the peak rate",
            "mfma_cycles": 2048, "read_cycles": round(reads, 1), "dma_cycles": round(dma, 1),
            "both_cycles": round(both, 1), "read_B_per_clk": round(192 * 1024 / reads, 1),
            "dma_B_per_clk": round(64 * 1024 / dma, 1)}


def gemm_operands(torch, b, prefix=""):
    """Each step GEMM's E4M3 operands as (A [rows, contraction], B [cols,
    contraction], output dtype), from a linear step's buffers."""
    return {prefix + "gemm_fprop": (b["qx"], b["qwT"], torch.bfloat16),
            prefix + "gemm_dgrad": (b["qdy"], b["qw"], torch.bfloat16),
            prefix + "gemm_wgrad": (b["qxT"], b["qdyT"], torch.float32)}


def blas_reference(torch, dev, ops, work):
    """hipBLASLt's plain FP8 GEMM (torch._scaled_mm, one tensor-wide scale of 1,
    no per-block rescale) on each step GEMM's own E4M3 operands and output
    dtype: a reference for what the matrix core reaches without the block
    scaling, timed back to back (median of 3 x 10 launches)."""
    out = {}
    one = torch.tensor(1.0, device=dev)
    f8 = torch.float8_e4m3fn
    for name, (a, b, odt) in ops.items():
        fn = lambda: torch._scaled_mm(a.view(f8), b.view(f8).t(), scale_a=one, scale_b=one, out_dtype=odt)
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 100.0)
        us = sorted(ts)[1]
        rate = work[name]["flop"] / (us * 1e-6)
        out[name] = {"us": round(us, 1), "TFLOP/s": round(rate / 1e12, 1), "frac_fp8_peak": round(rate / FP8_PEAK, 4)}
    return out


def probe_clock_mhz(torch, dev, iters=200000):
    """Median shader clock (MHz) over the CUs while every SIMD runs FP8 MFMAs
    and nothing else (libfgb_probe.so, built beside libfgb.so), or None if the
    probe is missing."""
    import ctypes
    L = _probe_lib()
    if L is None:
        return None
    mhz = ctypes.c_double(0.0)
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    if L.fgb_probe_clock(iters, ctypes.byref(mhz), st) != 0:
        return None
    return mhz.value


def clock_during_mhz(torch, dev, fn, kernel_ms, reps=3):
    """Median shader clock (MHz) while `fn` (one kernel launch) runs back to
    back: the kernel is queued on the current stream for about 4 windows, then
    single-wave sleeping samplers on a second stream (default priority) read
    s_memtime against the constant-rate counter over one window; the median of
    `reps` such samples.  None if the probe is missing."""
    import ctypes
    L = _probe_lib()
    if L is None:
        return None
    main_s = torch.cuda.current_stream(dev)
    side_s = torch.cuda.Stream(dev)
    window_us = max(200.0, min(2000.0, 2.0 * kernel_ms * 1e3))
    launches = max(4, int(4 * window_us / (kernel_ms * 1e3)) + 1)
    out = []
    for _ in range(reps):
        torch.cuda.synchronize()
        for _ in range(launches):
            fn()
        st = ctypes.c_void_p(side_s.cuda_stream)
        if L.fgb_probe_clock_begin(64, window_us, st) != 0:
            torch.cuda.synchronize()
            return None
        mhz = ctypes.c_double(0.0)
        rc = L.fgb_probe_clock_end(ctypes.byref(mhz), st)
        torch.cuda.synchronize()
        if rc != 0:
            return None
        out.append(mhz.value)
    return float(sorted(out)[len(out) // 2])


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(multi-GPU sharding is a design note only).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fine_grained_block_amd as fgb
    from fine_grained_block_amd import workloads as wl

    if args.workload == "quant_stress":
        quant_stress_main(args, np, torch, fgb, wl)
        return
    dev = torch.device("cuda:0")
    ue8m0 = args.recipe == "ue8m0"
    sr = args.rounding == "sr"
    if (ue8m0 or sr) and args.workload != "linear_dsv3_attn":
        print("bench.py: --recipe ue8m0 and --rounding sr apply to --workload linear_dsv3_attn", file=sys.stderr)
        sys.exit(2)
    cpu_inputs = None
    blas_ops = None
    if args.workload == "ffn_dense":
        up, down = wl.ffn_dense_up(), wl.ffn_dense_down()
        bu, bd = {}, {}
        kernels = prefixed(linear_step(fgb, torch, dev, up, bufs=bu), "up.") + \
            prefixed(linear_step(fgb, torch, dev, down, bufs=bd), "down.")
        blas_ops = {**gemm_operands(torch, bu, "up."), **gemm_operands(torch, bd, "down.")}
        config = {"workload": "ffn_dense fwd+bwd: up X[8192,7168] (Student-t(3)) W_up[7168,18432] "
                              "dY_up[8192,18432]; down H[8192,18432] (Student-t(3)) W_down[18432,7168] "
                              "dY_down[8192,7168]; 6 GEMMs, contraction up to 18432 (144 blocks)",
                  "M": up["M"], "d_model": up["K"], "d_ff": up["N"], "scales": "fp32", "rounding": "rn"}
        data = "synthetic (seeded Student-t(3) X and H, N(0,0.02) W, N(0,1e-3) dY; bf16)"
        cpu_inputs = ("ffn_dense", (up, down))
    elif args.workload == "linear_dsv3_attn":
        d = wl.linear_dsv3_attn()
        if ue8m0 and sr:
            print("bench.py: stochastic rounding uses absmax/448 scales (--recipe fp32)", file=sys.stderr)
            sys.exit(2)
        two_stage = ue8m0 and args.ue8m0_weights == "two-stage"
        bl = {}
        kernels = linear_step(fgb, torch, dev, d, separate_dy=args.separate_dy_casts, ue8m0=ue8m0, sr=sr,
                              two_stage=two_stage, bufs=bl)
        blas_ops = gemm_operands(torch, bl)
        config = {"workload": "linear_dsv3_attn fwd+bwd: X[4096,7168] W[7168,7168] dY[4096,7168]"
                              + (", power-of-two (UE8M0) scales" if ue8m0 else "")
                              + (" with the two-stage weight cast" if two_stage else "")
                              + (", stochastic rounding of the X, W and dY casts" if sr else ""),
                  "M": d["M"], "K": d["K"], "N": d["N"], "scales": args.recipe, "rounding": args.rounding}
        data = "synthetic (seeded N(0,0.02) X and W, N(0,1e-3) dY; bf16)"
        cpu_inputs = ("linear_dsv3_attn", d)
    else:
        d = wl.moe_grouped()
        kernels = moe_step(fgb, torch, dev, d)
        config = {"workload": "moe_grouped SwiGLU FFN fwd+bwd, one GPU's expert share: 32 experts, 8192 tokens "
                              "top-8 (Zipf 1.1 loads, 3 empty), W_gate/up [7168,2x2048], W_down [2048,7168] per "
                              "expert, SwiGLU casts fused",
                  "experts": d["E"], "routed_rows": int(np.sum(d["loads"])), "R_pad": d["R_pad"]}
        data = "synthetic (seeded N(0,1) X, N(0,0.02) W, N(0,1e-3) dY; bf16)"
        cpu_inputs = ("moe_grouped", d)

    overlap = args.schedule == "overlap"
    step = make_runner(torch, dev, kernels, overlap)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: per-kernel HIP events on the stream each kernel runs on
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in kernels] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for s in range(args.steps):
        step(ev[s])
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps
    per_kernel_ms = {name: float(np.mean([ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)]))
                     for i, (name, _, _, _, _) in enumerate(kernels)}
    work = {name: w for name, _, w, _, _ in kernels}

    # cold-cache step times, labelled as such: 10 warm-ups, then the median of 50
    # steps, each after a 1 GiB read scrub (outside its events) that evicts L2
    # and the 256 MB Infinity Cache
    cold = None
    if args.cold_iters > 0:
        scrub = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        sink = torch.empty((), dtype=torch.float32, device=dev)
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        cst, cev = [], []
        for _ in range(args.cold_iters):
            torch.sum(scrub, dim=(0,), out=sink)
            e = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in kernels]
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            step(e)
            b.record()
            torch.cuda.synchronize()
            cst.append(a.elapsed_time(b))
            cev.append([x.elapsed_time(y) for x, y in e])
        del scrub
        cold = {"what": f"median of {args.cold_iters} steps after 10 warm-ups, each step after a 1 GiB read "
                        "scrub outside its events (L2 and Infinity Cache cold at the step's start)",
                "ms_per_step": round(float(np.median(cst)), 4),
                "kernels_us": {name: round(float(np.median([c[i] for c in cev])) * 1e3, 2)
                               for i, (name, _, _, _, _) in enumerate(kernels)}}

    step_flop = sum(w.get("flop", 0.0) for w in work.values())
    quant_bytes = sum(w.get("bytes", 0) for w in work.values())
    value = step_flop / (ms_per_step * 1e-3) / 1e12
    kinfo = {}
    for name, ms in per_kernel_ms.items():
        if "flop" in work[name]:
            rate = work[name]["flop"] / (ms * 1e-3)
            kinfo[name] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(rate / 1e12, 1),
                           "frac_fp8_peak": round(rate / FP8_PEAK, 4)}
            if "roofline_us" in work[name]:
                # grouped: the per-expert max(compute, memory) bound summed over experts
                kinfo[name]["roofline_us"] = round(work[name]["roofline_us"], 1)
                kinfo[name]["frac_of_roofline"] = round(work[name]["roofline_us"] / (ms * 1e3), 4)
                kinfo[name]["experts_memory_bound"] = work[name]["experts_memory_bound"]
        else:
            rate = work[name]["bytes"] / (ms * 1e-3)
            kinfo[name] = {"us": round(ms * 1e3, 2), "GB/s": round(rate / 1e9, 1),
                           "frac_hbm_peak": round(rate / HBM_PEAK, 4), "bytes": work[name]["bytes"]}
    gemms = {k: v for k, v in per_kernel_ms.items() if "flop" in work[k]}
    dom = max(gemms, key=gemms.get)
    dom_rate = work[dom]["flop"] / (gemms[dom] * 1e-3)
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(dom_rate / 1e12, 1),
                "peak": FP8_PEAK / 1e12, "unit": "TFLOP/s", "frac": round(dom_rate / FP8_PEAK, 4),
                "traffic": traffic_record(dom)}
    # the shader clock while each GEMM runs back to back, and the GEMM's rate
    # against the MFMA peak at that clock
    fns = {name: fn for name, fn, _, _, _ in kernels}
    for name in gemms:
        c = clock_during_mhz(torch, dev, fns[name], gemms[name])
        if c:
            kinfo[name]["clock_mhz"] = round(c, 1)
            kinfo[name]["frac_at_clock"] = round(work[name]["flop"] / (gemms[name] * 1e-3) / (FP8_PEAK * c / 2400.0), 4)
    mhz = kinfo[dom].get("clock_mhz")
    mhz_probe = probe_clock_mhz(torch, dev)
    if mhz:
        # the MFMA peak scales with the clock: 5.0 PFLOP/s is quoted at 2.4 GHz
        roofline["clock_mhz"] = round(mhz, 1)
        roofline["frac_at_clock"] = round(dom_rate / (FP8_PEAK * mhz / 2400.0), 4)
        roofline["clock_how"] = ("median shader clock while the kernel runs back to back (sleeping "
                                 "single-wave samplers beside it: s_memtime ticks per s_memrealtime time)")
    if mhz_probe:
        roofline["clock_mhz_mfma_only"] = round(mhz_probe, 1)
    staging = probe_staging(torch, dev)
    if staging:
        roofline["staging_probe"] = staging
    want_blas = args.blas_reference or (args.workload == "ffn_dense" and not args.no_blas_reference)
    if want_blas and blas_ops is not None:
        blas_ops = {n: o for n, o in blas_ops.items() if n in kinfo}
        try:
            for name, v in blas_reference(torch, dev, blas_ops, work).items():
                kinfo[name]["hipblaslt_plain_fp8"] = v
        except Exception as e:      # a reference only: its failure must not cost the line
            roofline["hipblaslt_plain_fp8_error"] = f"{type(e).__name__}: {str(e)[:160]}"
    quant_ms = sum(v for k, v in per_kernel_ms.items() if "bytes" in work[k])
    config.update({"gemm_flop_per_step": step_flop, "quant_bytes_per_step": quant_bytes,
                   "schedule": ("overlap: casts " + ", ".join(n for n, _, _, lane, _ in kernels if lane == 1)
                                + " on a second stream") if overlap else "serial: one stream"})

    out = {
        "metric": "block-scaled FP8 GEMM TFLOP/s (% FP8 MFMA peak) + quant GB/s (% HBM) at 1 GPU",
        "value": round(value, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 x e4m3 -> fp32 accumulate (bf16 in/out, fp32 dW)",
        "data": data,
        "config": config,
        "quant_GBps": round(quant_bytes / (quant_ms * 1e-3) / 1e9, 1),
        "quant_frac_hbm_peak": round(quant_bytes / (quant_ms * 1e-3) / HBM_PEAK, 4),
        "roofline": roofline,
        "kernels": kinfo,
    }
    if cold is not None:
        cold["TFLOP/s"] = round(step_flop / (cold["ms_per_step"] * 1e-3) / 1e12, 1)
        out["cold"] = cold
    if args.workload == "ffn_dense" and not args.no_quant_stress:
        # the quantizers' HBM row on the stress tensor, so that this line carries it too
        out["quant_stress"] = quant_stress_summary(args, np, torch, fgb, wl)

    if args.copy_calibration:
        a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        c = torch.empty_like(a)
        for _ in range(3):          # elementwise: each launch reads 1 GiB and writes 1 GiB
            torch.neg(a, out=c)
        torch.cuda.synchronize()
        del a, c

    if not args.no_cpu_baseline:
        kind, inp = cpu_inputs
        if kind == "linear_dsv3_attn":
            out["cpu_baseline"] = cpu_baseline(inp, args.cpu_rows, ue8m0, sr)
        elif kind == "ffn_dense":
            out["cpu_baseline"] = cpu_baseline_tiles_linear(list(inp), args.cpu_tile_frac)
        else:
            out["cpu_baseline"] = cpu_baseline_tiles_moe(inp, args.cpu_tile_frac)
    emit(args, out)


def tile_sample(n, frac, g):
    """Element indices of a seeded sample of the 128-wide tiles of range(n):
    about frac of them (at least one), always the first and the last tile."""
    nt = -(-n // T)
    k = max(1, int(round(frac * nt)))
    pick = {0, nt - 1} if k >= 2 else {0}
    rest = [t for t in range(nt) if t not in pick]
    extra = max(0, k - len(pick))
    if extra and rest:
        pick |= set(g.choice(rest, size=min(extra, len(rest)), replace=False).tolist())
    idx = np.concatenate([np.arange(t * T, min(n, t * T + T)) for t in sorted(pick)])
    return idx.astype(np.int64), len(pick), nt


def host_info(oracle):
    model, ncpu = cpu_model()
    return {"cores": oracle.max_threads(), "cpu_model": model, "nproc": ncpu}


def quant_t1(oracle, x_bits):
    """GB/s of the oracle's 1x128 quantizer on x_bits with one thread."""
    threads = oracle.max_threads()
    oracle.set_num_threads(1)
    try:
        t = time.perf_counter()
        oracle.quantize_1x128(x_bits)
        dt = time.perf_counter() - t
    finally:
        oracle.set_num_threads(threads)
    R, C = x_bits.shape
    return {"quant_T1_GBps": round((R * C * 3 + 4 * R * (-(-C // T))) / dt / 1e9, 3),
            "quant_T1_what": f"oracle quantize_1x128 of [{R},{C}] on one thread ({dt:.2f} s)"}


def cpu_baseline_tiles_linear(ds, frac):
    """The CPU oracle on a seeded sample of the dense linears' output tiles:
    quantizers on the full tensors, then for every linear the Fprop, Dgrad and
    Wgrad outputs of frac of the 128x128 output tiles (half the tile rows x a
    quarter of the tile columns at frac = 1/8, first and last tiles included),
    each over the full contraction.  value = sampled GEMM FLOP / GEMM time."""
    import oracle
    g = np.random.default_rng(0)
    fr, fc = np.sqrt(frac * 2.0), np.sqrt(frac / 2.0)     # 1/2 x 1/4 at frac = 1/8
    tq = tg = 0.0
    qbytes = flop = 0.0
    parts = []
    for d in ds:
        M, K, N = d["M"], d["K"], d["N"]
        t0 = time.perf_counter()
        qx, sx = oracle.quantize_1x128(d["x"])
        q, qT, sw = oracle.quantize_128x128(d["w"])
        qdy, sdy = oracle.quantize_1x128(d["dy"])
        qdyT, sdyT = oracle.quantize_128x1(d["dy"])
        qxT, sxT = oracle.requant_128x1(qx, sx)
        tq += time.perf_counter() - t0
        qbytes += sum(v for k, v in algorithmic_bytes(M, K, N).items()
                      if k in ("quantize_1x128_x", "quantize_128x128_w", "quantize_1x128_dy",
                               "quantize_128x1_dy", "requant_128x1_x"))
        rows, nrt, ntm = tile_sample(M, fr, g)
        colsN, nct, ntn = tile_sample(N, fc, g)
        colsK, nck, ntk = tile_sample(K, fc, g)
        rowsK, nrk, _ = tile_sample(K, fr, g)
        t0 = time.perf_counter()
        oracle.gemm_fprop(qx, sx, qT, sw, rows=rows, cols=colsN)
        oracle.gemm_dgrad(qdy, sdy, q, sw, rows=rows, cols=colsK)
        oracle.gemm_wgrad(qxT, sxT, qdyT, sdyT, M, rows=rowsK, cols=colsN)
        tg += time.perf_counter() - t0
        flop += 2.0 * rows.size * colsN.size * K + 2.0 * rows.size * colsK.size * N + 2.0 * rowsK.size * colsN.size * M
        parts.append(f"[{M}x{K}x{N}] Fprop {nrt}/{ntm} x {nct}/{ntn} tiles, Dgrad {nrt}/{ntm} x {nck}/{ntk}, "
                     f"Wgrad {nrk}/{ntk} x {nct}/{ntn}")
    out = {"value": round(flop / tg / 1e12, 6), "unit": "TFLOP/s", "kind": "oracle",
           "sample": f"quantizers on the full tensors ({tq:.1f} s); GEMMs on a seeded sample of about {frac:g} of "
                     "the 128x128 output tiles, first and last tile rows and columns included, full contraction "
                     f"({tg:.1f} s): " + "; ".join(parts) + ". value = sampled GEMM FLOP / GEMM time",
           "sample_fraction": round(flop / sum(6.0 * d["M"] * d["K"] * d["N"] for d in ds), 4),
           "quant_GBps": round(qbytes / tq / 1e9, 3), "quant_s": round(tq, 2)}
    out.update(host_info(oracle))
    out.update(quant_t1(oracle, ds[0]["x"]))
    return out


def cpu_baseline_tiles_moe(d, frac):
    """The CPU oracle on one GPU's MoE expert share: the 1x128/128x1 casts of
    the grouped activations and gradients and both projections' expert weights
    on the full tensors, then the grouped Fprop, Dgrad and Wgrad of both
    projections on a seeded sample of about frac of every expert's 128x128
    output tiles (each expert's first and last tile rows, the first and last
    tile columns).  The backward GEMMs take the workload's dY tensors as their
    gradients.  value = sampled GEMM FLOP (routed rows) / GEMM time."""
    import oracle
    g = np.random.default_rng(0)
    fr, fc = np.sqrt(frac * 2.0), np.sqrt(frac / 2.0)
    offsets, loads, E = np.asarray(d["offsets"]), np.asarray(d["loads"]), d["E"]
    Dm, F2, F = d["d_model"], d["d_ff2"], d["d_ff"]
    t0 = time.perf_counter()
    qx, sx = oracle.quantize_1x128(d["x"])
    qxT, sxT = oracle.requant_128x1(qx, sx)
    qh, sh = oracle.quantize_1x128(d["h"])
    qhT, shT = oracle.requant_128x1(qh, sh)
    qdu, sdu = oracle.quantize_1x128(d["dy_up"])
    qduT, sduT = oracle.quantize_128x1(d["dy_up"])
    qdd, sdd = oracle.quantize_1x128(d["dy_down"])
    qddT, sddT = oracle.quantize_128x1(d["dy_down"])
    wu = [oracle.quantize_128x128(w) for w in d["w_up"]]
    wd = [oracle.quantize_128x128(w) for w in d["w_down"]]
    tq = time.perf_counter() - t0
    qwu, qwuT, swu = (np.stack([w[k] for w in wu]) for k in range(3))
    qwd, qwdT, swd = (np.stack([w[k] for w in wd]) for k in range(3))
    # rows: per expert, a sample of its own row tiles (its first and last included)
    rows, valid_rows = [], 0
    for e in range(E):
        a, n = int(offsets[e]), int(loads[e])
        if n == 0:
            continue
        idx, _, _ = tile_sample(n, fr, g)
        rows.append(a + idx)
        valid_rows += idx.size
    rows = np.concatenate(rows)
    cu, _, _ = tile_sample(F2, fc, g)          # gate/up output columns
    cd, _, _ = tile_sample(Dm, fc, g)          # down output columns / gate-up Dgrad columns
    cf, _, _ = tile_sample(F, fc, g)           # down Dgrad columns
    kD, _, _ = tile_sample(Dm, fr, g)          # Wgrad rows (gate/up: d_model)
    kF, _, _ = tile_sample(F, fr, g)           # Wgrad rows (down: d_ff)
    t0 = time.perf_counter()
    oracle.gemm_fprop_grouped(offsets, qx, sx, qwuT, swu, rows=rows, cols=cu)
    oracle.gemm_fprop_grouped(offsets, qh, sh, qwdT, swd, rows=rows, cols=cd)
    oracle.gemm_dgrad_grouped(offsets, qdd, sdd, qwd, swd, rows=rows, cols=cf)
    oracle.gemm_dgrad_grouped(offsets, qdu, sdu, qwu, swu, rows=rows, cols=cd)
    oracle.gemm_wgrad_grouped(offsets, qhT, shT, qddT, sddT, rows=kF, cols=cd)
    oracle.gemm_wgrad_grouped(offsets, qxT, sxT, qduT, sduT, rows=kD, cols=cu)
    tg = time.perf_counter() - t0
    routed = int(loads.sum())
    flop = (2.0 * valid_rows * (cu.size * Dm + cd.size * F + cf.size * Dm + cd.size * F2)
            + 2.0 * routed * (kF.size * cd.size + kD.size * cu.size))
    total = 2.0 * routed * Dm * F2 * 3 + 2.0 * routed * F * Dm * 3     # Fprop+Dgrad+Wgrad, both projections
    out = {"value": round(flop / tg / 1e12, 6), "unit": "TFLOP/s", "kind": "oracle",
           "sample": f"casts of X, H, both dY and all {E} experts' weights on the full tensors ({tq:.1f} s); "
                     f"grouped GEMMs of both projections on a seeded sample of about {frac:g} of every expert's "
                     f"128x128 output tiles ({valid_rows} of {routed} routed rows x about {fc:.2f} of the columns; "
                     f"Wgrad about {fr:.2f} x {fc:.2f} of each expert's tiles), full contraction ({tg:.1f} s). "
                     "value = sampled GEMM FLOP over routed rows / GEMM time",
           "sample_fraction": round(flop / total, 4),
           "quant_s": round(tq, 2)}
    out.update(host_info(oracle))
    out.update(quant_t1(oracle, d["x"][:8192]))
    return out


def cpu_baseline(d, rows_arg, ue8m0=False, sr=False):

    """The CPU oracle, as it stands, on a bounded sample of the same step: the
    three quantizers of X/dY and W on full tensors, then Fprop, Dgrad and Wgrad
    on a sample of output rows (all columns, full contraction).  Reported as the
    oracle's GEMM throughput in TFLOP/s over the sample, plus its quant GB/s."""
    import numpy as np

    import oracle
    M, K, N = d["M"], d["K"], d["N"]
    t0 = time.perf_counter()
    if ue8m0:
        dec = lambda e: oracle.e8m0_decode(e).astype(np.float32)
        qx, ex = oracle.quantize_1x128_ue8m0(d["x"])
        q, qT, ew = oracle.quantize_128x128_ue8m0(d["w"])
        qdy, edy = oracle.quantize_1x128_ue8m0(d["dy"])
        qdyT, edyT = oracle.quantize_128x1_ue8m0(d["dy"])
        qxT, exT = oracle.requant_128x1_ue8m0(qx, ex)
        sx, sw, sdy, sdyT, sxT = dec(ex), dec(ew), dec(edy), dec(edyT), dec(exT)
    elif sr:
        qx, sx = oracle.quantize_1x128_sr(d["x"], 0x5EED, 1)
        q, qT, sw = oracle.quantize_128x128_sr(d["w"], 0x5EED, 2)
        qdy, sdy = oracle.quantize_1x128_sr(d["dy"], 0x5EED, 3)
        qdyT, sdyT = oracle.quantize_128x1_sr(d["dy"], 0x5EED, 3)
        qxT, sxT = oracle.requant_128x1(qx, sx)
    else:
        qx, sx = oracle.quantize_1x128(d["x"])
        q, qT, sw = oracle.quantize_128x128(d["w"])
        qdy, sdy = oracle.quantize_1x128(d["dy"])
        qdyT, sdyT = oracle.quantize_128x1(d["dy"])
        qxT, sxT = oracle.requant_128x1(qx, sx)
    tq = time.perf_counter() - t0
    qbytes = sum(algorithmic_bytes(M, K, N).values())
    # size the GEMM sample so the oracle works ~15 s: time a 1/128 slice of each
    # GEMM's output rows first, then take the fraction f of the rows (f <= 1: the
    # whole step) that the target allows
    def run(frac, seed):
        g = np.random.default_rng(seed)
        nr, nk = max(1, int(round(frac * M))), max(1, int(round(frac * K)))
        rows = np.sort(g.choice(M, size=nr, replace=False))
        rowsK = np.sort(g.choice(K, size=nk, replace=False))
        t = time.perf_counter()
        oracle.gemm_fprop(qx, sx, qT, sw, rows=rows)
        oracle.gemm_dgrad(qdy, sdy, q, sw, rows=rows)
        oracle.gemm_wgrad(qxT, sxT, qdyT, sdyT, M, rows=rowsK)
        return time.perf_counter() - t, nr, nk

    frac = min(1.0, rows_arg / M) if rows_arg > 0 else None
    if frac is None:
        tp, _, _ = run(1.0 / 128, 1)
        frac = min(1.0, (1.0 / 128) * 15.0 / max(tp, 1e-6))
    tg, nr, nk = run(frac, 0)
    flop = 2.0 * nr * N * K + 2.0 * nr * K * N + 2.0 * nk * N * M
    what = "the whole step" if nr == M and nk == K else f"{nr}/{M} Fprop and Dgrad rows, {nk}/{K} Wgrad rows"
    return {"value": round(flop / tg / 1e12, 6), "unit": "TFLOP/s", "kind": "oracle",
            "sample": f"quantizers on the full tensors ({tq:.1f} s), then GEMMs over {what} "
                      f"(all columns, full contraction; {tg:.1f} s); value = GEMM FLOP / GEMM time",
            "quant_GBps": round(qbytes / tq / 1e9, 3), "quant_s": round(tq, 2),
            **host_info(oracle), **quant_t1(oracle, d["x"])}


if __name__ == "__main__":
    main()
