"""Benchmark of the dense long-sequence attention hot path on one MI355X.

One step = the whole path over one batch of synthetic input at the 15-second
clip scale (H = 40 heads, L = 109,000 tokens, d = 128):
  attn_fwd_bf16 on the BF16 workload (N(0,1), 3 of 128 channels x20 on Q, K),
  qk_prep_fp4 + attn_fwd_fp4qk on the FP4 workload (Student-t(3) Q, K with the
  same outliers, N(0,1) V).
value = attention FLOP of the step (2 x 4 H L^2 d) / step time, TFLOP/s.
Prints ONE JSON line (rank 0).  Inputs are resident in HBM before timing.
After the timed steps (outside them) the line also carries the extra paths
(fused-Q FP4, the backward, the NVFP4 linear, the other configurations), the
CPU oracle baseline and the standalone matrix-core probe's sustained BF16 MFMA
rate for random and all-zero operands (the attainable ceiling under this GPU's
power limit, against which roofline.achieved is also read).  The shader
clock and socket power are sampled with amd-smi while the timed steps run.  The step's prep
follows the BF16 launch, which streams 2.2 GB of other tensors through the
256 MB memory-side cache, so it starts cold; the separately timed
memory-bound calls (K-only prep, NVFP4 quantizer) are each preceded by a
512 MB write that evicts that cache, outside the timed interval.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--no-mfma-ceiling] [--mfma-ceiling]
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense BF16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
COPY_PROBE_BYTES = 1 << 30    # plain copy of known size that calibrates FETCH_SIZE / WRITE_SIZE
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_bf16_traffic.json")
METRIC = "attention TFLOP/s and % of MFMA peak at 109k tokens, BF16 and FP4-QK paths"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attn_flop(H, L, d=128):
    return 4.0 * H * float(L) * float(L) * d


def prep_bytes(H, L, d=128):
    # read Q and K once (2 B each) + write codes (d/2 B) and scales (d/16 B) for both
    return H * L * (2 * 2 * d + 2 * (d // 2 + d // 16))


def gen_inputs(torch, name):
    from long_sequence_dense_amd import inputs
    cfg = inputs.CONFIGS[name]
    out = {}
    for which in ("q", "k", "v"):
        t0 = time.time()
        bits = inputs.make_tensor(cfg, which)
        out[which] = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        del bits
        log("  %s.%s generated and uploaded in %.1f s" % (name, which, time.time() - t0))
    return cfg, out


KERNEL_SOURCES = ("attn_fwd.hip", "device_common.h", "nvfp4_quant.h", "lsd_internal.h")


def kernel_source_hash():
    """sha256 of the attention kernel's sources (the kernel file and the
    headers it includes) with comments and blank lines removed:
    counter-derived traffic is only reported for the code it was measured on."""
    import hashlib
    import re
    code = []
    for name in KERNEL_SOURCES:
        src = os.path.join(ROOT, "long_sequence_dense_amd", "csrc", name)
        lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in open(src).read().splitlines())
        code.append("\n".join(ln for ln in lines if ln))
    return hashlib.sha256("\n".join(code).encode()).hexdigest()


def stored_traffic():
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        t = json.load(open(TRAFFIC_FILE))
    except Exception:
        return None
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(H, L, d, gpu_rows=None):
    """Time the CPU oracle (as it stands) on a bounded sample of the workload
    (about 15 s of CPU work on 16 cores) and extrapolate a full step; returns
    the cpu_baseline object.  ``gpu_rows(name, heads, rows)`` returns the GPU
    step's outputs (float64) for those rows: the oracle values computed here
    are then also compared with them (``parity``)."""
    from long_sequence_dense_amd import inputs
    from oracle.attention import attention_fp64
    from oracle.nvfp4 import dequant_nvfp4, qk_prep_fp4
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    cfg = inputs.CONFIGS["clip15s"]
    heads = [0, 1]
    rows = inputs.sample_rows(L, 12288)
    q = inputs.make_tensor(cfg, "q", heads)
    k = inputs.make_tensor(cfg, "k", heads)
    v = inputs.make_tensor(cfg, "v", heads)
    f = lambda b: inputs.bf16_bits_to_f32(b).astype(np.float64)
    t0 = time.time()
    oref, _ = attention_fp64(f(q), f(k), f(v), cfg.scale, rows=rows)
    t_attn = time.time() - t0
    attn_rate = len(heads) * len(rows) * 4.0 * L * d / t_attn          # FLOP/s
    fcfg = inputs.CONFIGS["fp4"]
    prep_heads = [0, 1, 2, 3]
    qf = inputs.make_tensor(fcfg, "q", prep_heads)
    kf = inputs.make_tensor(fcfg, "k", prep_heads)
    t0 = time.time()
    ref = qk_prep_fp4(qf, kf)
    t_prep = time.time() - t0
    t_prep_head = t_prep / len(prep_heads)
    full_attn_s = attn_flop(H, L, d) / attn_rate
    step_s = 2 * full_attn_s + H * t_prep_head
    out = {
        "value": round(2 * attn_flop(H, L, d) / step_s / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": ("fp64 numpy oracle: BF16 attention for %d query rows x %d heads at L=%d "
                   "(%.1f s, %.2f GFLOP/s), NVFP4 prep of %d full heads of Q and K (%.1f s); "
                   "full step extrapolated to %.0f s (2 attention calls + %d heads of prep)"
                   % (len(rows), len(heads), L, t_attn, attn_rate / 1e9, len(prep_heads), t_prep,
                      step_s, H)),
    }
    if gpu_rows is not None:
        # Not timed: the same oracle rows against the GPU step's outputs, and
        # the FP4-QK error as a fraction of the quantization error on head 0:
        # ||O_gpu - O(same codes)|| / ||O(same codes) - O(exact)||.
        err = np.abs(gpu_rows("bf16", heads, rows) - oref)
        frows = inputs.sample_rows(L, 2048, seed=7)
        qh = dequant_nvfp4(ref["q_codes"][:1], ref["q_scales"][:1])
        kh = dequant_nvfp4(ref["k_codes"][:1], ref["k_scales"][:1])
        vf = f(inputs.make_tensor(fcfg, "v", [0]))
        o_same, _ = attention_fp64(qh, kh, vf, fcfg.scale, rows=frows)
        o_exact, _ = attention_fp64(f(qf[:1]), f(kf[:1]), vf, fcfg.scale, rows=frows)
        g5 = gpu_rows("fp4", [0], frows)
        e5 = np.abs(g5 - o_same)
        ratio = float(np.linalg.norm(g5 - o_same) / np.linalg.norm(o_same - o_exact))
        out["parity"] = {
            "attn_fwd_bf16": {"rows": "%d sampled rows x heads %s" % (len(rows), heads),
                              "max_abs": float(err.max()), "mean_abs": float(err.mean())},
            "attn_fwd_fp4qk": {"rows": "%d sampled rows of head 0" % len(frows),
                               "max_abs": float(e5.max()), "mean_abs": float(e5.mean()),
                               "error_over_quantization_error": ratio},
        }
    return out


LIN_M, LIN_N, LIN_K = 109000, 5120, 5120


def linear_operands(torch, dev):
    gen = torch.Generator(device=dev)
    gen.manual_seed(6)
    x = torch.randn((LIN_M, LIN_K), dtype=torch.float32, device=dev, generator=gen)
    ch = torch.randperm(LIN_K, generator=torch.Generator().manual_seed(6))[:round(0.02 * LIN_K)].to(dev)
    x[:, ch] *= 20.0
    x = x.to(torch.bfloat16)
    w = (torch.randn((LIN_N, LIN_K), dtype=torch.float32, device=dev, generator=gen) * LIN_K ** -0.5).to(torch.bfloat16)
    gx = float(x.float().abs().max().item()) / (6.0 * 448.0)
    gw = float(w.float().abs().max().item()) / (6.0 * 448.0)
    return x, w, gx, gw


def time_calls(torch, stream, fn, n=3, before=None):
    """One warm-up and n timed calls of fn on the launch stream (HIP events);
    `before`, if given, runs on the stream ahead of each call, outside the
    timed interval."""
    times = []
    for i in range(n + 1):
        if before is not None:
            before()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        b.synchronize()
        if i:
            times.append(a.elapsed_time(b))
    return sum(times) / len(times)


class MallFlush:
    """A 512 MB write on the launch stream: evicts the 256 MB memory-side
    cache, so that a separately timed memory-bound call cannot read its inputs
    from it warm from the previous call."""

    def __init__(self, torch, dev):
        self.buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        self.i = 0

    def __call__(self):
        self.i += 1
        self.buf.fill_(self.i & 0xFF)


class ClockSampler:
    """Samples the GPU's shader clock and socket power with `amd-smi metric -c
    -p` (the mean of the eight XCD clocks per sample) from a background thread
    while the timed steps run."""

    def __init__(self, interval=0.25, window="the timed steps (both attention launches and the prep)"):
        import threading
        self.interval = interval
        self.window = window
        self.samples = []
        self.error = None
        self.stop_event = threading.Event()
        self.thread = threading.Thread(target=self._run, daemon=True)

    def _one(self):
        import subprocess
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "-p", "--json"], stdout=subprocess.PIPE,
                           stderr=subprocess.PIPE, text=True, timeout=20)
        d = json.loads(r.stdout)["gpu_data"][0]
        vals = [float(v["clk"]["value"]) for k, v in d["clock"].items() if k.startswith("gfx_")]
        try:
            watts = float(d["power"]["socket_power"]["value"])
        except (KeyError, TypeError, ValueError):
            watts = None
        return sum(vals) / len(vals), watts

    def _run(self):
        while not self.stop_event.is_set():
            try:
                self.samples.append(self._one())
            except Exception as e:          # no amd-smi, other output: report the reason
                self.error = "%s: %s" % (type(e).__name__, e)
                return
            self.stop_event.wait(self.interval)

    def start(self):
        self.thread.start()
        return self

    def stop(self):
        self.stop_event.set()
        if self.thread.is_alive():
            self.thread.join(timeout=30)
        return self.summary()

    def summary(self):
        if not self.samples:
            return {"error": self.error or "no sample"}
        xs = [c for c, _ in self.samples]
        ws = [w for _, w in self.samples if w is not None]
        def median(v):
            v = sorted(v)
            return 0.5 * (v[(len(v) - 1) // 2] + v[len(v) // 2])
        rep = {"source": "amd-smi metric -c -p: mean of the 8 XCD shader clocks, socket power",
               "window": self.window,
               "samples": len(xs), "mean_mhz": round(sum(xs) / len(xs), 1), "median_mhz": round(median(xs), 1),
               "min_mhz": round(min(xs), 1), "max_mhz": round(max(xs), 1)}
        if ws:
            rep.update({"mean_socket_w": round(sum(ws) / len(ws), 1), "median_socket_w": round(median(ws), 1),
                        "max_socket_w": round(max(ws), 1)})
        return rep


def linear_path(torch, binding, stream, dev):
    x, w, gx, gw = linear_operands(torch, dev)
    M, N, K = LIN_M, LIN_N, LIN_K
    T = binding.NVFP4_TILED                      # the product's own load order
    xc, xs = binding.nvfp4_quantize(x, gx, layout=T, stream=stream)
    wc, ws = binding.nvfp4_quantize(w, gw, layout=T, stream=stream)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    flush = MallFlush(torch, dev)
    t_q = time_calls(torch, stream, lambda: binding.nvfp4_quantize(x, gx, xc, xs, layout=T, stream=stream),
                     before=flush)
    del flush
    t_l = time_calls(torch, stream, lambda: binding.nvfp4_linear(xc, xs, gx, wc, ws, gw, y, stream=stream,
                                                                 layout=T, M=M, N=N, K=K))
    assert not torch.isnan(y).any().item()
    qbytes = M * K * 2 + M * K // 2 + M * K // 16    # (the tiled padding of the last tile not counted)
    qg = qbytes / (t_q * 1e-3) / 1e9
    lf = 2.0 * M * N * K
    lt = lf / (t_l * 1e-3) / 1e12
    wl = "M=%d tokens, N=%d, K=%d" % (M, N, K)
    return {
        "nvfp4_quantize": {"ms": round(t_q, 4), "GB/s": round(qg, 1), "algorithmic_bytes": qbytes,
                           "frac_of_peak": round(qg / PEAK_HBM_GBS, 4), "workload": "X of " + wl + ", tiled code layout",
                           "in_value": False},
        "nvfp4_linear": {"ms": round(t_l, 3), "TFLOP/s": round(lt, 1), "algorithmic_flop": lf,
                         "frac_of_peak": round(lt / PEAK_BF16_TFLOPS, 4),
                         "mfma_precision": "fp16 (exact dequantization of NVFP4 X and W)",
                         "workload": wl + ", tiled code layout", "in_value": False},
    }


def config_path(torch, binding, stream, name, reps):
    """attn_fwd_bf16 on another configuration of the same method (not in
    value): seeded inputs generated on the host, one warm-up, ``reps`` timed
    calls on the launch stream."""
    cfg, x = gen_inputs(torch, name)
    o = torch.empty_like(x["q"])
    t = time_calls(torch, stream, lambda: binding.attn_fwd_bf16(x["q"], x["k"], x["v"], o, None, cfg.scale, stream),
                   n=reps)
    fl = attn_flop(cfg.H, cfg.L)
    tf = fl / (t * 1e-3) / 1e12
    del x, o
    return {"ms": round(t, 4), "TFLOP/s": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "workload": cfg.desc, "in_value": False}


def bw_ceiling():
    """Run the standalone HBM probe (built in-tree by the library's build
    step): read-only, copy and write-only passes with 16-byte accesses over a
    tensor of the prep's input size (1.116 GB) and its code and scale bytes,
    ordinary and non-temporal loads, the memory-side cache replaced by clean
    lines before each launch.  None if it is not built."""
    import subprocess
    exe = os.path.join(ROOT, "long_sequence_dense_amd", "hbm_ceiling_probe")
    if not os.path.exists(exe):
        log("hbm_ceiling_probe not built; skipped")
        return None
    log("running the HBM ceiling probe ...")
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    if r.returncode != 0:
        raise RuntimeError("hbm_ceiling_probe failed (%d): %s" % (r.returncode, r.stderr.strip()))
    return json.loads(r.stdout.strip().splitlines()[-1])


def operand_energy(torch, binding, stream, H, L, d, reps=20):
    """The shipped attn_fwd_bf16 on the same shape with different operand
    data: the 15-second inputs as generated, the same with V = 0 and with
    K = V = 0, and flat N(0,1) Q, K, V (no outlier channels).  Every case runs
    the same instructions; the shader clock and socket power are sampled
    during ``reps`` timed calls (after five untimed calls that bring the
    clock to its level under this load), so that cycles per launch (ms x
    median clock) and energy per launch (ms x median power) can be compared.
    Prints one JSON line."""
    cfg, x = gen_inputs(torch, "clip15s")
    o = torch.empty_like(x["q"])
    fl = attn_flop(H, L, d)
    gen = torch.Generator(device=x["q"].device)
    gen.manual_seed(11)

    def flat():
        return torch.randn((H, L, d), dtype=torch.float32, device=x["q"].device, generator=gen).to(torch.bfloat16)

    zeros = torch.zeros_like(x["v"])
    cases = [("15-second inputs as generated", lambda: (x["q"], x["k"], x["v"])),
             ("15-second inputs, V = 0", lambda: (x["q"], x["k"], zeros)),
             ("15-second inputs, K = V = 0", lambda: (x["q"], zeros, zeros)),
             ("flat N(0,1) Q, K, V", lambda: (flat(), flat(), flat()))]
    rows = []
    for name, make in cases:
        q, k, v = make()
        log("operand energy: %s ..." % name)
        for _ in range(5):
            binding.attn_fwd_bf16(q, k, v, o, None, cfg.scale, stream)
        torch.cuda.synchronize()
        sampler = ClockSampler(window="attn_fwd_bf16, " + name).start()
        t = time_calls(torch, stream, lambda: binding.attn_fwd_bf16(q, k, v, o, None, cfg.scale, stream), n=reps)
        clk = sampler.stop()
        row = {"inputs": name, "ms": round(t, 3), "TFLOP/s": round(fl / (t * 1e-3) / 1e12, 1), "clock": clk}
        if "median_mhz" in clk:
            row["mcycles_per_launch"] = round(t * clk["median_mhz"] / 1e3, 1)
        if "median_socket_w" in clk:
            row["socket_joules_per_launch"] = round(t * clk["median_socket_w"] / 1e3, 1)
            row["socket_pj_per_flop"] = round(t * 1e-3 * clk["median_socket_w"] / fl * 1e12, 3)
        rows.append(row)
        del q, k, v
    print(json.dumps({"operand_energy": rows, "kernel": "attn_fwd_bf16",
                      "shape": "H=%d, L=%d, d=%d" % (H, L, d), "calls_per_case": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=8)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mfma-ceiling", action="store_true",
                    help="skip the standalone MFMA ceiling probe (random vs zero operands) after the timed steps")
    ap.add_argument("--no-hbm-ceiling", action="store_true",
                    help="skip the standalone HBM ceiling probe (read-only, copy, write-only) after the timed steps")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only run the standalone MFMA ceiling probe and print its JSON line")
    ap.add_argument("--only", choices=["all", "bf16"], default="all",
                    help="bf16: time only attn_fwd_bf16 (for profiling runs)")
    ap.add_argument("--no-bwd", action="store_true",
                    help="skip the extra (not in value) timing of attn_bwd_bf16 and attn_bwd_fp4qk")
    ap.add_argument("--no-linear", action="store_true",
                    help="skip the extra (not in value) timing of the NVFP4 linear layer")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the extra (not in value) BF16 timings of the 24 x 8192 and 40 x 36,480 workloads")
    ap.add_argument("--bw-ceiling", action="store_true",
                    help="only run the standalone HBM probe (read-only, copy and write-only passes over "
                         "tensors of the prep's sizes: the ceilings its kernels are compared with) and "
                         "print its JSON line")
    ap.add_argument("--operand-energy", action="store_true",
                    help="time attn_fwd_bf16 on the benchmark shape with its inputs as generated, with V = 0, "
                         "with K = V = 0 and on flat N(0,1) inputs, sampling clock and power; prints one JSON line")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="for hardware-counter runs: one %d-byte torch copy (counter calibration), "
                         "then one launch of each kernel on the benchmark workload; no timing" % COPY_PROBE_BYTES)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(attention would shard by head with no exchange); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    if args.mfma_ceiling:
        print(json.dumps(mfma_ceiling()), flush=True)
        return
    if args.bw_ceiling:
        print(json.dumps(bw_ceiling()), flush=True)
        return

    import torch
    from long_sequence_dense_amd import binding
    assert torch.cuda.is_available(), "bench needs a GPU"
    binding.load_library()
    H, L, d = 40, 109000, 128
    if args.operand_energy:
        operand_energy(torch, binding, torch.cuda.current_stream(), H, L, d)
        return

    log("generating inputs (seeded, synthetic) ...")
    cfg4, x4 = gen_inputs(torch, "clip15s")
    cfg5, x5 = gen_inputs(torch, "fp4")
    dev = x4["q"].device
    o4 = torch.empty((H, L, d), dtype=torch.bfloat16, device=dev)
    o5 = torch.empty((H, L, d), dtype=torch.bfloat16, device=dev)
    prep = {
        "q_codes": torch.empty((H, L, d // 2), dtype=torch.uint8, device=dev),
        "q_scales": torch.empty((H, L, d // 16), dtype=torch.uint8, device=dev),
        "k_codes": torch.empty((H, L, d // 2), dtype=torch.uint8, device=dev),
        "k_scales": torch.empty((H, L, d // 16), dtype=torch.uint8, device=dev),
        "k_mean": torch.empty((H, d), dtype=torch.float32, device=dev),
    }
    ws = torch.empty(binding.qk_prep_fp4_workspace_bytes(H, L, d), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    ev = {n: [] for n in ("bf16", "prep", "fp4")}

    def step(record):
        def mark():
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            return e
        a = mark() if record else None
        binding.attn_fwd_bf16(x4["q"], x4["k"], x4["v"], o4, None, cfg4.scale, stream)
        if args.only == "bf16":
            if record:
                ev["bf16"].append((a, mark()))
            return
        b = mark() if record else None
        binding.qk_prep_fp4(x5["q"], x5["k"], prep, ws, stream)
        c = mark() if record else None
        binding.attn_fwd_fp4qk(prep["q_codes"], prep["q_scales"], prep["k_codes"], prep["k_scales"],
                               x5["v"], o5, None, cfg5.scale, stream)
        if record:
            e = mark()
            ev["bf16"].append((a, b))
            ev["prep"].append((b, c))
            ev["fp4"].append((c, e))

    if args.pmc_probe:
        a = torch.empty(COPY_PROBE_BYTES // 2, dtype=torch.int16, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)                                   # the calibration copy
        torch.cuda.synchronize()
        step(False)
        torch.cuda.synchronize()
        kflags = binding.PREP_SMOOTH_K | binding.PREP_ROTATE | binding.PREP_K_ONLY
        kprep = {key: prep[key] for key in ("k_codes", "k_scales", "k_mean")}
        binding.qk_prep_fp4_ex(None, x5["k"], kflags, kprep, ws, stream)
        binding.attn_fwd_fp4qk_fused_q(x5["q"], kprep["k_codes"], kprep["k_scales"], x5["v"], o5, None,
                                       cfg5.scale, stream)
        torch.cuda.synchronize()
        x, w, gx, gw = linear_operands(torch, dev)
        T = binding.NVFP4_TILED
        xc, xs = binding.nvfp4_quantize(x, gx, layout=T, stream=stream)
        wc, ws_ = binding.nvfp4_quantize(w, gw, layout=T, stream=stream)
        binding.nvfp4_linear(xc, xs, gx, wc, ws_, gw, stream=stream, layout=T, M=LIN_M, N=LIN_N, K=LIN_K)
        torch.cuda.synchronize()
        del x, w, xc, xs, wc, ws_
        # one training forward and backward of the BF16 path
        o32 = torch.empty((H, L, d), dtype=torch.float32, device=dev)
        ml = torch.empty((H, L, 2), dtype=torch.float32, device=dev)
        binding.attn_fwd_bf16_train(x4["q"], x4["k"], x4["v"], o4, None, o32, ml, cfg4.scale, stream)
        gen = torch.Generator(device=dev)
        gen.manual_seed(5)
        dout = torch.randn((H, L, d), dtype=torch.float32, device=dev, generator=gen).to(torch.bfloat16)
        binding.attn_bwd_bf16(x4["q"], x4["k"], x4["v"], o32, ml, dout, softmax_scale=cfg4.scale, stream=stream)
        torch.cuda.synchronize()
        log("pmc probe done")
        return

    log("warmup %d steps ..." % args.warmup)
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    log("timing %d steps ..." % args.steps)
    sampler = ClockSampler(window="the timed steps (attn_fwd_bf16 only)" if args.only == "bf16" else
                           "the timed steps (both attention launches and the prep)").start()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sclk = sampler.stop()
    log("timed region %.2f s" % wall)
    assert not torch.isnan(o4).any().item() and not torch.isnan(o5).any().item()

    def avg_ms(name):
        xs = [a.elapsed_time(b) for a, b in ev[name]]
        return sum(xs) / len(xs) if xs else None

    ms_step = wall * 1e3 / args.steps
    fl = attn_flop(H, L, d)
    step_flop = fl if args.only == "bf16" else 2 * fl
    value = step_flop / (ms_step * 1e-3) / 1e12
    t_bf16 = avg_ms("bf16")
    achieved = fl / (t_bf16 * 1e-3) / 1e12
    paths = {"attn_fwd_bf16": {"ms": round(t_bf16, 3), "TFLOP/s": round(achieved, 1),
                               "frac_of_peak": round(achieved / PEAK_BF16_TFLOPS, 4)}}
    if args.only != "bf16":
        t_prep, t_fp4 = avg_ms("prep"), avg_ms("fp4")
        gbs = prep_bytes(H, L, d) / (t_prep * 1e-3) / 1e9
        a4 = fl / (t_fp4 * 1e-3) / 1e12
        paths["qk_prep_fp4"] = {"ms": round(t_prep, 4), "GB/s": round(gbs, 1),
                                "algorithmic_bytes": prep_bytes(H, L, d),
                                "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}
        paths["attn_fwd_fp4qk"] = {"ms": round(t_fp4, 3), "TFLOP/s": round(a4, 1),
                                   "frac_of_peak": round(a4 / PEAK_BF16_TFLOPS, 4),
                                   "mfma_precision": "fp16 scores (exact dequantization of NVFP4 Q/K), bf16 P.V"}
    if args.only != "bf16":
        # Extra path, outside the step's value: the fused-Q form of the FP4
        # path (K-only prep, then attention that quantizes Q in its prologue)
        # on the same inputs; 1 warm-up + 3 timed calls of each part.
        log("timing the fused-Q FP4 path (3 calls) ...")
        kflags = binding.PREP_SMOOTH_K | binding.PREP_ROTATE | binding.PREP_K_ONLY
        kprep = {key: prep[key] for key in ("k_codes", "k_scales", "k_mean")}
        flush = MallFlush(torch, dev)
        t_kp = time_calls(torch, stream, lambda: binding.qk_prep_fp4_ex(None, x5["k"], kflags, kprep, ws, stream),
                          before=flush)
        del flush
        o5f = torch.empty_like(o5)
        t_fq = time_calls(torch, stream, lambda: binding.attn_fwd_fp4qk_fused_q(
            x5["q"], kprep["k_codes"], kprep["k_scales"], x5["v"], o5f, None, cfg5.scale, stream))
        same = bool(torch.equal(o5f.view(torch.int16), o5.view(torch.int16)))
        kbytes = H * L * (2 * d + d // 2 + d // 16)
        paths["qk_prep_fp4_k_only"] = {"ms": round(t_kp, 4), "GB/s": round(kbytes / (t_kp * 1e-3) / 1e9, 1),
                                       "algorithmic_bytes": kbytes,
                                       "frac_of_peak": round(kbytes / (t_kp * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                       "in_value": False}
        af = fl / (t_fq * 1e-3) / 1e12
        paths["attn_fwd_fp4qk_fused_q"] = {"ms": round(t_fq, 3), "TFLOP/s": round(af, 1),
                                           "frac_of_peak": round(af / PEAK_BF16_TFLOPS, 4),
                                           "output_bit_identical_to_two_call_path": same,
                                           "fused_path_ms": round(t_kp + t_fq, 3), "in_value": False}
        del o5f
    if args.only != "bf16" and not args.no_bwd:
        # Extra path, outside the step and its value: the backward of the BF16
        # path on the same inputs, dO ~ N(0, 1); 1 warm-up + 3 timed calls.
        log("timing attn_bwd_bf16 (3 calls) ...")
        o32 = torch.empty((H, L, d), dtype=torch.float32, device=dev)
        ml = torch.empty((H, L, 2), dtype=torch.float32, device=dev)
        binding.attn_fwd_bf16_train(x4["q"], x4["k"], x4["v"], o4, None, o32, ml, cfg4.scale, stream)
        gen = torch.Generator(device=dev)
        gen.manual_seed(5)
        dout = torch.randn((H, L, d), dtype=torch.float32, device=dev, generator=gen).to(torch.bfloat16)
        grads = [torch.empty((H, L, d), dtype=torch.bfloat16, device=dev) for _ in range(3)]
        bws = torch.empty(binding.attn_bwd_bf16_workspace_bytes(H, L, d), dtype=torch.uint8, device=dev)
        times = []
        for i in range(4):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            binding.attn_bwd_bf16(x4["q"], x4["k"], x4["v"], o32, ml, dout, *grads, softmax_scale=cfg4.scale,
                                  workspace=bws, stream=stream)
            b.record(stream)
            b.synchronize()
            if i:
                times.append(a.elapsed_time(b))
        t_bwd = sum(times) / len(times)
        bw = 2.5 * fl / (t_bwd * 1e-3) / 1e12
        paths["attn_bwd_bf16"] = {"ms": round(t_bwd, 3), "TFLOP/s": round(bw, 1),
                                  "frac_of_peak": round(bw / PEAK_BF16_TFLOPS, 4),
                                  "flop_convention": "2.5 x forward (5 of the 2HL^2d products); the kernels "
                                                     "compute 7 (S and dP for dK/dV and again for dQ)",
                                  "in_value": False}
        # The training-time FP4 backward on the FP4 path's tensors (the codes
        # of the step's prep, its training forward's outputs): 1 warm-up + 2 calls.
        log("timing attn_bwd_fp4qk (2 calls) ...")
        binding.attn_fwd_fp4qk_train(prep["q_codes"], prep["q_scales"], prep["k_codes"], prep["k_scales"], x5["v"],
                                     o5, None, o32, ml, cfg5.scale, stream)
        fws = torch.empty(binding.attn_bwd_fp4qk_workspace_bytes(H, L, d), dtype=torch.uint8, device=dev)
        t_fb = time_calls(torch, stream, lambda: binding.attn_bwd_fp4qk(
            prep["q_codes"], prep["q_scales"], prep["k_codes"], prep["k_scales"], x5["v"], o32, ml, dout, *grads,
            softmax_scale=cfg5.scale, workspace=fws, stream=stream), n=2)
        fb = 2.5 * fl / (t_fb * 1e-3) / 1e12
        paths["attn_bwd_fp4qk"] = {"ms": round(t_fb, 3), "TFLOP/s": round(fb, 1),
                                   "frac_of_peak": round(fb / PEAK_BF16_TFLOPS, 4),
                                   "flop_convention": "as attn_bwd_bf16; the time also covers the exact "
                                                      "dequantization of Q, K and the rotation of dQ, dK back",
                                   "in_value": False}
        del grads, dout, bws, fws, o32, ml
    if args.only != "bf16" and not args.no_linear:
        # Extra path, outside the step and its value: one NVFP4 W4A4 linear of
        # the same transformer at the 40 x 128 hidden size, over the clip's
        # tokens (X [109000, 5120], W [5120, 5120]); seeded device draws, X
        # N(0,1) with 2% of its channels x20, W N(0, 1/5120); static global
        # scales from the tensors' maxima.  1 warm-up + 3 timed calls each.
        log("timing nvfp4_quantize + nvfp4_linear (3 calls each) ...")
        r = linear_path(torch, binding, stream, dev)
        paths.update(r)
    if args.only != "bf16" and not args.no_configs:
        log("timing attn_fwd_bf16 on the mid and clip5s workloads ...")
        paths["attn_fwd_bf16_mid"] = config_path(torch, binding, stream, "mid", 50)
        paths["attn_fwd_bf16_clip5s"] = config_path(torch, binding, stream, "clip5s", 10)
    traffic = stored_traffic()
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded numpy draws, BF16)",
        "config": {"workload": "dense non-causal attention, 15-second clip scale: BF16 path + "
                               "NVFP4 prep + FP4-QK path" if args.only != "bf16" else "BF16 path only",
                   "H": H, "L": L, "d": d, "softmax_scale": "1/sqrt(128)",
                   "bf16_inputs": cfg4.desc, "fp4_inputs": cfg5.desc},
        "roofline": {"bound": "mfma", "kernel": "attn_fwd_bf16", "achieved": round(achieved, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "algorithmic_flop_per_launch": fl},
        "paths": paths,
        "sclk_during_timed_steps": sclk,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        def gpu_rows(name, heads, rows):
            from long_sequence_dense_amd import inputs
            t = o4 if name == "bf16" else o5
            idx_h = torch.tensor(heads, device=dev)
            idx_r = torch.from_numpy(np.asarray(rows)).to(dev)
            sel = t.index_select(0, idx_h).index_select(1, idx_r)
            bits = sel.view(torch.int16).cpu().numpy().view(np.uint16)
            return inputs.bf16_bits_to_f32(bits).astype(np.float64)

        res["cpu_baseline"] = cpu_baseline(H, L, d, gpu_rows if args.only != "bf16" else None)
        if "parity" in res["cpu_baseline"]:
            par = res["cpu_baseline"].pop("parity")
            for key, val in par.items():
                res["paths"][key]["parity_vs_oracle"] = val
    if not args.no_mfma_ceiling:
        ceil = mfma_ceiling()
        if ceil is not None:
            rnd = ceil["mfma_ceiling_bf16_TFLOP/s"]["random_operands"]
            ceil["attn_fwd_bf16_frac_of_random_operand_ceiling"] = round(res["roofline"]["achieved"] / rnd, 4)
        res["mfma_ceiling_probe"] = ceil
    if not args.no_hbm_ceiling:
        hbm = bw_ceiling()
        if hbm is not None and "qk_prep_fp4" in res["paths"]:
            copy = max(v["best"] for k, v in hbm["hbm_ceiling_GB/s"].items() if k.startswith("copy"))
            hbm["qk_prep_fp4_algorithmic_rate_frac_of_copy_ceiling"] = round(
                res["paths"]["qk_prep_fp4"]["GB/s"] / copy, 4)
        res["hbm_ceiling_probe"] = hbm
    print(json.dumps(res), flush=True)


def mfma_ceiling():
    """Run the standalone matrix-core probe (built in-tree by the library's
    build step): the dense BF16 MFMA rate this GPU sustains with nothing else
    running, for random and for all-zero operands.  None if it is not built."""
    import subprocess
    exe = os.path.join(ROOT, "long_sequence_dense_amd", "mfma_ceiling_probe")
    if not os.path.exists(exe):
        log("mfma_ceiling_probe not built; skipped")
        return None
    log("running the MFMA ceiling probe ...")
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    if r.returncode != 0:
        raise RuntimeError("mfma_ceiling_probe failed (%d): %s" % (r.returncode, r.stderr.strip()))
    return json.loads(r.stdout.strip().splitlines()[-1])


if __name__ == "__main__":
    main()
