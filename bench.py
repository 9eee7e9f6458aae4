"""Benchmark of the dense long-sequence attention hot path on one MI355X.

One step = the whole path over one batch of synthetic input at the 15-second
clip scale (H = 40 heads, L = 109,000 tokens, d = 128):
  attn_fwd_bf16 on the BF16 workload (N(0,1), 3 of 128 channels x20 on Q, K),
  qk_prep_fp4 + attn_fwd_fp4qk on the FP4 workload (Student-t(3) Q, K with the
  same outliers, N(0,1) V).
value = attention FLOP of the step (2 x 4 H L^2 d) / step time, TFLOP/s.
Prints ONE JSON line (rank 0).  Inputs are resident in HBM before timing.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
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


KERNEL_SOURCES = ("attn_fwd.hip", "device_common.h", "lsd_internal.h")


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


def cpu_baseline(H, L, d):
    """Time the CPU oracle (as it stands) on a bounded sample of the workload
    (about 15 s of CPU work on 16 cores) and extrapolate a full step; returns
    the cpu_baseline object."""
    from long_sequence_dense_amd import inputs
    from oracle.attention import attention_fp64
    from oracle.nvfp4 import qk_prep_fp4
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
    attention_fp64(f(q), f(k), f(v), cfg.scale, rows=rows)
    t_attn = time.time() - t0
    attn_rate = len(heads) * len(rows) * 4.0 * L * d / t_attn          # FLOP/s
    fcfg = inputs.CONFIGS["fp4"]
    prep_heads = [0, 1, 2, 3]
    qf = inputs.make_tensor(fcfg, "q", prep_heads)
    kf = inputs.make_tensor(fcfg, "k", prep_heads)
    t0 = time.time()
    qk_prep_fp4(qf, kf)
    t_prep = time.time() - t0
    t_prep_head = t_prep / len(prep_heads)
    full_attn_s = attn_flop(H, L, d) / attn_rate
    step_s = 2 * full_attn_s + H * t_prep_head
    return {
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


def time_calls(torch, stream, fn, n=3):
    times = []
    for i in range(n + 1):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        b.synchronize()
        if i:
            times.append(a.elapsed_time(b))
    return sum(times) / len(times)


def linear_path(torch, binding, stream, dev):
    x, w, gx, gw = linear_operands(torch, dev)
    M, N, K = LIN_M, LIN_N, LIN_K
    T = binding.NVFP4_TILED                      # the product's own load order
    xc, xs = binding.nvfp4_quantize(x, gx, layout=T, stream=stream)
    wc, ws = binding.nvfp4_quantize(w, gw, layout=T, stream=stream)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    t_q = time_calls(torch, stream, lambda: binding.nvfp4_quantize(x, gx, xc, xs, layout=T, stream=stream))
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=8)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["all", "bf16"], default="all",
                    help="bf16: time only attn_fwd_bf16 (for profiling runs)")
    ap.add_argument("--no-bwd", action="store_true",
                    help="skip the extra (not in value) timing of attn_bwd_bf16 and attn_bwd_fp4qk")
    ap.add_argument("--no-linear", action="store_true",
                    help="skip the extra (not in value) timing of the NVFP4 linear layer")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="for hardware-counter runs: one %d-byte torch copy (counter calibration), "
                         "then one launch of each kernel on the benchmark workload; no timing" % COPY_PROBE_BYTES)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(attention would shard by head with no exchange); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from long_sequence_dense_amd import binding
    assert torch.cuda.is_available(), "bench needs a GPU"
    binding.load_library()
    H, L, d = 40, 109000, 128

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
        x, w, gx, gw = linear_operands(torch, dev)
        T = binding.NVFP4_TILED
        xc, xs = binding.nvfp4_quantize(x, gx, layout=T, stream=stream)
        wc, ws_ = binding.nvfp4_quantize(w, gw, layout=T, stream=stream)
        binding.nvfp4_linear(xc, xs, gx, wc, ws_, gw, stream=stream, layout=T, M=LIN_M, N=LIN_N, K=LIN_K)
        torch.cuda.synchronize()
        log("pmc probe done")
        return

    log("warmup %d steps ..." % args.warmup)
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    log("timing %d steps ..." % args.steps)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
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
                                   "mfma_precision": "bf16 (exact dequantization of NVFP4 Q/K)"}
    if args.only != "bf16" and not args.no_bwd:
        # Extra path, outside the step and its value: the backward of the BF16
        # path on the same inputs, dO ~ N(0, 1); 1 warm-up + 3 timed calls.
        log("timing attn_bwd_bf16 (3 calls) ...")
        lse = torch.empty((H, L), dtype=torch.float32, device=dev)
        binding.attn_fwd_bf16(x4["q"], x4["k"], x4["v"], o4, lse, cfg4.scale, stream)
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
            binding.attn_bwd_bf16(x4["q"], x4["k"], x4["v"], o4, lse, dout, *grads, softmax_scale=cfg4.scale,
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
                                                     "compute 7 (S and dP again for dQ)",
                                  "in_value": False}
        # The training-time FP4 backward on the FP4 path's tensors (the codes
        # of the step's prep, its forward's output and LSE): 1 warm-up + 2 calls.
        log("timing attn_bwd_fp4qk (2 calls) ...")
        binding.attn_fwd_fp4qk(prep["q_codes"], prep["q_scales"], prep["k_codes"], prep["k_scales"], x5["v"], o5,
                               lse, cfg5.scale, stream)
        fws = torch.empty(binding.attn_bwd_fp4qk_workspace_bytes(H, L, d), dtype=torch.uint8, device=dev)
        t_fb = time_calls(torch, stream, lambda: binding.attn_bwd_fp4qk(
            prep["q_codes"], prep["q_scales"], prep["k_codes"], prep["k_scales"], x5["v"], o5, lse, dout, *grads,
            softmax_scale=cfg5.scale, workspace=fws, stream=stream), n=2)
        fb = 2.5 * fl / (t_fb * 1e-3) / 1e12
        paths["attn_bwd_fp4qk"] = {"ms": round(t_fb, 3), "TFLOP/s": round(fb, 1),
                                   "frac_of_peak": round(fb / PEAK_BF16_TFLOPS, 4),
                                   "flop_convention": "as attn_bwd_bf16; the time also covers the exact "
                                                      "dequantization of Q, K and the rotation of dQ, dK back",
                                   "in_value": False}
        del grads, dout, bws, fws
    if args.only != "bf16" and not args.no_linear:
        # Extra path, outside the step and its value: one NVFP4 W4A4 linear of
        # the same transformer at the 40 x 128 hidden size, over the clip's
        # tokens (X [109000, 5120], W [5120, 5120]); seeded device draws, X
        # N(0,1) with 2% of its channels x20, W N(0, 1/5120); static global
        # scales from the tensors' maxima.  1 warm-up + 3 timed calls each.
        log("timing nvfp4_quantize + nvfp4_linear (3 calls each) ...")
        r = linear_path(torch, binding, stream, dev)
        paths.update(r)
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
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        res["cpu_baseline"] = cpu_baseline(H, L, d)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
