"""Benchmark: diagonal-batched inference of one 131,072-token sequence.

Workload: the LLaMA-1B-shaped RMT (16 layers, d = 2048, 32 query / 8 KV heads
of 64, SwiGLU 8192, segments of 1024 tokens + 128 memory rows, 128 segments),
bf16 weights and activations with fp32 accumulation and an fp32 residual
stream, random weights and token ids from a fixed seed.

Prints one JSON line.  `value` is tokens/s of rmt_forward_diagonal over the
whole sequence with inputs already in HBM.  Alongside: the same GPU's
sequential per-cell path, per-stage GPU times (HIP events recorded on the
library's stream between launches), the grouped-GEMM fraction of the MI355X
bf16 dense MFMA peak, the isolated 1152 x 2048 x 8192 grouped GEMM at
G = 1, 4, 8, 16, the CPU oracle timed on a prefix of the sequence, and (as
`secondary`) the 8B-shaped RMT with fp16 operands, one timed step.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu] [--no-seq]
                    [--workload llama1b|llama8b|norm_swiglu_1b|encoder1b] [--dtype bf16|f16]

The default workload is the 1B-shaped one above; --workload selects the
8B-shaped RMT (32 layers, d = 4096, segments of 2048 + 128 rows, 64 segments,
131,072 tokens), the attention-free 1B-width stack (32 segments, 32,768
tokens) or the encoder-layer cell at the 1B width (pre-norm LayerNorm,
unmasked 32-head attention, 4x ReLU feed-forward; 128 segments, 131,072
tokens) instead.  Every GPU stage is also split into full diagonals (all
min(L, S) cells active) and ramp diagonals.
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

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "tokens/s for one 131K-token sequence; grouped-GEMM % of bf16 MFMA peak"
WORKLOADS = {"llama1b": "LLAMA_1B", "llama8b": "LLAMA_8B", "norm_swiglu_1b": "NORM_SWIGLU_1B",
             "encoder1b": "ENCODER_1B", "encoder1b_postnorm": "ENCODER_1B_POSTNORM",
             "tiny_linear_gelu": "TINY_LINEAR_GELU"}
PEAK_FP32_VALU_TFLOPS = 157.3  # MI355X fp32 vector (FMA) peak
# the encoder cell's stages, named by what they compute there
ENCODER_STAGE_NAMES = {"norm1": "layernorm1", "norm2": "layernorm2", "gateup": "ffn_w1", "down": "ffn_w2"}
# post-norm: the first norm-stage launch is the bf16 copy of A, the second stage holds both LayerNorms
POSTNORM_STAGE_NAMES = {"norm1": "cast_a_bf16", "norm2": "layernorms", "gateup": "ffn_w1", "down": "ffn_w2"}
GEMM_KERNELS = {
    "llama": {"qkv": "QKV stage, rows scaled by 1/rms + RoPE epilogue (gemm_bf16_kernel<1, ...>)",
              "oproj": "O stage + residual and RMSNorm side-output epilogue (gemm_bf16_kernel<7, ...>)",
              "gateup": "gate/up stage, rows scaled by 1/rms + SwiGLU epilogue (gemm_bf16_kernel<2, ...>)",
              "down": "down stage + residual and RMSNorm side-output epilogue (gemm_bf16_kernel<7, ...>)"},
    "encoder": {"qkv": "QKV stage + bias epilogue (gemm_bf16_kernel<4>)",
                "oproj": "O stage + bias + residual epilogue (gemm_bf16_kernel<6>)",
                "gateup": "W1 stage + bias + ReLU epilogue (gemm_bf16_kernel<5>)",
                "down": "W2 stage + bias + residual epilogue (gemm_bf16_kernel<6>)"},
    "norm_swiglu": {"gateup": "gate/up stage + SwiGLU epilogue (gemm_bf16_kernel<2>)",
                    "down": "down stage + residual epilogue (gemm_bf16_kernel<3>)"},
    "linear_gelu": {"linear": "fp32 linear + bias + GELU cell (linear_gelu_f32_kernel, VALU FMAs)"},
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def gen_layers(cfg, seed=0):
    import rmt_inputs as ri
    return ri.all_weights(cfg, seed, workers=8)


def code_hash(path):
    """sha256 prefix of a C++ source with its comments and blank space removed,
    so that the figure certifies the code, not its commentary."""
    import hashlib
    import re
    src = open(path).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    src = re.sub(r"\s+", " ", src).strip()
    return hashlib.sha256(src.encode()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per gate/up launch from the committed counter summary, used
    only while the GEMM code is the one the counters were taken on."""
    import re
    src = os.path.join(ROOT, "long_context_anti_amd", "csrc", "gemm_bf16.hip")
    summ = os.path.join(ROOT, "profiles", "llama1b_rmt_L16_S128_gateup_hbm_traffic.md")
    try:
        text = open(summ).read()
        h = code_hash(src)
        if f"code sha256 prefix: {h}" not in text:
            return None
        m = re.search(r"traffic \(bench roofline field\) = ([0-9.]+) GB \+ ([0-9.]+) GB", text)
        return round((float(m.group(1)) + float(m.group(2))) * 1e9) if m else None
    except OSError:
        return None


def timed_steps(fn, steps, stream):
    import torch
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, e0.elapsed_time(e1) / 1e3


def gemm_sweep(steps=20):
    """Isolated grouped GEMM, 1152 x 2048 x 8192 per group, distinct weights."""
    import torch
    import long_context_anti_amd as rmt
    import rmt_inputs as ri
    from rmt_inputs import device as rdev
    gc = ri.GROUPED_GEMM_1B
    A, B = ri.gemm_operands(gc, G=gc.G_max)
    A_d = rdev.bf16_tensor(A)
    W_d = rdev.bf16_tensor(B)
    B_d = torch.empty((gc.G_max, gc.N, gc.K), dtype=torch.bfloat16, device="cuda")
    rmt.pack_weight(W_d, B_d)
    del W_d
    C_d = torch.empty((gc.G_max, gc.M, gc.N), dtype=torch.bfloat16, device="cuda")
    out = {}
    st = torch.cuda.current_stream()
    for G in gc.G_sweep:
        fn = lambda: rmt.grouped_gemm(A_d[:G], B_d, list(range(G)), C_d[:G])  # noqa: E731
        for _ in range(3):
            fn()
        _, gpu_s = timed_steps(fn, steps, st)
        flops = 2.0 * G * gc.M * gc.N * gc.K
        tf = flops * steps / gpu_s / 1e12
        out[f"G{G}"] = {"us": round(gpu_s / steps * 1e6, 2), "tflops": round(tf, 1),
                        "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    # The same largest launch on all-zero operands: the instruction stream is
    # identical, only the bits the matrix cores and data paths toggle differ,
    # so a higher rate here is the clock the chip holds at lower power.
    G = gc.G_max
    A_d.zero_()
    B_d.zero_()
    fn = lambda: rmt.grouped_gemm(A_d[:G], B_d, list(range(G)), C_d[:G])  # noqa: E731
    for _ in range(3):
        fn()
    _, gpu_s = timed_steps(fn, steps, st)
    tf = 2.0 * G * gc.M * gc.N * gc.K * steps / gpu_s / 1e12
    out[f"G{G}_zero_operands"] = {"us": round(gpu_s / steps * 1e6, 2), "tflops": round(tf, 1),
                                  "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    return out


def secondary_llama8b(steps=1, warmup=1):
    """The LLaMA-8B-shaped workload (32 layers, d = 4096, 2048 + 128 rows, 64
    segments, 131,072 tokens) with fp16 operands, the precision that meets the
    2e-2 gate at that depth: tokens/s of the diagonal sweep and the grouped-GEMM
    stage rates from per-launch events.  No CPU leg, no sequential path."""
    import torch
    import long_context_anti_amd as rmt
    import rmt_inputs as ri
    from rmt_inputs import device as rdev

    cfg = ri.LLAMA_8B
    t0 = time.perf_counter()
    layers = gen_layers(cfg)
    embed = ri.embedding(cfg)
    dw = rdev.device_weights(cfg, layers, embed)
    del layers
    kw = rdev.model_kwargs(cfg)
    kw["dtype"] = rmt.RMT_F16
    model = rmt.RMTModel(**kw, weights=dw)
    tok_d = rdev.segment_inputs(cfg, ri.tokens(cfg, 0))
    mem0_d = rdev.f32_tensor(ri.initial_memory(cfg, 0))
    hidden = torch.empty((cfg.T, cfg.d), dtype=torch.float32, device="cuda")
    mem = torch.empty((cfg.L, cfg.m, cfg.d), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    diag = lambda: model.forward_diagonal(tok_d, mem0_d, hidden, mem)  # noqa: E731
    for _ in range(warmup):
        diag()
    torch.cuda.synchronize()
    log(f"[bench] {cfg.name} (fp16 operands): ready in {time.perf_counter() - t0:.1f} s")
    wall, _ = timed_steps(diag, steps, stream)
    model.enable_timing(True)
    timed_steps(diag, steps, stream)
    stages = model.stage_times()
    model.enable_timing(False)
    model.close()
    del dw, model
    torch.cuda.empty_cache()
    ms = {"ms": 0.0, "flops": 0.0}
    for k in ("qkv", "oproj", "gateup", "down"):
        ms["ms"] += stages[k]["ms"]
        ms["flops"] += stages[k]["flops"]
    tf = ms["flops"] / (ms["ms"] / 1e3) / 1e12
    gu = stages["gateup"]
    gu_tf = gu["flops"] / (gu["ms"] / 1e3) / 1e12
    log(f"[bench] {cfg.name}: {wall / steps * 1e3:.1f} ms/step")
    return {"workload": cfg.name, "dtype": "f16", "value": round(cfg.T * steps / wall, 1), "unit": "tokens/s",
            "steps": steps, "warmup": warmup, "ms_per_step": round(wall / steps * 1e3, 2),
            "grouped_gemm_stages": {"tflops": round(tf, 1), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)},
            "gateup": {"tflops": round(gu_tf, 1), "frac_bf16_peak": round(gu_tf / PEAK_BF16_TFLOPS, 4)}}


def cpu_baseline(cfg, layers, tokens, mem0, embed, gpu_hidden, gpu_mem_prefix_fn, S_prefix):
    """The CPU oracle as it stands, timed on a prefix of S_prefix segments."""
    from threadpoolctl import threadpool_info
    from oracle import rmt_oracle as orc
    threads = max([i.get("num_threads", 1) for i in threadpool_info()
                   if i.get("user_api") == "blas"] or [1])
    host_cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    h, m = orc.forward_sequential(cfg, layers, tokens[:S_prefix * cfg.n], mem0, embed)
    dt = time.perf_counter() - t0
    toks = S_prefix * cfg.n
    res = {"value": round(toks / dt, 2), "unit": "tokens/s", "cores": int(threads),
           "host_cores": host_cores, "blas_threads": int(threads), "kind": "oracle",
           "sample": f"first {S_prefix} of {cfg.S} segments through all {cfg.L} layers "
                     f"({toks} tokens, NumPy fp32, {dt:.1f} s); per-segment cost is constant in s",
           "seconds": round(dt, 2)}
    # the same prefix of the GPU's full-sequence run: segment s never reads later segments
    gh = gpu_hidden[:toks].astype(np.float64)
    res["parity_rel_l2_hidden_prefix"] = float(np.linalg.norm(gh - h) / np.linalg.norm(h))
    gm = gpu_mem_prefix_fn()
    if gm is not None:
        res["parity_rel_l2_mem_prefix"] = float(np.linalg.norm(gm - m) / np.linalg.norm(m))
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-seq", action="store_true", help="skip the sequential path")
    ap.add_argument("--no-sweep", action="store_true", help="skip the isolated grouped-GEMM sweep")
    ap.add_argument("--cpu-segments", type=int, default=4)
    ap.add_argument("--workload", default="llama1b", choices=sorted(WORKLOADS))
    ap.add_argument("--batch", type=int, default=1,
                    help="B sequences through the same diagonals (rmt_model_set_batch); "
                         "tokens/s then counts all B sequences")
    ap.add_argument("--dtype", default=None, choices=["bf16", "f16"],
                    help="16-bit operand type of the LLaMA-shaped cell (default: the workload's bf16); "
                         "f16 is the precision that meets the 2e-2 gate at the 8B shape")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the secondary LLaMA-8B-shaped measurement (fp16 operands) of the default run")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy, the reference for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the diagonal sweep is measured on a single "
              "MI355X (no multi-GPU path is built); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import long_context_anti_amd as rmt
    import rmt_inputs as ri
    from rmt_inputs import device as rdev

    cfg = getattr(ri, WORKLOADS[args.workload])
    llama = cfg.cell == ri.CELL_LLAMA
    encoder = cfg.cell == ri.CELL_ENCODER
    torch.cuda.set_device(0)
    t0 = time.perf_counter()
    layers = gen_layers(cfg)
    embed = ri.embedding(cfg) if llama else None
    B = args.batch
    # sequence 0 uses seed 0 (the one-sequence workload); sequence b seed b
    toks_b = [ri.tokens(cfg, b) if llama else ri.input_embeddings(cfg, b) for b in range(B)]
    mems_b = [ri.initial_memory(cfg, b) for b in range(B)]
    tokens, mem0 = toks_b[0], mems_b[0]
    log(f"[bench] {cfg.name}: inputs generated in {time.perf_counter() - t0:.1f} s")
    dw = rdev.device_weights(cfg, layers, embed)
    kw = rdev.model_kwargs(cfg)
    f16 = args.dtype == "f16"
    if f16:
        if not llama:
            print("--dtype f16 applies to the LLaMA-shaped workloads only", file=sys.stderr)
            sys.exit(2)
        kw["dtype"] = rmt.RMT_F16
    model = rmt.RMTModel(**kw, weights=dw)
    emb_dev = dw.get("embed")
    del dw
    if B == 1:
        tok_d = rdev.segment_inputs(cfg, tokens)
        mem0_d = rdev.f32_tensor(mem0)
    else:
        model.set_batch(B)
        tok_d = torch.stack([rdev.segment_inputs(cfg, x) for x in toks_b]).contiguous()
        mem0_d = rdev.f32_tensor(np.stack(mems_b))
    del toks_b, mems_b
    T = cfg.T
    hidden = torch.empty((B, T, cfg.d) if B > 1 else (T, cfg.d), dtype=torch.float32, device="cuda")
    mem = torch.empty((B, cfg.L, cfg.m, cfg.d) if B > 1 else (cfg.L, cfg.m, cfg.d),
                      dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    log(f"[bench] model on device: {model.device_bytes() / 2**30:.2f} GiB")

    diag = lambda: model.forward_diagonal(tok_d, mem0_d, hidden, mem)  # noqa: E731
    for i in range(args.warmup):
        diag()
    torch.cuda.synchronize()
    log("[bench] warmup done")

    # timed region: the forward pass alone
    wall, gpu_s = timed_steps(diag, args.steps, stream)
    log(f"[bench] diagonal: {wall / args.steps * 1e3:.1f} ms/step wall")
    # the same steps again with per-launch HIP events on the library's stream
    model.enable_timing(True)
    wall_ev, _ = timed_steps(diag, args.steps, stream)
    g_full = min(cfg.L, cfg.S)
    if B == 1:      # with B > 1 launches mix ramp and full cells, so no split
        full = model.stage_times(groups=(g_full, g_full))
        ramp = model.stage_times(groups=(1, g_full - 1))
    else:
        full = ramp = {k: {"ms": 0.0, "launches": 0, "flops": 0.0, "bytes": 0.0} for k in rmt._lib.STAGES}
    stages = model.stage_times()
    model.enable_timing(False)
    hidden_np = (hidden[0] if B > 1 else hidden).cpu().numpy()

    ms_step = wall / args.steps * 1e3
    tok_s = B * T * args.steps / wall

    def rates(v):
        e = {"ms_per_step": round(v["ms"] / args.steps, 3), "launches_per_step": v["launches"] // args.steps}
        if v["ms"] > 0 and v["flops"] > 0:
            tf = v["flops"] / (v["ms"] / 1e3) / 1e12
            e["tflops"] = round(tf, 1 if tf >= 1 else 6)
            if cfg.cell == ri.CELL_LINEAR_GELU:     # fp32 on the vector ALUs
                e["frac_fp32_valu_peak"] = round(tf / PEAK_FP32_VALU_TFLOPS, 6)
            else:
                e["frac_bf16_peak"] = round(tf / PEAK_BF16_TFLOPS, 4)
        if v["ms"] > 0 and v["bytes"] > 0:
            e["gbs"] = round(v["bytes"] / (v["ms"] / 1e3) / 1e9, 1)
            e["frac_hbm_peak"] = round(e["gbs"] / PEAK_HBM_GBS, 4)
        return e

    st_out = {}
    gemm = {k: {"ms": 0.0, "flops": 0.0, "launches": 0, "bytes": 0.0} for k in ("all", "full", "ramp")}
    for name, v in stages.items():
        if v["launches"] == 0:
            continue
        e = rates(v)
        if full[name]["launches"]:
            e["full_diagonals"] = rates(full[name])
        if ramp[name]["launches"]:
            e["ramp_diagonals"] = rates(ramp[name])
        st_out[name] = e
        if name in ("qkv", "oproj", "gateup", "down"):
            for key, src in (("all", v), ("full", full[name]), ("ramp", ramp[name])):
                for f in ("ms", "flops", "launches"):
                    gemm[key][f] += src[f]
    gemm_out = {}
    for key, v in gemm.items():
        if v["ms"] > 0:
            tf = v["flops"] / (v["ms"] / 1e3) / 1e12
            gemm_out[key if key != "all" else "all_diagonals"] = {
                "tflops": round(tf, 1), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    gemm_out["full_diagonals"] = gemm_out.pop("full", None)
    gemm_out["ramp_diagonals"] = gemm_out.pop("ramp", None)

    # the dominant kernel: the GEMM stage that takes the most time
    kind = ("llama" if llama else "encoder" if encoder else
            "linear_gelu" if cfg.cell == ri.CELL_LINEAR_GELU else "norm_swiglu")
    dom = max((s for s in GEMM_KERNELS[kind] if stages[s]["launches"]), key=lambda s: stages[s]["ms"])
    # the committed counter summary covers the 1B-shaped workload's gate/up kernel only
    traffic = (measured_traffic() if args.workload == "llama1b" and dom == "gateup" and not f16 and B == 1
               else None)
    gu = stages[dom]
    achieved = gu["flops"] / gu["launches"] / (gu["ms"] / 1e3 / gu["launches"]) / 1e12
    alu = kind == "linear_gelu"      # fp32 arithmetic on the vector ALUs, no matrix cores
    peak = PEAK_FP32_VALU_TFLOPS if alu else PEAK_BF16_TFLOPS
    roofline = {"kernel": ("" if alu else "grouped GEMM, ") + GEMM_KERNELS[kind][dom],
                "bound": "alu" if alu else "mfma", "achieved": round(achieved, 3), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 5), "traffic": traffic,
                "traffic_source": ("HBM-side bytes per launch from the committed rocprofv3 FETCH_SIZE / "
                                   "WRITE_SIZE summary profiles/llama1b_rmt_L16_S128_gateup_hbm_traffic.md, "
                                   "valid for the GEMM source hash recorded there (not measured in this run)")
                if traffic else None,
                "avg_launch_us": round(gu["ms"] / gu["launches"] * 1e3, 2),
                "flops_per_launch": gu["flops"] / gu["launches"]}

    config = {"workload": cfg.name, "layers": cfg.L, "segments": cfg.S, "segment_tokens": cfg.n,
              "memory_rows": cfg.m, "width": cfg.d}
    if llama or encoder:
        config.update({"heads": cfg.Hq, "kv_heads": cfg.Hkv, "head_dim": cfg.hd})
    if encoder:
        config["cell"] = (("post" if cfg.post_norm else "pre") +
                          "-norm encoder layer (LayerNorm, unmasked MHA, ReLU FFN, biases)")
    config.update({"ffn": cfg.F, "tokens": T, "path": "rmt_forward_diagonal"})
    props = torch.cuda.get_device_properties(0)
    device = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
              "compute_units": props.multi_processor_count,
              "hbm_gib": round(props.total_memory / 2**30, 1)}
    if B > 1:
        config["sequences"] = B
    if llama:
        config["vocab"] = cfg.V
    data = ("synthetic (seeded random weights, token ids uniform over the vocabulary)" if llama
            else "synthetic (seeded random weights and input embeddings)")
    dtype = "f32" if cfg.dtype != ri.BF16 else ("f16" if f16 else "bf16")
    result = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": data,
        "config": config,
        "roofline": roofline,
        "device": device,
        "grouped_gemm_stages": gemm_out,
        "ms_per_step_with_stage_events": round(wall_ev / args.steps * 1e3, 2),
        "stages": ({(POSTNORM_STAGE_NAMES if cfg.post_norm else ENCODER_STAGE_NAMES).get(k, k): v
                    for k, v in st_out.items()} if encoder else st_out),
    }

    if not args.no_seq:
        seq = lambda: model.forward_sequential(tok_d, mem0_d, hidden, mem)  # noqa: E731
        seq()
        torch.cuda.synchronize()
        w_s, _ = timed_steps(seq, 1, stream)
        result["sequential"] = {"value": round(B * T / w_s, 1), "unit": "tokens/s",
                                "ms_per_step": round(w_s * 1e3, 2),
                                "diagonal_speedup": round(w_s / (wall / args.steps), 3)}
        log(f"[bench] sequential: {w_s * 1e3:.1f} ms/step")

    if not args.no_sweep:
        result["grouped_gemm_sweep"] = {"workload": ri.GROUPED_GEMM_1B.name, **gemm_sweep()}
        log("[bench] grouped GEMM sweep done")

    if not args.no_cpu and B > 1:
        log("[bench] the CPU oracle leg runs at one sequence only; skipped for --batch > 1")
    elif not args.no_cpu:
        Sp = args.cpu_segments

        def gpu_mem_prefix():
            # memory after the prefix: rerun the GPU on exactly that prefix
            model.set_segments(Sp)
            mp = torch.empty_like(mem)
            hp = torch.empty((Sp * cfg.n, cfg.d), dtype=torch.float32, device="cuda")
            model.forward_diagonal(tok_d[:Sp * cfg.n], mem0_d, hp, mp)
            torch.cuda.synchronize()
            model.set_segments(cfg.S)
            return mp.cpu().numpy().astype(np.float64)

        log(f"[bench] CPU oracle on {Sp} segments ...")
        result["cpu_baseline"] = cpu_baseline(cfg, layers, tokens, mem0, embed, hidden_np,
                                              gpu_mem_prefix, Sp)
    model.close()
    del emb_dev
    if (not args.no_secondary and args.workload == "llama1b" and B == 1 and not f16
            and not args.calibrate_copy):
        result["secondary"] = secondary_llama8b()
    if args.calibrate_copy:
        src = torch.ones(256 * 2**20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
