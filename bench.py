"""Benchmark: GPTQ of one Llama-7B-shaped q_proj layer on one MI355X.

Workload (default): W [4096 x 4096] fp16 ~ N(0, 0.02); calibration X = 128
sequences x 2048 tokens x 4096 channels, bf16, Student-t(4) with 0.5 % of the
channels x30; 4-bit asymmetric, group 128, block 128, damp 0.01, natural order.
One step is the whole path on inputs already resident in HBM:
H = 0; H += 2 X^T X; damp + order + U; column loop with lazy updates; pack.

Prints one JSON line.  The roofline object is for the dominant stage (the
Hessian: the SYRK kernel plus its fixed-order split reduction), timed with HIP
events on the stream the library launches on.  The cpu_baseline object times
the float64 CPU oracle on a bounded sample of the same workload.  Two more
objects time the widened rows on the same inputs: w4a16_decode (the product on
the packed layer at one activation row) and awq (the activation-aware
quantization of the same layer from the same calibration tokens); a third,
block_sequential, times layer-by-layer GPTQ over a Llama-7B-shaped decoder
block on 32,768 of the calibration tokens.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="c2_llama7b_q_proj")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=16384,
                    help="tokens in the oracle's Hessian sample (result scaled to all tokens)")
    ap.add_argument("--cpu-rows", type=int, default=1024,
                    help="rows in the oracle's column-loop sample (result scaled to all rows)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "hessian_c2_traffic.json"))
    ap.add_argument("--no-extras", action="store_true",
                    help="report the GPTQ step only (no w4a16_decode, awq, block_sequential objects), "
                         "e.g. for a kernel trace of the step alone")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (for scaling the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


HESSIAN_SOURCE = os.path.join(ROOT, "post_weight_quantization_29_amd", "csrc", "hessian.hip")


def source_digest(path=HESSIAN_SOURCE):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def calibrate_copy(mib):
    """One copy kernel of a known size: it reads and writes mib MiB once each."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": n * 4, "bytes_written": n * 4}),
          flush=True)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(W, X, wl, args):
    """The oracle as it stands, on a bounded sample: its Hessian over the first
    cpu_tokens tokens (time scaled by n_tokens/cpu_tokens), its factor for the
    whole layer, its column loop over cpu_rows rows (time scaled by
    d_out/cpu_rows; rows are independent), and its packing."""
    import numpy as np
    import gptq_inputs as gi
    from oracle import gptq_ref as o

    layer, calib, q = wl.layers[0], wl.calib[0], wl.quant[0]
    cores = len(os.sched_getaffinity(0))
    nt = min(args.cpu_tokens, calib.n_tokens)
    xs = gi.to_float64(X[:nt], calib.dtype)
    t0 = time.perf_counter()
    Hs = o.hessian([xs], calib.d_in)
    t_h = (time.perf_counter() - t0) * (calib.n_tokens / nt)
    rows = min(args.cpu_rows, layer.d_out)
    W64 = gi.to_float64(W[:rows], layer.dtype)
    t0 = time.perf_counter()
    r = o.gptq(W64, Hs, bits=q.bits, group_size=q.group_size, block_size=q.block_size,
               damp_percent=q.damp_percent, desc_act=bool(q.desc_act))
    t_q = time.perf_counter() - t0
    # split the loop time from the factor time: time the factor alone
    t0 = time.perf_counter()
    Hd, _ = o.damp(Hs, q.damp_percent)
    o.hinv_factor(Hd)
    t_f = time.perf_counter() - t0
    t_loop = max(t_q - t_f, 0.0) * (layer.d_out / rows)
    t0 = time.perf_counter()
    o.pack_int4(r.codes)
    t_p = (time.perf_counter() - t0) * (layer.d_out / rows)
    total = t_h + t_f + t_loop + t_p
    weights = layer.d_out * layer.d_in
    return {
        "value": weights / total, "unit": "weights/s", "cores": cores, "kind": "oracle",
        "sample": (f"float64 numpy oracle: Hessian over {nt} of {calib.n_tokens} tokens "
                   f"(x{calib.n_tokens / nt:g}), factor of the full {calib.d_in}^2 H, column loop "
                   f"over {rows} of {layer.d_out} rows (x{layer.d_out / rows:g}); "
                   f"est. total {total:.1f} s per layer"),
        "stages_s": {"hessian": round(t_h, 3), "factor": round(t_f, 3), "loop": round(t_loop, 3),
                     "pack": round(t_p, 4)},
    }


def w4a16_measure(P, torch, packed, scales, zeros, group_size, reps=24):
    """Decode-shaped product on packed layers (one activation row, bf16 in, fp32
    out): the quantized layer of this step, and a 70B down_proj-shaped packed
    layer (8192 x 28672, random codes) for the HBM roofline; on the latter also
    a prefill shape (2048 activation rows, the MFMA path) against the bf16 MFMA
    peak.  The large layer
    is held in three copies used in turn, 3 x 132 MB, more than the 256 MB
    last-level cache, so each call streams its weights from HBM.  HIP events
    on the launch stream, mean over reps after a warm-up."""
    out = []
    dev = packed.device
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    big_rows, big_cols, G = 8192, 28672, 128

    def layer():
        return (torch.randint(-2**31, 2**31 - 1, (big_rows, big_cols // 8), dtype=torch.int32,
                              device=dev, generator=g),
                torch.rand((big_rows, big_cols // G), device=dev, generator=g) * 0.01 + 1e-3,
                torch.randint(0, 16, (big_rows, big_cols // G), dtype=torch.int32, device=dev,
                              generator=g))

    stream = torch.cuda.current_stream()
    for copies, gs in (([(packed, scales, zeros)], group_size), ([layer() for _ in range(3)], G)):
        pk, sc, zr = copies[0]
        d_out, d_in = pk.shape[0], pk.shape[1] * 8
        X = torch.randn((1, d_in), device=dev, generator=g).to(torch.bfloat16)
        Y = torch.empty((1, d_out), dtype=torch.float32, device=dev)
        for c in copies:
            P.gptq_w4a16_gemm(X, c[0], c[1], c[2], Y, group_size=gs)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            c = copies[i % len(copies)]
            P.gptq_w4a16_gemm(X, c[0], c[1], c[2], Y, group_size=gs)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        nbytes = pk.numel() * 4 + sc.numel() * 4 + zr.numel() * 4 + X.numel() * 2 + Y.numel() * 4
        out.append({"shape": f"{d_out}x{d_in}", "m": 1, "us": round(us, 2), "bytes": nbytes,
                    "GB_per_s": round(nbytes / us / 1e3, 1),
                    "frac_hbm": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4)})
        if len(copies) == 3:
            # prefill shape on the same copies: 2048 activation rows (the tiled MFMA product)
            mp = 2048
            Xp = torch.randn((mp, d_in), device=dev, generator=g).to(torch.bfloat16)
            Yp = torch.empty((mp, d_out), dtype=torch.float32, device=dev)
            for c in copies:
                P.gptq_w4a16_gemm(Xp, c[0], c[1], c[2], Yp, group_size=gs)
            e0.record(stream)
            for i in range(6):
                c = copies[i % 3]
                P.gptq_w4a16_gemm(Xp, c[0], c[1], c[2], Yp, group_size=gs)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / 6
            tf = 2.0 * mp * d_out * d_in / us / 1e6
            out.append({"shape": f"{d_out}x{d_in}", "m": mp, "us": round(us, 1), "TFLOP_per_s": round(tf, 1),
                        "frac_bf16_mfma": round(tf / PEAK_BF16_TFLOPS, 4)})
        del copies
    return out


def awq_measure(P, torch, Wg, Xg, reps=5):
    """The AWQ path on the same layer and calibration tokens (both already in
    HBM): the channel statistic over all tokens, the factor search (25
    candidates, top 5 %, 4-bit groups of 128), the scaled quantization and
    the packing.  HIP events on the launch stream, mean over reps after a
    warm-up.  The statistic reads X once (2 bytes per element): its HBM rate
    is reported against 8 TB/s."""
    d_out, d = Wg.shape
    N = Xg.shape[0]
    dev = Wg.device
    grid = P.AWQ_DEFAULT_GRID
    a = torch.zeros((d,), dtype=torch.float64, device=dev)
    s = torch.empty((d,), dtype=torch.float32, device=dev)
    scores = torch.empty((len(grid),), dtype=torch.float64, device=dev)
    best = torch.empty((1,), dtype=torch.int32, device=dev)
    codes = torch.empty((d_out, d), dtype=torch.uint8, device=dev)
    scales = torch.empty((d_out, d // 128), dtype=torch.float32, device=dev)
    zeros = torch.empty((d_out, d // 128), dtype=torch.int32, device=dev)
    packed = torch.empty((d_out, d // 8), dtype=torch.int32, device=dev)
    ws_a = torch.empty(P.gptq_awq_sumsq_workspace_size(N, d), dtype=torch.uint8, device=dev)
    ws_s = torch.empty(P.gptq_awq_search_workspace_size(d_out, d, 128), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def run(ev=None):
        if ev:
            ev[0].record(stream)
        a.zero_()
        P.gptq_awq_act_sumsq(a, Xg, ws_a)
        if ev:
            ev[1].record(stream)
        P.gptq_awq_search(Wg, a, s, scores, best, grid=grid, ws=ws_s)
        if ev:
            ev[2].record(stream)
        P.gptq_awq_quantize(Wg, s, codes, scales, zeros, None)
        if ev:
            ev[3].record(stream)
        P.gptq_pack_int4(codes, packed)
        if ev:
            ev[4].record(stream)

    run()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(reps)]
    for e in evs:
        run(e)
    torch.cuda.synchronize()
    names = ["statistic", "search", "quantize", "pack"]
    ms = {n: sum(e[k].elapsed_time(e[k + 1]) for e in evs) / reps for k, n in enumerate(names)}
    total = sum(ms.values())
    x_bytes = N * d * Xg.element_size()
    gbs = x_bytes / (ms["statistic"] / 1e3) / 1e9
    return {"stages_ms": {k: round(v, 4) for k, v in ms.items()}, "ms_per_layer": round(total, 4),
            "weights_per_s": d_out * d / (total / 1e3), "best_factor": float(grid[int(best.item())]),
            "statistic_GB_per_s": round(gbs, 1), "statistic_frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
            "grid": len(grid)}


def block_measure(P, torch, Xg, n_tokens=32768, seq_len=2048):
    """Layer-sequential GPTQ over one Llama-7B-shaped decoder block (d 4096,
    32 heads of 128, intermediate 11008; random fp16 weights N(0, 0.02)) on
    the first n_tokens calibration tokens (as fp32), 4-bit groups of 128:
    q/k/v share one Hessian and factor, then o, gate/up, down, each from the
    quantized stages before it.  HIP events per stage, one warm-up run."""
    from post_weight_quantization_29_amd import block as PB
    d, f, heads = 4096, 11008, 32
    dev = Xg.device
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    shapes = {"q": (d, d), "k": (d, d), "v": (d, d), "o": (d, d), "gate": (f, d), "up": (f, d),
              "down": (d, f)}
    W = {n: (torch.randn(s, device=dev, generator=g) * 0.02).half() for n, s in shapes.items()}
    x = Xg[:n_tokens].float().contiguous()
    cfg = P.make_config(bits=4, group_size=128)
    shape = PB.BlockShape(d, heads, f, seq_len)
    stream = torch.cuda.current_stream()

    def run(ev=None):
        if ev:
            ev[0].record(stream)
        x1, _, qz = PB.stage_qkv(x, W, cfg)
        if ev:
            ev[1].record(stream)
        attn, _, qo = PB.stage_o(x1, qz["q"].Q, qz["k"].Q, qz["v"].Q, W, cfg, shape)
        if ev:
            ev[2].record(stream)
        h, x2, _, qgu = PB.stage_gate_up(x, attn, qo["o"].Q, W, cfg)
        if ev:
            ev[3].record(stream)
        m, _, qd = PB.stage_down(x2, qgu["gate"].Q, qgu["up"].Q, W, cfg, shape)
        if ev:
            ev[4].record(stream)
        PB.block_output(m, h, qd["down"].Q)
        if ev:
            ev[5].record(stream)

    run()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    run(ev)
    torch.cuda.synchronize()
    names = ["qkv", "o", "gate_up", "down", "output"]
    ms = {n: ev[k].elapsed_time(ev[k + 1]) for k, n in enumerate(names)}
    total = sum(ms.values())
    weights = sum(a * b for a, b in shapes.values())
    return {"shape": {"d": d, "heads": heads, "f": f, "seq_len": seq_len, "n_tokens": n_tokens},
            "stages_ms": {k: round(v, 3) for k, v in ms.items()}, "ms_per_block": round(total, 3),
            "weights_per_s": weights / (total / 1e3)}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "single-GPU implementation: --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    import numpy as np
    import torch

    import gptq_inputs as gi
    import post_weight_quantization_29_amd as P

    wl = gi.workload(args.workload)
    layer, calib, q = wl.layers[0], wl.calib[0], wl.quant[0]
    d_out, d = layer.d_out, layer.d_in
    N = calib.n_tokens
    log(f"[bench] generating {args.workload}: W {d_out}x{d} {layer.dtype}, X {N}x{d} {calib.dtype}")
    t0 = time.time()
    W = gi.weight(layer, wl.config)
    X = gi.x_full(calib, wl.config)
    log(f"[bench] inputs generated in {time.time() - t0:.1f}s")

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
    if calib.dtype == "bf16":
        Xg = torch.from_numpy(X.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        Xg = torch.from_numpy(X).to(dev)
    Wg = torch.from_numpy(W).to(dev)
    assert Wg.dtype == tdt[layer.dtype]

    cfg = P.make_config(bits=q.bits, group_size=q.group_size, block_size=q.block_size,
                        damp_percent=q.damp_percent, desc_act=q.desc_act)
    G = d if q.group_size == -1 else q.group_size
    ng = (d + G - 1) // G
    H = torch.zeros((d, d), dtype=torch.float32, device=dev)
    # fp64 diagonal keys only where the column order needs them (desc_act);
    # without them damping takes mean(diag H) from H itself
    hdiag = torch.zeros((d,), dtype=torch.float64, device=dev) if q.desc_act else None
    U = torch.empty((d, d), dtype=torch.float32, device=dev)
    perm = torch.empty((d,), dtype=torch.int32, device=dev)
    codes = torch.empty((d_out, d), dtype=torch.uint8, device=dev)
    scales = torch.empty((d_out, ng), dtype=torch.float32, device=dev)
    zeros = torch.empty((d_out, ng), dtype=torch.int32, device=dev)
    g_idx = torch.empty((d,), dtype=torch.int32, device=dev)
    packed = torch.empty((d_out, d // 8), dtype=torch.int32, device=dev)
    ws_h = torch.empty(P.gptq_hessian_workspace_size(N, d), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(P.gptq_prepare_hinv_workspace_size(d), dtype=torch.uint8, device=dev)
    ws_q = torch.empty(P.gptq_quantize_workspace_size(d_out, d, cfg), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def rec(ev, i):
        if ev is not None:
            ev[i].record(stream)

    def step(ev=None):
        rec(ev, 0)
        H.zero_()
        if hdiag is not None:
            hdiag.zero_()
        rec(ev, 1)
        P.gptq_hessian_accumulate(H, Xg, hdiag, ws_h)
        rec(ev, 2)
        P.gptq_prepare_hinv(H, q.damp_percent, q.desc_act, U, perm, hdiag, ws_f)
        rec(ev, 3)
        P.gptq_quantize_layer(Wg, U, perm, cfg, codes, scales, zeros, g_idx, None, ws_q)
        rec(ev, 4)
        P.gptq_pack_int4(codes, packed)
        rec(ev, 5)

    for i in range(args.warmup):
        step()
        log(f"[bench] warmup {i + 1}/{args.warmup} done")
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    log(f"[bench] {args.steps} timed steps done in {wall:.3f}s")

    names = ["zero_h", "hessian", "prepare_hinv", "quantize", "pack"]
    st = {n: [] for n in names}
    for e in evs:
        for k, n in enumerate(names):
            st[n].append(e[k].elapsed_time(e[k + 1]))
    mean = {n: float(np.mean(v)) for n, v in st.items()}
    ms_step = wall * 1e3 / args.steps
    weights = d_out * d
    value = weights / (ms_step / 1e3)

    h_flops = float(N) * d * (d + 1)                  # lower triangle incl. diagonal
    achieved_tf = h_flops / (mean["hessian"] / 1e3) / 1e12
    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            tj = json.load(open(args.traffic_json))
            # counters taken on another kernel build do not describe this one
            if tj.get("workload") == args.workload and tj.get("source_sha256") == source_digest():
                traffic = tj.get("bytes_per_launch")
        except Exception:
            traffic = None

    out = {
        "metric": "GPTQ weights quantized/s per layer (+ Hessian TFLOP/s, % MFMA/HBM peak)",
        "value": value,
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32 (bf16 x bf16 -> fp32 Hessian)",
        "data": "synthetic",
        "config": {"workload": args.workload, "d_out": d_out, "d_in": d, "n_tokens": N,
                   "x_dtype": calib.dtype, "w_dtype": layer.dtype, "bits": q.bits,
                   "group_size": q.group_size, "block_size": q.block_size,
                   "damp_percent": q.damp_percent, "desc_act": q.desc_act,
                   "parallelism": "single GPU"},
        "stages_ms": {k: round(v, 4) for k, v in mean.items()},
        "hessian_tflops": achieved_tf,
        "weights_per_s_excl_hessian": weights / ((ms_step - mean["hessian"] - mean["zero_h"]) / 1e3),
        "roofline": {"bound": "mfma", "achieved": achieved_tf, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved_tf / PEAK_BF16_TFLOPS,
                     "traffic": traffic,
                     "kernel": ("gptq_hessian_accumulate: syrk16_kernel<bf16> + syrk_reduce_kernel<4, 512>"
                                + (" + diag_reduce_kernel (fp64 diagonal keys)" if q.desc_act else "")),
                     "work_per_launch": f"N*d*(d+1) = {h_flops:.4g} flop"},
    }
    if not args.no_extras:
        out["w4a16_decode"] = w4a16_measure(P, torch, packed, scales, zeros, q.group_size)
        out["awq"] = awq_measure(P, torch, Wg, Xg)
        out["block_sequential"] = block_measure(P, torch, Xg)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(W, X, wl, args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
