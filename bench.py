"""Benchmark: GPTQ of one linear layer on one MI355X.

Headline workload (default): the 70B-shaped down_proj, W [8192 x 28672] fp16
~ N(0, 0.015); calibration X = 128 sequences x 2048 tokens x 28672 channels
(262,144 tokens, 14 GiB), bf16, Student-t(3); 4-bit asymmetric, group 128,
block 128, damp 0.01, desc_act.  One step is the whole path on inputs already
resident in HBM: H = 0; H += 2 X^T X (one call over every token, with the
fp64 diagonal keys the desc_act order needs); damp + order + U; column loop
with lazy updates; pack.  X is generated on the host chunk by chunk (32,768
tokens at a time) and copied into one device buffer, so the host never holds
all of it.

Prints one JSON line.  `value` is weights quantized per second including the
Hessian (d_out * d_in / step time).  The roofline object is for the Hessian
call (the SYRK kernel plus its fixed-order split reduction and the fp64
diagonal), timed with HIP events on the stream the library launches on; the
`stages` object puts every stage against its own roof.  `hessian_streamed`
times the Hessian as eight calls of 32,768 tokens.  `per_config` measures the
other workloads' layers (Llama-7B q_proj, the Llama-7B MLP, the 13B desc_act
layers) stage by stage, with prepare_hinv amortized over the layers that share
one H.  The cpu_baseline object times the float64 CPU oracle on a bounded
sample of the headline workload.  w4a16_decode, awq and block_sequential time
the widened rows.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 MFMA
# fp32-accurate products as three fp16 MFMA products of split operands: the
# fp16 dense MFMA peak (2.5 PF, as bf16) over three
SPLIT_TFLOPS = 2500.0 / 3.0
PEAK_HBM_GBS = 8000.0
EXTRA_CONFIGS = ("c2_llama7b_q_proj", "c3_llama7b_mlp", "c4_13b_desc_act")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="c5_70b_down_proj")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=2048,
                    help="tokens in the oracle's Hessian sample (time scaled to all tokens)")
    ap.add_argument("--cpu-dim", type=int, default=6144,
                    help="leading channels in the oracle's factor and column-loop sample")
    ap.add_argument("--cpu-rows", type=int, default=64,
                    help="rows in the oracle's column-loop sample (time scaled to all rows)")
    ap.add_argument("--traffic-json", default=None,
                    help="FETCH_SIZE/WRITE_SIZE summary of the Hessian call (default: "
                         "profiles/hessian_<workload>_traffic.json)")
    ap.add_argument("--no-extras", action="store_true",
                    help="report the headline step only (no hessian_streamed, per_config, "
                         "w4a16_decode, awq, block_sequential), e.g. for a kernel trace of the step")
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


# ---------------------------------------------------------------- inputs

def upload_calib(torch, gi, cal, config, dev):
    """All calibration tokens of cal in one device buffer, drawn chunk by chunk."""
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[cal.dtype]
    X = torch.empty((cal.n_tokens, cal.d_in), dtype=tdt, device=dev)
    for c in range(gi.n_chunks(cal)):
        r0 = c * gi.CHUNK_TOKENS
        xc = gi.x_chunk(cal, config, c)
        t = torch.from_numpy(xc.view("int16") if cal.dtype == "bf16" else xc)
        X[r0:r0 + xc.shape[0]].copy_(t.to(dev).view(tdt))
        del xc, t
    return X


def upload_weight(torch, gi, layer, config, dev):
    W = gi.weight(layer, config)
    return W, torch.from_numpy(W).to(dev)


# ---------------------------------------------------------------- algorithmic work

def hessian_flops(n, d):
    return float(n) * d * (d + 1)           # lower triangle incl. the diagonal


def factor_flops(d):
    return 2.0 * d ** 3 / 3.0


def trailing_flops(d_out, d, B=128):
    # sum over blocks of 2 * d_out * B * (columns after the block)
    return sum(2.0 * d_out * min(B, d - b0) * (d - min(d, b0 + B)) for b0 in range(0, d, B))


def quantize_bytes(d_out, d, G):
    # read the fp32 work weight, write the u8 code and the fp32 error, scale+zero per group
    return d_out * d * (4.0 + 1.0 + 4.0 + 8.0 / G)


def pack_bytes(d_out, d):
    return d_out * d * 1.5


def stage_roofs(N, d_out, d, G):
    """Roof time (s) of each stage: max(flops / peak, bytes / HBM)."""
    r = {
        "hessian": max(hessian_flops(N, d) / (PEAK_BF16_TFLOPS * 1e12),
                       (2.0 * N * d + 8.0 * d * d) / (PEAK_HBM_GBS * 1e9)),
        "prepare_hinv": max(factor_flops(d) / (SPLIT_TFLOPS * 1e12), 16.0 * d * d / (PEAK_HBM_GBS * 1e9)),
        "quantize": max(trailing_flops(d_out, d) / (SPLIT_TFLOPS * 1e12),
                        quantize_bytes(d_out, d, G) / (PEAK_HBM_GBS * 1e9)),
        "pack": pack_bytes(d_out, d) / (PEAK_HBM_GBS * 1e9),
    }
    return r


# the factor's and the lazy update's large products run on bf16 MFMA as
# three-piece splits of their fp32 operands (six bf16 products per fp32 one)
SPLIT_NOTE = ("TFLOP/s counts the algorithm's fp32 flops; the roof is the fastest fp32-accurate product on the "
              "chip, three fp16 MFMA products of split operands (2.5 PF / 3 = 833 TFLOP/s), which the factor's and "
              "the lazy update's large products use (smaller ones run fp32 MFMA tiles); fp32_mfma_ratio is the rate "
              "over the fp32 MFMA peak (157.3), for context")


def stage_report(ms, N, d_out, d, G):
    """Each measured stage against its roof."""
    roofs = stage_roofs(N, d_out, d, G)
    out = {}
    if "hessian" in ms:
        tf = hessian_flops(N, d) / (ms["hessian"] / 1e3) / 1e12
        out["hessian"] = {"ms": round(ms["hessian"], 4), "TFLOP_per_s": round(tf, 1),
                          "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                          "roof_ms": round(roofs["hessian"] * 1e3, 4)}
    tf = factor_flops(d) / (ms["prepare_hinv"] / 1e3) / 1e12
    out["prepare_hinv"] = {"ms": round(ms["prepare_hinv"], 4), "TFLOP_per_s": round(tf, 2),
                           "frac_roof": round(tf / SPLIT_TFLOPS, 4),
                           "fp32_mfma_ratio": round(tf / PEAK_FP32_TFLOPS, 4),
                           "roof_ms": round(roofs["prepare_hinv"] * 1e3, 4), "note": SPLIT_NOTE}
    qb = quantize_bytes(d_out, d, G) / (ms["quantize"] / 1e3) / 1e9
    qt = trailing_flops(d_out, d) / (ms["quantize"] / 1e3) / 1e12
    out["quantize"] = {"ms": round(ms["quantize"], 4), "GB_per_s": round(qb, 1),
                       "frac_hbm": round(qb / PEAK_HBM_GBS, 4),
                       "trailing_TFLOP_per_s": round(qt, 2),
                       "frac_roof": round(qt / SPLIT_TFLOPS, 4),
                       "fp32_mfma_ratio": round(qt / PEAK_FP32_TFLOPS, 4),
                       "roof_ms": round(roofs["quantize"] * 1e3, 4), "note": SPLIT_NOTE}
    pb = pack_bytes(d_out, d) / (ms["pack"] / 1e3) / 1e9
    out["pack"] = {"ms": round(ms["pack"], 4), "GB_per_s": round(pb, 1),
                   "frac_hbm": round(pb / PEAK_HBM_GBS, 4), "roof_ms": round(roofs["pack"] * 1e3, 4)}
    return out, roofs


def timed(torch, fn, reps, stream):
    """Median of reps HIP-event timings (ms) on the launch stream, after one warm-up."""
    fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return statistics.median(ts)


def hessian_streamed_ms(torch, P, gi, H, hdiag, Xg, stream, reps=3):
    """The Hessian as the calibration arrives: eight calls of 32,768 tokens."""
    N = Xg.shape[0]
    chunk = gi.CHUNK_TOKENS
    ws = torch.empty(P.gptq_hessian_workspace_size(chunk, Xg.shape[1]), dtype=torch.uint8,
                     device=Xg.device)

    def run():
        H.zero_()
        if hdiag is not None:
            hdiag.zero_()
        for r0 in range(0, N, chunk):
            P.gptq_hessian_accumulate(H, Xg[r0:r0 + chunk], hdiag, ws)
    return timed(torch, run, reps, stream)


# ---------------------------------------------------------------- the other workloads

def measure_config(torch, P, gi, key, dev, keep_x=False):
    """Stage by stage on every layer of a workload (HIP events, median of 3):
    the Hessian of each distinct d_in (one call over all tokens, and eight
    32,768-token calls), prepare_hinv once per H, quantize and pack per layer
    and quantizer setting.  T_layer = prepare + quantize + pack; amortized:
    prepare divided over the layers (and settings) that share the H."""
    wl = gi.workload(key)
    stream = torch.cuda.current_stream()
    out = {"workload": key, "hessians": [], "layers": []}
    kept = None
    for cal in wl.calib:
        d, N = cal.d_in, cal.n_tokens
        t0 = time.time()
        Xg = upload_calib(torch, gi, cal, wl.config, dev)
        log(f"[bench] {key} d_in={d}: calibration generated in {time.time() - t0:.1f}s")
        desc = wl.quant[0].desc_act
        damp = wl.quant[0].damp_percent
        H = torch.zeros((d, d), dtype=torch.float32, device=dev)
        hdiag = torch.zeros((d,), dtype=torch.float64, device=dev) if desc else None
        ws_h = torch.empty(P.gptq_hessian_workspace_size(N, d), dtype=torch.uint8, device=dev)

        def hess():
            H.zero_()
            if hdiag is not None:
                hdiag.zero_()
            P.gptq_hessian_accumulate(H, Xg, hdiag, ws_h)
        t_h = timed(torch, hess, 3, stream)
        t_hs = hessian_streamed_ms(torch, P, gi, H, hdiag, Xg, stream)
        hess()
        del ws_h
        if keep_x and kept is None:
            kept = Xg
        else:
            del Xg
        torch.cuda.empty_cache()
        U = torch.empty((d, d), dtype=torch.float32, device=dev)
        perm = torch.empty((d,), dtype=torch.int32, device=dev)
        ws_f = torch.empty(P.gptq_prepare_hinv_workspace_size(d), dtype=torch.uint8, device=dev)
        t_f = timed(torch, lambda: P.gptq_prepare_hinv(H, damp, desc, U, perm, hdiag, ws_f), 3, stream)
        del ws_f
        tf_h = hessian_flops(N, d) / (t_h / 1e3) / 1e12
        layers = [ly for ly in wl.layers if ly.d_in == d]
        sharing = len(layers) * len(wl.quant)
        out["hessians"].append({
            "d_in": d, "n_tokens": N, "one_call_ms": round(t_h, 4), "TFLOP_per_s": round(tf_h, 1),
            "frac_bf16_peak": round(tf_h / PEAK_BF16_TFLOPS, 4),
            "streamed_8x32768_ms": round(t_hs, 4),
            "streamed_TFLOP_per_s": round(hessian_flops(N, d) / (t_hs / 1e3) / 1e12, 1),
            "prepare_hinv_ms": round(t_f, 4),
            "prepare_TFLOP_per_s": round(factor_flops(d) / (t_f / 1e3) / 1e12, 2),
            "shared_by": sharing})
        for layer in layers:
            _, Wg = upload_weight(torch, gi, layer, wl.config, dev)
            d_out = layer.d_out
            for q in wl.quant:
                cfg = P.make_config(bits=q.bits, group_size=q.group_size, block_size=q.block_size,
                                    damp_percent=q.damp_percent, desc_act=q.desc_act)
                G = d if q.group_size == -1 else q.group_size
                ng = (d + G - 1) // G
                codes = torch.empty((d_out, d), dtype=torch.uint8, device=dev)
                scales = torch.empty((d_out, ng), dtype=torch.float32, device=dev)
                zeros = torch.empty((d_out, ng), dtype=torch.int32, device=dev)
                g_idx = torch.empty((d,), dtype=torch.int32, device=dev)
                packed = torch.empty((d_out, d // 8), dtype=torch.int32, device=dev)
                ws_q = torch.empty(P.gptq_quantize_workspace_size(d_out, d, cfg), dtype=torch.uint8,
                                   device=dev)
                t_q = timed(torch, lambda: P.gptq_quantize_layer(Wg, U, perm, cfg, codes, scales, zeros,
                                                                 g_idx, None, ws_q), 3, stream)
                t_p = timed(torch, lambda: P.gptq_pack_int4(codes, packed), 3, stream)
                rep, roofs = stage_report({"prepare_hinv": t_f, "quantize": t_q, "pack": t_p},
                                          N, d_out, d, G)
                t_layer = t_f + t_q + t_p
                t_am = t_f / sharing + t_q + t_p
                w = d_out * d
                roof_excl = (roofs["prepare_hinv"] / sharing + roofs["quantize"] + roofs["pack"]) * 1e3
                out["layers"].append({
                    "layer": layer.name, "d_out": d_out, "d_in": d, "bits": q.bits,
                    "group_size": q.group_size, "desc_act": q.desc_act,
                    "quantize_ms": round(t_q, 4), "pack_ms": round(t_p, 4),
                    "T_layer_ms": round(t_layer, 4), "T_layer_amortized_ms": round(t_am, 4),
                    "weights_per_s": w / (t_layer / 1e3),
                    "weights_per_s_amortized": w / (t_am / 1e3),
                    "weights_per_s_incl_hessian_amortized": w / ((t_am + t_h / sharing) / 1e3),
                    "roofline_frac_amortized_excl_hessian": round(roof_excl / t_am, 4),
                    "stages": {k: v for k, v in rep.items() if k != "prepare_hinv"}})
                del codes, scales, zeros, g_idx, packed, ws_q
            del Wg
        del H, U, perm, hdiag
        torch.cuda.empty_cache()
        log(f"[bench] {key} d_in={d} measured")
    return out, kept


# ---------------------------------------------------------------- CPU oracle

def cpu_baseline(W, wl, args):
    """The oracle as it stands, on a bounded sample of the workload, each stage
    scaled by its own complexity to the whole layer:
      Hessian: cpu_tokens tokens at the full d_in            (x n_tokens / cpu_tokens)
      factor:  the leading cpu_dim x cpu_dim block of H_d      (x (d_in / cpu_dim)^3)
      loop:    cpu_rows rows over the leading cpu_dim columns  (x d_out / cpu_rows x (d_in / cpu_dim)^2,
               the loop's per-row work being its O(d_in^2) lazy updates)
      pack:    those rows' codes                              (x d_out * d_in / (cpu_rows * cpu_dim))"""
    import numpy as np
    import gptq_inputs as gi
    from oracle import gptq_ref as o

    layer, calib, q = wl.layers[0], wl.calib[0], wl.quant[0]
    d, d_out, N = layer.d_in, layer.d_out, calib.n_tokens
    cores = len(os.sched_getaffinity(0))
    nt = min(args.cpu_tokens, N)
    xs = gi.to_float64(gi.x_chunk(calib, wl.config, 0)[:nt], calib.dtype)
    t0 = time.perf_counter()
    Hs = o.hessian([xs], d)
    t_h = (time.perf_counter() - t0) * (N / nt)
    del xs
    ds = min(args.cpu_dim, d)
    Hsub = np.ascontiguousarray(Hs[:ds, :ds])
    del Hs
    t0 = time.perf_counter()
    prep = o.prepare(Hsub, q.damp_percent, bool(q.desc_act))
    t_f = (time.perf_counter() - t0) * (d / ds) ** 3
    rows = min(args.cpu_rows, d_out)
    W64 = gi.to_float64(W[:rows, :ds], layer.dtype)
    t0 = time.perf_counter()
    r = o.gptq(W64, Hsub, bits=q.bits, group_size=q.group_size, block_size=q.block_size,
               damp_percent=q.damp_percent, desc_act=bool(q.desc_act), prepared=prep)
    t_loop = (time.perf_counter() - t0) * (d_out / rows) * (d / ds) ** 2
    t0 = time.perf_counter()
    o.pack_int4(r.codes)
    t_p = (time.perf_counter() - t0) * (d_out * d) / (rows * ds)
    total = t_h + t_f + t_loop + t_p
    return {
        "value": d_out * d / total, "unit": "weights/s", "cores": cores, "kind": "oracle",
        "sample": (f"float64 numpy oracle on {cores} threads: Hessian over {nt} of {N} tokens at the "
                   f"full d_in {d} (x{N / nt:g}); prepare (order, damp, inverse, Cholesky) of the "
                   f"leading {ds}^2 block (x{(d / ds) ** 3:.1f}); column loop over {rows} of {d_out} "
                   f"rows on the leading {ds} columns (x{d_out / rows:g} x{(d / ds) ** 2:.1f}); "
                   f"est. total {total / 60:.1f} min per layer"),
        "stages_s": {"hessian": round(t_h, 2), "factor": round(t_f, 2), "loop": round(t_loop, 2),
                     "pack": round(t_p, 3)},
    }


# ---------------------------------------------------------------- widened rows

def w4a16_measure(P, torch, packed, scales, zeros, group_size, g_idx=None, reps=24):
    """Decode-shaped product on packed layers (one activation row, bf16 in, fp32
    out): the quantized layer of this step (held in three copies used in turn
    when it is small, so each call streams its weights from HBM rather than the
    256 MB last-level cache), read with contiguous groups and, when the layer
    has one, with its act-order g_idx (a group per column); and a prefill shape
    (2048 activation rows, the MFMA path) against the bf16 MFMA peak.  HIP
    events on the launch stream, mean over reps after a warm-up."""
    out = []
    dev = packed.device
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    stream = torch.cuda.current_stream()
    d_out, d_in = packed.shape[0], packed.shape[1] * 8
    nbytes_layer = packed.numel() * 4 + scales.numel() * 8
    copies = [(packed, scales, zeros)]
    while len(copies) * nbytes_layer < 384 * (1 << 20):
        copies.append((packed.clone(), scales.clone(), zeros.clone()))
    X = torch.randn((1, d_in), device=dev, generator=g).to(torch.bfloat16)
    Y = torch.empty((1, d_out), dtype=torch.float32, device=dev)
    for c in copies:
        P.gptq_w4a16_gemm(X, c[0], c[1], c[2], Y, group_size=group_size)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for gi_ in ([None] if g_idx is None else [None, g_idx]):
        if gi_ is not None:
            for c in copies:
                P.gptq_w4a16_gemm(X, c[0], c[1], c[2], Y, g_idx=gi_, group_size=group_size)
        e0.record(stream)
        for i in range(reps):
            c = copies[i % len(copies)]
            P.gptq_w4a16_gemm(X, c[0], c[1], c[2], Y, g_idx=gi_, group_size=group_size)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        # algorithmic bytes: codes, scales and zeros, X, Y (and g_idx with it)
        nbytes = nbytes_layer + X.numel() * 2 + Y.numel() * 4 + (0 if gi_ is None else gi_.numel() * 4)
        out.append({"shape": f"{d_out}x{d_in}", "m": 1, "groups": "contiguous" if gi_ is None else "g_idx",
                    "us": round(us, 2), "bytes": nbytes, "GB_per_s": round(nbytes / us / 1e3, 1),
                    "frac_hbm": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4)})
    mp = 2048
    Xp = torch.randn((mp, d_in), device=dev, generator=g).to(torch.bfloat16)
    Yp = torch.empty((mp, d_out), dtype=torch.float32, device=dev)
    P.gptq_w4a16_gemm(Xp, packed, scales, zeros, Yp, group_size=group_size)
    e0.record(stream)
    for i in range(6):
        c = copies[i % len(copies)]
        P.gptq_w4a16_gemm(Xp, c[0], c[1], c[2], Yp, group_size=group_size)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / 6
    tf = 2.0 * mp * d_out * d_in / us / 1e6
    out.append({"shape": f"{d_out}x{d_in}", "m": mp, "us": round(us, 1), "TFLOP_per_s": round(tf, 1),
                "frac_bf16_mfma": round(tf / PEAK_BF16_TFLOPS, 4)})
    del copies
    return out


def awq_measure(P, torch, Wg, Xg, reps=5):
    """The AWQ path on one layer and its calibration tokens (both already in
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
    return {"layer": f"{d_out}x{d}", "n_tokens": N,
            "stages_ms": {k: round(v, 4) for k, v in ms.items()}, "ms_per_layer": round(total, 4),
            "weights_per_s": d_out * d / (total / 1e3), "best_factor": float(grid[int(best.item())]),
            "statistic_GB_per_s": round(gbs, 1), "statistic_frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
            "grid": len(grid)}


def block_measure(P, torch, Xg, n_tokens=32768, seq_len=2048):
    """Layer-sequential GPTQ over one Llama-7B-shaped decoder block (d 4096,
    32 heads of 128, intermediate 11008; random fp16 weights N(0, 0.02)) on
    n_tokens calibration tokens (as fp32), 4-bit groups of 128: q/k/v share
    one Hessian and factor, then o, gate/up, down, each from the quantized
    stages before it.  HIP events per stage, one warm-up run."""
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


# ---------------------------------------------------------------- main

def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the GPTQ path here runs on one GPU: --gpus must be 1 (across "
                                   "GPUs it would shard X by tokens for H and W by output rows)",
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
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log(f"[bench] generating {args.workload}: W {d_out}x{d} {layer.dtype}, X {N}x{d} {calib.dtype}")
    t0 = time.time()
    W, Wg = upload_weight(torch, gi, layer, wl.config, dev)
    Xg = upload_calib(torch, gi, calib, wl.config, dev)
    log(f"[bench] inputs generated and copied in {time.time() - t0:.1f}s")

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
        torch.cuda.synchronize()
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
    stages, roofs = stage_report(mean, N, d_out, d, G)
    t_roof = sum(roofs.values()) * 1e3

    h_flops = hessian_flops(N, d)
    achieved_tf = h_flops / (mean["hessian"] / 1e3) / 1e12
    traffic = None
    tj_path = args.traffic_json or os.path.join(ROOT, "profiles", f"hessian_{args.workload}_traffic.json")
    if os.path.exists(tj_path):
        try:
            tj = json.load(open(tj_path))
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
        "dtype": ("fp32 (bf16 x bf16 -> fp32 Hessian; fp32 factor and lazy update, their large products as "
                  "two scaled fp16 pieces per operand on fp16 MFMA with fp32 accumulation; fp64 column loop)"),
        "data": "synthetic",
        "config": {"workload": args.workload, "d_out": d_out, "d_in": d, "n_tokens": N,
                   "x_dtype": calib.dtype, "w_dtype": layer.dtype, "bits": q.bits,
                   "group_size": q.group_size, "block_size": q.block_size,
                   "damp_percent": q.damp_percent, "desc_act": q.desc_act,
                   "parallelism": "single GPU"},
        "stages_ms": {k: round(v, 4) for k, v in mean.items()},
        "hessian_tflops": achieved_tf,
        "weights_per_s_excl_hessian": weights / ((ms_step - mean["hessian"] - mean["zero_h"]) / 1e3),
        "step_roofline": {"roof_ms": round(t_roof, 3), "frac": round(t_roof / ms_step, 4),
                          "roof_excl_hessian_ms": round(t_roof - roofs["hessian"] * 1e3, 3),
                          "frac_excl_hessian": round((t_roof - roofs["hessian"] * 1e3)
                                                     / (ms_step - mean["hessian"] - mean["zero_h"]), 4)},
        "stages": stages,
        "timing_note": ("stages_ms: HIP events around each stage of the timed steps on one stream, each stage "
                        "right after the one before, so prepare_hinv and quantize run at the clock the chip keeps "
                        "after the Hessian's full MFMA load (alone they run up to 15-20 % faster); per_config: "
                        "median of 3 after a warm-up, each prepare_hinv right after its Hessian calls"),
        "roofline": {"bound": "mfma", "achieved": achieved_tf, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved_tf / PEAK_BF16_TFLOPS,
                     "traffic": traffic,
                     "kernel": ("gptq_hessian_accumulate: syrk16_kernel<bf16> (tiles added into H directly "
                                "at one token split, else + syrk_reduce_kernel<4, 512>)"
                                + (" + sumsq_kernel pass (fp64 diagonal keys)" if q.desc_act else "")),
                     "work_per_launch": f"N*d*(d+1) = {h_flops:.4g} flop"},
    }
    if not args.no_extras:
        t_hs = hessian_streamed_ms(torch, P, gi, H, hdiag, Xg, stream)
        out["hessian_streamed"] = {"calls": (N + gi.CHUNK_TOKENS - 1) // gi.CHUNK_TOKENS,
                                   "tokens_per_call": gi.CHUNK_TOKENS, "ms": round(t_hs, 4),
                                   "TFLOP_per_s": round(h_flops / (t_hs / 1e3) / 1e12, 1)}
        log("[bench] streamed Hessian done")
        out["w4a16_decode"] = w4a16_measure(P, torch, packed, scales, zeros, q.group_size,
                                            g_idx=g_idx if q.desc_act else None)
        log("[bench] w4a16 done")
    del Xg, H, U, ws_h, ws_f, ws_q, codes, packed
    torch.cuda.empty_cache()
    if not args.no_extras:
        out["per_config"] = []
        for key in EXTRA_CONFIGS:
            res, kept = measure_config(torch, P, gi, key, dev, keep_x=(key == "c2_llama7b_q_proj"))
            out["per_config"].append(res)
            if kept is not None:
                wl2 = gi.workload(key)
                _, W2 = upload_weight(torch, gi, wl2.layers[0], wl2.config, dev)
                out["awq"] = awq_measure(P, torch, W2, kept)
                out["block_sequential"] = block_measure(P, torch, kept)
                del W2, kept
                torch.cuda.empty_cache()
                log("[bench] awq and block done")
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(W, wl, args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
