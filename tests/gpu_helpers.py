"""Helpers for the GPU parity tests: move seeded numpy inputs to the device,
run the C-ABI path, and compare with the oracle under the stated bar."""
from __future__ import annotations

import sys
from dataclasses import dataclass

import numpy as np

import gptq_inputs as gi
from oracle import gptq_ref as o


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    elif dtype == "f16":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16))
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to("cuda")


def gpu_hessian(x_chunks, x_dtype, d, with_diag=False, keys=True):
    """keys=False: no fp64 diagonal is requested (the kernels skip that work)."""
    import torch
    import post_weight_quantization_29_amd as P
    H = torch.zeros((d, d), dtype=torch.float32, device="cuda")
    hd = torch.zeros((d,), dtype=torch.float64, device="cuda") if keys else None
    for xc in x_chunks:
        P.gptq_hessian_accumulate(H, to_dev(xc, x_dtype), hd)
    torch.cuda.synchronize()
    return (H, hd) if with_diag else H


@dataclass
class Parity:
    agree: float
    n_disagree: int
    first_not_tie: int
    max_first_tie: float   # largest |w/scale - k - 1/2| at a row's first disagreement
    scale_rel: float
    zero_mismatch: int
    q_bad: int
    obj_gpu: float
    obj_oracle: float
    obj_rel: float


def compare_quant(ref: o.GPTQResult, W64, H64, codes, scales, zeros, Q, G, tie_tol=1e-3,
                  rows=None) -> Parity:
    """Codes: >= 99.9 % equal, each row's first disagreement a near-tie.
    Scales/zeros/Q compared on each row's groups before its first disagreement."""
    rows = np.arange(codes.shape[0]) if rows is None else rows
    rc = ref.codes[rows]
    codes = codes.astype(np.int64)
    dis = codes != rc
    agree = 1.0 - dis.mean()
    perm = ref.perm
    first_not_tie = 0
    max_first_tie = 0.0
    d = codes.shape[1]
    scale_rel = 0.0
    zero_mismatch = 0
    q_bad = 0
    for k, r in enumerate(rows):
        dp = dis[k][perm]                      # processing order
        idx = np.nonzero(dp)[0]
        first = idx[0] if idx.size else d
        if idx.size:
            t = ref.t_at_code[r, first]
            dist = abs((t - np.floor(t)) - 0.5)
            max_first_tie = max(max_first_tie, dist)
            if dist > tie_tol:
                first_not_tie += 1
        ng_ok = first // G                     # groups fully before the first disagreement
        if ng_ok > 0:
            sr = np.abs(scales[k, :ng_ok] - ref.scales[r, :ng_ok]) / np.abs(ref.scales[r, :ng_ok])
            scale_rel = max(scale_rel, float(sr.max()))
            zero_mismatch += int((zeros[k, :ng_ok] != ref.zeros[r, :ng_ok]).sum())
        if Q is not None and first > 0:
            cols = perm[:first]
            qo = ref.Q[r, cols]
            qg = Q[k, cols].astype(np.float64)
            tol = 1e-3 * np.abs(qo) + 1e-6 * np.abs(W64[r]).max()
            q_bad += int((np.abs(qg - qo) > tol).sum())
    obj_o = o.objective(W64[rows], ref.Q[rows], H64)
    obj_g = o.objective(W64[rows], Q.astype(np.float64), H64) if Q is not None else float("nan")
    return Parity(agree, int(dis.sum()), first_not_tie, max_first_tie, scale_rel, zero_mismatch,
                  q_bad, obj_g, obj_o, abs(obj_g - obj_o) / obj_o)


@dataclass
class GoldParity:
    agree: float
    n_disagree: int
    rows_with_flip: int
    first_not_tie: int
    scale_rel: float
    zero_mismatch: int
    q_bad: int

    def __str__(self):
        return (f"agree {self.agree:.6f} ({self.n_disagree} codes, {self.rows_with_flip} rows), "
                f"first not at a tie {self.first_not_tie}, scale rel {self.scale_rel:.1e}, "
                f"zero mismatches {self.zero_mismatch}, Q off {self.q_bad}")


def golden_codes(z, k3, d):
    nib = z[k3 + "codes_nib"]
    c = np.empty((nib.shape[0], 2 * nib.shape[1]), dtype=np.int64)
    c[:, 0::2] = nib & 0xF
    c[:, 1::2] = nib >> 4
    return c[:, :d]


def compare_golden(z, k3, d, perm, codes, scales, zeros, Q, G, tie_tol=1e-3) -> GoldParity:
    """The same bar as compare_quant against the oracle's stored results for
    sampled rows (golden file written by tests/golden/make_workload_goldens.py):
    codes >= 99.9 % equal with each row's first disagreement (processing
    order) at a position the oracle decided within tie_tol of a rounding tie;
    scales (relative), zero points (exact) and Q = scale * (code - zero)
    (relative, with the oracle's float64 scale) on each row's groups / columns
    before its first disagreement."""
    rc = golden_codes(z, k3, d)
    sc_o = z[k3 + "scales"]
    ze_o = z[k3 + "zeros"].astype(np.int64)
    ties = {}
    for r, p, dist in zip(z[k3 + "tie_row"], z[k3 + "tie_pos"], z[k3 + "tie_dist"]):
        ties[(int(r), int(p))] = float(dist)
    codes = codes.astype(np.int64)
    dis = codes != rc
    first_not_tie = rows_with_flip = zero_mismatch = q_bad = 0
    scale_rel = 0.0
    for k in range(codes.shape[0]):
        dp = dis[k][perm]
        idx = np.nonzero(dp)[0]
        first = int(idx[0]) if idx.size else d
        if idx.size:
            rows_with_flip += 1
            if ties.get((k, first), 1.0) > tie_tol:
                first_not_tie += 1
        ng_ok = first // G
        if ng_ok > 0:
            sr = np.abs(scales[k, :ng_ok] - sc_o[k, :ng_ok]) / np.abs(sc_o[k, :ng_ok])
            scale_rel = max(scale_rel, float(sr.max()))
            zero_mismatch += int((zeros[k, :ng_ok] != ze_o[k, :ng_ok]).sum())
        if first > 0:
            cols = perm[:first]
            g = np.arange(first) // G
            qo = sc_o[k, g] * (rc[k, cols] - ze_o[k, g]).astype(np.float64)
            qg = Q[k, cols].astype(np.float64)
            tol = 1e-3 * np.abs(qo) + 1e-6 * np.abs(sc_o[k]).max()
            q_bad += int((np.abs(qg - qo) > tol).sum())
    return GoldParity(1.0 - dis.mean(), int(dis.sum()), rows_with_flip, first_not_tie, scale_rel,
                      zero_mismatch, q_bad)
