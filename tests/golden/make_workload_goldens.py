"""Write the float64 oracle's results for the workloads at their full sizes.

For each workload of gptq_inputs (Llama-7B q_proj, the Llama-7B MLP, the 13B
desc_act layers, the 70B down_proj) this runs the oracle over ALL calibration
tokens (128 sequences x 2048 tokens, the GPTQ practice page at
m.lqnn.cn/news/117696, section 3.2) and stores, in
tests/golden/workloads/<key>.npz:

* per distinct d_in: the Hessian's diagonal and a 64 x 64 block of sampled
  channels (H = 2 X^T X in float64);
* per (d_in, damp, desc_act): the processing order, lambda, the factor's
  diagonal and a 64 x 64 block of sampled processing positions;
* per layer and quantizer setting, on sampled rows (rows are independent given
  H): the codes (two 4-bit codes per byte), scales, zero points, the positions
  whose value w/scale lay within 1e-2 of a rounding tie (with that distance),
  and per row the layer objective of GPTQ and of round-to-nearest.

It calls only the oracle and the seeded input generator, so no stored value
comes from the GPU path.  The float64 Hessian of the 70B down_proj is
2.2e14 flop; on 8 host cores the whole script takes about an hour and up to
~40 GB of memory.

Usage:  python tests/golden/make_workload_goldens.py [workload keys ...]
"""
from __future__ import annotations

import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import gptq_inputs as gi                      # noqa: E402
from oracle import gptq_ref as o              # noqa: E402

OUT = os.path.join(HERE, "workloads")
KEYS = ("c5_70b_down_proj", "c2_llama7b_q_proj", "c3_llama7b_mlp", "c4_13b_desc_act")
TIE_KEEP = 1e-2          # near-tie positions kept (the parity bar's window is 1e-3)
N_SAMPLE = 64            # sampled channels / processing positions for H and U


def rows_for(d_in: int) -> int:
    return 128 if d_in <= 8192 else 64


def sample(n: int, k: int, seed: int, must=()) -> np.ndarray:
    rng = np.random.default_rng(seed)
    s = set(int(v) for v in must)
    s.update(int(v) for v in rng.choice(n, size=min(n, k), replace=False))
    return np.array(sorted(s), dtype=np.int64)


def nibbles(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    assert c.max() <= 15
    if c.shape[1] % 2:
        c = np.concatenate([c, np.zeros((c.shape[0], 1), np.uint8)], axis=1)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def sha(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8)).hexdigest()


def log(*a):
    print(time.strftime("%H:%M:%S"), *a, flush=True)


def one_workload(key: str) -> None:
    wl = gi.workload(key)
    out = {"numpy_version": np.array(np.__version__), "n_tokens": np.int64(wl.calib[0].n_tokens)}
    for cal in wl.calib:
        d = cal.d_in
        pre = f"d{d}_"
        t0 = time.perf_counter()
        x0 = gi.x_chunk(cal, wl.config, 0)
        out[pre + "x0_sha256"] = np.array(sha(x0))
        del x0

        def widened():
            for c in range(gi.n_chunks(cal)):
                yield gi.to_float64(gi.x_chunk(cal, wl.config, c), cal.dtype)
                log(f"  {key} d={d}: chunk {c + 1}/{gi.n_chunks(cal)}")

        H = o.hessian(widened(), d)
        log(f"{key} d={d}: Hessian over {cal.n_tokens} tokens in {time.perf_counter() - t0:.0f} s")
        out[pre + "hdiag"] = np.diag(H).copy()
        hidx = sample(d, N_SAMPLE, 7000 + d, must=gi.outlier_channels(cal, wl.config)[:4])
        out[pre + "h_idx"] = hidx
        out[pre + "h_sub"] = H[np.ix_(hidx, hidx)]

        for damp, desc in sorted({(q.damp_percent, q.desc_act) for q in wl.quant}):
            t1 = time.perf_counter()
            prep = o.prepare(H, damp, bool(desc))
            log(f"{key} d={d}: factor in {time.perf_counter() - t1:.0f} s")
            p2 = f"{pre}desc{desc}_"
            out[p2 + "damp"] = np.float64(damp)
            out[p2 + "perm"] = prep.perm.astype(np.int32)
            out[p2 + "lam"] = np.float64(prep.lam)
            out[p2 + "u_diag"] = np.diag(prep.U).copy()
            uidx = sample(d, N_SAMPLE, 8000 + d, must=(0, d - 1))
            out[p2 + "u_idx"] = uidx
            out[p2 + "u_sub"] = prep.U[np.ix_(uidx, uidx)]
            for layer in wl.layers:
                if layer.d_in != d:
                    continue
                W = gi.weight(layer, wl.config)
                W64 = gi.to_float64(W, layer.dtype)
                rows = sample(layer.d_out, rows_for(d) - 2, 9000 + layer.seed_offset,
                              must=(0, layer.d_out - 1))
                out[f"{layer.name}_w_sha256"] = np.array(sha(W))
                for q in wl.quant:
                    if (q.damp_percent, q.desc_act) != (damp, desc):
                        continue
                    t2 = time.perf_counter()
                    ref = o.gptq(W64[rows], H, bits=q.bits, group_size=q.group_size,
                                 block_size=q.block_size, damp_percent=q.damp_percent,
                                 desc_act=bool(q.desc_act), prepared=prep, sym=bool(q.sym))
                    G = d if q.group_size == -1 else q.group_size
                    _, Qr = o.rtn(W64[rows], bits=q.bits, group_size=q.group_size,
                                  perm=prep.perm, sym=bool(q.sym))
                    k3 = f"{layer.name}_b{q.bits}_g{q.group_size}_"
                    out[k3 + "rows"] = rows
                    out[k3 + "codes_nib"] = nibbles(ref.codes)
                    out[k3 + "scales"] = ref.scales
                    out[k3 + "zeros"] = ref.zeros.astype(np.int16)
                    t = ref.t_at_code
                    dist = np.abs((t - np.floor(t)) - 0.5)
                    tr, tp = np.nonzero(dist <= TIE_KEEP)
                    assert len(rows) < 32768 and d < 32768
                    out[k3 + "tie_row"] = tr.astype(np.int16)
                    out[k3 + "tie_pos"] = tp.astype(np.int16)       # processing order
                    out[k3 + "tie_dist"] = dist[tr, tp].astype(np.float32)
                    out[k3 + "obj_rows"] = o.objective_rows(W64[rows], ref.Q, H)
                    out[k3 + "rtn_obj_rows"] = o.objective_rows(W64[rows], Qr, H)
                    out[k3 + "err_sq"] = ref.err_sq
                    log(f"{key} {layer.name} {q.bits}-bit G{G}: {len(rows)} rows in "
                        f"{time.perf_counter() - t2:.0f} s, objective {out[k3 + 'obj_rows'].sum():.6g} "
                        f"(RTN {out[k3 + 'rtn_obj_rows'].sum():.6g})")
                del W, W64
            del prep
        del H
    os.makedirs(OUT, exist_ok=True)
    path = os.path.join(OUT, key + ".npz")
    np.savez_compressed(path + ".tmp.npz", **out)
    os.replace(path + ".tmp.npz", path)
    log(f"wrote {path} ({os.path.getsize(path) / 1e6:.2f} MB)")


def main(argv) -> int:
    keys = argv[1:] or list(KEYS)
    for k in keys:
        one_workload(k)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
