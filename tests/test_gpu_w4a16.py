"""GPU parity of the product on the packed layer (gptq_w4a16_gemm) against the
float64 oracle.  The packed codes, scales, zeros and g_idx are drawn by the test
(or, end to end, each side quantizes the same layer itself).  The dequantized
weights are defined exactly (fp32 scale*(code - zero), ties-to-even to the
activation type), so only the fp32 accumulation order and the output rounding
separate the two sides."""
from __future__ import annotations

import numpy as np
import pytest

import gptq_inputs as gi
from oracle import gptq_ref as o

from gpu_helpers import gpu_hessian, say, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

_TT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import post_weight_quantization_29_amd as P
    P.lib()
    yield


def _layer(d_out, d_in, G, desc, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 16, size=(d_out, d_in))
    Ge = d_in if G == -1 else G
    ng = (d_in + Ge - 1) // Ge
    scales = rng.uniform(1e-3, 2e-2, size=(d_out, ng)).astype(np.float32)
    zeros = rng.integers(0, 16, size=(d_out, ng)).astype(np.int32)
    perm = rng.permutation(d_in) if desc else np.arange(d_in)
    g_idx = np.empty(d_in, dtype=np.int32)
    g_idx[perm] = np.arange(d_in) // Ge
    return o.pack_int4(codes), scales, zeros, g_idx


def _check(Y, Yref, bound, y_dtype):
    # the output's own rounding (at most half a step, a step being up to 2^-7 of
    # the value in bf16 and 2^-10 in f16) plus the fp32 accumulation order
    ulp = {"f32": 0.0, "f16": 2.0 ** -10, "bf16": 2.0 ** -7}[y_dtype]
    err = np.abs(Y - Yref)
    tol = 1e-5 * bound + ulp * np.abs(Yref) + 1e-30
    say(f"  max |dY| / tol = {np.max(err / tol):.3f}")
    assert np.all(err <= tol)


CASES = [
    # m, d_out, d_in, G, desc(g_idx path), x_dtype, y_dtype
    (1, 256, 256, 128, 0, "bf16", "f32"),
    (3, 300, 1024, 64, 1, "f16", "f32"),
    (8, 4096, 4096, 128, 0, "bf16", "bf16"),
    (13, 100, 512, -1, 0, "bf16", "f16"),
    (5, 70, 4104, 8, 1, "f16", "f16"),
    (2, 33, 96, 32, 0, "f16", "bf16"),
    # long rows, one or two activation rows: the activations shared through LDS
    # (d_out not a multiple of 4: the last workgroup's extra rows are not stored)
    (1, 130, 9216, 128, 0, "bf16", "f32"),
    (2, 70, 8192, 64, 0, "f16", "bf16"),
    # the same with a group per column (act order, g_idx): the rows' (scale,
    # zero) tables in LDS; more groups than the tables hold: the per-wave form
    (1, 130, 8192, 32, 1, "bf16", "f32"),
    (2, 70, 9216, 64, 1, "f16", "bf16"),
    (1, 40, 12800, 8, 1, "bf16", "f32"),
    # 32 or more activation rows: the tiled MFMA product
    (200, 300, 1024, 64, 1, "f16", "f32"),
    (128, 4096, 4096, 128, 0, "bf16", "bf16"),
    (100, 70, 4104, 8, 1, "bf16", "f16"),
    (333, 129, 640, -1, 0, "f16", "f16"),
    (2048, 4096, 4096, 128, 0, "bf16", "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"m{c[0]}_{c[1]}x{c[2]}_g{c[3]}_idx{c[4]}_{c[5]}_{c[6]}" for c in CASES])
def test_w4a16_parity(case):
    import post_weight_quantization_29_amd as P
    m, d_out, d_in, G, desc, xd, yd = case
    say(f"[w4a16] {case}")
    packed, scales, zeros, g_idx = _layer(d_out, d_in, G, desc, seed=m * 1000 + d_in)
    rng = np.random.default_rng(d_out)
    X = gi.cast_storage(rng.standard_normal((m, d_in)).astype(np.float32), xd)
    X64 = gi.to_float64(X, xd)
    Yref = o.w4a16_matmul(X64, packed, scales, zeros, g_idx, dtype=xd)
    bound = np.abs(X64) @ np.abs(o.dequantize16(packed, scales, zeros, g_idx, d_in, xd)).T
    Y = torch.empty((m, d_out), dtype=_TT[yd], device="cuda")
    P.gptq_w4a16_gemm(to_dev(X, xd), torch.from_numpy(packed.view(np.int32)).cuda(),
                      torch.from_numpy(scales).cuda(), torch.from_numpy(zeros).cuda(), Y,
                      g_idx=torch.from_numpy(g_idx).cuda() if desc else None, group_size=G)
    torch.cuda.synchronize()
    _check(Y.float().cpu().numpy().astype(np.float64), Yref, bound, yd)


def test_w4a16_70b_down_proj_shape_sampled_rows():
    """8192 x 28672 with a desc_act g_idx, one activation row (decode)."""
    import post_weight_quantization_29_amd as P
    d_out, d_in, G = 8192, 28672, 128
    packed, scales, zeros, g_idx = _layer(d_out, d_in, G, 1, seed=77)
    rng = np.random.default_rng(78)
    X = gi.cast_storage(rng.standard_normal((1, d_in)).astype(np.float32), "bf16")
    Y = torch.empty((1, d_out), dtype=torch.float32, device="cuda")
    P.gptq_w4a16_gemm(to_dev(X, "bf16"), torch.from_numpy(packed.view(np.int32)).cuda(),
                      torch.from_numpy(scales).cuda(), torch.from_numpy(zeros).cuda(), Y,
                      g_idx=torch.from_numpy(g_idx).cuda())
    torch.cuda.synchronize()
    rows = np.sort(rng.choice(d_out, 96, replace=False))
    X64 = gi.to_float64(X, "bf16")
    Yref = o.w4a16_matmul(X64, packed[rows], scales[rows], zeros[rows], g_idx, dtype="bf16")
    bound = np.abs(X64) @ np.abs(o.dequantize16(packed[rows], scales[rows], zeros[rows], g_idx, d_in,
                                               "bf16")).T
    _check(Y.cpu().numpy()[:, rows].astype(np.float64), Yref, bound, "f32")


def test_w4a16_70b_gate_proj_shape_batch16_sampled_rows():
    """28672 x 8192 with contiguous groups and 16 activation rows (four output
    rows per wave, each activation load shared by them)."""
    import post_weight_quantization_29_amd as P
    d_out, d_in, G, m = 28672, 8192, 128, 16
    packed, scales, zeros, g_idx = _layer(d_out, d_in, G, 0, seed=79)
    rng = np.random.default_rng(80)
    X = gi.cast_storage(rng.standard_normal((m, d_in)).astype(np.float32), "bf16")
    Y = torch.empty((m, d_out), dtype=torch.bfloat16, device="cuda")
    P.gptq_w4a16_gemm(to_dev(X, "bf16"), torch.from_numpy(packed.view(np.int32)).cuda(),
                      torch.from_numpy(scales).cuda(), torch.from_numpy(zeros).cuda(), Y,
                      group_size=G)
    torch.cuda.synchronize()
    rows = np.sort(rng.choice(d_out, 96, replace=False))
    X64 = gi.to_float64(X, "bf16")
    Yref = o.w4a16_matmul(X64, packed[rows], scales[rows], zeros[rows], g_idx, dtype="bf16")
    bound = np.abs(X64) @ np.abs(o.dequantize16(packed[rows], scales[rows], zeros[rows], g_idx, d_in,
                                               "bf16")).T
    _check(Y.float().cpu().numpy()[:, rows].astype(np.float64), Yref, bound, "bf16")


@pytest.mark.parametrize("m, xd", [(1, "bf16"), (2, "f16"), (64, "bf16")])
def test_w4a16_zero_points_at_and_beyond_1024(m, xd):
    """Natural groups whose zero points lie far outside the 4-bit grid (an
    all-positive or all-negative group's zero point is not clamped), mixed
    with ordinary ones: one or two activation rows over long rows (the
    activations shared through LDS) and the tiled MFMA product.  The weights
    scale * (code - zero) then reach ~1500 scale steps, and Y meets the same
    bar as on ordinary grids."""
    import post_weight_quantization_29_amd as P
    d_out, d_in, G = 70, 9216, 128
    packed, scales, zeros, g_idx = _layer(d_out, d_in, G, 0, seed=4242 + m)
    rng = np.random.default_rng(4243 + m)
    special = np.array([-1500, -1025, -1024, -1023, -7, 0, 15, 1023, 1024, 1025, 1500], dtype=np.int32)
    zeros = rng.choice(special, size=zeros.shape).astype(np.int32)
    X = gi.cast_storage(rng.standard_normal((m, d_in)).astype(np.float32), xd)
    X64 = gi.to_float64(X, xd)
    Yref = o.w4a16_matmul(X64, packed, scales, zeros, g_idx, dtype=xd)
    bound = np.abs(X64) @ np.abs(o.dequantize16(packed, scales, zeros, g_idx, d_in, xd)).T
    Y = torch.empty((m, d_out), dtype=torch.float32, device="cuda")
    P.gptq_w4a16_gemm(to_dev(X, xd), torch.from_numpy(packed.view(np.int32)).cuda(),
                      torch.from_numpy(scales).cuda(), torch.from_numpy(zeros).cuda(), Y, group_size=G)
    torch.cuda.synchronize()
    _check(Y.cpu().numpy().astype(np.float64), Yref, bound, "f32")


def test_w4a16_end_to_end_small_layer():
    """Quantize, pack and multiply on each side (the 256 x 256 workload)."""
    import post_weight_quantization_29_amd as P
    wl = gi.workload("c1_tiny_256")
    W = gi.weight(wl.layers[0], wl.config)
    X = gi.x_full(wl.calib[0], wl.config)
    q = wl.quant[0]
    H64 = o.hessian([X.astype(np.float64)], 256)
    ref = o.gptq(W.astype(np.float64), H64, bits=4, group_size=q.group_size)
    Hg, hd = gpu_hessian([X], "f32", 256, with_diag=True)
    cfg = P.make_config(bits=4, group_size=q.group_size)
    res = P.quantize_layer_outputs(torch.from_numpy(W).cuda(), Hg, cfg, hdiag=hd)
    assert np.array_equal(res.codes.cpu().numpy(), ref.codes)
    xa = gi.cast_storage(np.random.default_rng(5).standard_normal((4, 256)).astype(np.float32), "bf16")
    Y = torch.empty((4, 256), dtype=torch.float32, device="cuda")
    P.gptq_w4a16_gemm(to_dev(xa, "bf16"), res.packed, res.scales, res.zeros, Y, group_size=q.group_size)
    torch.cuda.synchronize()
    X64 = gi.to_float64(xa, "bf16")
    pk = o.pack_int4(ref.codes)
    Yref = o.w4a16_matmul(X64, pk, ref.scales.astype(np.float32), ref.zeros, ref.g_idx, dtype="bf16")
    bound = np.abs(X64) @ np.abs(o.dequantize16(pk, ref.scales.astype(np.float32), ref.zeros,
                                               ref.g_idx, 256, "bf16")).T
    # the two sides' scales agree to ~1e-7 relative, so allow that on top
    _check(Y.cpu().numpy().astype(np.float64), Yref, bound * 30.0, "f32")
