"""Pins for the CPU oracle: each checks it against something other than itself
(closed forms, the pages' worked example, brute force, identities of the method).

No GPU is needed; sizes are small.
"""
import json
import os

import numpy as np
import pytest

import gptq_inputs as gi
from oracle import gptq_ref as o

HERE = os.path.dirname(os.path.abspath(__file__))


def _case(d_out=16, d_in=64, n=1024, seed=1, **kw):
    c = gi.random_case(d_out, d_in, n, seed, **kw)
    return gi.to_float64(c.W, c.w_dtype), gi.to_float64(c.X, c.x_dtype)


# ---------------------------------------------------------------- P1 Hessian

def test_hessian_closed_form_orthogonal_columns():
    rng = np.random.default_rng(0)
    q, _ = np.linalg.qr(rng.standard_normal((200, 7)))
    s = np.array([1.0, 2.0, 0.5, 3.0, 1.5, 0.25, 4.0])
    X = q * s                                       # orthogonal columns with norms s
    H = o.hessian([X[:50], X[50:]], 7)
    np.testing.assert_allclose(H, 2.0 * np.diag(s ** 2), atol=1e-13)


def test_hessian_closed_form_constant():
    X = np.full((37, 5), 3.0)
    H = o.hessian([X], 5)
    np.testing.assert_allclose(H, np.full((5, 5), 2.0 * 37 * 9.0), rtol=0, atol=0)


def test_hessian_elementwise_loops_tiny():
    rng = np.random.default_rng(3)
    X = rng.integers(-4, 5, size=(6, 4)).astype(np.float64)
    H = o.hessian([X[:2], X[2:5], X[5:]], 4)
    for i in range(4):
        for j in range(4):
            acc = 0.0
            for t in range(6):
                acc += X[t, i] * X[t, j]
            assert H[i, j] == 2.0 * acc


def test_hessian_chunking_and_bf16_widening():
    c = gi.random_case(4, 32, 3000, 11, x_dtype="bf16", dist="t")
    X = gi.to_float64(c.X, "bf16")
    H1 = o.hessian([X], 32)
    H2 = o.hessian([X[i:i + 700] for i in range(0, 3000, 700)], 32)
    np.testing.assert_allclose(H1, H2, rtol=1e-12)
    assert np.array_equal(H1, H1.T)
    np.testing.assert_allclose(np.diag(H1), 2.0 * (X ** 2).sum(0), rtol=1e-12)


# ---------------------------------------------------------------- P2 damping, P3 order

def test_damp_closed_form():
    H = np.diag([1.0, 2.0, 3.0, 4.0]) + 0.5
    Hd, lam = o.damp(H, 0.01)
    assert lam == pytest.approx(0.01 * 3.0)
    np.testing.assert_allclose(Hd - H, lam * np.eye(4), atol=1e-15)


def test_act_order_descending_stable():
    H = np.diag([1.0, 3.0, 3.0, 2.0, 5.0])
    assert list(o.act_order(H, True)) == [4, 1, 2, 3, 0]
    assert list(o.act_order(H, False)) == [0, 1, 2, 3, 4]


def test_desc_act_equals_natural_order_on_permuted_inputs():
    W, X = _case(12, 48, 800, seed=5, outlier_frac=0.1, outlier_factor=10.0)
    H = o.hessian([X], 48)
    r = o.gptq(W, H, bits=4, group_size=16, block_size=16, desc_act=True)
    p = r.perm
    r2 = o.gptq(W[:, p], H[np.ix_(p, p)], bits=4, group_size=16, block_size=16, desc_act=False)
    assert np.array_equal(r.codes[:, p], r2.codes)
    np.testing.assert_allclose(r.Q[:, p], r2.Q, rtol=1e-12, atol=1e-15)
    # g_idx: original column -> processing-order group
    assert np.array_equal(r.g_idx[p], np.arange(48) // 16)


# ---------------------------------------------------------------- P4 the factor U

def test_factor_identities():
    W, X = _case(4, 40, 500, seed=2)
    H = o.hessian([X], 40)
    Hd, _ = o.damp(H, 0.01)
    U = o.hinv_factor(Hd)
    assert np.allclose(np.tril(U, -1), 0)
    assert np.all(np.diag(U) > 0)
    np.testing.assert_allclose(U.T @ U @ Hd, np.eye(40), atol=1e-10)
    # U equals the flip of the inverse of the Cholesky factor of the flipped H
    J = np.eye(40)[::-1]
    M = np.linalg.cholesky(J @ Hd @ J)
    np.testing.assert_allclose(U, J @ np.linalg.inv(M) @ J, rtol=1e-9, atol=1e-14)


def test_factor_2x2_closed_form():
    a, b, c = 4.0, 1.0, 3.0
    U = o.hinv_factor(np.array([[a, b], [b, c]]))
    det = a * c - b * b
    u11 = np.sqrt(c / det)
    np.testing.assert_allclose(U, [[u11, -b / det / u11], [0.0, 1.0 / np.sqrt(c)]], rtol=1e-14)


def test_factor_diagonal_closed_form():
    h = np.array([2.0, 8.0, 0.5])
    np.testing.assert_allclose(o.hinv_factor(np.diag(h)), np.diag(1 / np.sqrt(h)), rtol=1e-15)


def test_factor_rows_are_obq_directions():
    """Row q of U is the q-th column of inv(Hd restricted to {q..d-1}),
    divided by the square root of its diagonal entry (the OBQ update direction
    for the weights not yet quantized)."""
    _, X = _case(1, 9, 300, seed=4)
    Hd, _ = o.damp(o.hessian([X], 9), 0.01)
    U = o.hinv_factor(Hd)
    for q in range(9):
        Finv = np.linalg.inv(Hd[q:, q:])
        np.testing.assert_allclose(U[q, q:], Finv[0] / np.sqrt(Finv[0, 0]), rtol=1e-10)


def test_not_pd_without_damping_on_rank_deficient_h():
    _, X = _case(1, 32, 16, seed=6)         # 16 tokens < 32 channels: H singular
    H = o.hessian([X], 32)
    Hd, _ = o.damp(H, 0.0)
    with pytest.raises(o.NotPositiveDefinite):
        o.hinv_factor(Hd - 1e-9 * np.eye(32))
    with pytest.raises(o.NotPositiveDefinite):
        o.hinv_factor(np.full((3, 3), np.nan))


# ---------------------------------------------------------------- P5 the grid

@pytest.mark.parametrize("decision", ["f32", "f64"])
def test_minmax_worked_example_from_page(decision):
    with open(os.path.join(HERE, "golden", "minmax_2bit_heights.json")) as f:
        g = json.load(f)
    maxq = (1 << g["bits"]) - 1
    seg = np.array([[g["group_min"], g["value"], 1.9, g["group_max"]]])
    s, z = o.group_params(seg, maxq, decision)
    levels = s[0] * (np.arange(maxq + 1) - z[0])
    np.testing.assert_allclose(np.round(levels, 2), g["levels_printed_2dp"], atol=1e-12)
    c, q = o.quantize(np.array([g["value"]]), s, z, maxq, decision)
    assert q[0] == pytest.approx(g["expected_level"], abs=1e-6)
    assert abs(g["value"] - q[0]) == pytest.approx(g["expected_abs_error"], abs=1e-6)
    assert 0 <= c[0] <= maxq


def test_degenerate_groups():
    for a, expect_scale, expect_zero in [(0.3, 0.3 / 15, 0), (-0.3, 0.3 / 15, 15), (0.0, 1.0, 0)]:
        seg = np.full((1, 8), a)
        s, z = o.group_params(seg, 15, "f64")
        assert s[0] == pytest.approx(expect_scale) and z[0] == expect_zero
        c, q = o.quantize(seg[0], s, z, 15, "f64")
        np.testing.assert_allclose(q, a, atol=1e-15)


def test_codes_in_range_and_q_on_grid():
    W, X = _case(32, 96, 600, seed=9, outlier_frac=0.05, outlier_factor=20.0)
    H = o.hessian([X], 96)
    for bits in (3, 4):
        r = o.gptq(W, H, bits=bits, group_size=32, block_size=32, desc_act=True)
        assert r.codes.min() >= 0 and r.codes.max() <= (1 << bits) - 1
        s = r.scales[:, r.g_idx]
        z = r.zeros[:, r.g_idx]
        np.testing.assert_allclose(r.Q, s * (r.codes - z), rtol=0, atol=0)


# ---------------------------------------------------------------- P6 brute force LS

def _brute_force_sequential(W, Hd, bits, G, decision="f64", sym=False):
    """Independent route: before deciding column j, the not-yet-quantized weights
    are set to the minimizer of (v - w)^T Hd (v - w) with all earlier columns fixed
    to their quantized values (least squares on A with A^T A = Hd)."""
    d_out, d = W.shape
    A = np.linalg.cholesky(Hd).T                      # A^T A = Hd
    maxq = (1 << bits) - 1
    codes = np.zeros((d_out, d), dtype=np.int64)
    Q = np.zeros((d_out, d))
    for r in range(d_out):
        w = W[r]
        fixed = np.zeros(d, dtype=bool)
        vals = np.zeros(d)
        s = z = None
        for j in range(d):
            free = ~fixed
            # minimize || A[:, free] u + A[:, fixed] (vals_f - w_f) - A[:, free] w_free ... ||
            rhs = -(A[:, fixed] @ (vals[fixed] - w[fixed]))
            u, *_ = np.linalg.lstsq(A[:, free], rhs, rcond=None)
            v = w.copy()
            v[fixed] = vals[fixed]
            v[free] = w[free] + u
            if j % G == 0:
                s, z = o.group_params(v[None, j:min(j + G, d)], maxq, decision, sym)
            c, q = o.quantize(v[j:j + 1], s, z, maxq, decision)
            codes[r, j] = c[0]
            Q[r, j] = q[0]
            fixed[j] = True
            vals[j] = q[0]
    return codes, Q


@pytest.mark.parametrize("G,B", [(4, 4), (4, 8), (8, 4), (12, 12)])
def test_gptq_equals_sequential_least_squares(G, B):
    W, X = _case(5, 12, 200, seed=21, correlated_rank=4, noise=0.3)
    H = o.hessian([X], 12)
    r = o.gptq(W, H, bits=3, group_size=G, block_size=B, damp_percent=0.01, decision="f64")
    Hd, _ = o.damp(H, 0.01)
    codes, Q = _brute_force_sequential(W, Hd, 3, G)
    assert np.array_equal(r.codes, codes)
    np.testing.assert_allclose(r.Q, Q, rtol=1e-9, atol=1e-12)


def test_single_obq_step_least_squares():
    """One OBQ step: fixing w_0 to q_0 and re-fitting the others by least squares
    on X gives exactly -e_0 * U[0, 1:] (no damping, H = 2 X^T X is PD)."""
    _, X = _case(1, 8, 400, seed=23, correlated_rank=3, noise=0.2)
    H = o.hessian([X], 8)
    U = o.hinv_factor(H)
    w = np.linspace(-0.05, 0.04, 8)
    q0 = 0.01
    e0 = (w[0] - q0) / U[0, 0]
    delta = -e0 * U[0, 1:]
    u, *_ = np.linalg.lstsq(X[:, 1:], -X[:, 0] * (q0 - w[0]), rcond=None)
    np.testing.assert_allclose(delta, u, rtol=1e-9, atol=1e-14)


# ---------------------------------------------------------------- P7 .. P14

@pytest.mark.parametrize("G", [16, 32, 64, 128])
def test_lazy_batch_is_exact(G):
    W, X = _case(24, 128, 700, seed=31, correlated_rank=8, noise=0.5)
    H = o.hessian([X], 128)
    r1 = o.gptq(W, H, bits=4, group_size=G, block_size=1)
    r2 = o.gptq(W, H, bits=4, group_size=G, block_size=32)
    assert np.array_equal(r1.codes, r2.codes)
    np.testing.assert_allclose(r1.Q, r2.Q, rtol=1e-12)


@pytest.mark.parametrize("desc_act", [False, True])
def test_diagonal_hessian_reduces_to_rtn(desc_act):
    W, X = _case(16, 64, 500, seed=41)
    h = np.diag(o.hessian([X], 64))
    for H in (np.eye(64), np.diag(h)):
        r = o.gptq(W, H, bits=4, group_size=16, block_size=32, desc_act=desc_act)
        c, Q = o.rtn(W, bits=4, group_size=16, perm=r.perm)
        assert np.array_equal(r.codes, c)
        np.testing.assert_array_equal(r.Q, Q)


def test_error_sum_equals_damped_quadratic_form():
    W, X = _case(16, 64, 500, seed=43, outlier_frac=0.05, outlier_factor=20.0)
    H = o.hessian([X], 64)
    r = o.gptq(W, H, bits=4, group_size=32, block_size=32, desc_act=True)
    Hd, _ = o.damp(H[np.ix_(r.perm, r.perm)], 0.01)
    D = W[:, r.perm] - r.Q_p
    np.testing.assert_allclose(r.err_sq, np.einsum("ij,jk,ik->i", D, Hd, D), rtol=1e-10)


def test_objective_equals_output_error():
    W, X = _case(8, 32, 300, seed=45)
    H = o.hessian([X], 32)
    r = o.gptq(W, H, bits=4, group_size=32, block_size=32)
    direct = float(np.sum(((W - r.Q) @ X.T) ** 2))
    assert o.objective(W, r.Q, H) == pytest.approx(direct, rel=1e-12)


@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("kind", ["iid", "correlated", "outliers"])
def test_gptq_not_worse_than_rtn(bits, kind):
    kw = dict(iid={}, correlated=dict(correlated_rank=16, noise=0.2),
              outliers=dict(outlier_frac=0.01, outlier_factor=20.0, dist="t"))[kind]
    W, X = _case(64, 256, 2048, seed=51 + bits, **kw)
    H = o.hessian([X], 256)
    r = o.gptq(W, H, bits=bits, group_size=128)
    _, Qr = o.rtn(W, bits=bits, group_size=128)
    assert o.objective(W, r.Q, H) <= o.objective(W, Qr, H)


def test_scale_invariance():
    W, X = _case(16, 64, 400, seed=61, correlated_rank=6)
    H = o.hessian([X], 64)
    r = o.gptq(W, H, bits=4, group_size=32, block_size=32)
    r4 = o.gptq(W, 4.0 * H, bits=4, group_size=32, block_size=32)
    assert np.array_equal(r.codes, r4.codes)         # power of two: bitwise identical path
    r3 = o.gptq(W, 3.7 * H, bits=4, group_size=32, block_size=32)
    assert (r3.codes == r.codes).mean() >= 0.999


def test_rows_are_independent():
    W, X = _case(20, 64, 400, seed=63, correlated_rank=6)
    H = o.hessian([X], 64)
    r = o.gptq(W, H, bits=4, group_size=32, block_size=32, desc_act=True)
    rows = [3, 7, 19, 0]
    rs = o.gptq(W[rows], H, bits=4, group_size=32, block_size=32, desc_act=True)
    assert np.array_equal(rs.codes, r.codes[rows])
    np.testing.assert_array_equal(rs.scales, r.scales[rows])


def test_exhaustive_search_bounds_tiny():
    W, X = _case(1, 6, 60, seed=65, correlated_rank=2, noise=0.3)
    H = o.hessian([X], 6)
    r = o.gptq(W, H, bits=2, group_size=6, block_size=6, damp_percent=0.0, decision="f64")
    cr, Qr = o.rtn(W, bits=2, group_size=6, decision="f64")
    s, z = r.scales[0, 0], r.zeros[0, 0]
    best = np.inf
    for idx in range(4 ** 6):
        c = np.array([(idx >> (2 * k)) & 3 for k in range(6)])
        best = min(best, o.objective(W, (s * (c - z))[None, :], H))
    g = o.objective(W, r.Q, H)
    assert best <= g + 1e-15
    assert g <= o.objective(W, Qr, H) + 1e-15


# ---------------------------------------------------------------- packing

def test_pack_layout_and_roundtrip():
    codes = np.arange(8, dtype=np.int64)[None, :]
    assert o.pack_int4(codes)[0, 0] == 0x76543210
    rng = np.random.default_rng(0)
    c = rng.integers(0, 16, size=(5, 64))
    p = o.pack_int4(c)
    assert p.dtype == np.uint32 and p.nbytes * 2 == c.size   # 0.5 byte per weight
    assert np.array_equal(o.unpack_int4(p, 64), c)


# ---------------------------------------------------------------- quantizer variants

def test_sym_grid_closed_form():
    """Symmetric grid: [-m, m], m = max |w|, scale = 2m/maxq, zero = (maxq+1)/2."""
    seg = np.array([[-1.0, 0.5, 0.25, 0.0]])
    s, z = o.group_params(seg, 15, "f64", sym=True)
    assert s[0] == 2.0 / 15 and z[0] == 8
    c, q = o.quantize(seg[0], s, z, 15, "f64")
    # -1/s = -7.5 rounds half to even to -8; 0.5/s = 3.75 -> 4; 0.25/s = 1.875 -> 2
    assert list(c) == [0, 12, 10, 8]
    np.testing.assert_allclose(q, [-16 / 15, 8 / 15, 4 / 15, 0.0], rtol=0, atol=1e-15)
    # the positive end: 0.9/0.12 = 7.5 -> 8, code 16 clamps to 15 -> 7 * 0.12
    s2, z2 = o.group_params(np.array([[0.3, 0.9]]), 15, "f64", sym=True)
    assert s2[0] == pytest.approx(0.12, abs=1e-16) and z2[0] == 8
    c2, q2 = o.quantize(np.array([0.9]), s2, z2, 15, "f64")
    assert c2[0] == 15 and q2[0] == pytest.approx(0.84, abs=1e-15)
    # all-zero group: scale 1, the middle code, value 0 (2-bit: zero = 2)
    s3, z3 = o.group_params(np.zeros((1, 4)), 3, "f64", sym=True)
    assert s3[0] == 1.0 and z3[0] == 2
    assert o.quantize(np.zeros(4), s3, z3, 3, "f64")[1].tolist() == [0.0] * 4


@pytest.mark.parametrize("G,B", [(4, 4), (12, 12)])
def test_sym_gptq_equals_sequential_least_squares(G, B):
    W, X = _case(5, 12, 200, seed=25, correlated_rank=4, noise=0.3)
    H = o.hessian([X], 12)
    r = o.gptq(W, H, bits=3, group_size=G, block_size=B, damp_percent=0.01, decision="f64", sym=True)
    Hd, _ = o.damp(H, 0.01)
    codes, Q = _brute_force_sequential(W, Hd, 3, G, sym=True)
    assert np.array_equal(r.codes, codes)
    np.testing.assert_allclose(r.Q, Q, rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("bits,sym", [(2, False), (8, False), (4, True), (2, True), (8, True)])
def test_variants_diag_h_is_rtn_and_codes_in_range(bits, sym):
    W, X = _case(16, 64, 500, seed=47, outlier_frac=0.05, outlier_factor=20.0)
    h = np.diag(o.hessian([X], 64))
    r = o.gptq(W, np.diag(h), bits=bits, group_size=16, block_size=32, desc_act=True, sym=sym)
    c, Q = o.rtn(W, bits=bits, group_size=16, perm=r.perm, sym=sym)
    assert np.array_equal(r.codes, c)
    assert c.min() >= 0 and c.max() <= (1 << bits) - 1
    H = o.hessian([X], 64)
    g = o.gptq(W, H, bits=bits, group_size=16, block_size=32, sym=sym)
    _, Qr = o.rtn(W, bits=bits, group_size=16, sym=sym)
    if bits >= 3:
        # not a theorem: the compensation is greedy and each group's grid comes
        # from already-compensated weights; on a 4-level grid this input's
        # compensated groups widen enough that GPTQ ends above RTN
        assert o.objective(W, g.Q, H) <= o.objective(W, Qr, H)
    if sym:
        assert np.all(g.zeros == (1 << (bits - 1)))


def test_pack_dense_layouts():
    # 3 bits: code 10 sits at bit 30 and straddles words 0 and 1
    c = np.zeros((1, 32), dtype=np.int64)
    c[0, 10] = 5                                   # 0b101
    p = o.pack_dense(c, 3)
    assert p.shape == (1, 3) and p[0, 0] == (1 << 30) and p[0, 1] == 1 and p[0, 2] == 0
    assert np.all(o.pack_dense(np.full((1, 32), 7), 3) == 0xFFFFFFFF)
    # 2 bits and 8 bits
    c2 = np.zeros((1, 16), dtype=np.int64)
    c2[0, :3] = [3, 1, 2]
    assert o.pack_dense(c2, 2)[0, 0] == 0x27
    assert o.pack_dense(np.array([[1, 2, 3, 250]]), 8)[0, 0] == 0xFA030201
    # 4 bits is pack_int4's layout
    rng = np.random.default_rng(3)
    c4 = rng.integers(0, 16, size=(4, 64))
    assert np.array_equal(o.pack_dense(c4, 4), o.pack_int4(c4))
    for bits, cols in ((2, 48), (3, 96), (8, 20)):
        r = rng.integers(0, 1 << bits, size=(6, cols))
        p = o.pack_dense(r, bits)
        assert p.nbytes * 8 == r.size * bits             # bits/8 byte per weight
        assert np.array_equal(o.unpack_dense(p, cols, bits), r)


# ---------------------------------------------------------------- using the packed layer

def test_w4a16_matmul_equals_dequantized_gptq_output():
    """The packed codes + scales/zeros/g_idx of a GPTQ run dequantize to its Q
    exactly, and the product is X Q^T (element loops on a tiny case)."""
    W, X = _case(12, 64, 300, seed=51, outlier_frac=0.05, outlier_factor=20.0)
    H = o.hessian([X], 64)
    r = o.gptq(W, H, bits=4, group_size=16, block_size=32, desc_act=True)
    packed = o.pack_int4(r.codes)
    Wq = o.dequantize(packed, r.scales, r.zeros, r.g_idx, 64)
    np.testing.assert_array_equal(Wq, r.Q)
    x = X[:3]
    Y = o.w4a16_matmul(x, packed, r.scales, r.zeros, r.g_idx)
    for i in range(3):
        for j in range(12):
            ref = sum(x[i, c] * r.Q[j, c] for c in range(64))
            assert Y[i, j] == pytest.approx(ref, rel=1e-12, abs=1e-15)


def test_dequantize16_rounding():
    """scale * (code - zero) in float32, then ties-to-even to the 16-bit type."""
    packed = o.pack_int4(np.array([[3, 0, 15, 8, 1, 2, 4, 5]]))
    g = np.zeros(8, dtype=np.int64)
    s = np.array([[1.0 + 2.0 ** -8]], dtype=np.float32)      # one bf16 ulp above 1 is 2^-7
    z = np.array([[1]])
    w = o.dequantize16(packed, s, z, g, 8, "bf16")[0]
    # code 3: 2*(1+2^-8) = 2 + 2^-7 is a tie between 2 and 2 + 2^-6 -> even -> 2
    assert w[0] == 2.0
    # code 0: -(1+2^-8): tie between -1 and -(1+2^-7) -> even -> -1
    assert w[1] == -1.0
    # code 15: 14*(1+2^-8) = 14 + 14/256 -> nearest bf16 step (1/16 at 14) -> 14.0625
    assert w[2] == 14.0625
    wf = o.dequantize16(packed, s, z, g, 8, "f16")[0]
    assert wf[0] == np.float64(np.float16(2.0 + 2.0 ** -7))
    np.testing.assert_array_equal(o.dequantize16(packed, np.array([[0.5]], np.float32), z, g, 8, "bf16"),
                                  o.dequantize(packed, np.array([[0.5]]), z, g, 8))
