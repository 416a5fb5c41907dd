"""CPU oracle: GPTQ post-training quantization of one linear layer, float64 numpy.

TEST INFRASTRUCTURE.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library and never reads anything the HIP library produced.

Sources (five web pages on GPTQ/AWQ; short names used below):
  [P2] "大模型压缩量化技术：GPTQ 与 AWQ 原理详解 + Python 实战教程"
       section 二 (min-max uniform grid and its worked example), section 三
       (quantize one weight, let the remaining ones absorb the error).
  [P4] "AWQ与GPTQ谁更强？ms-swift量化模块深度评测" (zero_point=True means
       an asymmetric grid; damp_percent guards against a singular Hessian).
  [P3] "告别显存焦虑：用AWQ和GPTQ在消费级显卡上跑通7B大模型" section 4.3
       (raise damp_percent when the factorization breaks down).
  [P5] the GPTQ practice page at m.lqnn.cn/news/117696:
       section 2.1 (OBQ: the Hessian comes from the layer's calibration
       activations; quantize one weight, move the others along the H^-1 column),
       section 2.2 (fixed column order by the Hessian diagonal, lazy batch of
       128 columns, Cholesky factor of H^-1), section 3.3 (bits, group_size =
       128 consecutive columns sharing one scale and zero point, desc_act,
       damp_percent).

Readings of open points:
  * H = 2 X^T X over all calibration tokens, no 1/N (codes are invariant to a
    positive scaling of H).
  * damp: lambda = damp_percent * mean(diag H), H_d = H + lambda I.
  * desc_act order: stable sort by descending diag(H); ties keep the lower
    original index first.  The page's "from back to front" is read as garble.
  * The triangular factor: U upper with U^T U = H_d^-1 (the page's
    "lower-triangular" factor is U^T).
  * The printed OBQ update drops the quantized value; the step used is
    delta = -(w_q - quant(w_q)) / [H^-1]_qq * H^-1[:, q].
  * Group scale/zero are taken from the current (already compensated) weights
    at the group's first column, groups contiguous in processing order.
  * Min-max grid, zero point = rint(-min/scale) not clamped; a degenerate group
    (max == min == a) uses the range [min(a,0), max(a,0)]; a == 0 gives
    scale 1, zero 0.
  * Round half to even for both roundings; true division.
  * Every quantity is float64, the integer decisions (each zero point and each
    code) included: rint(-min/scale) and rint(w/scale) of float64 values with
    true float64 division.  ``decision="f32"`` (float32 operands for those two
    roundings only) is kept for a pin showing that the page's worked example
    does not depend on that precision; nothing else uses it.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Iterable, Optional, Tuple

import numpy as np

try:  # dsyrk halves the Hessian's flops; it is a plain library primitive for A A^T
    from scipy.linalg.blas import dsyrk as _dsyrk
except Exception:  # pragma: no cover
    _dsyrk = None


class NotPositiveDefinite(ArithmeticError):
    """The damped Hessian has no Cholesky factor (a pivot <= 0 or NaN).
    The remedy the pages give is a larger damp_percent ([P3] 4.3, [P4])."""


# ----------------------------------------------------------------------------
# 1. Hessian  ([P5] 2.1: built from the layer's calibration activations)
# ----------------------------------------------------------------------------

def hessian(chunks: Iterable[np.ndarray], d_in: int) -> np.ndarray:
    """H = sum over chunks of 2 * Xc^T Xc, with Xc token-major [tokens, d_in]
    already widened to float64."""
    H = np.zeros((d_in, d_in), dtype=np.float64, order="F")
    n = 0
    for xc in chunks:
        xc = np.asarray(xc, dtype=np.float64)
        assert xc.ndim == 2 and xc.shape[1] == d_in
        n += xc.shape[0]
        if _dsyrk is not None:
            # Fortran view of the C-ordered chunk is Xc^T; dsyrk(a) = a a^T.
            H = _dsyrk(2.0, np.asfortranarray(xc.T), beta=1.0, c=H, trans=0,
                       lower=1, overwrite_c=1)
        else:  # pragma: no cover
            H += 2.0 * (xc.T @ xc)
    if _dsyrk is not None:
        # dsyrk filled the lower triangle: copy it to the upper one, a band of
        # columns at a time (no full-size temporaries at large d)
        for c0 in range(0, d_in, 1024):
            c1 = min(d_in, c0 + 1024)
            H[c0:c1, c1:] = H[c1:, c0:c1].T
            blk = H[c0:c1, c0:c1]
            blk[np.triu_indices(c1 - c0, 1)] = blk.T[np.triu_indices(c1 - c0, 1)]
    return np.ascontiguousarray(H)


# ----------------------------------------------------------------------------
# 2. damping and column order  ([P5] 3.3 damp_percent, desc_act; [P5] 2.2 "first")
# ----------------------------------------------------------------------------

def damp(H: np.ndarray, damp_percent: float) -> Tuple[np.ndarray, float]:
    lam = float(damp_percent) * float(np.mean(np.diag(H)))
    Hd = H.copy()
    Hd[np.diag_indices_from(Hd)] += lam
    return Hd, lam


def act_order(H: np.ndarray, desc_act: bool) -> np.ndarray:
    """Processing order -> original column.  Identity unless desc_act, then
    descending diag(H) with ties broken by the lower original index."""
    return order_from_keys(np.diag(H), desc_act)


def order_from_keys(keys: np.ndarray, desc_act: bool) -> np.ndarray:
    """The same order from the diagonal alone (keys = diag(H))."""
    d = keys.shape[0]
    if not desc_act:
        return np.arange(d, dtype=np.int64)
    return np.argsort(-np.asarray(keys, dtype=np.float64), kind="stable").astype(np.int64)


# ----------------------------------------------------------------------------
# 3. factor of the inverse  ([P5] 2.2 "third": Cholesky of H^-1)
# ----------------------------------------------------------------------------

def hinv_factor(Hd: np.ndarray) -> np.ndarray:
    """U upper triangular with positive diagonal and U^T U = Hd^-1, by the
    plain route: invert, then Cholesky (lower L with L L^T = Hd^-1), U = L^T."""
    try:
        np.linalg.cholesky(Hd)                  # positive-definiteness test
    except np.linalg.LinAlgError as exc:
        raise NotPositiveDefinite(str(exc)) from None
    if not np.all(np.isfinite(Hd)):
        raise NotPositiveDefinite("non-finite Hessian")
    Hinv = np.linalg.inv(Hd)
    try:
        L = np.linalg.cholesky(Hinv)
    except np.linalg.LinAlgError as exc:       # pragma: no cover
        raise NotPositiveDefinite(str(exc)) from None
    return np.ascontiguousarray(L.T)


# ----------------------------------------------------------------------------
# 4. the min-max asymmetric grid  ([P2] section 二; [P5] 3.3; [P4] zero_point)
# ----------------------------------------------------------------------------

def _f(x, decision):
    return np.asarray(x, dtype=np.float32 if decision == "f32" else np.float64)


def group_params(seg: np.ndarray, maxq: int, decision: str = "f64", sym: bool = False):
    """Per row of seg [rows, g]: scale = (max - min)/maxq, zero = rint(-min/scale).
    Returns (scale, zero) with scale in the decision precision and zero an
    integer-valued array of the same type.

    sym ([P4]'s GptqConfig sym=True; the pages define no formula, the plainest
    symmetric reading is taken): the grid spans [-m, m] with
    m = max(|min|, |max|), scale = 2m/maxq, and the zero point is the middle
    code (maxq + 1)/2; an all-zero group gets scale 1."""
    xmin = _f(seg.min(axis=-1), decision)
    xmax = _f(seg.max(axis=-1), decision)
    zero_t = _f(0.0, decision)
    if sym:
        m = np.maximum(np.abs(xmin), np.abs(xmax))
        scale = np.where(m == zero_t, _f(1.0, decision), (m + m) / _f(maxq, decision))
        zero = np.full_like(scale, (maxq + 1) // 2)
        return scale.astype(xmin.dtype), zero.astype(xmin.dtype)
    deg = xmax == xmin
    xmin = np.where(deg, np.minimum(xmin, zero_t), xmin)
    xmax = np.where(deg, np.maximum(xmax, zero_t), xmax)
    both0 = xmax == xmin                        # the group is all zeros
    rng = np.where(both0, _f(maxq, decision), xmax - xmin)
    scale = rng / _f(maxq, decision)            # 1 for an all-zero group
    zero = np.rint(-xmin / scale)
    return scale.astype(xmin.dtype), (zero + zero_t).astype(xmin.dtype)


def quantize(w: np.ndarray, scale, zero, maxq: int, decision: str = "f64"):
    """code = clamp(rint(w/scale) + zero, 0, maxq) taken in the decision
    precision; q = scale*(code - zero) returned in float64."""
    t = _f(w, decision) / _f(scale, decision)
    c = np.clip(np.rint(t) + _f(zero, decision), 0, maxq)
    q = np.asarray(scale, dtype=np.float64) * (c.astype(np.float64) - np.asarray(zero, np.float64))
    return c.astype(np.int64), q


# ----------------------------------------------------------------------------
# 5. the column loop  ([P5] 2.1 OBQ step, 2.2 fixed order + lazy batch)
# ----------------------------------------------------------------------------

@dataclass
class GPTQResult:
    codes: np.ndarray      # [d_out, d_in] int64, original column order
    Q: np.ndarray          # [d_out, d_in] float64 dequantized, original order
    scales: np.ndarray     # [d_out, n_groups], processing-order groups
    zeros: np.ndarray      # [d_out, n_groups] int64
    perm: np.ndarray       # [d_in] processing order -> original column
    g_idx: np.ndarray      # [d_in] original column -> group
    U: np.ndarray          # [d_in, d_in] factor used (processing order)
    lam: float
    err_sq: np.ndarray     # [d_out] sum over columns of e_j^2
    codes_p: np.ndarray    # codes in processing order
    Q_p: np.ndarray        # Q in processing order
    t_at_code: np.ndarray  # w/scale + zero at the moment each code was decided (processing order)


def n_groups(d_in: int, group_size: int) -> int:
    G = d_in if group_size == -1 else group_size
    return (d_in + G - 1) // G


@dataclass
class Prepared:
    """The steps that depend on H only: processing order, damping, factor."""
    perm: np.ndarray
    lam: float
    U: np.ndarray


def prepare(H: np.ndarray, damp_percent: float = 0.01, desc_act: bool = False) -> Prepared:
    """Order ([P5] 2.2 "first"), damp ([P5] 3.3), then the factor of the damped,
    permuted H's inverse ([P5] 2.2 "third")."""
    perm = act_order(H, desc_act)
    Hd, lam = damp(H[np.ix_(perm, perm)], damp_percent)
    return Prepared(perm=perm, lam=lam, U=hinv_factor(Hd))


def gptq(W: np.ndarray, H: np.ndarray, *, bits: int = 4, group_size: int = 128,
         block_size: int = 128, damp_percent: float = 0.01, desc_act: bool = False,
         decision: str = "f64", prepared: Optional[Prepared] = None,
         sym: bool = False) -> GPTQResult:
    """The column loop.  ``prepared`` (from ``prepare(H, damp_percent,
    desc_act)``) lets several quantizer settings share one H's order and
    factor; without it they are computed here."""
    W64 = np.asarray(W, dtype=np.float64)
    d_out, d = W64.shape
    assert H.shape == (d, d)
    maxq = (1 << bits) - 1
    G = d if group_size == -1 else int(group_size)
    B = int(block_size)

    prep = prepared if prepared is not None else prepare(H, damp_percent, desc_act)
    perm, lam, U = prep.perm, prep.lam, prep.U

    Wp = W64[:, perm].copy()
    codes_p = np.zeros((d_out, d), dtype=np.int64)
    Qp = np.zeros((d_out, d), dtype=np.float64)
    tcode = np.zeros((d_out, d), dtype=np.float64)
    ng = n_groups(d, group_size)
    scales = np.zeros((d_out, ng), dtype=np.float64)
    zeros = np.zeros((d_out, ng), dtype=np.int64)
    err_sq = np.zeros(d_out, dtype=np.float64)
    s = z = None
    for b0 in range(0, d, B):
        b1 = min(b0 + B, d)
        Err = np.zeros((d_out, b1 - b0), dtype=np.float64)
        for j in range(b0, b1):
            if j % G == 0:
                s, z = group_params(Wp[:, j:min(j + G, d)], maxq, decision, sym)
                scales[:, j // G] = s
                zeros[:, j // G] = z.astype(np.int64)
            w = Wp[:, j]
            c, q = quantize(w, s, z, maxq, decision)
            tcode[:, j] = (_f(w, decision) / _f(s, decision)).astype(np.float64) + z
            e = (w - q) / U[j, j]
            Wp[:, j + 1:b1] -= np.outer(e, U[j, j + 1:b1])
            Err[:, j - b0] = e
            codes_p[:, j] = c
            Qp[:, j] = q
            err_sq += e * e
        if b1 < d:
            Wp[:, b1:] -= Err @ U[b0:b1, b1:]

    inv = np.empty_like(perm)
    inv[perm] = np.arange(d)
    g_idx = np.empty(d, dtype=np.int64)
    g_idx[perm] = np.arange(d) // G
    return GPTQResult(codes=codes_p[:, inv], Q=Qp[:, inv], scales=scales, zeros=zeros,
                      perm=perm, g_idx=g_idx, U=U, lam=lam, err_sq=err_sq,
                      codes_p=codes_p, Q_p=Qp, t_at_code=tcode)


def rtn(W: np.ndarray, *, bits: int = 4, group_size: int = 128,
        perm: Optional[np.ndarray] = None, decision: str = "f64", sym: bool = False):
    """Round-to-nearest baseline ([P2] section 二, the naive min-max grid; [P5]
    2.3 compares GPTQ against it): same grid and grouping, no compensation.
    Returns (codes, Q) in original column order."""
    W64 = np.asarray(W, dtype=np.float64)
    d_out, d = W64.shape
    maxq = (1 << bits) - 1
    G = d if group_size == -1 else int(group_size)
    perm = np.arange(d) if perm is None else np.asarray(perm)
    Wp = W64[:, perm]
    codes_p = np.zeros((d_out, d), dtype=np.int64)
    Qp = np.zeros((d_out, d), dtype=np.float64)
    for g0 in range(0, d, G):
        g1 = min(g0 + G, d)
        s, z = group_params(Wp[:, g0:g1], maxq, decision, sym)
        for j in range(g0, g1):
            c, q = quantize(Wp[:, j], s, z, maxq, decision)
            codes_p[:, j] = c
            Qp[:, j] = q
    inv = np.empty_like(perm)
    inv[perm] = np.arange(d)
    return codes_p[:, inv], Qp[:, inv]


# ----------------------------------------------------------------------------
# 6. objective and packing
# ----------------------------------------------------------------------------

def objective_rows(W: np.ndarray, Q: np.ndarray, H: np.ndarray) -> np.ndarray:
    """Per output row r: ||(W_r - Q_r) X^T||^2 = 1/2 D_r H D_r^T with D = W - Q
    and the undamped H = 2 X^T X (rows are independent, so the layer's error is
    their sum)."""
    D = np.asarray(W, np.float64) - np.asarray(Q, np.float64)
    return 0.5 * np.sum((D @ H) * D, axis=1)


def objective(W: np.ndarray, Q: np.ndarray, H: np.ndarray) -> float:
    """Layer reconstruction error ||(W - Q) X^T||_F^2 = 1/2 tr(D H D^T) with
    D = W - Q and the undamped H = 2 X^T X."""
    return float(np.sum(objective_rows(W, Q, H)))


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Eight 4-bit codes per 32-bit word, the first column in the lowest nibble
    (0.5 byte per weight at 4 bits, [P5] section 1.1)."""
    codes = np.asarray(codes, dtype=np.uint32) & np.uint32(0xF)
    rows, cols = codes.shape
    assert cols % 8 == 0
    c = codes.reshape(rows, cols // 8, 8)
    out = np.zeros((rows, cols // 8), dtype=np.uint32)
    for k in range(8):
        out |= c[:, :, k] << np.uint32(4 * k)
    return out


def unpack_int4(packed: np.ndarray, cols: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint32)
    rows = packed.shape[0]
    out = np.zeros((rows, cols), dtype=np.int64)
    for k in range(8):
        out[:, k::8] = (packed >> np.uint32(4 * k)) & np.uint32(0xF)
    return out


def pack_dense(codes: np.ndarray, bits: int) -> np.ndarray:
    """Dense packing of bits-wide codes (2, 3, 4 or 8): each row is one bit
    stream, code k in bits [k*bits, (k+1)*bits) counted from the least
    significant bit of word 0, so a 3-bit code may straddle two words
    (3/8 byte per weight, [P5] section 1.1's accounting).  cols*bits must be
    a multiple of 32.  At 4 bits this is pack_int4's layout."""
    codes = np.asarray(codes, dtype=np.uint64)
    rows, cols = codes.shape
    assert bits in (2, 3, 4, 8) and (cols * bits) % 32 == 0
    nw = cols * bits // 32
    out = np.zeros((rows, nw), dtype=np.uint64)
    mask = np.uint64((1 << bits) - 1)
    for k in range(cols):
        pos = k * bits
        w, sh = pos // 32, pos % 32
        v = codes[:, k] & mask
        out[:, w] |= (v << np.uint64(sh)) & np.uint64(0xFFFFFFFF)
        if sh + bits > 32:                      # the high part goes to the next word
            out[:, w + 1] |= v >> np.uint64(32 - sh)
    return out.astype(np.uint32)


def unpack_dense(packed: np.ndarray, cols: int, bits: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint64)
    rows = packed.shape[0]
    out = np.zeros((rows, cols), dtype=np.int64)
    for k in range(cols):
        pos = k * bits
        w, sh = pos // 32, pos % 32
        v = packed[:, w] >> np.uint64(sh)
        if sh + bits > 32:
            v |= packed[:, w + 1] << np.uint64(32 - sh)
        out[:, k] = (v & np.uint64((1 << bits) - 1)).astype(np.int64)
    return out


# ----------------------------------------------------------------------------
# 7. using the packed layer: y = x W_q^T  ([P5] 4.3: at inference the 4-bit
#    weights are dequantized to 16-bit and multiplied; the saving is in the
#    bytes moved)
# ----------------------------------------------------------------------------

def dequantize(packed: np.ndarray, scales: np.ndarray, zeros: np.ndarray, g_idx: np.ndarray,
               cols: int) -> np.ndarray:
    """W_q[r][c] = scales[r][g_idx[c]] * (code[r][c] - zeros[r][g_idx[c]]), float64,
    codes from pack_int4's layout."""
    codes = unpack_int4(packed, cols).astype(np.float64)
    g = np.asarray(g_idx, dtype=np.int64)
    return np.asarray(scales, np.float64)[:, g] * (codes - np.asarray(zeros, np.float64)[:, g])


def _round16(a32: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> nearest (ties to even) 16-bit value of dtype, as float64."""
    a32 = np.asarray(a32, dtype=np.float32)
    if dtype == "f16":
        return a32.astype(np.float16).astype(np.float64)
    u = a32.view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return (r.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def dequantize16(packed: np.ndarray, scales: np.ndarray, zeros: np.ndarray, g_idx: np.ndarray,
                 cols: int, dtype: str) -> np.ndarray:
    """The weights as the product uses them: [P5] 4.3 has the 4-bit weights
    dequantized to a 16-bit type first.  Each is the float32 product
    scale * (code - zero) rounded to dtype ("f16" or "bf16")."""
    codes = unpack_int4(packed, cols)
    g = np.asarray(g_idx, dtype=np.int64)
    s32 = np.asarray(scales, dtype=np.float32)[:, g]
    cz = (codes - np.asarray(zeros, dtype=np.int64)[:, g]).astype(np.float32)
    return _round16(s32 * cz, dtype)


def w4a16_matmul(X: np.ndarray, packed: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
                 g_idx: np.ndarray, dtype: Optional[str] = None) -> np.ndarray:
    """Y [m x d_out] = X [m x d_in] @ W^T in float64, W = dequantize (dtype None)
    or dequantize16 (dtype "f16"/"bf16")."""
    X64 = np.asarray(X, dtype=np.float64)
    d_in = X64.shape[1]
    Wd = (dequantize(packed, scales, zeros, g_idx, d_in) if dtype is None
          else dequantize16(packed, scales, zeros, g_idx, d_in, dtype))
    return X64 @ Wd.T
