"""CPU oracle: activation-aware weight quantization (AWQ) of one linear layer,
float64 numpy.

TEST INFRASTRUCTURE.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library and never reads anything the HIP library produced.

Sources (short names as in gptq_ref):
  [P1] "GPTQ/AWQ量化导出：让大模型在消费级显卡上跑起来" (bxzpzcl.cn/news/361031),
       the AWQ steps after the GPTQ description:
       per input channel the RMS of the calibration activations; the most
       active top-k % of channels (5 % by default) get a larger scaling factor
       so that quantization keeps more of them; at inference the factor is
       multiplied back, so the layer computes the same function.
  [P2] "大模型压缩量化技术：GPTQ 与 AWQ 原理详解 + Python 实战教程", section 四:
       find the channels with large activations from calibration statistics,
       multiply their weights by a factor s > 1, quantize, divide the matching
       activations by s at inference; the factor is chosen as the best one;
       no backpropagation and no Hessian.
  [P4] "AWQ与GPTQ谁更强？ms-swift量化模块深度评测": AwqConfig(bits=4,
       group_size=128, zero_point=True), i.e. 4-bit asymmetric groups of 128.

Readings of open points:
  * Statistic: a_j = sum_t x_tj^2 over the calibration tokens (the RMS squared
    times N; the ranking and the argmin below do not depend on the 1/N).
  * Salient set: the k channels with the largest a_j, ties to the lower index,
    k = top_frac * d_in rounded to nearest (halves up), computed in float64
    from top_frac's float32 value.
  * Scaling: s_j = sigma for salient channels, 1 otherwise; the quantized
    weights are the min-max group grid of gptq_ref (asymmetric, zero point not
    clamped) applied to fp32(fp32(w) * fp32(s_j)), and the layer's effective
    weights are Qhat_ij = scale * (code - zero) / s_j.  [P4]'s opposite
    direction (non-salient channels scaled down) is the same transform up to a
    per-group factor, to which the min-max grid is invariant (pinned for a
    factor of 2, where the products are exact).
  * "The best factor": the sigma of a candidate grid that minimizes
    E(sigma) = sum_j a_j sum_i (W_ij - Qhat_ij)^2, the layer's output error
    sum_t ||x_t (W - Qhat)^T||^2 when the channels are uncorrelated (pinned
    against that output error for inputs with orthogonal columns).  Ties go
    to the earlier candidate.  The grid is an input; the default is
    1, 1.125, ..., 4 (25 candidates, 1 included, so E(best) <= E(RTN)).
  * Integer decisions (zero points, codes) in float32 as in gptq_ref; the
    error sum in float64.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Iterable, Sequence

import numpy as np

from . import gptq_ref as g

DEFAULT_GRID = tuple(1.0 + 0.125 * k for k in range(25))
DEFAULT_TOP_FRAC = 0.05


def act_sumsq(chunks: Iterable[np.ndarray], d_in: int) -> np.ndarray:
    """a_j = sum over all tokens of x_tj^2 ([P1] step 1: the per-channel RMS is
    sqrt(a_j / N)).  Chunks are [tokens, d_in] arrays of any float type."""
    a = np.zeros(d_in)
    for x in chunks:
        x64 = np.asarray(x, dtype=np.float64)
        a += np.einsum("tj,tj->j", x64, x64)
    return a


def n_salient(top_frac: float, d_in: int) -> int:
    """k = top_frac * d_in rounded to the nearest integer (halves up), from
    top_frac's float32 value in float64: 5 % of 4096 channels is 205."""
    k = int(np.floor(np.float64(np.float32(top_frac)) * d_in + 0.5))
    return max(0, min(d_in, k))


def salient_mask(a: np.ndarray, top_frac: float) -> np.ndarray:
    """The top-k channels by a_j ([P1] step 2), ties to the lower index."""
    a = np.asarray(a, dtype=np.float64)
    k = n_salient(top_frac, a.shape[0])
    order = np.argsort(-a, kind="stable")
    mask = np.zeros(a.shape[0], dtype=bool)
    mask[order[:k]] = True
    return mask


def channel_scales(mask: np.ndarray, sigma: float) -> np.ndarray:
    """s_j = sigma on salient channels, 1 elsewhere (float32)."""
    return np.where(mask, np.float32(sigma), np.float32(1.0)).astype(np.float32)


@dataclass
class AWQQuant:
    codes: np.ndarray    # [d_out, d_in] int64
    scales: np.ndarray   # [d_out, n_groups] float32 (grid of the scaled weights)
    zeros: np.ndarray    # [d_out, n_groups] float32, integer-valued
    Qhat: np.ndarray     # [d_out, d_in] float64 effective weights scale*(code-zero)/s_j


def quantize_scaled(W: np.ndarray, s: np.ndarray, *, bits: int = 4,
                    group_size: int = 128) -> AWQQuant:
    """[P2] section 四 steps 2-4: multiply channel j's weights by s_j, quantize
    with the plain group grid (round to nearest, no compensation), divide by
    s_j again for the effective weights."""
    W32 = np.asarray(W, dtype=np.float32)
    s32 = np.asarray(s, dtype=np.float32)
    Ws = (W32 * s32[None, :]).astype(np.float32)          # fp32 products
    d_out, d = Ws.shape
    maxq = (1 << bits) - 1
    G = d if group_size == -1 else int(group_size)
    ng = (d + G - 1) // G
    codes = np.zeros((d_out, d), dtype=np.int64)
    Qs = np.zeros((d_out, d))
    scales = np.zeros((d_out, ng), dtype=np.float32)
    zeros = np.zeros((d_out, ng), dtype=np.float32)
    for gi in range(ng):
        c0, c1 = gi * G, min(d, (gi + 1) * G)
        sc, z = g.group_params(Ws[:, c0:c1].astype(np.float64), maxq, "f32")
        scales[:, gi], zeros[:, gi] = sc, z
        codes[:, c0:c1], Qs[:, c0:c1] = g.quantize(Ws[:, c0:c1].astype(np.float64), sc[:, None],
                                                   z[:, None], maxq, "f32")
    Qhat = Qs / s32.astype(np.float64)[None, :]
    return AWQQuant(codes, scales, zeros, Qhat)


def weighted_error(W: np.ndarray, Qhat: np.ndarray, a: np.ndarray) -> float:
    """E = sum_j a_j sum_i (W_ij - Qhat_ij)^2."""
    D = np.asarray(W, dtype=np.float64) - Qhat
    return float(np.sum(np.asarray(a, dtype=np.float64)[None, :] * D * D))


@dataclass
class AWQResult:
    best: int                 # index into the grid
    sigma: float
    scores: np.ndarray        # E(sigma_k) for every candidate
    s: np.ndarray             # [d_in] float32 channel factors of the best candidate
    quant: AWQQuant           # the layer quantized with them


def awq(W: np.ndarray, a: np.ndarray, *, bits: int = 4, group_size: int = 128,
        top_frac: float = DEFAULT_TOP_FRAC, grid: Sequence[float] = DEFAULT_GRID) -> AWQResult:
    """Statistics -> salient channels -> the best factor on the grid -> the
    layer quantized with it ([P1] steps 1-4, [P2] section 四)."""
    mask = salient_mask(a, top_frac)
    grid32 = np.asarray(grid, dtype=np.float32)
    scores = np.empty(len(grid32))
    for k, sg in enumerate(grid32):
        q = quantize_scaled(W, channel_scales(mask, sg), bits=bits, group_size=group_size)
        scores[k] = weighted_error(W, q.Qhat, a)
    best = int(np.argmin(scores))                       # first minimum
    s = channel_scales(mask, grid32[best])
    return AWQResult(best, float(grid32[best]), scores, s,
                     quantize_scaled(W, s, bits=bits, group_size=group_size))
