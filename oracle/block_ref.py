"""CPU oracle: layer-sequential GPTQ over one Llama-shaped decoder block,
float64 numpy.

TEST INFRASTRUCTURE.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library and never reads anything the HIP library produced.

Sources (short names as in gptq_ref):
  [P1] "GPTQ/AWQ量化导出：让大模型在消费级显卡上跑起来": a calibration forward
       pass collects each layer's input activations; quantization starts at
       the first layer and moves on to the next one until all are done.
  [P2] "大模型压缩量化技术：GPTQ 与 AWQ 原理详解 + Python 实战教程", GPTQ's
       "layer by layer": one layer (a Transformer block) at a time, its
       curvature information from running the calibration data through it.
  [P5] the GPTQ practice page, section 2.1: the Hessian of a layer comes from
       that layer's calibration inputs, H = 2 X^T X.

Readings of open points:
  * The block is Llama's decoder layer (the pages quantize Llama/Qwen-style
    models): RMSNorm (eps 1e-6, weight gamma), q/k/v projections, rotary
    position embedding (rotate-half pairs (i, i + hd/2), theta_i =
    base^(-2i/hd), base 10000, position = index within the sequence), causal
    softmax attention with scale 1/sqrt(hd) per head, o projection, residual,
    RMSNorm, SwiGLU MLP (silu(x W_g^T) * (x W_u^T)) W_d^T, residual.
  * "Layer by layer" inside the block follows the order in which the
    sub-layers consume their inputs: q, k, v (one input, so one shared H) ->
    o -> gate, up (one shared H) -> down.  Every sub-layer's calibration
    inputs are computed with the already quantized sub-layers before it
    (the quantized weights are the dequantized Q = scale * (code - zero)),
    and the block's output (with all seven quantized) is the next block's
    calibration input.
  * The forward between sub-layers runs in float64 here and in fp32 on the
    GPU (no 16-bit rounding of activations).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional

import numpy as np

from . import gptq_ref as g

EPS = 1e-6
ROPE_BASE = 10000.0
SUBLAYERS = ("q", "k", "v", "o", "gate", "up", "down")


@dataclass
class BlockShape:
    d: int          # hidden size
    n_heads: int
    f: int          # MLP intermediate size
    seq_len: int    # tokens per calibration sequence (positions restart at 0)

    @property
    def hd(self) -> int:
        return self.d // self.n_heads


def rmsnorm(x: np.ndarray, gamma: Optional[np.ndarray] = None, eps: float = EPS) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gamma, per token (row)."""
    x = np.asarray(x, dtype=np.float64)
    y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return y if gamma is None else y * np.asarray(gamma, dtype=np.float64)[None, :]


def rope(x: np.ndarray, n_heads: int, seq_len: int, base: float = ROPE_BASE) -> np.ndarray:
    """Rotary embedding of q or k [T, d]: in each head, pair (i, i + hd/2) is
    rotated by angle p * base^(-2i/hd), p = token index within its sequence."""
    x = np.asarray(x, dtype=np.float64)
    T, d = x.shape
    hd = d // n_heads
    half = hd // 2
    pos = (np.arange(T) % seq_len).astype(np.float64)
    inv = base ** (-2.0 * np.arange(half) / hd)
    ang = pos[:, None] * inv[None, :]                       # [T, half]
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty_like(x)
    for h in range(n_heads):
        a = x[:, h * hd:h * hd + half]
        b = x[:, h * hd + half:(h + 1) * hd]
        out[:, h * hd:h * hd + half] = a * c - b * s
        out[:, h * hd + half:(h + 1) * hd] = b * c + a * s
    return out


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_heads: int,
                     seq_len: int) -> np.ndarray:
    """Per sequence and head: softmax(q k^T / sqrt(hd)) over positions <= the
    query's, times v."""
    T, d = q.shape
    hd = d // n_heads
    out = np.zeros((T, d))
    mask = np.tril(np.ones((seq_len, seq_len), dtype=bool))
    for s0 in range(0, T, seq_len):
        for h in range(n_heads):
            cols = slice(h * hd, (h + 1) * hd)
            qs, ks, vs = q[s0:s0 + seq_len, cols], k[s0:s0 + seq_len, cols], v[s0:s0 + seq_len, cols]
            sc = (qs @ ks.T) / np.sqrt(hd)
            sc = np.where(mask[:len(qs), :len(qs)], sc, -np.inf)
            sc = sc - sc.max(axis=1, keepdims=True)
            p = np.exp(sc)
            p /= p.sum(axis=1, keepdims=True)
            out[s0:s0 + seq_len, cols] = p @ vs
    return out


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def linear(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """y = x W^T."""
    return np.asarray(x, np.float64) @ np.asarray(W, np.float64).T


@dataclass
class BlockWeights:
    W: Dict[str, np.ndarray]                 # the seven projection matrices, [d_out, d_in]
    gamma1: Optional[np.ndarray] = None
    gamma2: Optional[np.ndarray] = None


def block_forward(x: np.ndarray, bw: BlockWeights, shape: BlockShape) -> Dict[str, np.ndarray]:
    """The block with the given weights; returns every sub-layer's input and
    the block output: x1 (q/k/v input), attn (o input), x2 (gate/up input),
    m (down input), h (residual after attention), y (output)."""
    x = np.asarray(x, np.float64)
    W = bw.W
    x1 = rmsnorm(x, bw.gamma1)
    q = rope(linear(x1, W["q"]), shape.n_heads, shape.seq_len)
    k = rope(linear(x1, W["k"]), shape.n_heads, shape.seq_len)
    v = linear(x1, W["v"])
    attn = causal_attention(q, k, v, shape.n_heads, shape.seq_len)
    h = x + linear(attn, W["o"])
    x2 = rmsnorm(h, bw.gamma2)
    m = silu(linear(x2, W["gate"])) * linear(x2, W["up"])
    y = h + linear(m, W["down"])
    return dict(x1=x1, attn=attn, h=h, x2=x2, m=m, y=y)


@dataclass
class SequentialResult:
    H: Dict[str, np.ndarray]                 # the Hessian each sub-layer was quantized with
    quant: Dict[str, g.GPTQResult]
    acts: Dict[str, np.ndarray] = field(default_factory=dict)   # x1, attn, h, x2, m, y


Quantizer = Callable[[np.ndarray, np.ndarray], g.GPTQResult]


def sequential_gptq(x: np.ndarray, bw: BlockWeights, shape: BlockShape, quantize: Quantizer
                    ) -> SequentialResult:
    """[P1]/[P2] layer by layer inside the block: each sub-layer's H from its
    calibration inputs computed with the quantized sub-layers before it."""
    x = np.asarray(x, np.float64)
    W = bw.W
    H, Qr = {}, {}
    x1 = rmsnorm(x, bw.gamma1)
    Hqkv = g.hessian([x1], shape.d)
    for n in ("q", "k", "v"):
        H[n] = Hqkv
        Qr[n] = quantize(W[n], Hqkv)
    q = rope(linear(x1, Qr["q"].Q), shape.n_heads, shape.seq_len)
    k = rope(linear(x1, Qr["k"].Q), shape.n_heads, shape.seq_len)
    v = linear(x1, Qr["v"].Q)
    attn = causal_attention(q, k, v, shape.n_heads, shape.seq_len)
    H["o"] = g.hessian([attn], shape.d)
    Qr["o"] = quantize(W["o"], H["o"])
    h = x + linear(attn, Qr["o"].Q)
    x2 = rmsnorm(h, bw.gamma2)
    Hgu = g.hessian([x2], shape.d)
    for n in ("gate", "up"):
        H[n] = Hgu
        Qr[n] = quantize(W[n], Hgu)
    m = silu(linear(x2, Qr["gate"].Q)) * linear(x2, Qr["up"].Q)
    H["down"] = g.hessian([m], shape.f)
    Qr["down"] = quantize(W["down"], H["down"])
    y = h + linear(m, Qr["down"].Q)
    return SequentialResult(H, Qr, dict(x1=x1, attn=attn, h=h, x2=x2, m=m, y=y))


def gptq_quantizer(bits: int = 4, group_size: int = 128, damp_percent: float = 0.01,
                   desc_act: bool = False) -> Quantizer:
    def qz(W, H):
        return g.gptq(np.asarray(W, np.float64), H, bits=bits, group_size=group_size,
                      damp_percent=damp_percent, desc_act=desc_act)
    return qz
