"""Layer-sequential GPTQ over one Llama decoder block: allocation and call
sequencing only; every step (norms, projections, attention, Hessians,
factorizations, column loops) runs in libgptq.so.

Order (the pages' "layer by layer", inside the block in the order the
sub-layers consume their inputs): q, k, v share one Hessian (one input) and
one factor; o; gate and up share one; down.  Each sub-layer's calibration
inputs are computed with the already quantized sub-layers before it (their
dequantized Q), and the block output with all seven quantized is the next
block's calibration input.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import torch

from . import _lib as L
from .layer import GPTQLayerResult, quantize_layer_outputs

SUBLAYERS = ("q", "k", "v", "o", "gate", "up", "down")


@dataclass
class BlockShape:
    d: int
    n_heads: int
    f: int
    seq_len: int


@dataclass
class BlockResult:
    quant: Dict[str, GPTQLayerResult]
    y: torch.Tensor                                   # block output with every sub-layer quantized
    H: Dict[str, torch.Tensor] = field(default_factory=dict)
    acts: Dict[str, torch.Tensor] = field(default_factory=dict)


def _hessian(x: torch.Tensor):
    d = x.shape[1]
    H = torch.zeros((d, d), dtype=torch.float32, device=x.device)
    hd = torch.zeros((d,), dtype=torch.float64, device=x.device)
    L.gptq_hessian_accumulate(H, x, hd)
    return H, hd


def _quantize_group(names, W, H, hd, cfg, pack=True) -> Dict[str, GPTQLayerResult]:
    """Sub-layers with one input: one factor, then one column loop each."""
    d = H.shape[0]
    U = torch.empty((d, d), dtype=torch.float32, device=H.device)
    perm = torch.empty((d,), dtype=torch.int32, device=H.device)
    L.gptq_prepare_hinv(H, cfg.damp_percent, cfg.desc_act, U, perm, hd)
    return {n: quantize_layer_outputs(W[n], H, cfg, with_q=True, pack=pack, U=U, perm=perm, hdiag=hd)
            for n in names}


def stage_qkv(x: torch.Tensor, W: Dict[str, torch.Tensor], cfg: L.gptq_config,
              gamma1: Optional[torch.Tensor] = None):
    """x1 = RMSNorm(x); one H (and one factor) for q, k, v."""
    T, d = x.shape
    x1 = torch.empty((T, d), dtype=torch.float32, device=x.device)
    L.gptq_rmsnorm(x, x1, gamma1)
    H, hd = _hessian(x1)
    return x1, H, _quantize_group(("q", "k", "v"), W, H, hd, cfg, True)


def stage_o(x1: torch.Tensor, Qq: torch.Tensor, Qk: torch.Tensor, Qv: torch.Tensor,
            W: Dict[str, torch.Tensor], cfg: L.gptq_config, shape: BlockShape,
            rope_base: float = 10000.0):
    """The o projection's input: attention with the given (quantized) q, k, v."""
    attn = torch.empty_like(x1)
    L.gptq_block_attention(x1, Qq, Qk, Qv, attn, shape.n_heads, shape.seq_len, rope_base)
    H, hd = _hessian(attn)
    return attn, H, _quantize_group(("o",), W, H, hd, cfg, True)


def stage_gate_up(x: torch.Tensor, attn: torch.Tensor, Qo: torch.Tensor, W: Dict[str, torch.Tensor],
                  cfg: L.gptq_config, gamma2: Optional[torch.Tensor] = None):
    """h = x + attn Qo^T; x2 = RMSNorm(h); one H for gate and up."""
    h = torch.empty_like(x)
    L.gptq_linear(attn, Qo, h, R=x)
    x2 = torch.empty_like(x)
    L.gptq_rmsnorm(h, x2, gamma2)
    H, hd = _hessian(x2)
    return h, x2, H, _quantize_group(("gate", "up"), W, H, hd, cfg, True)


def stage_down(x2: torch.Tensor, Qg: torch.Tensor, Qu: torch.Tensor, W: Dict[str, torch.Tensor],
               cfg: L.gptq_config, shape: BlockShape):
    """m = silu(x2 Qg^T) * (x2 Qu^T), the down projection's input."""
    T = x2.shape[0]
    f32 = dict(dtype=torch.float32, device=x2.device)
    gt = torch.empty((T, shape.f), **f32)
    up = torch.empty((T, shape.f), **f32)
    L.gptq_linear(x2, Qg, gt)
    L.gptq_linear(x2, Qu, up)
    m = torch.empty((T, shape.f), **f32)
    L.gptq_swiglu(gt, up, m)
    del gt, up
    H, hd = _hessian(m)
    return m, H, _quantize_group(("down",), W, H, hd, cfg, True)


def block_output(m: torch.Tensor, h: torch.Tensor, Qd: torch.Tensor) -> torch.Tensor:
    y = torch.empty_like(h)
    L.gptq_linear(m, Qd, y, R=h)
    return y


def quantize_block_sequential(x: torch.Tensor, W: Dict[str, torch.Tensor], shape: BlockShape,
                              cfg: L.gptq_config, gamma1: Optional[torch.Tensor] = None,
                              gamma2: Optional[torch.Tensor] = None, rope_base: float = 10000.0,
                              keep: bool = False) -> BlockResult:
    """x: [T, d] fp32 calibration hidden states (T a multiple of seq_len);
    W: the seven projections [d_out, d_in] (fp32/fp16/bf16).  Each stage
    runs with the quantized sub-layers of the stages before it."""
    x1, H1, quant = stage_qkv(x, W, cfg, gamma1)
    attn, H2, qo = stage_o(x1, quant["q"].Q, quant["k"].Q, quant["v"].Q, W, cfg, shape, rope_base)
    quant.update(qo)
    h, x2, H3, qgu = stage_gate_up(x, attn, quant["o"].Q, W, cfg, gamma2)
    quant.update(qgu)
    m, H4, qd = stage_down(x2, quant["gate"].Q, quant["up"].Q, W, cfg, shape)
    quant.update(qd)
    y = block_output(m, h, quant["down"].Q)
    Hs, acts = {}, {}
    if keep:
        Hs = dict(q=H1, k=H1, v=H1, o=H2, gate=H3, up=H3, down=H4)
        acts = dict(x1=x1, attn=attn, h=h, x2=x2, m=m)
    return BlockResult(quant, y, Hs, acts)
