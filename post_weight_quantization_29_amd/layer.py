"""Convenience wrapper: allocate outputs and chain the C-ABI calls for one layer.

Only allocation and call sequencing live here; the arithmetic is in libgptq.so.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib as L


@dataclass
class GPTQLayerResult:
    codes: torch.Tensor      # [d_out, d_in] uint8, original column order
    scales: torch.Tensor     # [d_out, n_groups] fp32 (processing-order groups)
    zeros: torch.Tensor      # [d_out, n_groups] int32
    g_idx: torch.Tensor      # [d_in] int32
    perm: torch.Tensor       # [d_in] int32, processing order -> original column
    U: torch.Tensor          # [d_in, d_in] fp32
    Q: Optional[torch.Tensor]
    packed: Optional[torch.Tensor]


def alloc_outputs(d_out: int, d_in: int, group_size: int, device, with_q: bool = True):
    G = d_in if group_size == -1 else group_size
    ng = (d_in + G - 1) // G
    return dict(
        codes=torch.empty((d_out, d_in), dtype=torch.uint8, device=device),
        scales=torch.empty((d_out, ng), dtype=torch.float32, device=device),
        zeros=torch.empty((d_out, ng), dtype=torch.int32, device=device),
        g_idx=torch.empty((d_in,), dtype=torch.int32, device=device),
        Q=torch.empty((d_out, d_in), dtype=torch.float32, device=device) if with_q else None,
    )


def quantize_layer_outputs(W: torch.Tensor, H: torch.Tensor, cfg: L.gptq_config,
                           with_q: bool = True, pack: bool = True,
                           U: Optional[torch.Tensor] = None,
                           perm: Optional[torch.Tensor] = None,
                           hdiag: Optional[torch.Tensor] = None) -> GPTQLayerResult:
    """prepare_hinv (unless U/perm are given, e.g. shared by several layers
    with one H) -> quantize_layer -> pack_int4 (when bits <= 4)."""
    d_out, d_in = W.shape
    dev = W.device
    if U is None or perm is None:
        U = torch.empty((d_in, d_in), dtype=torch.float32, device=dev)
        perm = torch.empty((d_in,), dtype=torch.int32, device=dev)
        L.gptq_prepare_hinv(H, cfg.damp_percent, cfg.desc_act, U, perm, hdiag)
    out = alloc_outputs(d_out, d_in, cfg.group_size, dev, with_q)
    L.gptq_quantize_layer(W, U, perm, cfg, out["codes"], out["scales"], out["zeros"],
                          out["g_idx"], out["Q"])
    packed = None
    if pack and cfg.bits <= 4 and d_in % 8 == 0:
        packed = torch.empty((d_out, d_in // 8), dtype=torch.int32, device=dev)
        L.gptq_pack_int4(out["codes"], packed)
    return GPTQLayerResult(out["codes"], out["scales"], out["zeros"], out["g_idx"], perm, U,
                           out["Q"], packed)


@dataclass
class AWQLayerResult:
    s: torch.Tensor          # [d_in] fp32 channel factors (activations are divided by them)
    best: int                # index of the chosen factor in the grid
    scores: torch.Tensor     # [n_grid] fp64 activation-weighted error of every candidate
    codes: torch.Tensor      # [d_out, d_in] uint8
    scales: torch.Tensor     # [d_out, n_groups] fp32
    zeros: torch.Tensor      # [d_out, n_groups] int32
    Qhat: Optional[torch.Tensor]
    packed: Optional[torch.Tensor]


def awq_quantize_layer(W: torch.Tensor, x_chunks, bits: int = 4, group_size: int = 128,
                       top_frac: float = 0.05, grid=L.AWQ_DEFAULT_GRID, with_q: bool = True,
                       pack: bool = True, a: Optional[torch.Tensor] = None) -> AWQLayerResult:
    """gptq_awq_act_sumsq over the calibration chunks (unless the statistic a
    is given) -> gptq_awq_search -> gptq_awq_quantize -> gptq_pack_int4."""
    d_out, d_in = W.shape
    dev = W.device
    if a is None:
        a = torch.zeros((d_in,), dtype=torch.float64, device=dev)
        for x in x_chunks:
            L.gptq_awq_act_sumsq(a, x)
    s = torch.empty((d_in,), dtype=torch.float32, device=dev)
    scores = torch.empty((len(grid),), dtype=torch.float64, device=dev)
    best = torch.empty((1,), dtype=torch.int32, device=dev)
    L.gptq_awq_search(W, a, s, scores, best, bits=bits, group_size=group_size, top_frac=top_frac,
                      grid=grid)
    G = d_in if group_size == -1 else group_size
    ng = (d_in + G - 1) // G
    codes = torch.empty((d_out, d_in), dtype=torch.uint8, device=dev)
    scales = torch.empty((d_out, ng), dtype=torch.float32, device=dev)
    zeros = torch.empty((d_out, ng), dtype=torch.int32, device=dev)
    Qhat = torch.empty((d_out, d_in), dtype=torch.float32, device=dev) if with_q else None
    L.gptq_awq_quantize(W, s, codes, scales, zeros, Qhat, bits=bits, group_size=group_size)
    packed = None
    if pack and bits <= 4 and d_in % 8 == 0:
        packed = torch.empty((d_out, d_in // 8), dtype=torch.int32, device=dev)
        L.gptq_pack_int4(codes, packed)
    return AWQLayerResult(s, int(best.item()), scores, codes, scales, zeros, Qhat, packed)
