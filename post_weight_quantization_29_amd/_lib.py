"""ctypes binding of libgptq.so: the C-ABI calls under the same names.

Argument marshalling only: torch tensors are passed as device pointers and the
current HIP stream; every step runs in the library's kernels.  Workspaces are
allocated through torch when the caller does not pass one.  There is no CPU
fallback: a missing library raises immediately.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("GPTQ_MI355X_LIB", os.path.join(_PKG, "libgptq.so"))

GPTQ_F32, GPTQ_F16, GPTQ_BF16 = 0, 1, 2
OK, ERR_INVALID_ARG, ERR_NOT_PD, ERR_HIP, ERR_WORKSPACE, ERR_UNSUPPORTED = 0, -1, -2, -3, -4, -5

_DTYPE = {torch.float32: GPTQ_F32, torch.float16: GPTQ_F16, torch.bfloat16: GPTQ_BF16}


class GPTQError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class NotPositiveDefinite(GPTQError):
    pass


class gptq_config(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("damp_percent", ctypes.c_float),
                ("desc_act", ctypes.c_int32), ("sym", ctypes.c_int32),
                ("per_block_steps", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libgptq.so not found at {LIB_PATH}; build it with "
                              f"`python -m post_weight_quantization_29_amd.build_lib`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        sig = {
            "gptq_hessian_workspace_size": (sz, [i64, i32]),
            "gptq_hessian_accumulate": (ctypes.c_int, [vp, vp, vp, ctypes.c_int, i64, i32, vp, sz, vp]),
            "gptq_hessian_noalloc_scratch_bytes": (sz, []),
            "gptq_hessian_accumulate_noalloc": (ctypes.c_int, [vp, vp, vp, ctypes.c_int, i64, i32, vp]),
            "gptq_prepare_hinv_workspace_size": (sz, [i32]),
            "gptq_prepare_hinv": (ctypes.c_int, [vp, vp, i32, ctypes.c_float, i32, vp, vp, vp, sz, vp]),
            "gptq_quantize_workspace_size": (sz, [i32, i32, ctypes.POINTER(gptq_config)]),
            "gptq_quantize_layer": (ctypes.c_int, [vp, ctypes.c_int, i32, i32, vp, vp,
                                                   ctypes.POINTER(gptq_config), vp, vp, vp, vp, vp,
                                                   vp, sz, vp]),
            "gptq_pack_int4": (ctypes.c_int, [vp, i64, i64, vp, vp]),
            "gptq_pack_dense": (ctypes.c_int, [vp, i64, i64, i32, vp, vp]),
            "gptq_w4a16_gemm": (ctypes.c_int, [vp, ctypes.c_int, i64, i32, vp, vp, vp, vp, i32, i32,
                                               i32, vp, ctypes.c_int, vp]),
            "gptq_awq_sumsq_workspace_size": (sz, [i64, i32]),
            "gptq_awq_act_sumsq": (ctypes.c_int, [vp, vp, ctypes.c_int, i64, i32, vp, sz, vp]),
            "gptq_awq_search_workspace_size": (sz, [i32, i32, i32]),
            "gptq_awq_search": (ctypes.c_int, [vp, ctypes.c_int, i32, i32, vp, i32, i32, ctypes.c_float,
                                               ctypes.POINTER(ctypes.c_float), i32, vp, vp, vp, vp, sz,
                                               vp]),
            "gptq_awq_quantize": (ctypes.c_int, [vp, ctypes.c_int, i32, i32, vp, i32, i32, vp, vp, vp,
                                                 vp, vp]),
            "gptq_rmsnorm": (ctypes.c_int, [vp, ctypes.c_int, i64, i32, vp, ctypes.c_float, vp, vp]),
            "gptq_linear_workspace_size": (sz, [i32, i32]),
            "gptq_linear": (ctypes.c_int, [vp, i64, i32, vp, i32, vp, vp, vp, sz, vp]),
            "gptq_block_attention_workspace_size": (sz, [i64, i32, i32, i32]),
            "gptq_block_attention": (ctypes.c_int, [vp, i64, i32, i32, i32, vp, vp, vp, ctypes.c_float,
                                                    vp, vp, sz, vp]),
            "gptq_swiglu": (ctypes.c_int, [vp, vp, i64, vp, vp]),
            "gptq_layer_error_workspace_size": (sz, [i32, i32]),
            "gptq_layer_error": (ctypes.c_int, [vp, vp, ctypes.c_int, vp, i32, i32,
                                                ctypes.POINTER(ctypes.c_double), vp, sz, vp]),
            "gptq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "gptq_abi_version": (ctypes.c_int, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


EXPORTED = ("gptq_hessian_workspace_size", "gptq_hessian_accumulate",
            "gptq_hessian_noalloc_scratch_bytes", "gptq_hessian_accumulate_noalloc",
            "gptq_prepare_hinv_workspace_size", "gptq_prepare_hinv",
            "gptq_quantize_workspace_size", "gptq_quantize_layer", "gptq_pack_int4",
            "gptq_pack_dense", "gptq_w4a16_gemm", "gptq_awq_sumsq_workspace_size",
            "gptq_awq_act_sumsq", "gptq_awq_search_workspace_size", "gptq_awq_search",
            "gptq_awq_quantize", "gptq_rmsnorm", "gptq_linear_workspace_size", "gptq_linear",
            "gptq_block_attention_workspace_size", "gptq_block_attention", "gptq_swiglu",
            "gptq_layer_error_workspace_size", "gptq_layer_error", "gptq_status_string",
            "gptq_abi_version")


def _check(st: int, what: str) -> None:
    if st == OK:
        return
    msg = f"{what}: {lib().gptq_status_string(st).decode()}"
    if st == ERR_NOT_PD:
        raise NotPositiveDefinite(st, msg)
    raise GPTQError(st, msg)


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ws(nbytes: int, ws: Optional[torch.Tensor], device, stream=None) -> torch.Tensor:
    """The caller's workspace, or a fresh one from torch's caching allocator.
    A fresh one is allocated on the stream the call's work goes to, so that
    the allocator reuses its memory only after that work (the call may return
    before its kernels have run)."""
    if ws is not None:
        return ws
    if stream is None:
        return torch.empty(max(1, nbytes), dtype=torch.uint8, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(max(1, nbytes), dtype=torch.uint8, device=device)


def make_config(bits: int = 4, group_size: int = 128, block_size: int = 128,
                damp_percent: float = 0.01, desc_act: int = 0, sym: int = 0,
                per_block_steps: int = 0) -> gptq_config:
    return gptq_config(bits, group_size, block_size, damp_percent, int(desc_act), int(sym),
                       int(per_block_steps))


# ---------------------------------------------------------------- C-ABI calls

def gptq_hessian_workspace_size(n_tokens: int, d_in: int) -> int:
    return int(lib().gptq_hessian_workspace_size(n_tokens, d_in))


def gptq_hessian_accumulate(H: torch.Tensor, X: torch.Tensor, hdiag: Optional[torch.Tensor] = None,
                            ws: Optional[torch.Tensor] = None, stream=None) -> None:
    """H [d, d] fp32 += 2 X^T X for X [n_tokens, d] (fp32 / fp16 / bf16);
    hdiag [d] fp64 (optional) += the same diagonal summed in fp64."""
    _dev(H, "H"); _dev(X, "X")
    n, d = X.shape
    assert H.dtype == torch.float32 and tuple(H.shape) == (d, d)
    if hdiag is not None:
        _dev(hdiag, "hdiag")
        assert hdiag.dtype == torch.float64 and hdiag.numel() == d
    need = gptq_hessian_workspace_size(n, d)
    ws = _ws(need, ws, X.device, stream)
    _check(lib().gptq_hessian_accumulate(_ptr(H), _ptr(hdiag), _ptr(X), _DTYPE[X.dtype], n, d,
                                         _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "gptq_hessian_accumulate")


def gptq_hessian_noalloc_scratch_bytes() -> int:
    return int(lib().gptq_hessian_noalloc_scratch_bytes())


def gptq_hessian_accumulate_noalloc(H: torch.Tensor, X: torch.Tensor,
                                    hdiag: Optional[torch.Tensor] = None, stream=None) -> None:
    """gptq_hessian_accumulate with the partial sums in the library's static
    per-device scratch array (no allocation at all; d_in <= 11,264)."""
    _dev(H, "H"); _dev(X, "X")
    n, d = X.shape
    assert H.dtype == torch.float32 and tuple(H.shape) == (d, d)
    if hdiag is not None:
        _dev(hdiag, "hdiag")
        assert hdiag.dtype == torch.float64 and hdiag.numel() == d
    _check(lib().gptq_hessian_accumulate_noalloc(_ptr(H), _ptr(hdiag), _ptr(X), _DTYPE[X.dtype], n, d,
                                                 _stream(stream)), "gptq_hessian_accumulate_noalloc")


def gptq_prepare_hinv_workspace_size(d_in: int) -> int:
    return int(lib().gptq_prepare_hinv_workspace_size(d_in))


def gptq_prepare_hinv(H: torch.Tensor, damp_percent: float, desc_act: int, U: torch.Tensor,
                      perm: torch.Tensor, hdiag: Optional[torch.Tensor] = None,
                      ws: Optional[torch.Tensor] = None, stream=None) -> None:
    _dev(H, "H"); _dev(U, "U"); _dev(perm, "perm")
    d = H.shape[0]
    assert H.dtype == U.dtype == torch.float32 and perm.dtype == torch.int32
    if hdiag is not None:
        _dev(hdiag, "hdiag")
        assert hdiag.dtype == torch.float64 and hdiag.numel() == d
    ws = _ws(gptq_prepare_hinv_workspace_size(d), ws, H.device, stream)
    _check(lib().gptq_prepare_hinv(_ptr(H), _ptr(hdiag), d, float(damp_percent), int(desc_act),
                                   _ptr(U), _ptr(perm), _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)), "gptq_prepare_hinv")


def gptq_quantize_workspace_size(d_out: int, d_in: int, cfg: gptq_config) -> int:
    return int(lib().gptq_quantize_workspace_size(d_out, d_in, ctypes.byref(cfg)))


def gptq_quantize_layer(W: torch.Tensor, U: torch.Tensor, perm: torch.Tensor, cfg: gptq_config,
                        codes: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
                        g_idx: torch.Tensor, Q: Optional[torch.Tensor] = None,
                        ws: Optional[torch.Tensor] = None, stream=None) -> None:
    for t, nm in ((W, "W"), (U, "U"), (perm, "perm"), (codes, "codes"), (scales, "scales"),
                  (zeros, "zeros"), (g_idx, "g_idx")):
        _dev(t, nm)
    if Q is not None:
        _dev(Q, "Q")
    d_out, d_in = W.shape
    assert codes.dtype == torch.uint8 and scales.dtype == torch.float32
    assert zeros.dtype == torch.int32 and g_idx.dtype == torch.int32
    ws = _ws(gptq_quantize_workspace_size(d_out, d_in, cfg), ws, W.device, stream)
    _check(lib().gptq_quantize_layer(_ptr(W), _DTYPE[W.dtype], d_out, d_in, _ptr(U), _ptr(perm),
                                     ctypes.byref(cfg), _ptr(codes), _ptr(scales), _ptr(zeros),
                                     _ptr(g_idx), _ptr(Q), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream(stream)), "gptq_quantize_layer")


def gptq_pack_int4(codes: torch.Tensor, packed: torch.Tensor, stream=None) -> None:
    _dev(codes, "codes"); _dev(packed, "packed")
    rows, cols = codes.shape
    assert packed.dtype == torch.int32 or packed.dtype == torch.uint32
    _check(lib().gptq_pack_int4(_ptr(codes), rows, cols, _ptr(packed), _stream(stream)),
           "gptq_pack_int4")


def gptq_pack_dense(codes: torch.Tensor, packed: torch.Tensor, bits: int, stream=None) -> None:
    _dev(codes, "codes"); _dev(packed, "packed")
    rows, cols = codes.shape
    assert packed.dtype == torch.int32 or packed.dtype == torch.uint32
    _check(lib().gptq_pack_dense(_ptr(codes), rows, cols, int(bits), _ptr(packed), _stream(stream)),
           "gptq_pack_dense")


def gptq_w4a16_gemm(X: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
                    Y: torch.Tensor, g_idx: Optional[torch.Tensor] = None, group_size: int = 128,
                    stream=None) -> None:
    for t, n in ((X, "X"), (packed, "packed"), (scales, "scales"), (zeros, "zeros"), (Y, "Y")):
        _dev(t, n)
    m, d_in = X.shape
    d_out, n_groups = scales.shape
    assert Y.shape == (m, d_out) and zeros.shape == scales.shape
    if g_idx is not None:
        _dev(g_idx, "g_idx")
    _check(lib().gptq_w4a16_gemm(_ptr(X), _DTYPE[X.dtype], m, d_in, _ptr(packed), _ptr(scales),
                                 _ptr(zeros), _ptr(g_idx) if g_idx is not None else None,
                                 int(group_size), n_groups, d_out, _ptr(Y), _DTYPE[Y.dtype],
                                 _stream(stream)), "gptq_w4a16_gemm")


AWQ_DEFAULT_GRID = tuple(1.0 + 0.125 * k for k in range(25))


def gptq_awq_sumsq_workspace_size(n_tokens: int, d_in: int) -> int:
    return int(lib().gptq_awq_sumsq_workspace_size(n_tokens, d_in))


def gptq_awq_act_sumsq(a: torch.Tensor, X: torch.Tensor, ws: Optional[torch.Tensor] = None,
                       stream=None) -> None:
    _dev(a, "a"); _dev(X, "X")
    n, d_in = X.shape
    assert a.dtype == torch.float64 and a.shape == (d_in,)
    ws = _ws(gptq_awq_sumsq_workspace_size(n, d_in), ws, X.device, stream)
    _check(lib().gptq_awq_act_sumsq(_ptr(a), _ptr(X), _DTYPE[X.dtype], n, d_in, _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream)),
           "gptq_awq_act_sumsq")


def gptq_awq_search_workspace_size(d_out: int, d_in: int, group_size: int = 128) -> int:
    return int(lib().gptq_awq_search_workspace_size(d_out, d_in, group_size))


def gptq_awq_search(W: torch.Tensor, a: torch.Tensor, s_out: torch.Tensor, scores: torch.Tensor,
                    best: Optional[torch.Tensor] = None, bits: int = 4, group_size: int = 128,
                    top_frac: float = 0.05, grid=AWQ_DEFAULT_GRID, ws: Optional[torch.Tensor] = None,
                    stream=None) -> None:
    for t, n in ((W, "W"), (a, "a"), (s_out, "s_out"), (scores, "scores")):
        _dev(t, n)
    d_out, d_in = W.shape
    g = (ctypes.c_float * len(grid))(*[float(v) for v in grid])
    ws = _ws(gptq_awq_search_workspace_size(d_out, d_in, group_size), ws, W.device, stream)
    _check(lib().gptq_awq_search(_ptr(W), _DTYPE[W.dtype], d_out, d_in, _ptr(a), bits, group_size,
                                 float(top_frac), g, len(grid), _ptr(s_out), _ptr(scores), _ptr(best),
                                 _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "gptq_awq_search")


def gptq_awq_quantize(W: torch.Tensor, s: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                      zeros: torch.Tensor, Qhat: Optional[torch.Tensor] = None, bits: int = 4,
                      group_size: int = 128, stream=None) -> None:
    for t, n in ((W, "W"), (s, "s"), (codes, "codes"), (scales, "scales"), (zeros, "zeros")):
        _dev(t, n)
    d_out, d_in = W.shape
    _check(lib().gptq_awq_quantize(_ptr(W), _DTYPE[W.dtype], d_out, d_in, _ptr(s), bits, group_size,
                                   _ptr(codes), _ptr(scales), _ptr(zeros), _ptr(Qhat),
                                   _stream(stream)), "gptq_awq_quantize")


def gptq_rmsnorm(X: torch.Tensor, Y: torch.Tensor, gamma: Optional[torch.Tensor] = None,
                 eps: float = 1e-6, stream=None) -> None:
    _dev(X, "X"); _dev(Y, "Y")
    n, d = X.shape
    assert Y.dtype == torch.float32 and Y.shape == (n, d)
    _check(lib().gptq_rmsnorm(_ptr(X), _DTYPE[X.dtype], n, d, _ptr(gamma), float(eps), _ptr(Y),
                              _stream(stream)), "gptq_rmsnorm")


def gptq_linear_workspace_size(d_out: int, d_in: int) -> int:
    return int(lib().gptq_linear_workspace_size(d_out, d_in))


def gptq_linear(X: torch.Tensor, W: torch.Tensor, Y: torch.Tensor, R: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None, stream=None) -> None:
    _dev(X, "X"); _dev(W, "W"); _dev(Y, "Y")
    n, d_in = X.shape
    d_out = W.shape[0]
    assert W.shape == (d_out, d_in) and Y.shape == (n, d_out)
    assert X.dtype == W.dtype == Y.dtype == torch.float32
    ws = _ws(gptq_linear_workspace_size(d_out, d_in), ws, X.device, stream)
    _check(lib().gptq_linear(_ptr(X), n, d_in, _ptr(W), d_out, _ptr(R), _ptr(Y), _ptr(ws),
                             ws.numel() * ws.element_size(), _stream(stream)), "gptq_linear")


def gptq_block_attention_workspace_size(n_tokens: int, d: int, n_heads: int, seq_len: int) -> int:
    return int(lib().gptq_block_attention_workspace_size(n_tokens, d, n_heads, seq_len))


def gptq_block_attention(x1: torch.Tensor, Wq: torch.Tensor, Wk: torch.Tensor, Wv: torch.Tensor,
                         out: torch.Tensor, n_heads: int, seq_len: int, rope_base: float = 10000.0,
                         ws: Optional[torch.Tensor] = None, stream=None) -> None:
    for t, n in ((x1, "x1"), (Wq, "Wq"), (Wk, "Wk"), (Wv, "Wv"), (out, "out")):
        _dev(t, n)
    T, d = x1.shape
    ws = _ws(gptq_block_attention_workspace_size(T, d, n_heads, seq_len), ws, x1.device, stream)
    _check(lib().gptq_block_attention(_ptr(x1), T, d, n_heads, seq_len, _ptr(Wq), _ptr(Wk), _ptr(Wv),
                                      float(rope_base), _ptr(out), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(stream)),
           "gptq_block_attention")


def gptq_swiglu(G: torch.Tensor, U: torch.Tensor, M: torch.Tensor, stream=None) -> None:
    _dev(G, "G"); _dev(U, "U"); _dev(M, "M")
    assert G.shape == U.shape == M.shape
    _check(lib().gptq_swiglu(_ptr(G), _ptr(U), G.numel(), _ptr(M), _stream(stream)), "gptq_swiglu")


def gptq_layer_error_workspace_size(d_out: int, d_in: int) -> int:
    return int(lib().gptq_layer_error_workspace_size(d_out, d_in))


def gptq_layer_error(H: torch.Tensor, W: torch.Tensor, Q: torch.Tensor,
                     ws: Optional[torch.Tensor] = None, stream=None) -> float:
    _dev(H, "H"); _dev(W, "W"); _dev(Q, "Q")
    d_out, d_in = W.shape
    ws = _ws(gptq_layer_error_workspace_size(d_out, d_in), ws, W.device, stream)
    out = ctypes.c_double(0.0)
    _check(lib().gptq_layer_error(_ptr(H), _ptr(W), _DTYPE[W.dtype], _ptr(Q), d_out, d_in,
                                  ctypes.byref(out), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream)), "gptq_layer_error")
    return float(out.value)


def gptq_status_string(status: int) -> str:
    return lib().gptq_status_string(status).decode()


def gptq_abi_version() -> int:
    return int(lib().gptq_abi_version())
