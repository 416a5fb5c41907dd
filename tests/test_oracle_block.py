"""Pins of the block oracle (oracle/block_ref.py): each piece of the Llama
decoder layer against closed forms, invariants or brute force, and the
layer-sequential pipeline against the plain block forward."""
from __future__ import annotations

import math
from types import SimpleNamespace

import numpy as np
import pytest

from oracle import block_ref as B
from oracle import gptq_ref as g


def test_rmsnorm_closed_form():
    x = np.full((2, 8), 3.0)
    x[1] *= -1
    y = B.rmsnorm(x)
    assert np.allclose(y, np.sign(x) * 3.0 / math.sqrt(9.0 + B.EPS), rtol=1e-15)
    gam = np.arange(1, 9, dtype=float)
    assert np.allclose(B.rmsnorm(x, gam), y * gam, rtol=1e-15)


def test_rope_identity_norms_and_relative_positions():
    rng = np.random.default_rng(0)
    heads, hd, S = 2, 8, 16
    x = rng.standard_normal((S, heads * hd))
    r = B.rope(x, heads, S)
    assert np.allclose(r[0], x[0])                           # position 0: no rotation
    for h in range(heads):                                    # each (i, i + hd/2) pair keeps its norm
        a, b = x[:, h * hd:h * hd + hd // 2], x[:, h * hd + hd // 2:(h + 1) * hd]
        ra, rb = r[:, h * hd:h * hd + hd // 2], r[:, h * hd + hd // 2:(h + 1) * hd]
        assert np.allclose(a * a + b * b, ra * ra + rb * rb)
    q, k = rng.standard_normal(heads * hd), rng.standard_normal(heads * hd)

    def dot_at(m, n):
        X = np.zeros((S, heads * hd))
        Y = np.zeros((S, heads * hd))
        X[m], Y[n] = q, k
        return float(B.rope(X, heads, S)[m] @ B.rope(Y, heads, S)[n])
    assert dot_at(5, 2) == pytest.approx(dot_at(11, 8), rel=1e-12)
    assert dot_at(5, 2) != pytest.approx(dot_at(5, 3), rel=1e-6)
    # a 2-element head rotated by angle p (theta_0 = 1)
    one = B.rope(np.tile([[1.0, 0.0]], (4, 1)), 1, 4)
    assert np.allclose(one, np.stack([np.cos(np.arange(4)), np.sin(np.arange(4))], axis=1))


def test_causal_attention_brute_force_and_special_cases():
    rng = np.random.default_rng(1)
    heads, hd, S = 2, 4, 3
    q, k, v = (rng.standard_normal((2 * S, heads * hd)) for _ in range(3))
    out = B.causal_attention(q, k, v, heads, S)
    for s0 in (0, S):
        for h in range(heads):
            c = slice(h * hd, (h + 1) * hd)
            for i in range(S):
                w = [math.exp(float(q[s0 + i, c] @ k[s0 + j, c]) / math.sqrt(hd)) for j in range(i + 1)]
                ref = sum(w[j] * v[s0 + j, c] for j in range(i + 1)) / sum(w)
                assert np.allclose(out[s0 + i, c], ref, rtol=1e-12)
    assert np.allclose(out[[0, S]], v[[0, S]])                # first position attends to itself
    zero = B.causal_attention(np.zeros_like(q), k, v, heads, S)
    assert np.allclose(zero[2], v[:3].mean(axis=0))            # uniform weights: prefix mean


def test_silu_values():
    assert B.silu(np.array([0.0]))[0] == 0.0
    assert B.silu(np.array([1.0]))[0] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert B.silu(np.array([-40.0]))[0] == pytest.approx(0.0, abs=1e-15)


def _block(rng, shape):
    d, f = shape.d, shape.f
    W = {n: rng.standard_normal((d, d)) * 0.05 for n in ("q", "k", "v", "o")}
    W["gate"], W["up"] = rng.standard_normal((f, d)) * 0.05, rng.standard_normal((f, d)) * 0.05
    W["down"] = rng.standard_normal((d, f)) * 0.05
    return B.BlockWeights(W)


def test_sequential_with_identity_quantizer_is_the_plain_forward():
    rng = np.random.default_rng(2)
    shape = B.BlockShape(d=16, n_heads=2, f=24, seq_len=8)
    bw = _block(rng, shape)
    x = rng.standard_normal((3 * shape.seq_len, shape.d))
    ident = lambda W, H: SimpleNamespace(Q=np.asarray(W, np.float64))
    res = B.sequential_gptq(x, bw, shape, ident)
    ref = B.block_forward(x, bw, shape)
    for key in ("x1", "attn", "h", "x2", "m", "y"):
        assert np.allclose(res.acts[key], ref[key], rtol=1e-13, atol=1e-14), key
    assert res.H["q"] is res.H["k"] is res.H["v"] and res.H["gate"] is res.H["up"]
    assert np.allclose(res.H["down"], 2.0 * ref["m"].T @ ref["m"])
    assert np.allclose(res.H["o"], 2.0 * ref["attn"].T @ ref["attn"])


def test_sequential_propagates_quantized_outputs():
    """The o projection's calibration input comes from the quantized q/k/v:
    it differs from the unquantized block's, and equals the attention of the
    dequantized weights."""
    rng = np.random.default_rng(3)
    shape = B.BlockShape(d=32, n_heads=2, f=48, seq_len=16)
    bw = _block(rng, shape)
    x = rng.standard_normal((4 * shape.seq_len, shape.d))
    res = B.sequential_gptq(x, bw, shape, B.gptq_quantizer(bits=3, group_size=16))
    plain = B.block_forward(x, bw, shape)
    assert not np.allclose(res.acts["attn"], plain["attn"], rtol=1e-6)
    Wq = {n: res.quant[n].Q for n in B.SUBLAYERS}
    deq = B.block_forward(x, B.BlockWeights(Wq), shape)
    for key in ("attn", "x2", "m", "y"):
        assert np.allclose(res.acts[key], deq[key], rtol=1e-12, atol=1e-13), key
    for n in B.SUBLAYERS:                                     # each sub-layer is GPTQ on its own H
        r = g.gptq(bw.W[n], res.H[n], bits=3, group_size=16)
        assert np.array_equal(r.codes, res.quant[n].codes)
