"""Pins of the AWQ oracle (oracle/awq_ref.py) against what the pages and the
mathematics fix, independent of the oracle's own formulas:

* the statistic against element loops and a constant input;
* the salient set on hand-worked examples (ties to the lower index);
* no scaling (factor 1) is exactly the round-to-nearest baseline of gptq_ref;
* the inference identity of the pages' step 4: (x / s) Q(W s)^T = x Qhat^T;
* the score equals the layer's output error ||X (W - Qhat)^T||^2 computed
  from the activations themselves when the channels are orthogonal, and the
  search picks the candidate with the smallest such error (brute force);
* the opposite scaling direction of the ms-swift review (non-salient channels
  scaled down) gives the same effective weights for a factor of 2;
* on inputs with a few dominant channels the searched factor beats
  round-to-nearest on the true output error;
* planted mistakes in the oracle each fail one of these pins.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import awq_ref as a
from oracle import gptq_ref as g


def _orthogonal_acts(rng, n, d, amp):
    """X [n x d] with X^T X = diag(amp^2) (up to rounding): orthonormal
    columns times per-channel amplitudes."""
    Qm, _ = np.linalg.qr(rng.standard_normal((n, d)))
    return Qm * amp[None, :]


def test_sumsq_element_loops_and_constant():
    rng = np.random.default_rng(0)
    X = rng.standard_normal((7, 5)).astype(np.float32)
    ref = [0.0] * 5
    for t in range(7):
        for j in range(5):
            ref[j] += float(X[t, j]) * float(X[t, j])
    assert np.allclose(a.act_sumsq([X[:3], X[3:]], 5), ref, rtol=1e-15, atol=0)
    C = np.full((11, 4), 0.5)
    assert np.array_equal(a.act_sumsq([C], 4), np.full(4, 11 * 0.25))


def test_salient_hand_examples():
    v = np.array([3.0, 1.0, 3.0, 2.0, 0.0])
    assert a.n_salient(0.4, 5) == 2 and a.n_salient(0.6, 5) == 3 and a.n_salient(0.05, 4096) == 205
    assert a.salient_mask(v, 0.4).tolist() == [True, False, True, False, False]
    assert a.salient_mask(v, 0.6).tolist() == [True, False, True, True, False]
    assert a.salient_mask(np.ones(4), 0.5).tolist() == [True, True, False, False]
    assert not a.salient_mask(v, 0.0).any() and a.salient_mask(v, 1.0).all()


@pytest.mark.parametrize("G", [8, 32, -1])
def test_factor_one_is_rtn(G):
    rng = np.random.default_rng(1)
    W = (rng.standard_normal((6, 64)) * 0.02).astype(np.float16).astype(np.float64)
    q = a.quantize_scaled(W, np.ones(64, np.float32), bits=4, group_size=G)
    # AWQ's grid is taken on the fp32 products W*s, so with s = 1 it is the
    # round-to-nearest grid with its decisions in float32
    codes, Q = g.rtn(W, bits=4, group_size=G, decision="f32")
    assert np.array_equal(q.codes, codes) and np.array_equal(q.Qhat, Q)


def test_inference_identity():
    rng = np.random.default_rng(2)
    W = rng.standard_normal((5, 48)) * 0.02
    s = a.channel_scales(rng.random(48) < 0.2, 2.5)
    q = a.quantize_scaled(W, s, bits=4, group_size=16)
    x = rng.standard_normal((3, 48))
    G = 16
    Qs = np.repeat(q.scales.astype(np.float64), G, axis=1) * (q.codes - np.repeat(q.zeros, G, axis=1))
    lhs = (x / s.astype(np.float64)[None, :]) @ Qs.T
    assert np.allclose(lhs, x @ q.Qhat.T, rtol=1e-12, atol=1e-15)


def test_score_is_output_error_for_orthogonal_channels():
    rng = np.random.default_rng(3)
    d = 32
    amp = np.exp(rng.normal(0, 1.0, d))
    X = _orthogonal_acts(rng, 64, d, amp)
    W = rng.standard_normal((4, d)) * 0.02
    s = a.channel_scales(a.salient_mask(amp ** 2, 0.25), 1.75)
    q = a.quantize_scaled(W, s, bits=3, group_size=8)
    direct = float(np.sum((X @ (W - q.Qhat).T) ** 2))
    assert a.weighted_error(W, q.Qhat, a.act_sumsq([X], d)) == pytest.approx(direct, rel=1e-10)


def test_search_brute_force_tiny():
    rng = np.random.default_rng(4)
    d = 16
    amp = np.ones(d)
    amp[[3, 11]] = 20.0
    X = _orthogonal_acts(rng, 40, d, amp)
    W = rng.standard_normal((3, d)) * 0.02
    grid = [1.0, 1.5, 2.0, 3.0]
    res = a.awq(W, a.act_sumsq([X], d), bits=3, group_size=8, top_frac=2 / 16, grid=grid)
    assert res.s[[3, 11]].tolist() == [res.sigma] * 2 and np.all(np.delete(res.s, [3, 11]) == 1.0)
    errs = []
    for sg in grid:
        s = np.ones(d, np.float32)
        s[[3, 11]] = sg
        Qh = a.quantize_scaled(W, s, bits=3, group_size=8).Qhat
        errs.append(float(np.sum((X @ (W - Qh).T) ** 2)))
    assert res.best == int(np.argmin(errs))
    assert np.allclose(res.scores, errs, rtol=1e-9)


def test_opposite_direction_same_weights():
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((4, 64)) * 0.02).astype(np.float16).astype(np.float64)
    mask = rng.random(64) < 0.1
    up = a.channel_scales(mask, 2.0)
    down = np.where(mask, np.float32(1.0), np.float32(0.5)).astype(np.float32)
    qu = a.quantize_scaled(W, up, bits=4, group_size=16)
    qd = a.quantize_scaled(W, down, bits=4, group_size=16)
    assert np.array_equal(qu.codes, qd.codes) and np.array_equal(qu.Qhat, qd.Qhat)


def test_awq_beats_rtn_with_dominant_channels():
    rng = np.random.default_rng(6)
    d, n = 256, 2048
    X = rng.standard_normal((n, d))
    hot = rng.choice(d, 8, replace=False)
    X[:, hot] *= 30.0
    W = rng.standard_normal((64, d)) * 0.02
    res = a.awq(W, a.act_sumsq([X], d), bits=4, group_size=128, top_frac=8 / 256)
    assert set(np.flatnonzero(res.s != 1.0)) == set(hot) and res.sigma > 1.0
    _, Qr = g.rtn(W, bits=4, group_size=128)
    err = lambda Q: float(np.sum((X @ (W - Q).T) ** 2))
    assert err(res.quant.Qhat) < 0.9 * err(Qr)
    assert res.scores[res.best] <= res.scores[0]      # the grid holds factor 1


def _pins_fail():
    failed = 0
    for fn, args in ((test_salient_hand_examples, ()), (test_inference_identity, ()),
                     (test_score_is_output_error_for_orthogonal_channels, ()),
                     (test_search_brute_force_tiny, ()), (test_awq_beats_rtn_with_dominant_channels, ())):
        try:
            fn(*args)
        except AssertionError:
            failed += 1
    return failed


@pytest.mark.parametrize("mutation", ["no_divide", "smallest_channels", "unweighted_score",
                                      "worst_candidate"])
def test_planted_mistakes_fail_a_pin(mutation, monkeypatch):
    if mutation == "no_divide":
        orig = a.quantize_scaled

        def bad(W, s, **kw):
            q = orig(W, s, **kw)
            q.Qhat = q.Qhat * np.asarray(s, np.float64)[None, :]
            return q
        monkeypatch.setattr(a, "quantize_scaled", bad)
    elif mutation == "smallest_channels":
        monkeypatch.setattr(a, "salient_mask",
                            lambda v, f: np.isin(np.arange(len(v)),
                                                 np.argsort(np.asarray(v), kind="stable")[:a.n_salient(f, len(v))]))
    elif mutation == "unweighted_score":
        monkeypatch.setattr(a, "weighted_error",
                            lambda W, Q, v: float(np.sum((np.asarray(W, np.float64) - Q) ** 2)))
    elif mutation == "worst_candidate":
        orig_awq = a.awq

        def bad_awq(W, v, **kw):
            r = orig_awq(W, v, **kw)
            r.best = int(np.argmax(r.scores))
            r.sigma = float(np.asarray(kw.get("grid", a.DEFAULT_GRID), np.float32)[r.best])
            r.s = np.where(r.s != 1.0, np.float32(r.sigma), np.float32(1.0)).astype(np.float32)
            r.quant = a.quantize_scaled(W, r.s, bits=kw.get("bits", 4), group_size=kw.get("group_size", 128))
            return r
        monkeypatch.setattr(a, "awq", bad_awq)
    assert _pins_fail() >= 1
