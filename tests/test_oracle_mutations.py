"""Plant a plausible mistake in the oracle (on the CPU) and check that at least
one pin fails, so that the pins are known to be sensitive to it."""
import numpy as np
import pytest

from oracle import gptq_ref as o
import test_oracle_pins as pins


def _orig(name):
    return getattr(o, name)


def _mut_factor_lower(Hd):            # transposed factor: the lower triangle
    return _orig_hinv(Hd).T.copy()


def _mut_factor_of_h(Hd):             # factor of H instead of H^-1
    return np.linalg.cholesky(Hd).T.copy()


def _mut_factor_unit_diag(Hd):        # drop the division by the pivot U_jj
    U = _orig_hinv(Hd).copy()
    np.fill_diagonal(U, 1.0)
    return U


def _mut_zero_clamped(seg, maxq, decision="f32"):
    s, z = _orig_gp(seg, maxq, decision)
    return s, np.clip(z, 0, maxq)


def _mut_round_up(w, scale, zero, maxq, decision="f32"):
    t = np.asarray(w, np.float64) / np.asarray(scale, np.float64)
    c = np.clip(np.ceil(t) + zero, 0, maxq)
    return c.astype(np.int64), np.asarray(scale, np.float64) * (c - zero)


def _mut_no_damp(H, damp_percent):
    return H.copy(), 0.0


def _mut_ascending(H, desc_act):
    d = H.shape[0]
    return np.argsort(np.diag(H), kind="stable") if desc_act else np.arange(d)


def _mut_hessian_no_two(chunks, d_in):
    return 0.5 * _orig_hess(chunks, d_in)


_orig_hinv = o.hinv_factor
_orig_gp = o.group_params
_orig_hess = o.hessian

MUTATIONS = [
    ("hinv_factor", _mut_factor_lower, [pins.test_gptq_equals_sequential_least_squares]),
    ("hinv_factor", _mut_factor_of_h, [pins.test_factor_2x2_closed_form]),
    ("hinv_factor", _mut_factor_unit_diag, [pins.test_gptq_equals_sequential_least_squares,
                                             pins.test_error_sum_equals_damped_quadratic_form]),
    ("group_params", _mut_zero_clamped, [pins.test_minmax_worked_example_from_page]),
    ("quantize", _mut_round_up, [pins.test_minmax_worked_example_from_page]),
    ("damp", _mut_no_damp, [pins.test_damp_closed_form]),
    ("act_order", _mut_ascending, [pins.test_act_order_descending_stable]),
    ("hessian", _mut_hessian_no_two, [pins.test_hessian_closed_form_orthogonal_columns]),
]

_ARGS = {
    pins.test_gptq_equals_sequential_least_squares: dict(G=4, B=4),
    pins.test_minmax_worked_example_from_page: dict(decision="f32"),
}


@pytest.mark.parametrize("name,mut,detectors", MUTATIONS,
                         ids=[f"{m[0]}:{m[1].__name__}" for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, mut, detectors):
    monkeypatch.setattr(o, name, mut)
    caught = False
    for det in detectors:
        try:
            det(**_ARGS.get(det, {}))
        except (AssertionError, o.NotPositiveDefinite, np.linalg.LinAlgError):
            caught = True
    assert caught, f"no pin detected the mutation of {name}"
