"""Plant plausible mistakes in the oracle (on the CPU) and check the pins catch each.

Each mutant replaces one internal step of ``oracle.attention`` (score, mask,
softmax, head grouping) with a wrong variant via monkeypatch. A mutant must
fail at least one pin other than the scalar brute-force comparison, so that
the invariants and closed forms alone would expose it.
"""

import numpy as np
import pytest

import oracle
from oracle import attention as sdpa_mod
from tests import oracle_pins


def _scores_no_scale(qh, kh, scale, causal, row0):
    return _orig_scores(qh, kh, 1.0, causal, row0)


def _scores_negated(qh, kh, scale, causal, row0):
    return _orig_scores(qh, kh, -scale, causal, row0)


def _scores_mask_excludes_diag(qh, kh, scale, causal, row0):
    s = scale * (qh @ kh.T)
    if causal:
        i = np.arange(row0, row0 + qh.shape[0])[:, None]
        j = np.arange(kh.shape[0])[None, :]
        s = np.where(j >= i, -np.inf, s)
    return s


def _scores_mask_upper(qh, kh, scale, causal, row0):
    s = scale * (qh @ kh.T)
    if causal:
        i = np.arange(row0, row0 + qh.shape[0])[:, None]
        j = np.arange(kh.shape[0])[None, :]
        s = np.where(j < i, -np.inf, s)
    return s


def _scores_transposed(qh, kh, scale, causal, row0):
    return _orig_scores(kh, qh, scale, causal, row0).T


def _softmax_wrong_axis(s):
    m = np.max(s, axis=0, keepdims=True)
    w = np.exp(s - m)
    return w / np.sum(w, axis=0, keepdims=True)


def _softmax_unnormalised(s):
    return np.exp(s - np.max(s, axis=1, keepdims=True))


def _softmax_no_exp(s):
    w = np.where(np.isinf(s), 0.0, s - np.min(np.where(np.isinf(s), np.inf, s), axis=1, keepdims=True))
    return w / np.sum(w, axis=1, keepdims=True)


def _kv_head_modulo(hq, Hq, Hkv):
    return hq % Hkv


_orig_shift = sdpa_mod._query_shift


def _shift_bottom_right_as_top_left(causal, Sq, Skv):
    r = _orig_shift(causal, Sq, Skv)
    return 0 if r is not None else None


def _shift_bottom_right_off_by_one(causal, Sq, Skv):
    r = _orig_shift(causal, Sq, Skv)
    return r + 1 if (r is not None and causal in (2, "bottom_right")) else r


_orig_scores = sdpa_mod._scores

MUTANTS = {
    "score_without_scale": ("_scores", _scores_no_scale),
    "score_sign_flipped": ("_scores", _scores_negated),
    "mask_hides_diagonal": ("_scores", _scores_mask_excludes_diag),
    "mask_upper_triangle": ("_scores", _scores_mask_upper),
    "scores_transposed": ("_scores", _scores_transposed),
    "softmax_over_queries": ("_softmax_rows", _softmax_wrong_axis),
    "softmax_not_normalised": ("_softmax_rows", _softmax_unnormalised),
    "softmax_without_exp": ("_softmax_rows", _softmax_no_exp),
    "kv_head_modulo": ("kv_head_of", _kv_head_modulo),
    "bottom_right_as_top_left": ("_query_shift", _shift_bottom_right_as_top_left),
    "bottom_right_off_by_one": ("_query_shift", _shift_bottom_right_off_by_one),
}

PINS = [p for p in oracle_pins.ALL_PINS if p is not oracle_pins.pin_brute_force]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(sdpa_mod, attr, fn)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(oracle.sdpa)
        except Exception:
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
