"""Pins of the fp64 log-sum-exp and backward oracle (CPU only), and mutants.

The backward oracle (oracle/backward.py) writes the chain rule through
softmax(scale Q K^T [+ mask]) V out by hand. Nothing below reuses that
derivation: the gradients are checked against torch's autograd in float64,
central finite differences of the (separately pinned) forward oracle, a
closed form for one query and two keys, and invariants that follow from the
softmax itself (adding a constant to a row of scores changes nothing; rows
of P sum to 1). Source: the codelab "Accelerate attention on GPU with cuDNN
and TransformerEngine", §1 (the formula and the role of the scale for the
softmax gradients), §7 (mask), §9 (head grouping), §10 (FP8 for training).

Each mutant plants one plausible mistake in a step of the backward oracle and
must fail at least one pin.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as bwd


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


MODES = (False, True, "bottom_right")


def _case(seed, B, Sq, Skv, Hq, Hkv, D):
    return (_rand(seed, B, Sq, Hq, D), _rand(seed + 1, B, Skv, Hkv, D), _rand(seed + 2, B, Skv, Hkv, D),
            _rand(seed + 3, B, Sq, Hq, D))


def _torch_mask(causal, Sq, Skv):
    """Boolean keep-mask from torch.tril: query i keeps keys j <= i + shift."""
    if causal is False:
        return None
    shift = 0 if causal is True else Skv - Sq
    return torch.ones(Sq, Skv, dtype=torch.bool).tril(diagonal=shift)


def pin_bwd_torch_autograd(backward, lse_fn):
    """torch autograd through its float64 CPU scaled_dot_product_attention,
    with K/V repeated over the query heads of each group (autograd then sums
    the group's contributions itself)."""
    for (B, Sq, Skv, Hq, Hkv, D) in [(2, 19, 19, 4, 2, 8), (1, 7, 23, 4, 1, 16), (2, 23, 9, 2, 2, 5)]:
        q, k, v, do = _case(100 + Sq, B, Sq, Skv, Hq, Hkv, D)
        for causal in MODES:
            if causal == "bottom_right" and Sq > Skv:
                continue
            tq = torch.from_numpy(q).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
            tk = torch.from_numpy(k).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
            tv = torch.from_numpy(v).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
            rk = tk.repeat_interleave(Hq // Hkv, dim=1)
            rv = tv.repeat_interleave(Hq // Hkv, dim=1)
            o = torch.nn.functional.scaled_dot_product_attention(tq, rk, rv, attn_mask=_torch_mask(causal, Sq, Skv),
                                                                 scale=0.41)
            o.backward(torch.from_numpy(do).permute(0, 2, 1, 3))
            dq, dk, dv = backward(q, k, v, do, scale=0.41, causal=causal)
            for got, t in ((dq, tq), (dk, tk), (dv, tv)):
                np.testing.assert_allclose(got, t.grad.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-11)


def pin_bwd_finite_differences(backward, lse_fn):
    """Every gradient element equals the central difference of the pinned
    forward oracle's loss sum(dout * sdpa) (step 1e-5, error O(1e-10))."""
    q, k, v, do = _case(7, 1, 3, 4, 2, 1, 3)
    h = 1e-5
    for causal in MODES:
        grads = backward(q, k, v, do, scale=0.8, causal=causal)
        for which, g in enumerate(grads):
            x = [q, k, v]
            for idx in np.ndindex(x[which].shape):
                xp = [a.copy() for a in x]
                xm = [a.copy() for a in x]
                xp[which][idx] += h
                xm[which][idx] -= h
                fp = np.sum(do * oracle.sdpa(*xp, scale=0.8, causal=causal))
                fm = np.sum(do * oracle.sdpa(*xm, scale=0.8, causal=causal))
                assert abs((fp - fm) / (2 * h) - g[idx]) < 1e-8, (causal, which, idx)


def pin_bwd_two_keys_closed_form(backward, lse_fn):
    """One query and two keys (D = 1): with s_j = c q k_j and p = sigmoid(s_1 - s_2),
    o = p v_1 + (1 - p) v_2, so by hand dq = g (v1 - v2) p (1 - p) c (k1 - k2),
    dk1 = -dk2 = g (v1 - v2) p (1 - p) c q, dv1 = g p, dv2 = g (1 - p), and
    lse = log(e^{s_1} + e^{s_2})."""
    qv, k1, k2, v1, v2, g, c = 0.7, 1.3, -0.4, 2.0, -1.5, 0.9, 0.6
    p = 1.0 / (1.0 + math.exp(-(c * qv * k1 - c * qv * k2)))
    q = np.array([qv]).reshape(1, 1, 1, 1)
    k = np.array([k1, k2]).reshape(1, 2, 1, 1)
    v = np.array([v1, v2]).reshape(1, 2, 1, 1)
    do = np.array([g]).reshape(1, 1, 1, 1)
    dq, dk, dv = backward(q, k, v, do, scale=c, causal=False)
    jac = g * (v1 - v2) * p * (1 - p) * c
    assert abs(dq[0, 0, 0, 0] - jac * (k1 - k2)) < 1e-14
    assert abs(dk[0, 0, 0, 0] - jac * qv) < 1e-14 and abs(dk[0, 1, 0, 0] + jac * qv) < 1e-14
    assert abs(dv[0, 0, 0, 0] - g * p) < 1e-14 and abs(dv[0, 1, 0, 0] - g * (1 - p)) < 1e-14
    lse = lse_fn(q, k, scale=c, causal=False)
    assert abs(lse[0, 0, 0] - math.log(math.exp(c * qv * k1) + math.exp(c * qv * k2))) < 1e-14


def pin_bwd_row_shift_invariance(backward, lse_fn):
    """Adding a constant to a row of scores changes no weight, so each row of
    dS sums to 0 and the key gradients of every KV head sum to zero over the
    keys; rows of P sum to 1, so the value gradients sum to the sum of dout
    over the queries of the group."""
    B, Sq, Skv, Hq, Hkv, D = 2, 13, 17, 6, 2, 4
    q, k, v, do = _case(21, B, Sq, Skv, Hq, Hkv, D)
    for causal in MODES:
        dq, dk, dv = backward(q, k, v, do, scale=0.5, causal=causal)
        np.testing.assert_allclose(dk.sum(axis=1), 0.0, rtol=0, atol=1e-12)
        G = Hq // Hkv
        want = do.sum(axis=1).reshape(B, Hkv, G, D).sum(axis=2)
        np.testing.assert_allclose(dv.sum(axis=1), want, rtol=0, atol=1e-12)


def pin_bwd_key_translation(backward, lse_fn):
    """Moving every key by one vector u adds scale <q_i, u> to each score of
    row i, which the softmax ignores: the output, dQ, dK and dV are
    unchanged, and lse moves by exactly scale <q_i, u>."""
    q, k, v, do = _case(31, 1, 9, 9, 2, 1, 5)
    u = _rand(35, 5)
    for causal in MODES:
        a = backward(q, k, v, do, scale=0.7, causal=causal)
        b = backward(q, k + u, v, do, scale=0.7, causal=causal)
        for x, y in zip(a, b):
            np.testing.assert_allclose(x, y, rtol=0, atol=1e-11)
        la = lse_fn(q, k, scale=0.7, causal=causal)
        lb = lse_fn(q, k + u, scale=0.7, causal=causal)
        np.testing.assert_allclose(lb - la, 0.7 * np.einsum("bshd,d->bhs", q, u), rtol=0, atol=1e-12)


def pin_bwd_scale_zero(backward, lse_fn):
    """scale = 0: uniform weights over the visible keys, so dQ = dK = 0,
    dV_j = sum over visible rows i of dout_i / n_i, and lse_i = log n_i with
    n_i the number of keys row i sees (§7: i + 1 for the top-left mask)."""
    Sq, Skv = 6, 6
    q, k, v, do = _case(41, 1, Sq, Skv, 1, 1, 3)
    for causal in (False, True):
        dq, dk, dv = backward(q, k, v, do, scale=0.0, causal=causal)
        assert np.all(dq == 0) and np.all(dk == 0)
        n = np.arange(1, Sq + 1) if causal else np.full(Sq, Skv)
        for j in range(Skv):
            rows = [i for i in range(Sq) if (not causal or j <= i)]
            want = sum(do[0, i, 0] / n[i] for i in rows)
            np.testing.assert_allclose(dv[0, j, 0], want, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse_fn(q, k, scale=0.0, causal=causal)[0, 0], np.log(n), rtol=0, atol=1e-14)


def pin_bwd_single_key_and_first_row(backward, lse_fn):
    """A row that sees one key has weight exactly 1 there: no gradient flows
    to its query, lse = scale <q, k_0>. With one key in all, dK = 0 and dV
    sums dout. Under the top-left mask row 0 sees only key 0 (§7), and keys
    after the last query's position get no gradient at all."""
    q, k, v, do = _case(51, 2, 5, 1, 2, 2, 4)
    dq, dk, dv = backward(q, k, v, do, scale=0.9, causal=False)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_allclose(dv[:, 0], do.sum(axis=1), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse_fn(q, k, scale=0.9, causal=False),
                               0.9 * np.einsum("bshd,bhd->bhs", q, k[:, 0]), rtol=0, atol=1e-13)
    q, k, v, do = _case(55, 1, 4, 9, 2, 1, 4)
    dq, dk, dv = backward(q, k, v, do, scale=0.9, causal=True)
    assert np.all(dq[:, 0] == 0)
    assert np.all(dk[:, 4:] == 0) and np.all(dv[:, 4:] == 0)


def pin_bwd_gqa_is_summed_mha(backward, lse_fn):
    """§9: GQA is MHA with each KV head repeated over its group, so its dQ is
    that MHA's dQ and its dK, dV are that MHA's summed over the group."""
    B, S, Hq, Hkv, D = 1, 11, 6, 2, 4
    q, k, v, do = _case(61, B, S, S, Hq, Hkv, D)
    G = Hq // Hkv
    for causal in MODES:
        dq, dk, dv = backward(q, k, v, do, scale=0.6, causal=causal)
        mq, mk, mv = backward(q, np.repeat(k, G, axis=2), np.repeat(v, G, axis=2), do, scale=0.6, causal=causal)
        np.testing.assert_allclose(dq, mq, rtol=0, atol=1e-13)
        np.testing.assert_allclose(dk, mk.reshape(B, S, Hkv, G, D).sum(axis=3), rtol=0, atol=1e-13)
        np.testing.assert_allclose(dv, mv.reshape(B, S, Hkv, G, D).sum(axis=3), rtol=0, atol=1e-13)


def pin_lse_rebuilds_forward(backward, lse_fn):
    """P = exp(S - lse) has rows summing to 1 and P V equals the pinned
    forward oracle, for every mask and grouping."""
    B, Sq, Skv, Hq, Hkv, D = 2, 9, 14, 4, 2, 6
    q, k, v, _ = _case(71, B, Sq, Skv, Hq, Hkv, D)
    for causal in MODES:
        lse = lse_fn(q, k, scale=0.45, causal=causal)
        out = oracle.sdpa(q, k, v, scale=0.45, causal=causal)
        shift = 0 if causal is True else Skv - Sq
        keep = np.arange(Skv)[None, :] <= np.arange(Sq)[:, None] + shift
        for b in range(B):
            for h in range(Hq):
                g = h // (Hq // Hkv)
                s = 0.45 * q[b, :, h] @ k[b, :, g].T
                p = np.exp(s - lse[b, h][:, None])
                if causal is not False:
                    p = np.where(keep, p, 0.0)
                np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-13)
                np.testing.assert_allclose(p @ v[b, :, g], out[b, :, h], rtol=0, atol=1e-12)


BWD_PINS = [pin_bwd_torch_autograd, pin_bwd_finite_differences, pin_bwd_two_keys_closed_form,
            pin_bwd_row_shift_invariance, pin_bwd_key_translation, pin_bwd_scale_zero,
            pin_bwd_single_key_and_first_row, pin_bwd_gqa_is_summed_mha, pin_lse_rebuilds_forward]


@pytest.mark.parametrize("pin", BWD_PINS, ids=lambda p: p.__name__)
def test_backward_oracle_pin(pin):
    pin(oracle.sdpa_backward, oracle.sdpa_lse)


def test_backward_shapes_and_errors():
    q, k, v, do = _case(81, 2, 0, 5, 4, 2, 8)
    dq, dk, dv = oracle.sdpa_backward(q, k, v, do, scale=1.0, causal=True)
    assert dq.shape == q.shape and np.all(dk == 0) and np.all(dv == 0)
    with pytest.raises(ValueError):
        oracle.sdpa_backward(q, k, v, do[:, :, :2], scale=1.0, causal=False)
    with pytest.raises(ValueError):
        oracle.sdpa_lse(_rand(1, 1, 6, 2, 8), _rand(2, 1, 5, 2, 8), scale=1.0, causal="bottom_right")


# ---- mutants: one plausible mistake each, planted on the CPU --------------------------------

_orig = {name: getattr(bwd, name) for name in ("_softmax_grad", "_head_grads", "_accumulate", "_row_lse")}


def _grad_no_rowsum(p, dp):
    return p * dp


def _grad_rowsum_sign(p, dp):
    return p * (dp + np.sum(p * dp, axis=1, keepdims=True))


def _grad_column_sum(p, dp):
    return p * (dp - np.sum(p * dp, axis=0, keepdims=True))


def _grads_dq_no_scale(p, ds, qh, kh, doh, scale):
    dq, dk, dv = _orig["_head_grads"](p, ds, qh, kh, doh, scale)
    return ds @ kh, dk, dv


def _grads_dk_uses_dq_side(p, ds, qh, kh, doh, scale):
    dq, dk, dv = _orig["_head_grads"](p, ds, qh, kh, doh, scale)
    return dq, scale * (ds @ qh) if ds.shape[0] == ds.shape[1] else dk * 0.5, dv


def _grads_dv_untransposed(p, ds, qh, kh, doh, scale):
    dq, dk, dv = _orig["_head_grads"](p, ds, qh, kh, doh, scale)
    return dq, dk, (p @ doh) if p.shape[0] == p.shape[1] else dv * 2.0


def _grads_dk_sign(p, ds, qh, kh, doh, scale):
    dq, dk, dv = _orig["_head_grads"](p, ds, qh, kh, doh, scale)
    return dq, -dk, dv


def _accumulate_overwrites(acc, b, g, part):
    acc[b, :, g, :] = part


def _lse_no_max(s):
    m = np.max(s, axis=1)
    return np.log(np.sum(np.exp(s - m[:, None]), axis=1))


def _lse_log2(s):
    return _orig["_row_lse"](s) / math.log(2.0)


MUTANTS = {
    "softmax_grad_no_rowsum": ("_softmax_grad", _grad_no_rowsum),
    "softmax_grad_rowsum_sign": ("_softmax_grad", _grad_rowsum_sign),
    "softmax_grad_column_sum": ("_softmax_grad", _grad_column_sum),
    "dq_missing_scale": ("_head_grads", _grads_dq_no_scale),
    "dk_untransposed": ("_head_grads", _grads_dk_uses_dq_side),
    "dv_untransposed": ("_head_grads", _grads_dv_untransposed),
    "dk_sign": ("_head_grads", _grads_dk_sign),
    "group_overwrites": ("_accumulate", _accumulate_overwrites),
    "lse_drops_max": ("_row_lse", _lse_no_max),
    "lse_log2": ("_row_lse", _lse_log2),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(bwd, attr, fn)
    failed = []
    for pin in BWD_PINS:
        try:
            pin(oracle.sdpa_backward, oracle.sdpa_lse)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
