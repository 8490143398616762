"""Pins that tie the fp64 oracle to facts that do not come from the oracle.

Each pin takes the SDPA function under test (normally ``oracle.sdpa``) and
raises AssertionError when it disagrees with a closed form, an invariant of
the definition, hand-derived values, brute force, or an independent library
routine. ``tests/test_oracle.py`` runs them on the oracle, and
``tests/test_oracle_mutants.py`` plants plausible mistakes in the oracle to
show that each mistake is caught.

Source: the codelab "Accelerate attention on GPU with cuDNN and
TransformerEngine" — §1 (formula, weights summing to 1, output shaped like
Q), §7 (causal mask: first position sees only itself, last sees all), §9
(MHA / GQA / MQA broadcast, output shape unchanged; the key-value-cache
inference use that the bottom-right causal alignment serves).
"""

import json
import math
import os

import numpy as np
import torch

import oracle
from oracle import attention as sdpa_mod

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def pin_golden(fn):
    """Hand-derived closed-form cases (tests/golden/hand_worked.json)."""
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        q, k, v, want = (np.array(c[x], dtype=np.float64) for x in ("q", "k", "v", "out"))
        got = fn(q, k, v, scale=c["scale"], causal=c["causal"])
        assert got.shape == want.shape, c["name"]
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12, err_msg=c["name"])


def pin_weights_sum_to_one(fn=None):
    """§1 step 2: the weights of each row sum to 1; causal weights above the
    diagonal are exactly 0 (§7)."""
    q, k = _rand(1, 2, 37, 4, 16), _rand(2, 2, 37, 2, 16)
    for causal in (False, True):
        for hq in range(4):
            w = oracle.attention_weights(q, k, scale=0.3, causal=causal, b=1, hq=hq)
            assert np.max(np.abs(w.sum(axis=1) - 1.0)) < 1e-12
            assert np.all(w >= 0)
            if causal:
                assert np.all(np.triu(w, 1) == 0.0)


def pin_output_shape(fn):
    """§1 step 4 and §9: the output has Q's shape for MHA, GQA and MQA alike
    (the codelab's q (2, 64, 8, 64) with 8, 2 and 1 KV heads)."""
    q = _rand(3, 2, 64, 8, 64)
    for hkv in (8, 2, 1):
        k, v = _rand(4, 2, 64, hkv, 64), _rand(5, 2, 64, hkv, 64)
        assert fn(q, k, v, scale=0.125, causal=False).shape == q.shape


def pin_causal_first_row(fn):
    """§7: with the mask, position 0 attends only to itself, so its output is
    exactly V[0] of its KV head."""
    q, k, v = _rand(6, 2, 19, 4, 8), _rand(7, 2, 19, 2, 8), _rand(8, 2, 19, 2, 8)
    out = fn(q, k, v, scale=0.9, causal=True)
    for hq in range(4):
        assert np.array_equal(out[:, 0, hq, :], v[:, 0, hq // 2, :])


def pin_causal_last_row(fn):
    """§7: the last position sees every key, so causal and full attention
    agree on it; and the first row differs (the mask is really applied)."""
    q, k, v = _rand(9, 1, 23, 2, 8), _rand(10, 1, 23, 2, 8), _rand(11, 1, 23, 2, 8)
    c = fn(q, k, v, scale=0.5, causal=True)
    f = fn(q, k, v, scale=0.5, causal=False)
    np.testing.assert_allclose(c[:, -1], f[:, -1], rtol=0, atol=1e-12)
    assert np.max(np.abs(c[:, 0] - f[:, 0])) > 1e-2


def pin_constant_v(fn):
    """The output is a convex combination of V rows, so constant V rows give
    that constant back."""
    q, k = _rand(12, 2, 17, 4, 8), _rand(13, 2, 17, 2, 8)
    row = _rand(14, 8)
    v = np.broadcast_to(row, (2, 17, 2, 8)).copy()
    for causal in (False, True):
        out = fn(q, k, v, scale=0.7, causal=causal)
        np.testing.assert_allclose(out, np.broadcast_to(row, out.shape), rtol=0, atol=1e-12)


def pin_gqa_is_repeated_mha(fn):
    """§9 reading: GQA equals MHA with each KV head repeated G times along the
    head axis (contiguous groups); MQA is the Hkv = 1 case."""
    q = _rand(15, 2, 21, 8, 8)
    for hkv in (4, 2, 1):
        k, v = _rand(16, 2, 21, hkv, 8), _rand(17, 2, 21, hkv, 8)
        rk, rv = (np.repeat(x, 8 // hkv, axis=2) for x in (k, v))
        for causal in (False, True):
            a = fn(q, k, v, scale=0.4, causal=causal)
            b = fn(q, rk, rv, scale=0.4, causal=causal)
            np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def pin_scale_zero_prefix_mean(fn):
    """Closed form: with scale 0 all visible scores are equal, so the output is
    the mean of the visible V rows (the prefix mean under the mask)."""
    q, k, v = _rand(18, 1, 11, 2, 4), _rand(19, 1, 11, 2, 4), _rand(20, 1, 11, 2, 4)
    full = fn(q, k, v, scale=0.0, causal=False)
    np.testing.assert_allclose(full, np.broadcast_to(v.mean(axis=1, keepdims=True), full.shape),
                               rtol=0, atol=1e-12)
    cz = fn(q, k, v, scale=0.0, causal=True)
    pref = np.cumsum(v, axis=1) / np.arange(1, 12)[None, :, None, None]
    np.testing.assert_allclose(cz, pref, rtol=0, atol=1e-12)


def pin_single_key(fn):
    """Closed form: with Skv = 1 every query returns V[0]."""
    q, k, v = _rand(21, 2, 5, 3, 4), _rand(22, 2, 1, 3, 4), _rand(23, 2, 1, 3, 4)
    out = fn(q, k, v, scale=1.3, causal=False)
    np.testing.assert_allclose(out, np.broadcast_to(v, out.shape), rtol=0, atol=1e-15)


def pin_two_keys_sigmoid(fn):
    """Closed form: two keys give sigma(s0 - s1) v0 + sigma(s1 - s0) v1 with
    s_j = scale * q . k_j, and sigma(x) = 1 / (1 + exp(-x))."""
    q, k, v = _rand(24, 1, 3, 1, 5), _rand(25, 1, 2, 1, 5), _rand(26, 1, 2, 1, 5)
    sc = 0.8
    out = fn(q, k, v, scale=sc, causal=False)
    for i in range(3):
        s0 = sc * float(np.dot(q[0, i, 0], k[0, 0, 0]))
        s1 = sc * float(np.dot(q[0, i, 0], k[0, 1, 0]))
        w0 = 1.0 / (1.0 + math.exp(-(s0 - s1)))
        w1 = 1.0 / (1.0 + math.exp(-(s1 - s0)))
        np.testing.assert_allclose(out[0, i, 0], w0 * v[0, 0, 0] + w1 * v[0, 1, 0], rtol=0, atol=1e-14)


def pin_shift_and_affine(fn):
    """Softmax is invariant to adding the same vector u to every key (each
    score of a row shifts by the same q . u), and the output is affine
    equivariant in V: V -> a V + c gives O -> a O + c."""
    q, k, v = _rand(27, 2, 13, 2, 6), _rand(28, 2, 13, 2, 6), _rand(29, 2, 13, 2, 6)
    u = _rand(30, 6)
    for causal in (False, True):
        base = fn(q, k, v, scale=0.6, causal=causal)
        np.testing.assert_allclose(fn(q, k + u, v, scale=0.6, causal=causal), base, rtol=0, atol=1e-12)
        np.testing.assert_allclose(fn(q, k, -2.5 * v + 0.75, scale=0.6, causal=causal),
                                   -2.5 * base + 0.75, rtol=0, atol=1e-12)


def pin_key_permutation(fn):
    """Without a mask nothing depends on key order: permuting keys jointly in
    K and V leaves the output unchanged."""
    q, k, v = _rand(31, 1, 9, 2, 4), _rand(32, 1, 14, 2, 4), _rand(33, 1, 14, 2, 4)
    perm = np.random.default_rng(34).permutation(14)
    a = fn(q, k, v, scale=0.9, causal=False)
    b = fn(q, k[:, perm], v[:, perm], scale=0.9, causal=False)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def pin_brute_force(fn):
    """The vectorised result matches scalar pure-Python loops on tiny inputs,
    for every mask and grouping variant (including Sq != Skv)."""
    for (B, Sq, Skv, Hq, Hkv, D) in [(1, 3, 3, 1, 1, 2), (2, 5, 7, 4, 2, 3), (1, 9, 4, 4, 1, 8),
                                     (2, 6, 6, 2, 2, 5)]:
        q, k, v = _rand(B + Sq, B, Sq, Hq, D), _rand(Skv + 1, B, Skv, Hkv, D), _rand(D + 7, B, Skv, Hkv, D)
        for causal in (False, True, "bottom_right"):
            if causal == "bottom_right" and Sq > Skv:
                continue
            got = fn(q, k, v, scale=0.37, causal=causal)
            want = np.array(oracle.brute_sdpa(q.tolist(), k.tolist(), v.tolist(), scale=0.37, causal=causal))
            np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def pin_torch_cpu_library(fn):
    """Independent library routine: torch's CPU scaled_dot_product_attention
    in float64 on (B, H, S, D)-transposed inputs with KV heads repeated."""
    B, S, Hq, Hkv, D = 2, 33, 4, 2, 16
    q, k, v = _rand(35, B, S, Hq, D), _rand(36, B, S, Hkv, D), _rand(37, B, S, Hkv, D)
    for causal in (False, True):
        got = fn(q, k, v, scale=1 / math.sqrt(D), causal=causal)
        tq = torch.from_numpy(q).permute(0, 2, 1, 3).contiguous()
        tk = torch.from_numpy(np.repeat(k, Hq // Hkv, axis=2)).permute(0, 2, 1, 3).contiguous()
        tv = torch.from_numpy(np.repeat(v, Hq // Hkv, axis=2)).permute(0, 2, 1, 3).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
        np.testing.assert_allclose(got, ref.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-10)
    # Bottom-right alignment against torch's lower-right causal bias, Sq < Skv.
    from torch.nn.attention.bias import causal_lower_right
    Sq = 7
    q = _rand(41, B, Sq, Hq, D)
    got = fn(q, k, v, scale=1 / math.sqrt(D), causal="bottom_right")
    tq = torch.from_numpy(q).permute(0, 2, 1, 3).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=causal_lower_right(Sq, S))
    np.testing.assert_allclose(got, ref.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-10)


def pin_rows_match_full(fn=None):
    """Sampled single rows (used at full problem sizes) equal the full result."""
    q, k, v = _rand(38, 2, 40, 4, 8), _rand(39, 2, 40, 2, 8), _rand(40, 2, 40, 2, 8)
    for causal in (False, True, "bottom_right"):
        for qq in (q, q[:, 11:]):
            full = oracle.sdpa(qq, k, v, scale=0.5, causal=causal, row_chunk=7)
            rows = [(0, 0, 0), (1, qq.shape[1] - 1, 3), (1, 17, 2), (0, 25, 1)]
            got = oracle.sdpa_rows(qq, k, v, rows, scale=0.5, causal=causal)
            for n, (b, i, h) in enumerate(rows):
                np.testing.assert_allclose(got[n], full[b, i, h], rtol=0, atol=1e-13)


def pin_bottom_right_is_cache_suffix(fn):
    """§9 key-value-cache reading: the Sq new queries at the end of a
    sequence of Skv tokens, attending with bottom-right alignment, give
    exactly the last Sq rows of causal self-attention over the whole
    sequence (§7 mask), whatever Sq is."""
    B, S, Hq, Hkv, D = 2, 29, 4, 2, 8
    qf, k, v = _rand(42, B, S, Hq, D), _rand(43, B, S, Hkv, D), _rand(44, B, S, Hkv, D)
    full = fn(qf, k, v, scale=0.45, causal=True)
    for Sq in (1, 2, 5, 16, 29):
        got = fn(qf[:, S - Sq:], k, v, scale=0.45, causal="bottom_right")
        np.testing.assert_allclose(got, full[:, S - Sq:], rtol=0, atol=1e-12)


def pin_bottom_right_limits(fn):
    """Bottom-right alignment at its two ends: one query sees every key (the
    same as no mask), and Sq == Skv is the ordinary §7 mask."""
    q1, k, v = _rand(45, 1, 1, 2, 8), _rand(46, 1, 13, 1, 8), _rand(47, 1, 13, 1, 8)
    np.testing.assert_allclose(fn(q1, k, v, scale=0.7, causal="bottom_right"),
                               fn(q1, k, v, scale=0.7, causal=False), rtol=0, atol=1e-13)
    q = _rand(48, 1, 13, 2, 8)
    np.testing.assert_allclose(fn(q, k, v, scale=0.7, causal="bottom_right"),
                               fn(q, k, v, scale=0.7, causal=True), rtol=0, atol=1e-13)


ALL_PINS = [pin_golden, pin_weights_sum_to_one, pin_output_shape, pin_causal_first_row,
            pin_causal_last_row, pin_constant_v, pin_gqa_is_repeated_mha, pin_scale_zero_prefix_mean,
            pin_single_key, pin_two_keys_sigmoid, pin_shift_and_affine, pin_key_permutation,
            pin_brute_force, pin_torch_cpu_library, pin_rows_match_full, pin_bottom_right_is_cache_suffix,
            pin_bottom_right_limits]
