"""Plain fp64 log-sum-exp and backward pass of SDPA (test infrastructure only).

The forward is out = softmax(scale Q K^T [+ mask]) V ([Attention codelab §1],
§4, §7, §9). The codelab motivates the scale by keeping the softmax out of
saturation, where its gradients vanish ([Attention codelab §1]), and names
E5M2 as the FP8 format of the backward pass ([Attention codelab §10]). This
module writes the gradients of that forward out by the chain rule, one
(batch, query head) at a time, with no tiling and no recomputation tricks:

    S  = scale Q K^T, masked entries -inf          (per head, Sq x Skv)
    P  = softmax(S) along keys;  O = P V
    dV = P^T dO                                     (summed over the query
    dP = dO V^T                                      heads that share a KV head)
    dS = P * (dP - rowsum(P * dP))                  (softmax Jacobian, row-wise)
    dQ = scale dS K
    dK = scale dS^T Q                               (summed like dV)

and the log-sum-exp of each row, lse_i = log sum_j exp(S_ij) (natural
logarithm), the quantity a fused forward keeps so that a backward pass can
rebuild P = exp(S - lse) without another max and sum over the keys.

Score, mask, softmax, head grouping and the causal readings are the forward
oracle's own steps (:mod:`oracle.attention`). Pins:
tests/test_oracle_backward.py (torch autograd in float64, central finite
differences of the forward oracle, closed forms and invariants).
"""

import numpy as np

from . import attention as fwd

__all__ = ["sdpa_lse", "sdpa_backward"]


def _head_probs(qh, kh, scale, shift):
    """Masked scaled scores S and their row softmax P for one head."""
    s = fwd._scores(qh, kh, scale, shift is not None, shift or 0)
    return s, fwd._softmax_rows(s)


def _row_lse(s):
    """log sum_j exp(s_ij) per row, with the row maximum taken out first."""
    m = np.max(s, axis=1)
    return m + np.log(np.sum(np.exp(s - m[:, None]), axis=1))


def _softmax_grad(p, dp):
    """dS = P * (dP - rowsum(P * dP)): a row softmax's Jacobian applied to dP."""
    return p * (dp - np.sum(p * dp, axis=1, keepdims=True))


def _head_grads(p, ds, qh, kh, doh, scale):
    """(dQ, dK, dV) contributions of one query head: scale dS K, scale dS^T Q, P^T dO."""
    return scale * (ds @ kh), scale * (ds.T @ qh), p.T @ doh


def _accumulate(acc, b, g, part):
    """A KV head's gradient is the sum over the query heads that read it."""
    acc[b, :, g, :] += part


def sdpa_lse(q, k, *, scale, causal):
    """Row log-sum-exp of the masked scaled scores, shape (B, Hq, Sq).

    lse[b, h, i] = log(sum_j exp(scale <q_bih, k_bjg>)) over the keys j that
    the mask leaves visible, g the KV head of query head h.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, Sq, Hq, D, Skv, Hkv = fwd._check_shapes(q, k, k)
    shift = fwd._query_shift(causal, Sq, Skv)
    out = np.empty((B, Hq, Sq), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            s, _ = _head_probs(q[b, :, h, :], k[b, :, fwd.kv_head_of(h, Hq, Hkv), :], scale, shift)
            out[b, h] = _row_lse(s)
    return out


def sdpa_backward(q, k, v, dout, *, scale, causal):
    """Gradients (dQ, dK, dV) of sum(dout * sdpa(q, k, v)) in fp64.

    Shapes follow the forward: q, dout, dQ (B, Sq, Hq, D); k, v, dK, dV
    (B, Skv, Hkv, D). Each KV head's gradient sums the contributions of the
    Hq / Hkv query heads that read it.
    """
    q, k, v, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    B, Sq, Hq, D, Skv, Hkv = fwd._check_shapes(q, k, v)
    if dout.shape != q.shape:
        raise ValueError(f"dout {dout.shape} must have q's shape {q.shape}")
    shift = fwd._query_shift(causal, Sq, Skv)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = fwd.kv_head_of(h, Hq, Hkv)
            qh, kh, vh, doh = q[b, :, h, :], k[b, :, g, :], v[b, :, g, :], dout[b, :, h, :]
            _, p = _head_probs(qh, kh, scale, shift)
            ds = _softmax_grad(p, doh @ vh.T)
            dqh, dkh, dvh = _head_grads(p, ds, qh, kh, doh, scale)
            dq[b, :, h, :] = dqh
            _accumulate(dk, b, g, dkh)
            _accumulate(dv, b, g, dvh)
    return dq, dk, dv
