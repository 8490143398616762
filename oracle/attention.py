"""Plain fp64 scaled dot-product attention (test infrastructure only).

The oracle is the textbook definition written out, with no tiling, no online
softmax and no fusion: it materialises the full score and weight matrices the
way the unfused computation of [Attention codelab §4] does, so a reader can
check it against the formula of [Attention codelab §1] by eye.

Layout follows [Attention codelab §3]: Q is (B, T, N, H) and K, V are
(B, S, K, H) with K <= N; this file names them (B, Sq, Hq, D) and
(B, Skv, Hkv, D). The output has Q's shape ([Attention codelab §1], step 4).

Readings taken where the pages are silent (each is pinned by a test):

* Causal alignment when Sq != Skv: the pages only ever use Sq == Skv. The
  reading for ``causal=True`` (also ``"top_left"``, 1) is the literal lower
  triangle of the Sq x Skv score matrix (key j visible to query i iff
  j <= i), called top-left alignment.
* ``causal="bottom_right"`` (also 2) is the key-value-cache reading of the
  grouped / multi-query inference use the pages motivate [Attention codelab
  §9]: the Sq queries are the last Sq positions of a sequence of Skv tokens,
  so query i sits at position Skv - Sq + i and sees keys j <= Skv - Sq + i.
  It needs Sq <= Skv (every query then sees at least key 0). With Sq == Skv
  both readings coincide.
* Grouping of query heads onto KV heads [Attention codelab §9]: contiguous
  groups, query head h reads KV head h // (Hq // Hkv). This equals repeating
  each KV head Hq // Hkv times in a row along the head axis.
* Softmax stabilisation: the row maximum is subtracted before exp; in exact
  arithmetic this does not change the result.
"""

import math

import numpy as np

__all__ = ["kv_head_of", "query_shift", "attention_weights", "sdpa", "sdpa_rows", "sdpa_one_row", "brute_sdpa"]


def kv_head_of(hq, Hq, Hkv):
    """KV head read by query head ``hq`` [Attention codelab §9].

    The codelab's GQA example has 8 query heads and 2 KV heads, "each shared
    by 4 query heads"; the order of sharing is not stated. Reading taken:
    contiguous groups of G = Hq // Hkv query heads share one KV head.
    """
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    return hq // (Hq // Hkv)


def _query_shift(causal, Sq, Skv):
    """None without a mask, else the position of query row 0.

    ``False``/0: no mask. ``True``/1/``"top_left"``: query i at position i.
    ``"bottom_right"``/2: query i at position Skv - Sq + i (requires
    Sq <= Skv).
    """
    if causal is False or causal == 0 or causal is None:
        return None
    if causal is True or causal == 1 or causal == "top_left":
        return 0
    if causal == 2 or causal == "bottom_right":
        if Sq > Skv:
            raise ValueError(f"bottom-right causal alignment needs Sq <= Skv (got {Sq} > {Skv})")
        return Skv - Sq
    raise ValueError(f"unknown causal mode {causal!r}")


def query_shift(causal, Sq, Skv):
    """Public form of the causal reading: None (no mask) or the position of
    query row 0, for callers that evaluate single rows with
    :func:`sdpa_one_row`."""
    return _query_shift(causal, Sq, Skv)


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D (B, S, H, D)")
    B, Sq, Hq, D = q.shape
    Bk, Skv, Hkv, Dk = k.shape
    if k.shape != v.shape:
        raise ValueError(f"k {k.shape} and v {v.shape} differ")
    if Bk != B or Dk != D:
        raise ValueError(f"q {q.shape} and k {k.shape} disagree on B or D")
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    return B, Sq, Hq, D, Skv, Hkv


def _scores(qh, kh, scale, causal, row0):
    """Score step + causal mask for queries at positions row0 .. row0+len(qh)-1.

    Score = scale * Q K^T ([Attention codelab §1] steps 1-2, §4). With
    ``causal`` the entries with key index j > query position i are set to
    -inf, the lower-triangular mask of [Attention codelab §7].
    """
    s = scale * (qh @ kh.T)
    if causal:
        i = np.arange(row0, row0 + qh.shape[0])[:, None]
        j = np.arange(kh.shape[0])[None, :]
        s = np.where(j > i, -np.inf, s)
    return s


def _softmax_rows(s):
    """Softmax along the key axis ([Attention codelab §4], axis=-1)."""
    m = np.max(s, axis=1, keepdims=True)
    w = np.exp(s - m)
    return w / np.sum(w, axis=1, keepdims=True)


def attention_weights(q, k, *, scale, causal, b=0, hq=0):
    """The (Sq, Skv) weight matrix softmax(scale Q K^T [+ mask]) of one head.

    Returned for the query head ``hq`` of batch ``b``; each row sums to 1
    ([Attention codelab §1], step 2).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    g = kv_head_of(hq, Hq, Hkv)
    shift = _query_shift(causal, Sq, Skv)
    return _softmax_rows(_scores(q[b, :, hq, :], k[b, :, g, :], scale, shift is not None, shift or 0))


def sdpa(q, k, v, *, scale, causal, row_chunk=1024):
    """softmax(scale Q K^T [+ causal mask]) V in fp64, layout (B, S, H, D).

    [Attention codelab §1] formula and four steps; [Attention codelab §4]
    computation order (score, scale, softmax over keys, weights @ V);
    [Attention codelab §7] mask; [Attention codelab §9] head broadcast.

    Inputs are converted to float64 first (callers pass values that were
    already rounded to the GPU's input type). Query rows are processed
    ``row_chunk`` at a time so a 16384 x 16384 head does not need 2 GiB at
    once; each row's result does not depend on the chunking.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Sq, Hq, D, Skv, Hkv = _check_shapes(q, k, v)
    out = np.empty((B, Sq, Hq, D), dtype=np.float64)
    if B * Sq * Hq * D == 0:
        return out
    if Skv == 0:
        raise ValueError("Skv must be >= 1 when Sq > 0")
    shift = _query_shift(causal, Sq, Skv)
    for b in range(B):
        for hq in range(Hq):
            g = kv_head_of(hq, Hq, Hkv)
            kh = k[b, :, g, :]
            vh = v[b, :, g, :]
            for r0 in range(0, Sq, row_chunk):
                qh = q[b, r0:r0 + row_chunk, hq, :]
                p = _softmax_rows(_scores(qh, kh, scale, shift is not None, (shift or 0) + r0))
                out[b, r0:r0 + qh.shape[0], hq, :] = p @ vh
    return out


def sdpa_one_row(qvec, kh, vh, *, i, scale, causal):
    """Output vector of one query vector at position ``i`` against one head.

    ``qvec`` is (D,), ``kh`` and ``vh`` are that head's (Skv, D) keys and
    values; with a true ``causal`` the mask hides keys j > i, where ``i`` is
    the query's position (for bottom-right alignment the caller passes
    Skv - Sq + row). Same definition as :func:`sdpa`, for one row.
    """
    qh = np.asarray(qvec, dtype=np.float64).reshape(1, -1)
    kh = np.asarray(kh, dtype=np.float64)
    vh = np.asarray(vh, dtype=np.float64)
    p = _softmax_rows(_scores(qh, kh, scale, bool(causal), i))
    return (p @ vh)[0]


def sdpa_rows(q, k, v, rows, *, scale, causal):
    """Output vectors O[b, i, hq, :] for a list of (b, i, hq) triples.

    The same definition as :func:`sdpa`, evaluated one query row at a time, so
    sampled outputs of a full-size problem can be checked without computing
    every row. Returns an array of shape (len(rows), D).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, Sq, Hq, D, Skv, Hkv = _check_shapes(q, k, v)
    shift = _query_shift(causal, Sq, Skv)
    res = np.empty((len(rows), D), dtype=np.float64)
    for n, (b, i, hq) in enumerate(rows):
        g = kv_head_of(hq, Hq, Hkv)
        res[n] = sdpa_one_row(q[b, i, hq, :], k[b, :, g, :], v[b, :, g, :], i=(shift or 0) + i, scale=scale,
                              causal=shift is not None)
    return res


def brute_sdpa(q, k, v, *, scale, causal):
    """Scalar pure-Python SDPA for tiny inputs (nested lists or arrays).

    No numpy arithmetic at all: every score is a Python dot product, the
    softmax is exp(s - max) / sum, and each output element is a weighted sum,
    written directly from [Attention codelab §1]. Used to pin :func:`sdpa`.
    ``causal`` takes the same values as in :func:`sdpa`.
    """
    B = len(q)
    Sq = len(q[0]) if B else 0
    Hq = len(q[0][0]) if Sq else 0
    D = len(q[0][0][0]) if Hq else 0
    Skv = len(k[0])
    Hkv = len(k[0][0])
    G = Hq // Hkv
    shift = _query_shift(causal, Sq, Skv)
    out = [[[[0.0] * D for _ in range(Hq)] for _ in range(Sq)] for _ in range(B)]
    for b in range(B):
        for i in range(Sq):
            for h in range(Hq):
                g = h // G
                s = []
                for j in range(Skv):
                    if shift is not None and j > shift + i:
                        continue
                    dot = 0.0
                    for d in range(D):
                        dot += float(q[b][i][h][d]) * float(k[b][j][g][d])
                    s.append((j, scale * dot))
                m = max(x for _, x in s)
                e = [(j, math.exp(x - m)) for j, x in s]
                tot = sum(x for _, x in e)
                for d in range(D):
                    acc = 0.0
                    for j, x in e:
                        acc += (x / tot) * float(v[b][j][g][d])
                    out[b][i][h][d] = acc
    return out
