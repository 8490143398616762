"""GPU parity of the row log-sum-exp output and of the backward pass, against
the fp64 oracle (oracle.sdpa_lse, oracle.sdpa_backward).

The oracle sees the same seeded input codes (decoded by its own codecs) and
computes the exact gradients of sum(dout * sdpa(q, k, v)); nothing it uses
comes from the GPU. The GPU backward takes the GPU forward's out and lse, as
a training step would.

Bounds. lse: 1e-5 for float32 inputs; 2e-2 for bf16 / f16 (the forward sums
weights rounded to the input type: relative error of the row sum below
2^-8, so |d lse| < 4e-3). Gradients (bf16 / f16), per tensor: max-abs error
at most 2^-7 max |exact| + 2^-9, plus, for dq, the error it inherits from
Delta (below). Rounding model: each gradient element is rounded once to the
output type (at most 2^-9 of its size), and the weights P and the score
gradients dS enter the products rounded to the input type (2^-9 relative
each), errors that grow with the gradient's own scale and, summed over many
keys or rows with mixed signs, stay within a small multiple of that rounding
at the largest element (measured: 1.6 to 1.8 times 2^-9 of max |exact| on
dq, dk and dv); 2^-7 = 4 times 2^-9 leaves about twice the measured error
as headroom, and 2^-9 is an absolute floor for tensors whose exact values
are all tiny. Delta_i = rowsum(dO_i * O_i) is formed from the forward's
output rounded to the input type, an error of about 2^-9 sqrt(sum_d
(dO_id O_id)^2) (independent roundings of the D terms; three times that is
taken), and dq_i = scale sum_j P_ij (dP_ij - Delta_i) k_j carries it times
scale (P K)_i, the weighted mean of the keys: small for zero-mean keys,
large when the keys share an offset (the drifting-keys stress input). The
oracle gives O and P K (attention with the keys as values) exactly.
"""

import numpy as np
import pytest
import torch

import oracle
from scaled_dot_product_09_amd import attn, workload
from scaled_dot_product_09_amd.workload import Workload
from tests import helpers

pytestmark = pytest.mark.gpu

LSE_TOL = {"f32": 1e-5, "bf16": 2e-2, "f16": 2e-2, "e4m3": 2e-2}


def W(dtype, B, Hq, Hkv, Sq, Skv, D, causal, seed=5):
    tag = {False: "", True: "_causal", "bottom_right": "_br"}[causal]
    return Workload(f"{dtype}_b{B}_hq{Hq}_hkv{Hkv}_sq{Sq}_skv{Skv}_d{D}{tag}", dtype, B, Hq, Hkv, Sq, Skv, D,
                    causal, seed)


def grad_tol(ref):
    return 2.0 ** -7 * (float(np.max(np.abs(ref))) if ref.size else 0.0) + 2.0 ** -9


LSE_CASES = [
    W("f32", 1, 4, 2, 100, 100, 64, True),
    W("f32", 2, 2, 1, 33, 70, 128, "bottom_right"),
    W("f32", 1, 2, 2, 50, 20, 32, False),
    W("bf16", 2, 8, 2, 300, 300, 128, True),
    W("bf16", 1, 4, 1, 7, 500, 128, "bottom_right"),
    W("bf16", 1, 4, 4, 130, 257, 64, False),
    W("bf16", 1, 4, 2, 200, 200, 32, True),
    W("f16", 1, 8, 2, 100, 100, 128, True),
    W("e4m3", 1, 4, 2, 150, 150, 128, True),
    W("e4m3", 1, 4, 1, 9, 300, 64, "bottom_right"),
    W("bf16", 1, 4, 2, 600, 600, 128, True),        # forward with folded row blocks
    W("f16", 1, 2, 2, 700, 900, 64, "bottom_right"),
]


@pytest.mark.parametrize("w", LSE_CASES, ids=lambda w: w.name)
def test_lse_parity(w):
    print(f"case {w.name}", flush=True)
    q, k, v, desc = workload.make_inputs(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    fp8 = w.dtype == "e4m3"
    out, lse = attn.fwd_lse(qd, kd, vd, causal=w.causal, scale=w.scale, descales=desc if fp8 else None)
    ref_out = attn.fwd(qd, kd, vd, causal=w.causal, scale=w.scale, descales=desc if fp8 else None)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)            # same kernel, same output
    want = oracle.sdpa_lse(helpers.to_f64(q, w.dtype, desc[0]), helpers.to_f64(k, w.dtype, desc[1]), scale=w.scale,
                           causal=w.causal)
    err = helpers.max_abs_err(lse.cpu().numpy().astype(np.float64), want)
    print(f"  lse max-abs {err:.3e}", flush=True)
    assert err <= LSE_TOL[w.dtype], err


def run_backward(w, q, k, v, g, *, scale=None):
    dev = torch.device("cuda:0")
    scale = w.scale if scale is None else scale
    qd, kd, vd, gd = q.to(dev), k.to(dev), v.to(dev), g.to(dev)
    out, lse = attn.fwd_lse(qd, kd, vd, causal=w.causal, scale=scale)
    dq, dk, dv = attn.bwd(qd, kd, vd, out, gd, lse, causal=w.causal, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def delta_term(f64_inputs, scale, causal):
    """The bound on dq's error inherited from Delta (see the module
    docstring): max over rows of scale * 3 * 2^-9 * sqrt(sum_d (dO O)^2)
    * max_d |(P K)_id|, from the oracle's exact O and P K."""
    qf, kf, vf, gf = f64_inputs
    o = helpers.oracle_sdpa_threaded(qf, kf, vf, scale=scale, causal=causal)
    pk = helpers.oracle_sdpa_threaded(qf, kf, kf, scale=scale, causal=causal)
    e = 3 * 2.0 ** -9 * np.sqrt(np.sum((gf * o) ** 2, axis=-1))
    return float(np.max(abs(scale) * e * np.max(np.abs(pk), axis=-1))) if e.size else 0.0


def check_grads(w, got, want, f64_inputs, scale=None):
    scale = w.scale if scale is None else scale
    extra = {"dq": delta_term(f64_inputs, scale, w.causal), "dk": 0.0, "dv": 0.0}
    for name, a, b in zip(("dq", "dk", "dv"), got, want):
        a = helpers.out_to_f64(a)
        err, tol = helpers.max_abs_err(a, b), grad_tol(b) + extra[name]
        print(f"  {name} max-abs {err:.3e} (max |exact| {np.max(np.abs(b)) if b.size else 0:.3f}, bound {tol:.3e}"
              f"{f', Delta term {extra[name]:.3e}' if extra[name] else ''})", flush=True)
        assert err <= tol, (name, err, tol)


BWD_CASES = [
    W("bf16", 1, 4, 2, 200, 200, 128, True),        # ragged in every tiling (64-key tiles, 128-key blocks, 32-row steps)
    W("bf16", 2, 4, 4, 130, 130, 64, False),
    W("bf16", 1, 8, 1, 77, 300, 128, "bottom_right"),   # MQA, Sq < Skv
    W("bf16", 1, 2, 1, 300, 77, 64, True),          # top-left mask with Sq > Skv: rows past Skv see every key
    W("bf16", 1, 4, 2, 256, 256, 32, True),
    W("bf16", 1, 4, 1, 5, 400, 128, "bottom_right"),    # decode shape: rows of several heads share a wave
    W("bf16", 1, 8, 2, 1, 1, 64, False),            # one key: dq = dk = 0
    W("bf16", 2, 4, 2, 64, 64, 128, False),
    W("f16", 1, 8, 2, 160, 160, 128, True),
    W("f16", 1, 4, 4, 97, 150, 64, "bottom_right"),
    W("f16", 2, 4, 1, 65, 65, 32, True),            # f16 head dim 32, MQA
    W("bf16", 1, 4, 2, 1, 700, 128, "bottom_right"),    # one decode query, keys in 6 blocks of 128 (ragged)
    W("bf16", 1, 2, 2, 129, 383, 64, False),        # one row past a step, keys past three blocks
    W("bf16", 3, 8, 4, 100, 100, 128, True),        # three batches, G = 2
]


@pytest.mark.parametrize("w", BWD_CASES, ids=lambda w: w.name)
def test_backward_parity(w):
    print(f"case {w.name}", flush=True)
    q, k, v, _ = workload.make_inputs(w)
    g = workload.make_dout(w)
    got = run_backward(w, q, k, v, g)
    f64 = tuple(helpers.to_f64(x, w.dtype) for x in (q, k, v, g))
    want = oracle.sdpa_backward(*f64, scale=w.scale, causal=w.causal)
    check_grads(w, got, want, f64)


@pytest.mark.parametrize("dtype,D,causal", [("bf16", 128, True), ("f16", 64, False), ("bf16", 64, "bottom_right")])
def test_backward_growing_row_maxima(dtype, D, causal):
    """Keys drift along the sequence so that every row's scores rise by about
    15 in exp2 terms per 64 keys, to about 2^140 at the last of 600 keys: the
    weights are rebuilt from the forward's lse at scores whose plain
    exponentials would overflow float32.

    The rise comes mostly from queries with a large mean (2 per component)
    and only a small drift of the keys (at most ~4-6 per component): dQ =
    scale dS K inherits the error of Delta = rowsum(dO * out), formed from the
    forward's rounded output, multiplied by the size of the keys, which no
    kernel can avoid when keys share a large common offset."""
    w = W(dtype, 1, 4, 2, 600, 600, D, causal, seed=33)
    print(f"case {w.name} (drifting keys)", flush=True)
    rng = np.random.default_rng(33)
    slope = 0.081 / np.sqrt(D)            # 2 sqrt(D) slope log2(e) = 0.234 per key
    qn = 2.0 + 0.5 * rng.standard_normal((1, 600, 4, D))
    kn = 0.5 * rng.standard_normal((1, 600, 2, D)) + slope * np.arange(600)[None, :, None, None]
    vn = rng.standard_normal((1, 600, 2, D))
    td = workload.TORCH_DTYPE[dtype]
    q, k, v = (torch.from_numpy(x.astype(np.float32)).to(td) for x in (qn, kn, vn))
    g = workload.make_dout(w)
    got = run_backward(w, q, k, v, g)
    f64 = tuple(helpers.to_f64(x, w.dtype) for x in (q, k, v, g))
    want = oracle.sdpa_backward(*f64, scale=w.scale, causal=w.causal)
    check_grads(w, got, want, f64)


FP8_CASES = [
    W("e4m3", 1, 4, 2, 200, 200, 128, True),
    W("e4m3", 1, 4, 4, 130, 257, 64, False),
    W("e4m3", 1, 8, 1, 33, 300, 128, "bottom_right"),
    W("e4m3", 2, 4, 2, 64, 64, 64, True),
]


@pytest.mark.parametrize("w", FP8_CASES, ids=lambda w: w.name)
def test_backward_fp8_parity(w):
    """E4M3 q, k, v and an E5M2 dout, each with its per-tensor descale; the
    oracle differentiates on the decoded values. Same bound as bf16: the
    codes are widened exactly and the descales only scale."""
    print(f"case {w.name}", flush=True)
    q, k, v, desc = workload.make_inputs(w)
    g, gdesc = workload.make_dout(w)
    dev = torch.device("cuda:0")
    qd, kd, vd, gd = q.to(dev), k.to(dev), v.to(dev), g.to(dev)
    out, lse = attn.fwd_lse(qd, kd, vd, causal=w.causal, scale=w.scale, descales=desc)
    got = attn.bwd(qd, kd, vd, out, gd, lse, causal=w.causal, scale=w.scale, descales=(*desc, gdesc))
    torch.cuda.synchronize()
    f64 = (helpers.to_f64(q, "e4m3", desc[0]), helpers.to_f64(k, "e4m3", desc[1]),
           helpers.to_f64(v, "e4m3", desc[2]), helpers.to_f64(g, "e5m2", gdesc))
    want = oracle.sdpa_backward(*f64, scale=w.scale, causal=w.causal)
    check_grads(w, got, want, f64)


def test_backward_negative_and_zero_scale():
    w = W("bf16", 1, 4, 2, 96, 96, 64, True)
    q, k, v, _ = workload.make_inputs(w)
    g = workload.make_dout(w)
    for scale in (-0.2, 0.0):
        print(f"scale {scale}", flush=True)
        got = run_backward(w, q, k, v, g, scale=scale)
        f64 = tuple(helpers.to_f64(x, w.dtype) for x in (q, k, v, g))
        want = oracle.sdpa_backward(*f64, scale=scale, causal=w.causal)
        check_grads(w, got, want, f64, scale=scale)


def test_backward_no_query_rows_zeroes_dk_dv():
    """Sq = 0: nothing reads the keys, so dk and dv are written as 0."""
    dev = torch.device("cuda:0")
    q = torch.zeros(1, 0, 4, 64, dtype=torch.bfloat16, device=dev)
    k = torch.randn(1, 50, 2, 64, device=dev).to(torch.bfloat16)
    lse = torch.zeros(1, 4, 0, device=dev)
    dk = torch.full_like(k, 7.0)
    dv = torch.full_like(k, 7.0)
    attn.bwd(q, k, k, q, q, lse, causal=False, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)


def test_backward_is_deterministic():
    w = W("bf16", 1, 8, 2, 300, 300, 128, True)
    q, k, v, _ = workload.make_inputs(w)
    g = workload.make_dout(w)
    a = run_backward(w, q, k, v, g)
    b = run_backward(w, q, k, v, g)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_full_size_headline():
    """Causal GQA, B=2, Hq=32, Hkv=8, S=4096, D=128, bf16: every gradient
    element of all 16 (batch, KV head) groups (each group's four query heads
    and its shared K/V head) against the oracle, computed group by group in a
    thread pool; and two sums that hold exactly for every group: the key
    gradients of a KV head sum to zero over the keys, and its value gradients
    sum to the group's dout summed over the rows."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    w = workload.WORKLOADS["bf16_gqa_b2_hq32_hkv8_s4096_d128_causal_bwd"]
    print(f"case {w.name}", flush=True)
    q, k, v, _ = workload.make_inputs(w)
    g = workload.make_dout(w)
    dq, dk, dv = run_backward(w, q, k, v, g)
    G = w.Hq // w.Hkv
    qf, kf, vf, gf = (helpers.to_f64(x, "bf16") for x in (q, k, v, g))
    want = [np.empty(qf.shape), np.empty(kf.shape), np.empty(vf.shape)]

    def group(bg):
        b, hkv = bg
        hs = slice(hkv * G, (hkv + 1) * G)
        r = oracle.sdpa_backward(qf[b:b + 1, :, hs], kf[b:b + 1, :, hkv:hkv + 1], vf[b:b + 1, :, hkv:hkv + 1],
                                 gf[b:b + 1, :, hs], scale=w.scale, causal=True)
        want[0][b:b + 1, :, hs] = r[0]
        want[1][b:b + 1, :, hkv:hkv + 1] = r[1]
        want[2][b:b + 1, :, hkv:hkv + 1] = r[2]

    with threadpool_limits(1):
        with ThreadPoolExecutor(max_workers=16) as ex:
            list(ex.map(group, [(b, h) for b in range(w.B) for h in range(w.Hkv)]))
    check_grads(w, (dq, dk, dv), want, (qf, kf, vf, gf))
    # Sums over keys (float64 of the rounded gradients) for every (batch, KV head).
    dk64 = dk.double().sum(dim=1).cpu().numpy()
    dv64 = dv.double().sum(dim=1).cpu().numpy()
    gsum = helpers.to_f64(g, "bf16").sum(axis=1).reshape(w.B, w.Hkv, G, w.D).sum(axis=2)
    err_k = float(np.max(np.abs(dk64)))
    err_v = float(np.max(np.abs(dv64 - gsum)))
    print(f"  |sum_j dk| max {err_k:.3e}; |sum_j dv - sum_i dout| max {err_v:.3e}", flush=True)
    # Each of the 4096 rounded terms is off by at most 2^-9 of its size.
    assert err_k <= 4096 * 2.0 ** -9 * float(dk.abs().max()), err_k
    assert err_v <= 4096 * 2.0 ** -9 * float(dv.abs().max()) + 1e-3 * float(np.max(np.abs(gsum))), err_v
