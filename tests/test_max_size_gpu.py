"""GPU parity at the largest accepted tensor size.

K and V each hold one KV head of 16,777,213 keys x 128 (2^31 - 384 elements,
4 GiB - 768 bytes of bfloat16: a tensor of 2^31 elements is rejected), so the
key offsets the kernels form run up to just below 2^32 bytes, and the last key
tile is ragged. Four query heads (MQA) of two decode rows each (bottom-right
causal: row 0 sees every key but the last, row 1 all of them).

Expected values in closed form (the oracle's full-row path would need the
whole 16 M x 128 key matrix in float64): every key is zero except one
"needle" per query head near the end of the span, k[J_h] = 340 e_h, and query
head h is q = e_h, so head h scores 340 / sqrt(128) on its needle and 0 on
every other visible key. With E_h = exp(340 / sqrt(128)) and n visible keys,

    out[i, h] = (E_h v[J_h] + sum_{visible j != J_h} v[j]) / (E_h + n - 1),

evaluated in float64 from V's exact values (multiples of 1/8 in [-1, 1]).
A kernel that missed a needle, or read keys at wrapped offsets, would return
about the mean of V instead of v[J_h]. Checked with and without split keys.
"""

import math

import numpy as np
import pytest
import torch

from scaled_dot_product_09_amd import attn

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
SKV = (1 << 24) - 3
D = 128
HQ = 4
NEEDLE = 340.0                                   # a bfloat16 value
J = [SKV - 2 - 1000 * h for h in range(HQ)]       # needle of query head h


@pytest.fixture(scope="module")
def inputs():
    assert SKV * D < (1 << 31)
    k = torch.zeros((1, SKV, 1, D), dtype=torch.bfloat16, device=DEV)
    for h in range(HQ):
        k[0, J[h], 0, h] = NEEDLE
    v = torch.empty((1, SKV, 1, D), dtype=torch.bfloat16, device=DEV)
    d = torch.arange(D, dtype=torch.int32, device=DEV)[None, :]
    step = 1 << 20
    for j0 in range(0, SKV, step):
        j = torch.arange(j0, min(j0 + step, SKV), dtype=torch.int32, device=DEV)[:, None]
        v[0, j0:j0 + j.shape[0], 0, :] = (((j * 7 + d * 13) % 17 - 8).to(torch.float32) / 8).to(torch.bfloat16)
    q = torch.zeros((1, 2, HQ, D), dtype=torch.bfloat16, device=DEV)
    for h in range(HQ):
        q[0, :, h, h] = 1.0
    # Column sums of V over the first SKV - 1 keys and over all of them, in float64 (exact).
    s_all = torch.zeros(D, dtype=torch.float64, device=DEV)
    for j0 in range(0, SKV - 1, step):
        s_all += v[0, j0:min(j0 + step, SKV - 1), 0, :].double().sum(dim=0)
    sums = [s_all.cpu().numpy(), (s_all + v[0, SKV - 1, 0, :].double()).cpu().numpy()]
    torch.cuda.synchronize()
    yield q, k, v, sums
    del k, v
    torch.cuda.empty_cache()


def expected(v, sums):
    e = math.exp(NEEDLE / math.sqrt(D))
    want = np.zeros((1, 2, HQ, D))
    for i in range(2):
        n = SKV - 1 + i
        for h in range(HQ):
            vj = v[0, J[h], 0, :].double().cpu().numpy()
            want[0, i, h] = (e * vj + (sums[i] - vj)) / (e + n - 1)
    return want


@pytest.mark.parametrize("n_split", [None, "auto"])
def test_largest_kv_head(inputs, n_split):
    q, k, v, sums = inputs
    print(f"case max-size MQA decode, Skv={SKV}, n_split={n_split}", flush=True)
    out = attn.fwd(q, k, v, causal="bottom_right", n_split=n_split)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    want = expected(v, sums)
    err = float(np.max(np.abs(got - want)))
    print(f"  max-abs {err:.3e}", flush=True)
    assert err <= 2e-2, err
    # The answer is essentially the needle's value row, unlike V's mean.
    assert float(np.max(np.abs(want[0, :, :, :] - v[0, J, 0, :].double().cpu().numpy()[None]))) < 1e-4


def test_largest_query_tensor():
    """q and out of 2^31 - 384 elements (16,777,213 query rows of one head,
    D = 128) against 70 keys, top-left causal: query offsets run up to just
    below 2^32 bytes. Sampled rows against the fp64 oracle (each needs only
    its own query row and the 70 keys), among them the first and last rows
    and rows on either side of the 2 GiB offset."""
    from tests import helpers
    print(f"case max-size query tensor, Sq={SKV}, Skv=70", flush=True)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(41)
    q = torch.empty((1, SKV, 1, D), dtype=torch.bfloat16, device=DEV)
    step = 1 << 20
    for i0 in range(0, SKV, step):
        n = min(step, SKV - i0)
        q[0, i0:i0 + n, 0, :] = torch.randn((n, D), generator=gen, device=DEV).to(torch.bfloat16)
    kv = torch.randn((2, 1, 70, 1, D), generator=gen, device=DEV).to(torch.bfloat16)
    k, v = kv[0].contiguous(), kv[1].contiguous()
    out = attn.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    half = (1 << 30) // D                        # the row starting at byte 2^31
    rows = sorted({0, 1, 63, 69, 70, 71, half - 1, half, half + 1, SKV - 65, SKV - 2, SKV - 1,
                   *np.random.default_rng(41).integers(0, SKV, 16).tolist()})
    idx = torch.tensor(rows, device=DEV)
    got = helpers.out_to_f64(out[0, idx, 0, :])
    qs = q[0, idx, 0, :].cpu()
    kc, vc = k.cpu(), v.cpu()
    want = np.stack([oracle_row(qs[r], kc, vc, i) for r, i in enumerate(rows)])
    err = helpers.max_abs_err(got, want)
    print(f"  {len(rows)} rows, max-abs {err:.3e}", flush=True)
    assert err <= 2e-2, err


def oracle_row(qrow, k, v, i):
    import oracle
    from tests import helpers
    return oracle.sdpa_one_row(helpers.to_f64(qrow, "bf16"), helpers.to_f64(k[0, :, 0], "bf16"),
                               helpers.to_f64(v[0, :, 0], "bf16"), i=i, scale=1.0 / math.sqrt(D), causal=True)
