"""Seeded synthetic inputs and the named workloads (no attention arithmetic).

This module draws the inputs that both the GPU library and the CPU oracle
receive. It holds none of the attention computation: it only draws random
numbers, rounds them to the input number format with torch's own converters,
and counts the work of each workload.

Input recipe (the codelab "Accelerate attention on GPU with cuDNN and
TransformerEngine" draws Q, K and V as i.i.d. standard normals in float32 in
§3, §8, §9 and §10, then casts with ``astype(bfloat16)`` in §6):

* Q, K, V i.i.d. N(0, 1), drawn as float32 from
  ``numpy.random.Generator(PCG64)`` seeded by ``SeedSequence(seed).spawn(3)``
  (child streams 0, 1, 2 for Q, K, V);
* bfloat16 / float16 inputs: round to nearest even (torch's ``.to(dtype)``);
* E4M3 inputs: per-tensor scale s = 448 / amax(|x|) in float32 (amax == 0
  gives s = 1), codes = round-to-nearest-even of x * s as ``float8_e4m3fn``,
  and the dequantisation factor 1 / s, also float32, goes to the kernel.

Layout is contiguous (B, S, H, D), as in §3 of the codelab.
"""

from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "PAGE_SHAPES", "draw_normal", "make_inputs", "make_dout", "metric_flops",
           "bwd_metric_flops", "workload_flops", "io_bytes", "to_layout"]

DTYPES = ("f32", "bf16", "f16", "e4m3")
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16,
               "e4m3": torch.float8_e4m3fn}
ELEM_BYTES = {"f32": 4, "bf16": 2, "f16": 2, "e4m3": 1}
E4M3_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Skv: int
    D: int
    causal: object          # False, True (top-left lower triangle) or "bottom_right"
    seed: int
    note: str = field(default="", compare=False)
    n_split: object = None  # None: attn_fwd; "auto" or an int: the split-key entry point
    layout: str = "bshd"    # storage of q, k, v, out on the GPU: "bshd" (dense) or "bhsd" (transposed views)
    direction: str = "fwd"  # "fwd": the forward pass; "bwd": the backward pass (attn_bwd) of that forward
    scaling: str = "amax"   # FP8 only: "amax" (codes cast with the tensor's own amax) or "delayed"
                            # (a whole delayed-scaling step: bf16 -> E4M3 casts with device-side
                            # scaling states, the forward reading its factors on the device, update)

    @property
    def scale(self):
        """1 / sqrt(D), the codelab's default scale (§4)."""
        return 1.0 / float(np.sqrt(self.D))

    @property
    def out_dtype(self):
        return "bf16" if self.dtype == "e4m3" else self.dtype


def _mqa_seq(S):
    return Workload(f"bf16_mqa_b1_hq32_hkv1_s{S}_d128_causal", "bf16", 1, 32, 1, S, S, 128, True, S,
                    "MQA sequence sweep; seed = S, following the codelab's key(seq_len) (§8)")


def _mqa_batch(B):
    return Workload(f"bf16_mqa_b{B}_hq32_hkv1_s1024_d128_causal_bsweep", "bf16", B, 32, 1, 1024, 1024, 128,
                    True, B + 100, "MQA batch sweep; seed = B + 100, following the codelab's key(bs + 100) (§8)")


WORKLOADS = {w.name: w for w in [
    Workload("f32_mha_b1_h2_s128_d64", "f32", 1, 2, 2, 128, 128, 64, False, 0,
             "fp32 correctness case; seed 0 as the codelab's key(0) (§3)"),
    Workload("bf16_mha_b4_h16_s2048_d64_causal", "bf16", 4, 16, 16, 2048, 2048, 64, True, 2048,
             "MHA causal, head dim 64"),
    Workload("bf16_gqa_b2_hq32_hkv8_s4096_d128_causal", "bf16", 2, 32, 8, 4096, 4096, 128, True, 42,
             "headline: GQA, 4 query heads per KV head; seed 42 as the codelab's GQA cell (§9)"),
    _mqa_seq(1024), _mqa_seq(4096), _mqa_seq(16384),
    _mqa_batch(1), _mqa_batch(8), _mqa_batch(32),
    Workload("e4m3_mha_b4_h16_s4096_d128_causal", "e4m3", 4, 16, 16, 4096, 4096, 128, True, 9000,
             "FP8 E4M3 inputs, bf16 output; seed 9000 as the codelab's FP8 cell (§10)"),
    # Key-value-cache (decode) form of the GQA / MQA inference use of §9: a few
    # new queries at the end of a long cached sequence, bottom-right causal,
    # keys split over workgroups. Seeds: Skv + B.
    Workload("bf16_gqa_decode_b8_hq32_hkv8_sq1_skv16384", "bf16", 8, 32, 8, 1, 16384, 128, "bottom_right",
             16384 + 8, "decode: one new token per sequence, 16384-token cache, GQA", n_split="auto"),
    Workload("bf16_mqa_decode_b32_hq32_hkv1_sq4_skv8192", "bf16", 32, 32, 1, 4, 8192, 128, "bottom_right",
             8192 + 32, "decode: four new tokens per sequence, 8192-token cache, MQA", n_split="auto"),
    # More head dimensions and layouts: head dim 32; the headline shape with
    # q, k, v, out stored as (B, H, S, D) and handed over as strided views.
    Workload("bf16_mha_b4_h32_s2048_d32_causal", "bf16", 4, 32, 32, 2048, 2048, 32, True, 32,
             "head dim 32; seed 32"),
    Workload("bf16_gqa_b2_hq32_hkv8_s4096_d128_causal_bhsd", "bf16", 2, 32, 8, 4096, 4096, 128, True, 42,
             "headline shape, (B, H, S, D) storage, strided entry point", layout="bhsd"),
    # Backward pass (the gradients the scale of §1 exists to keep alive) of
    # the headline and of the MHA head-dim-64 forward; dout drawn by make_dout.
    Workload("bf16_gqa_b2_hq32_hkv8_s4096_d128_causal_bwd", "bf16", 2, 32, 8, 4096, 4096, 128, True, 42,
             "backward of the headline forward", direction="bwd"),
    Workload("bf16_mha_b4_h16_s2048_d64_causal_bwd", "bf16", 4, 16, 16, 2048, 2048, 64, True, 2048,
             "backward, MHA, head dim 64", direction="bwd"),
    Workload("e4m3_mha_b4_h16_s4096_d128_causal_bwd", "e4m3", 4, 16, 16, 4096, 4096, 128, True, 9000,
             "backward of the FP8 forward: E4M3 q, k, v, E5M2 dout, bf16 gradients", direction="bwd"),
    Workload("e4m3_delayed_mha_b4_h16_s4096_d128_causal", "e4m3", 4, 16, 16, 4096, 4096, 128, True, 9000,
             "FP8 forward step under delayed scaling (casts + attention + scale update)", scaling="delayed"),
]}

HEADLINE = "bf16_gqa_b2_hq32_hkv8_s4096_d128_causal"

# Shapes the codelab itself runs: the default (B=4, T=S=128, N=8, H=64) of §3
# and the MHA / GQA / MQA example of §9 (q (2,64,8,64), k/v with 8, 2, 1 heads).
PAGE_SHAPES = [
    Workload("page_default_f32", "f32", 4, 8, 8, 128, 128, 64, False, 0),
    Workload("page_default_bf16", "bf16", 4, 8, 8, 128, 128, 64, False, 0),
    Workload("page_default_bf16_causal", "bf16", 4, 8, 8, 128, 128, 64, True, 0),
    Workload("page_mha", "bf16", 2, 8, 8, 64, 64, 64, False, 42),
    Workload("page_gqa", "bf16", 2, 8, 2, 64, 64, 64, False, 42),
    Workload("page_mqa", "bf16", 2, 8, 1, 64, 64, 64, False, 42),
]


def draw_normal(seed, shapes):
    """float32 N(0,1) arrays of the given shapes from seed's child streams."""
    children = np.random.SeedSequence(seed).spawn(len(shapes))
    return [np.random.Generator(np.random.PCG64(c)).standard_normal(s, dtype=np.float32)
            for c, s in zip(children, shapes)]


def _quantise_e4m3(x32):
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0)
    s = np.float32(1.0) if amax == 0 else np.float32(np.float32(E4M3_MAX) / amax)
    codes = torch.from_numpy(x32 * s).to(torch.float8_e4m3fn)
    return codes, float(np.float32(1.0) / s)


def make_inputs(w, *, seed=None, shapes=None):
    """Draw (q, k, v, descales) for workload ``w`` as CPU torch tensors.

    ``shapes`` overrides the (B, Sq, Hq, D) / (B, Skv, Hkv, D) shapes (used by
    tests on reduced sizes). ``descales`` is (1, 1, 1) except for E4M3 inputs.
    """
    seed = w.seed if seed is None else seed
    if shapes is None:
        shapes = [(w.B, w.Sq, w.Hq, w.D), (w.B, w.Skv, w.Hkv, w.D), (w.B, w.Skv, w.Hkv, w.D)]
    x = draw_normal(seed, shapes)
    if w.dtype == "e4m3":
        qs, ks, vs = (_quantise_e4m3(a) for a in x)
        return qs[0], ks[0], vs[0], (qs[1], ks[1], vs[1])
    t = [torch.from_numpy(a).to(TORCH_DTYPE[w.dtype]) for a in x]
    return t[0], t[1], t[2], (1.0, 1.0, 1.0)


E5M2_MAX = 57344.0


def make_dout(w, seed_offset=1000):
    """The loss gradient dout for a backward workload: N(0, 1) float32 of q's
    shape from the seed w.seed + 1000 (first child stream), rounded to the
    input type like q. For E4M3 workloads the gradient is FP8 E5M2 instead:
    returns (codes, descale), with the per-tensor scale s = 57344 / amax in
    float32, codes = nearest-even E5M2 of g * s (torch's converter), and
    descale = 1 / s."""
    g = draw_normal(w.seed + seed_offset, [(w.B, w.Sq, w.Hq, w.D)])[0]
    if w.dtype == "e4m3":
        amax = np.float32(np.max(np.abs(g))) if g.size else np.float32(0)
        s = np.float32(1.0) if amax == 0 else np.float32(np.float32(E5M2_MAX) / amax)
        return torch.from_numpy(g * s).to(torch.float8_e5m2), float(np.float32(1.0) / s)
    return torch.from_numpy(g).to(TORCH_DTYPE[w.dtype])


def to_layout(x, layout):
    """A (B, S, H, D) tensor in the workload's storage: itself for "bshd"; for
    "bhsd" a (B, S, H, D) view of dense (B, H, S, D) storage of the same
    values (so the library sees a strided layout)."""
    if layout == "bshd":
        return x
    if layout == "bhsd":
        return x.transpose(1, 2).contiguous().transpose(1, 2)
    raise ValueError(layout)


def metric_flops(B, Hq, Sq, Skv, D, causal):
    """Attention forward FLOPs as the metric counts them: 4 B Hq Sq Skv D,
    halved for a (top-left) causal mask (QK^T and PV, 2 flops per
    multiply-add). For bottom-right alignment, whose queries see nearly every
    key when Sq << Skv, the visible (query, key) pairs are counted exactly:
    Sq (Skv - Sq) + Sq (Sq + 1) / 2 per head."""
    if causal == "bottom_right":
        pairs = Sq * (Skv - Sq) + Sq * (Sq + 1) / 2
        return 4.0 * B * Hq * D * pairs
    f = 4.0 * B * Hq * Sq * Skv * D
    return f / 2 if causal else f


def bwd_metric_flops(B, Hq, Sq, Skv, D, causal):
    """Backward FLOPs as counted for the metric: the five products the
    gradients need (S = Q K^T, dP = dO V^T, dV = P^T dO, dK = dS^T Q,
    dQ = dS K), i.e. 2.5 times the forward's two. The kernels compute S and
    dP twice (7 products); the recomputation is not counted."""
    return 2.5 * metric_flops(B, Hq, Sq, Skv, D, causal)


def workload_flops(w):
    f = metric_flops if w.direction == "fwd" else bwd_metric_flops
    return f(w.B, w.Hq, w.Sq, w.Skv, w.D, w.causal)


def io_bytes(w):
    """Algorithmic HBM bytes of one call. Forward: Q, K, V read once, O
    written once (a delayed-scaling step adds its casts: bf16 read, codes
    written). Backward: Q, K, V, O, dO and the row log-sum-exp read once,
    dQ, dK, dV written once (and the per-row Delta written and read)."""
    e = ELEM_BYTES[w.dtype]
    o = ELEM_BYTES[w.out_dtype]
    nq, nk = w.B * w.Sq * w.Hq * w.D, w.B * w.Skv * w.Hkv * w.D
    if w.direction == "bwd":
        rows = w.B * w.Hq * w.Sq
        g = 2   # gradients are 16-bit (bf16 for FP8 inputs)
        return nq * (e + o + e + g) + nk * (2 * e + 2 * g) + 3 * rows * 4
    if w.scaling == "delayed":   # plus the casts: bf16 in, E4M3 codes out
        return nq * (e + o) + 2 * nk * e + (nq + 2 * nk) * (2 + 1)
    return nq * (e + o) + 2 * nk * e
