"""Number-format codecs used by the oracle (test infrastructure only).

The GPU receives inputs as raw 16-bit or 8-bit codes. The oracle decodes those
same codes itself, from the format definitions below, instead of trusting any
library's interpretation of them:

* bfloat16: the top 16 bits of an IEEE-754 binary32 (1 sign, 8 exponent,
  7 fraction bits). The codelab converts with ``astype(bfloat16)``
  [Attention codelab §6], which rounds to nearest, ties to even.
* float16: IEEE-754 binary16 (1 sign, 5 exponent bits with bias 15,
  10 fraction bits, subnormals, inf, NaN).
* E4M3 [Attention codelab §10]: 4 exponent bits and 3 mantissa bits for the
  forward pass. The reading taken is the OCP 8-bit floating point
  specification's E4M3 ("E4M3FN"): exponent bias 7, subnormals, no
  infinities, NaN only at S.1111.111, largest finite magnitude 448. The
  per-tensor scale follows the codelab's recipe with margin 0 and the
  maximum of the abs-max history; a single forward call has a one-entry
  history, so the scale is 448 / amax(|x|), with amax == 0 giving scale 1.

* E5M2 [Attention codelab §10]: 5 exponent bits and 2 mantissa bits, the
  FP8 format the codelab names for the backward pass (gradients). Reading
  taken: the OCP 8-bit floating point specification's E5M2, an IEEE-style
  format: exponent bias 15, subnormals, infinities at S.11111.00, NaN at
  S.11111.{01,10,11}, largest finite magnitude 57344. Its per-tensor scale
  follows the same recipe as E4M3's: s = 57344 / amax(|x|).

Every function is pinned in ``tests/test_codecs.py`` (all 65536 / 256 codes,
closed forms, and a cross-check against torch's own converters).
"""

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "f16_bits_to_f64",
    "e4m3_bits_to_f64",
    "f64_to_bf16_bits",
    "f64_to_e4m3_bits",
    "e4m3_amax_scale",
    "E4M3_MAX",
    "e5m2_bits_to_f64",
    "f64_to_e5m2_bits",
    "e5m2_amax_scale",
    "E5M2_MAX",
]

E4M3_MAX = 448.0
E5M2_MAX = 57344.0


def bf16_bits_to_f64(bits):
    """Decode bfloat16 codes (any integer array) to float64, exactly.

    A bfloat16 code is the upper half of a binary32 word, so placing it in the
    high 16 bits of a uint32 gives the same number as a binary32.
    """
    b = np.asarray(bits).astype(np.uint32) & np.uint32(0xFFFF)
    with np.errstate(invalid="ignore"):
        return (b << np.uint32(16)).view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits):
    """Decode IEEE binary16 codes to float64 from the field definitions."""
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    sub = sign * f * 2.0 ** -24                       # e == 0: f/1024 * 2^-14
    nor = sign * (1.0 + f / 1024.0) * np.exp2(e.astype(np.float64) - 15.0)
    special = np.where(f == 0, sign * np.inf, np.nan)  # e == 31
    return np.where(e == 0, sub, np.where(e == 31, special, nor))


def e4m3_bits_to_f64(bits):
    """Decode OCP E4M3 (E4M3FN) codes to float64 from the field definitions.

    value = (-1)^s * 2^(e-7) * (1 + m/8) for e in 1..15 (except the NaN code),
    (-1)^s * 2^-6 * (m/8) for e == 0, NaN for e == 15 and m == 7.
    """
    b = np.asarray(bits).astype(np.int64) & 0xFF
    sign = np.where((b >> 7) & 1, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    sub = sign * (m / 8.0) * 2.0 ** -6
    nor = sign * (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    val = np.where(e == 0, sub, nor)
    return np.where((e == 15) & (m == 7), np.nan, val)


def f64_to_bf16_bits(x):
    """Round binary32 values to bfloat16 codes, to nearest with ties to even.

    ``x`` is first taken as binary32 (the codelab draws float32 and casts).
    For a finite word w, the retained half is w >> 16 and the discarded half
    is w & 0xFFFF; adding 0x7FFF plus the retained half's lowest bit before
    the shift rounds up exactly when the discarded half exceeds one half ulp,
    or equals it and the retained half is odd. NaN maps to a quiet NaN code.
    """
    w = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (w >> np.uint64(16)) & np.uint64(1)
    r = ((w + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint32)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r = np.where(nan, (w >> np.uint64(16)).astype(np.uint32) | np.uint32(0x40), r)
    return r.astype(np.uint16)


def _e4m3_positive_table():
    """The 127 finite non-negative E4M3 values, indexed by their code."""
    return e4m3_bits_to_f64(np.arange(0x7F))


def f64_to_e4m3_bits(x):
    """Encode values to E4M3 codes: nearest, ties to even code, saturating.

    Written from the definition: among the finite E4M3 magnitudes pick the one
    nearest |x|; on a tie pick the code whose lowest bit is 0; magnitudes
    beyond 448 saturate to 448. NaN maps to the NaN code 0x7F with x's sign.
    """
    x = np.asarray(x, dtype=np.float64)
    table = _e4m3_positive_table()                     # increasing in the code
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(table, a, side="left")        # table[hi-1] < a <= table[hi]
    hi = np.clip(hi, 0, len(table) - 1)
    lo = np.clip(hi - 1, 0, len(table) - 1)
    dlo = a - table[lo]
    dhi = table[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == table[hi], hi, code)
    sign = np.where(np.signbit(x), 0x80, 0)
    code = np.where(np.isnan(x), 0x7F, code)
    return (code | sign).astype(np.uint8)


def e4m3_amax_scale(x):
    """Per-tensor quantisation scale s = 448 / amax(|x|) as binary32.

    The recipe of [Attention codelab §10] uses margin 0 and the maximum over
    its abs-max history; for one forward call that history holds the current
    tensor's abs-max only. An all-zero tensor gets s = 1. The dequantisation
    factor handed to the kernel is 1 / s, also as binary32.
    """
    amax = np.float32(np.max(np.abs(np.asarray(x, dtype=np.float32)))) if np.size(x) else np.float32(0)
    if amax == 0 or not np.isfinite(amax):
        return np.float32(1.0)
    return np.float32(np.float32(E4M3_MAX) / amax)


def e5m2_bits_to_f64(bits):
    """Decode OCP E5M2 codes to float64 from the field definitions.

    value = (-1)^s * 2^(e-15) * (1 + m/4) for e in 1..30, (-1)^s * 2^-14 * (m/4)
    for e == 0; e == 31 is infinity (m == 0) or NaN (m != 0).
    """
    b = np.asarray(bits).astype(np.int64) & 0xFF
    sign = np.where((b >> 7) & 1, -1.0, 1.0)
    e = (b >> 2) & 0x1F
    m = (b & 0x3).astype(np.float64)
    sub = sign * (m / 4.0) * 2.0 ** -14
    nor = sign * (1.0 + m / 4.0) * np.exp2(e.astype(np.float64) - 15.0)
    special = np.where(m == 0, sign * np.inf, np.nan)
    return np.where(e == 0, sub, np.where(e == 31, special, nor))


def f64_to_e5m2_bits(x):
    """Encode values to E5M2 codes: nearest, ties to even code, saturating.

    Among the finite E5M2 magnitudes pick the one nearest |x|; on a tie the
    code whose lowest bit is 0; magnitudes beyond 57344 (infinities included)
    saturate to 57344, as a scaled gradient must stay finite. NaN maps to
    the NaN code S.11111.10.
    """
    x = np.asarray(x, dtype=np.float64)
    table = e5m2_bits_to_f64(np.arange(0x7C))          # the 124 finite non-negative values, by code
    a = np.minimum(np.abs(x), E5M2_MAX)
    a = np.where(np.isnan(a), 0.0, a)
    hi = np.clip(np.searchsorted(table, a, side="left"), 0, len(table) - 1)
    lo = np.clip(hi - 1, 0, len(table) - 1)
    dlo = a - table[lo]
    dhi = table[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == table[hi], hi, code)
    code = np.where(np.isnan(x), 0x7E, code)
    sign = np.where(np.signbit(x), 0x80, 0)
    return (code | sign).astype(np.uint8)


def e5m2_amax_scale(x):
    """Per-tensor quantisation scale s = 57344 / amax(|x|) as binary32
    (amax == 0 gives 1); the dequantisation factor is 1 / s."""
    amax = np.float32(np.max(np.abs(np.asarray(x, dtype=np.float32)))) if np.size(x) else np.float32(0)
    if amax == 0 or not np.isfinite(amax):
        return np.float32(1.0)
    return np.float32(np.float32(E5M2_MAX) / amax)
