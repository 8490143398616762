"""FP8 delayed scaling, written out plainly (test infrastructure only).

[Attention codelab §10] runs attention in FP8 under TransformerEngine's
delayed-scaling recipe: it keeps an absolute-maximum history per tensor and
derives the scaling factors from it, with margin 0, the HYBRID format pair
(E4M3 for the forward pass, E5M2 for the backward pass), a history of 1024
entries and the maximum as the reduction over the history.

Reading taken of the parts the codelab leaves open (the recipe's usual
meaning):

* A tensor's state is (history[1024], scale, scale_inv). It starts with an
  all-zero history and scale = scale_inv = 1.
* A step quantises the tensor with the *current* scale (delayed: computed
  from earlier steps): codes = encode(float32(x * scale)), nearest-even and
  saturating at the format's largest finite value; and records amax(|x|) of
  this step in history slot (step mod 1024).
* The update after the step sets amax = max(history) and, when amax is
  finite and positive and the quotient s = float32(fmax / amax) / 2^margin
  (margin 0: fmax / amax, one binary32 division) is finite too, scale = s
  and scale_inv = float32(1 / scale); otherwise both stay. (The quotient
  overflows for amax below fmax / FLT_MAX, about 1.3e-36 for E4M3; the
  codelab's recipe states no rule for it, and keeping the last finite scale
  keeps scale_inv a usable, non-zero dequantisation factor.) The step counter then advances and the slot the next
  step writes is cleared, so the history always holds the last (up to) 1024
  recorded amaxes.

Pins: tests/test_oracle_fp8_scaling.py.
"""

import numpy as np

from .codecs import E4M3_MAX, E5M2_MAX, f64_to_e4m3_bits, f64_to_e5m2_bits

__all__ = ["AMAX_HISTORY_LEN", "FORMAT_MAX", "DelayedScalingState", "quantize_with_scale"]

AMAX_HISTORY_LEN = 1024
FORMAT_MAX = {"e4m3": E4M3_MAX, "e5m2": E5M2_MAX}


def quantize_with_scale(x, scale, fmt):
    """FP8 codes of float32(x * scale), nearest-even, saturating (uint8 array)."""
    with np.errstate(invalid="ignore", over="ignore"):
        y = np.asarray(x, dtype=np.float32) * np.float32(scale)  # one binary32 product per element
    return f64_to_e4m3_bits(y) if fmt == "e4m3" else f64_to_e5m2_bits(y)


class DelayedScalingState:
    """The per-tensor state of the delayed-scaling recipe (margin 0, max over
    a history of AMAX_HISTORY_LEN)."""

    def __init__(self, fmt, history_len=AMAX_HISTORY_LEN, margin=0):
        if fmt not in FORMAT_MAX:
            raise ValueError(fmt)
        self.fmt = fmt
        self.history = np.zeros(history_len, dtype=np.float32)
        self.scale = np.float32(1.0)
        self.scale_inv = np.float32(1.0)
        self.step = 0
        self.margin = margin

    def quantize(self, x):
        """Codes of x under the current scale; records amax(|x|) for this step."""
        x = np.asarray(x, dtype=np.float32)
        codes = quantize_with_scale(x, self.scale, self.fmt)
        amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
        slot = self.step % len(self.history)
        self.history[slot] = np.maximum(self.history[slot], amax)   # NaN propagates
        return codes

    def update(self):
        """New scale from the history's maximum; advance to the next step."""
        amax = np.float32(np.max(self.history))
        if np.isfinite(amax) and amax > 0:
            with np.errstate(over="ignore"):
                s = np.float32(np.float32(FORMAT_MAX[self.fmt]) / amax)
                s = np.float32(s / np.float32(2.0 ** self.margin))
            if np.isfinite(s):
                self.scale = s
                self.scale_inv = np.float32(np.float32(1.0) / s)
        self.step += 1
        self.history[self.step % len(self.history)] = np.float32(0.0)
