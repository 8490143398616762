"""Pins of the FP8 delayed-scaling oracle (CPU only), and mutants.

The recipe of the codelab's §10 (TransformerEngine's DelayedScaling with
margin 0, the HYBRID E4M3 / E5M2 pair, a 1024-entry amax history reduced
with max) is checked against facts that do not come from the oracle: the
first step casts with scale 1; after a step with amax a the scale is the
binary32 quotient fmax / a; the scale follows the brute-force maximum of the
last 1024 recorded amaxes over a long random sequence; zero, infinite and NaN
maxima leave the scale alone; codes equal torch's own FP8 casts of the
binary32 products, saturated.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8_scaling as fs


def test_first_step_uses_unit_scale_and_saturates():
    st = oracle.DelayedScalingState("e4m3")
    x = np.array([0.5, -600.0, 447.9, 1e-4], np.float32)
    codes = st.quantize(x)
    assert np.array_equal(codes, oracle.f64_to_e4m3_bits(x))              # scale 1
    assert oracle.e4m3_bits_to_f64(codes[1]) == -448.0                     # saturated
    st.update()
    assert st.scale == np.float32(448.0) / np.float32(600.0)
    assert st.scale_inv == np.float32(1.0) / st.scale


def test_scale_is_fmax_over_history_max_e5m2():
    st = oracle.DelayedScalingState("e5m2")
    for a in (3.0, 7.5, 2.0):
        st.quantize(np.array([a, -a / 2], np.float32))
        st.update()
    assert st.scale == np.float32(57344.0) / np.float32(7.5)


def test_window_is_the_last_1024_amaxes():
    rng = np.random.default_rng(5)
    amaxes = np.exp(rng.normal(0, 2, 3000)).astype(np.float32)
    amaxes[10] = 1e6                                                       # leaves the window at step 1034
    st = oracle.DelayedScalingState("e4m3")
    for t, a in enumerate(amaxes):
        st.quantize(np.array([a, -a * 0.5, 0.25 * a], np.float32))
        st.update()
        window = amaxes[max(0, t - 1023): t + 1]
        assert st.scale == np.float32(np.float32(448.0) / np.float32(window.max())), t


def test_delayed_scale_is_used_by_the_next_step():
    st = oracle.DelayedScalingState("e4m3")
    st.quantize(np.array([2.0], np.float32))
    st.update()
    x = np.array([1.0, -3.0], np.float32)
    codes = st.quantize(x)                                                 # scale from step 0: 224
    want = torch.from_numpy(np.clip(x * np.float32(224.0), -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(codes, want.numpy())


def test_zero_inf_nan_amax_keep_the_scale():
    for bad in (0.0, np.inf, np.nan):
        st = oracle.DelayedScalingState("e4m3")
        st.quantize(np.array([4.0], np.float32))
        st.update()
        s0 = st.scale
        for _ in range(3):
            st.quantize(np.array([bad, 0.0], np.float32))
            st.update()
            if bad == 0.0:
                assert st.scale == s0                      # 4.0 is still in the history
            else:
                assert st.scale == s0                      # non-finite maximum: unchanged


def test_tiny_amax_keeps_a_finite_scale():
    """amax = 1e-37: fmax / amax overflows binary32, so the update keeps the
    last finite scale (here 1) and its non-zero inverse; the next cast of
    zeros and tiny values gives ordinary codes (0 for zero), no NaN codes."""
    for fmt, fmax in (("e4m3", 448.0), ("e5m2", 57344.0)):
        st = oracle.DelayedScalingState(fmt)
        st.quantize(np.array([1e-37, 0.0, -1e-38], np.float32))
        st.update()
        assert np.float32(fmax) / np.float32(1e-37) == np.inf    # the quotient does overflow
        assert st.scale == np.float32(1.0) and st.scale_inv == np.float32(1.0)
        codes = st.quantize(np.array([0.0, -0.0, 1e-37, 2.0], np.float32))
        want = torch.from_numpy(np.array([0.0, -0.0, 1e-37, 2.0], np.float32)).to(
            torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2).view(torch.uint8).numpy()
        assert np.array_equal(codes, want), (codes, want)


def test_codes_match_torch_casts():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal(20000) * 30).astype(np.float32)
    for fmt, fmax, dt in (("e4m3", 448.0, torch.float8_e4m3fn), ("e5m2", 57344.0, torch.float8_e5m2)):
        scale = np.float32(fmax / 50.0)
        y = np.clip(x * scale, -fmax, fmax)
        want = torch.from_numpy(y).to(dt).view(torch.uint8).numpy()
        assert np.array_equal(oracle.quantize_with_scale(x, scale, fmt), want)


# ---- mutants -------------------------------------------------------------------------------------

def _update_mean(self):
    amax = np.float32(np.mean(self.history[self.history > 0])) if np.any(self.history > 0) else np.float32(0)
    if amax > 0:
        self.scale = np.float32(np.float32(fs.FORMAT_MAX[self.fmt]) / amax)
        self.scale_inv = np.float32(1.0) / self.scale
    self.step += 1
    self.history[self.step % len(self.history)] = 0


def _update_no_clear(self):
    amax = np.float32(np.max(self.history))
    if np.isfinite(amax) and amax > 0:
        self.scale = np.float32(np.float32(fs.FORMAT_MAX[self.fmt]) / amax)
        self.scale_inv = np.float32(1.0) / self.scale
    self.step += 1


def _update_current_only(self):
    amax = np.float32(self.history[self.step % len(self.history)])
    if np.isfinite(amax) and amax > 0:
        self.scale = np.float32(np.float32(fs.FORMAT_MAX[self.fmt]) / amax)
        self.scale_inv = np.float32(1.0) / self.scale
    self.step += 1
    self.history[self.step % len(self.history)] = 0


def _update_any_quotient(self):
    amax = np.float32(np.max(self.history))
    if np.isfinite(amax) and amax > 0:
        with np.errstate(over="ignore", divide="ignore"):
            self.scale = np.float32(np.float32(fs.FORMAT_MAX[self.fmt]) / amax)
            self.scale_inv = np.float32(1.0) / self.scale
    self.step += 1
    self.history[self.step % len(self.history)] = 0


def _quantize_with_amax_first(self, x):
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x)))
    self.history[self.step % len(self.history)] = amax
    s = np.float32(np.float32(fs.FORMAT_MAX[self.fmt]) / amax) if amax > 0 else self.scale
    return fs.quantize_with_scale(x, s, self.fmt)                # current, not delayed, scale


PINS = [test_first_step_uses_unit_scale_and_saturates, test_scale_is_fmax_over_history_max_e5m2,
        test_window_is_the_last_1024_amaxes, test_delayed_scale_is_used_by_the_next_step,
        test_zero_inf_nan_amax_keep_the_scale, test_tiny_amax_keeps_a_finite_scale]
MUTANTS = {"mean_not_max": ("update", _update_mean), "slot_never_cleared": ("update", _update_no_clear),
           "no_history": ("update", _update_current_only), "current_scale": ("quantize", _quantize_with_amax_first),
           "overflowing_scale_adopted": ("update", _update_any_quotient)}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_scaling_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(fs.DelayedScalingState, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, name
