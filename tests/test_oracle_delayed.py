"""Pins for the oracle's delayed scaling with an amax history (CPU only).

Independent facts used: current scaling is the special case of a history
that holds exactly this tensor's amax; an all-zero history means s = 1 (the
amax == 0 rule); the scale depends on the history only through its maximum
(order and ring position do not matter); after L further steps an old amax
has left a history of length L; an element above the recorded amax
saturates to the format maximum and is counted (closed form below); the
recorded amax is the finite maximum of |x| (numpy).
"""
import numpy as np
import pytest

import oracle
import synth


def _np_amax(xbits):
    f = synth.bf16_bits_to_f32(xbits)
    f = np.abs(f[np.isfinite(f)])
    return np.float32(f.max()) if f.size else np.float32(0)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_history_of_own_amax_is_current_scaling(fmt):
    x = synth.with_outliers_bf16(11, (256, 384))
    a = oracle.amax(x)[0]
    q, qt, s, ctr, new, pos = oracle.quantize_delayed(x, fmt, [a], 0, want_t=True)
    q2, qt2, s2, ctr2 = oracle.quantize(x, fmt, oracle.TENSOR, oracle.FROM_AMAX, want_t=True)
    assert s[0] == s2[0]
    assert np.array_equal(q, q2) and np.array_equal(qt, qt2)
    assert ctr == ctr2
    assert new[0] == a and pos == 0


def test_zero_history_means_unit_scale():
    x = synth.small_shape_bf16(12, (64, 200))
    q, _, s, ctr, new, pos = oracle.quantize_delayed(x, oracle.E4M3, np.zeros(4, np.float32), 2)
    assert s[0] == 1.0
    q2, _, _, ctr2 = oracle.quantize(x, oracle.E4M3, oracle.TENSOR, oracle.GIVEN, np.array([1.0], np.float32))
    assert np.array_equal(q, q2) and ctr == ctr2
    assert new[2] == _np_amax(x) and pos == 3


def test_scale_depends_on_history_max_only():
    x = synth.small_shape_bf16(13, (32, 160))
    h = np.array([0.5, 3.0, 1.25, 2.0], np.float32)
    ref = oracle.quantize_delayed(x, oracle.E5M2, h, 0)
    for perm_seed in range(3):
        hp = np.random.default_rng(perm_seed).permutation(h)
        for p in range(4):
            out = oracle.quantize_delayed(x, oracle.E5M2, hp, p)
            assert out[2][0] == ref[2][0] == oracle.scale_from_amax(oracle.E5M2, 3.0)
            assert np.array_equal(out[0], ref[0])


def test_history_rolls_over():
    L = 3
    h, pos = np.zeros(L, np.float32), 0
    amaxes = [8.0, 1.0, 2.0, 4.0, 0.5]
    scales = []
    for a in amaxes:
        x = synth.f32_to_bf16_bits(np.array([[a, 0.0]], np.float32))
        _, _, s, _, h, pos = oracle.quantize_delayed(x, oracle.E4M3, h, pos)
        scales.append(s[0])
    # the scale of step t comes from the amaxes of steps t-L .. t-1
    assert scales[0] == 1.0
    assert scales[1] == scales[2] == scales[3] == oracle.scale_from_amax(oracle.E4M3, 8.0)
    assert scales[4] == oracle.scale_from_amax(oracle.E4M3, 4.0)      # 8.0 has left the history
    assert sorted(h.tolist()) == [0.5, 2.0, 4.0] and pos == len(amaxes) % L


@pytest.mark.parametrize("fmt,fmax,code", [(oracle.E4M3, 448.0, 0x7E), (oracle.E5M2, 57344.0, 0x7B)])
def test_growth_past_history_saturates_and_counts(fmt, fmax, code):
    # history amax 1.0 -> s = 1/fmax exactly representable? s = fl32(1/fmax);
    # an element of 2.0 gives v = fl32(2/s) ~ 2 fmax, far above the largest
    # value that still rounds to fmax, so it saturates and is counted.
    vals = np.array([2.0, -2.0, 1.0, -0.5, 3.0, 0.0], np.float32)
    x = synth.f32_to_bf16_bits(vals).reshape(2, 3)
    q, _, s, ctr, new, _ = oracle.quantize_delayed(x, fmt, [1.0], 0)
    assert s[0] == oracle.scale_from_amax(fmt, 1.0)
    flat = q.reshape(-1)
    assert flat[0] == code and flat[1] == 0x80 | code and flat[4] == code
    assert flat[2] == code                      # |x| == history amax lands on fmax, not counted
    assert ctr["saturated"] == 3
    assert new[0] == 3.0


def test_recorded_amax_ignores_nonfinite():
    x = synth.small_shape_bf16(14, (16, 128))
    x[0, 0] = 0x7F80
    x[3, 5] = 0xFFC1
    _, _, _, ctr, new, _ = oracle.quantize_delayed(x, oracle.E4M3, [0.25, 0.0], 1)
    assert new[1] == _np_amax(x) and new[0] == np.float32(0.25)
    assert ctr["nan"] == 1 and ctr["saturated"] >= 1
