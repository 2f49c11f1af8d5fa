"""Pins for Smooth-QK calibration: closed forms, exact invariance of Q K^T, the gate."""
import numpy as np

from oracle import smooth


def test_closed_form_toy_maxima():
    q_cal = np.zeros((2, 3, 4), dtype=np.float16)
    k_cal = np.zeros((1, 3, 4), dtype=np.float16)
    k_cal[0, 1, :] = [16, 1, 1, 1]
    k_cal[0, 2, 3] = -1
    q_cal[0, 0, :] = [1, 4, 1, 1]
    q_cal[1, 2, :] = [-1, 1, 1, 4]
    s, inv, gate = smooth.calibrate(q_cal, k_cal, alpha=0.5, tau=4.0)
    # rho = 16 / median(16, 1, 1, 1) = 16 >= 4 -> on; s = sqrt(aK / aQ)
    assert gate
    assert np.allclose(s[0], [4.0, 0.5, 1.0, 0.5], rtol=0, atol=0)
    assert np.array_equal(inv, (1.0 / s.astype(np.float64)).astype(np.float32))
    s2, _, _ = smooth.calibrate(q_cal, k_cal, alpha=0.25, tau=4.0)
    assert np.allclose(s2[0, 0], 16 ** 0.25 / 1.0 ** 0.75, rtol=1e-7)


def test_gate_off_gives_ones():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((4, 64, 32)).astype(np.float16)
    k = rng.standard_normal((2, 64, 32)).astype(np.float16)
    s, inv, gate = smooth.calibrate(q, k, tau=4.0)
    assert not gate and np.all(s == 1) and np.all(inv == 1)


def test_rescale_is_equivalent_in_exact_arithmetic():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((4, 16, 64))
    k = rng.standard_normal((2, 16, 64))
    k[:, :, [3, 40]] *= 30
    s, inv, gate = smooth.calibrate(q.astype(np.float16), k.astype(np.float16))
    assert gate
    s64 = s.astype(np.float64)
    for h in range(4):
        g = h // 2
        lhs = (q[h] * s64[g]) @ (k[g] / s64[g]).T
        assert np.allclose(lhs, q[h] @ k[g].T, rtol=1e-12, atol=1e-12)
    # the migration balances the channel maxima when alpha = 1/2
    a_q, a_k = smooth.channel_maxima(q.astype(np.float16), k.astype(np.float16))
    assert np.allclose(a_q * s64, a_k / s64, rtol=1e-6)


def test_apply_rounds_once_to_fp32():
    x = np.array([[[[1.0009765625, -3.0]]]], dtype=np.float16)  # 1 + 2^-10
    sc = np.array([[1.0 + 2.0 ** -20, 3.0]], dtype=np.float32)
    y = smooth.apply(x, sc, [0])
    assert y.dtype == np.float32
    exact = (1 + 2.0 ** -10) * (1 + 2.0 ** -20)
    assert y[0, 0, 0, 0] == np.float32(exact) and y[0, 0, 0, 1] == -9.0
