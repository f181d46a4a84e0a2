"""Pins for the causal depthwise conv1d + SiLU oracle (``oracle.ConvOracle``).

Each ``pin_*`` raises ``AssertionError`` if the oracle disagrees with a fact fixed
outside it: numpy's own convolution routine, the identity and shift kernels, the
sigmoid written through tanh, split and decode invariances, linearity and
causality.  ``test_oracle_conv_pins.py`` runs them on the committed oracle and on
deliberately broken builds.

The operation ("Understanding Mamba", aiattnstudio.link, sections 3.2 and 5.2):
a depthwise nn.Conv1d with kernel K, padding K - 1 and bias, first L outputs kept,
then SiLU.  numpy.convolve(a, v) computes sum_m a[m] v[n - m] (a true convolution),
so the cross-correlation of nn.Conv1d is numpy.convolve with the kernel reversed.
"""

from __future__ import annotations

import numpy as np


def ref_silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z * 0.5 * (1.0 + np.tanh(0.5 * z))


def random_conv_case(rng, batch=2, L=23, D=5, K=4, with_state=True, with_bias=True):
    x = rng.standard_normal((batch, L, D))
    w = rng.standard_normal((D, K))
    bias = rng.standard_normal(D) if with_bias else None
    st = rng.standard_normal((batch, D, K - 1)) if with_state else None
    return x, w, bias, st


def pin_numpy_convolve(orc):
    """pre equals numpy.convolve of the state-extended input with the reversed kernel."""
    rng = np.random.default_rng(1)
    for K in (1, 2, 3, 4):
        for with_state in (False, True):
            x, w, bias, st = random_conv_case(rng, K=K, with_state=with_state)
            pre, u, st_out = orc.conv(x, w, bias, st)
            batch, L, D = x.shape
            for b in range(batch):
                for d in range(D):
                    head = st[b, d] if st is not None else np.zeros(K - 1)
                    xe = np.concatenate([head, x[b, :, d]])           # length L + K - 1
                    full = np.convolve(xe, w[d][::-1], mode="valid")  # length L
                    ref = full + (bias[d] if bias is not None else 0.0)
                    assert np.allclose(pre[b, :, d], ref, rtol=1e-13, atol=1e-13), (K, b, d)
                    assert np.allclose(st_out[b, d], xe[L:], rtol=0, atol=0), (K, b, d)
            assert np.allclose(u, ref_silu(pre), rtol=1e-14, atol=1e-300)


def pin_identity_and_shift(orc):
    """w = e_{K-1}: pre = x + bias; w = e_k: pre_t = x_{t-(K-1-k)} (state or zero before 0)."""
    rng = np.random.default_rng(2)
    K = 4
    x, _, bias, st = random_conv_case(rng, L=9, D=3, K=K)
    for k in range(K):
        w = np.zeros((3, K))
        w[:, k] = 1.0
        pre, _, _ = orc.conv(x, w, None, st)
        lag = K - 1 - k
        for t in range(9):
            s = t - lag
            exp = x[:, s, :] if s >= 0 else st[:, :, K - 1 + s]
            assert np.array_equal(pre[:, t, :], exp), (k, t)
    w = np.zeros((3, K))
    w[:, K - 1] = 1.0
    pre, u, _ = orc.conv(x, w, bias, st)
    assert np.array_equal(pre, x + bias)


def pin_zero_padding(orc):
    """Without a state the inputs before t = 0 are zero (nn.Conv1d's padding)."""
    rng = np.random.default_rng(3)
    x, w, bias, _ = random_conv_case(rng, L=6, K=4, with_state=False)
    pre0, _, _ = orc.conv(x, w, bias, None)
    pre1, _, _ = orc.conv(x, w, bias, np.zeros((x.shape[0], x.shape[2], 3)))
    assert np.array_equal(pre0, pre1)
    # t = 0 sees only the newest tap
    assert np.allclose(pre0[:, 0, :], bias + w[:, 3] * x[:, 0, :], rtol=1e-15, atol=1e-15)


def pin_split_invariance(orc):
    """conv(x[0:L]) == conv(x[0:k]) then conv(x[k:L], state = state_out), bitwise,
    including first segments shorter than K - 1."""
    rng = np.random.default_rng(4)
    x, w, bias, st = random_conv_case(rng, L=30, K=4)
    pre, u, st_end = orc.conv(x, w, bias, st)
    for k in (0, 1, 2, 3, 7, 29, 30):
        p1, u1, s1 = orc.conv(x[:, :k], w, bias, st)
        p2, u2, s2 = orc.conv(x[:, k:], w, bias, s1)
        assert np.array_equal(np.concatenate([p1, p2], axis=1), pre), k
        assert np.array_equal(np.concatenate([u1, u2], axis=1), u), k
        assert np.array_equal(s2, st_end), k


def pin_decode_equals_prefill(orc):
    """L chained single-token steps reproduce the prefill and its final state exactly."""
    rng = np.random.default_rng(5)
    x, w, bias, st = random_conv_case(rng, L=12, K=4)
    pre, u, st_end = orc.conv(x, w, bias, st)
    state = st.copy()
    for t in range(12):
        p, uu, state = orc.step(state, x[:, t, :], w, bias)
        assert np.array_equal(p, pre[:, t, :]), t
        assert np.array_equal(uu, u[:, t, :]), t
    assert np.array_equal(state, st_end)


def pin_linearity_causality(orc):
    """pre - bias is linear in (x, state); outputs before t ignore inputs from t on."""
    rng = np.random.default_rng(6)
    x1, w, _, s1 = random_conv_case(rng, L=15, K=4)
    x2, _, _, s2 = random_conv_case(rng, L=15, K=4)
    a, c = 0.7, -1.9
    p1, _, _ = orc.conv(x1, w, None, s1)
    p2, _, _ = orc.conv(x2, w, None, s2)
    p12, _, _ = orc.conv(a * x1 + c * x2, w, None, a * s1 + c * s2)
    assert np.allclose(p12, a * p1 + c * p2, rtol=1e-12, atol=1e-12)
    x3 = x1.copy()
    x3[:, 9:, :] += 5.0
    q1, _, _ = orc.conv(x1, w, None, s1)
    q3, _, _ = orc.conv(x3, w, None, s1)
    assert np.array_equal(q1[:, :9], q3[:, :9])
    assert not np.allclose(q1[:, 9:], q3[:, 9:])


PINS = [pin_numpy_convolve, pin_identity_and_shift, pin_zero_padding, pin_split_invariance,
        pin_decode_equals_prefill, pin_linearity_causality]
