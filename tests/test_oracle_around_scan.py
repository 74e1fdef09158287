"""Pins of the oracle's stages around the scan ("Nemotron Kernels: From Inference
To Backpropagation", Kernel 1 "Forward And Inference": causal Conv1D + SiLU before
the selective scan, gated group RMSNorm after it).

Short causal depthwise convolution + SiLU:
- the pre-activation is numpy.convolve of each channel's samples with the
  reversed weights ('valid' over the K-1 leading samples), and the activation is
  v * scipy.special.expit(v);
- width 1 reduces to an elementwise affine map; a unit impulse returns the
  reversed weights (the filter's impulse response);
- causality: later samples never change earlier outputs; a split run carried
  across the boundary by the final samples equals the whole run bit for bit;
- SiLU(0) = 0 and SiLU(v) - SiLU(-v) = v;
- the backward equals central finite differences (u, w, bias, initial samples),
  so the overlapping-window sums are checked.
Gated group RMSNorm:
- with eps = 0 and unit scale each group's output has mean square 1, is
  invariant to positive scaling of y and odd in y;
- a zero gate gives zero; a constant group gives w * c / sqrt(c^2 + eps);
- groups are independent;
- the backward equals central finite differences (y, z, w).
"""
import numpy as np
import pytest
from scipy.special import expit

from oracle import oracle

EPS_FD = 1e-6


def _conv_problem(b=2, t=9, c=3, k=4, seed=0, init=True):
    r = np.random.default_rng(seed)
    return (r.standard_normal((b, t, c)), r.standard_normal((c, k)) * 0.7, r.standard_normal(c),
            r.standard_normal((b, k - 1, c)) if init else None)


def test_conv_matches_numpy_convolve_and_expit():
    u, w, bias, init = _conv_problem(seed=1)
    out, fin = oracle.conv1d_silu(u, w, bias, init)
    B, T, C = u.shape
    K = w.shape[1]
    for b in range(B):
        for c in range(C):
            ext = np.concatenate([init[b, :, c], u[b, :, c]])
            v = bias[c] + np.convolve(ext, w[c, ::-1], mode="valid")
            assert v.shape == (T,)
            np.testing.assert_allclose(out[b, :, c], v * expit(v), rtol=1e-13, atol=1e-14)
            np.testing.assert_array_equal(fin[b, :, c], ext[T:])
    assert fin.shape == (B, K - 1, C)


def test_conv_width_one_and_impulse_response():
    u, w, bias, _ = _conv_problem(k=1, seed=2, init=False)
    out, _ = oracle.conv1d_silu(u, w, bias)
    v = u * w[:, 0] + bias
    np.testing.assert_allclose(out, v * expit(v), rtol=1e-13, atol=1e-14)
    # impulse at t0 in channel 1, zero bias: pre-activations are the reversed weights
    K, T, t0 = 4, 10, 3
    w = np.random.default_rng(3).standard_normal((2, K))
    u = np.zeros((1, T, 2))
    u[0, t0, 1] = 1.0
    out, _ = oracle.conv1d_silu(u, w, np.zeros(2))
    v = np.zeros(T)
    v[t0:t0 + K] = w[1, ::-1]
    np.testing.assert_allclose(out[0, :, 1], v * expit(v), rtol=1e-14, atol=0)
    np.testing.assert_array_equal(out[0, :, 0], np.zeros(T))


def test_silu_values():
    v = np.linspace(-30, 30, 61)
    u = v[None, :, None]
    pos, _ = oracle.conv1d_silu(u, np.ones((1, 1)), np.zeros(1))
    neg, _ = oracle.conv1d_silu(-u, np.ones((1, 1)), np.zeros(1))
    assert pos[0, 30, 0] == 0.0
    np.testing.assert_allclose(pos[0, :, 0] - neg[0, :, 0], v, rtol=0, atol=1e-13)


def test_conv_causal_and_split_runs():
    u, w, bias, init = _conv_problem(t=12, seed=4)
    out, fin = oracle.conv1d_silu(u, w, bias, init)
    u2 = u.copy()
    u2[:, 7:] += 5.0
    out2, _ = oracle.conv1d_silu(u2, w, bias, init)
    np.testing.assert_array_equal(out[:, :7], out2[:, :7])
    assert not np.array_equal(out[:, 7:], out2[:, 7:])
    o1, f1 = oracle.conv1d_silu(u[:, :5], w, bias, init)
    o2, f2 = oracle.conv1d_silu(u[:, 5:], w, bias, f1)
    np.testing.assert_array_equal(np.concatenate([o1, o2], axis=1), out)
    np.testing.assert_array_equal(f2, fin)
    # shorter than the window: the final samples mix init and input
    o3, f3 = oracle.conv1d_silu(u[:, :2], w, bias, init)
    np.testing.assert_array_equal(f3, np.concatenate([init[:, 2:], u[:, :2]], axis=1))


def _fd(loss, x, eps=EPS_FD):
    g = np.empty_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + eps
        lp = loss()
        x[i] = old - eps
        lm = loss()
        x[i] = old
        g[i] = (lp - lm) / (2 * eps)
    return g


def _scaled(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def test_conv_backward_equals_finite_differences():
    u, w, bias, init = _conv_problem(b=2, t=6, c=2, k=3, seed=5)
    dout = np.random.default_rng(6).standard_normal(u.shape)
    g = oracle.conv1d_silu_bwd(u, w, bias, dout, init)

    def loss():
        return float(np.sum(dout * oracle.conv1d_silu(u, w, bias, init)[0]))

    for name, arr in (("du", u), ("dw", w), ("dbias", bias), ("dinit", init)):
        err = _scaled(g[name], _fd(loss, arr))
        assert err <= 1e-7, (name, err)


def _norm_problem(rows=4, C=12, seed=0):
    r = np.random.default_rng(seed)
    return r.standard_normal((rows, C)), r.standard_normal((rows, C)), r.standard_normal(C)


def test_rmsnorm_invariants():
    y, z, _ = _norm_problem(seed=7)
    G = 3
    S = y.shape[1] // G
    out = oracle.gated_rmsnorm(y, z, np.ones(12), G, eps=0.0)
    ms = (out.reshape(-1, G, S) ** 2).mean(axis=2)
    np.testing.assert_allclose(ms, 1.0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(oracle.gated_rmsnorm(3.5 * y, z, np.ones(12), G, eps=0.0), out,
                               rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(oracle.gated_rmsnorm(-y, z, np.ones(12), G, eps=0.0), -out,
                               rtol=0, atol=0)


def test_rmsnorm_special_cases_and_group_independence():
    y, z, w = _norm_problem(seed=8)
    G = 4
    np.testing.assert_array_equal(oracle.gated_rmsnorm(y, np.zeros_like(z), w, G), np.zeros_like(y))
    # a constant gated group: out = w * c / sqrt(c^2 + eps)
    z40 = np.full_like(z, 40.0)  # SiLU(40) = 40 * (1 - 4e-18) = 40 in fp64
    c = 0.3
    yc = np.full_like(y, c / 40.0)
    out = oracle.gated_rmsnorm(yc, z40, w, G, eps=1e-5)
    np.testing.assert_allclose(out, np.broadcast_to(w * c / np.sqrt(c * c + 1e-5), y.shape),
                               rtol=1e-12, atol=0)
    base = oracle.gated_rmsnorm(y, z, w, G)
    y2 = y.copy()
    y2[:, 3:6] += 1.0  # group 1 of 4 (3 channels each)
    out2 = oracle.gated_rmsnorm(y2, z, w, G)
    changed = np.any(out2 != base, axis=0)
    assert list(np.nonzero(changed)[0]) == [3, 4, 5]


def test_rmsnorm_backward_equals_finite_differences():
    y, z, w = _norm_problem(rows=3, C=8, seed=9)
    G = 2
    dout = np.random.default_rng(10).standard_normal(y.shape)
    g = oracle.gated_rmsnorm_bwd(y, z, w, dout, G, eps=1e-3)

    def loss():
        return float(np.sum(dout * oracle.gated_rmsnorm(y, z, w, G, eps=1e-3)))

    for name, arr in (("dy", y), ("dz", z), ("dw", w)):
        err = _scaled(g[name], _fd(loss, arr))
        assert err <= 1e-7, (name, err)
