"""Pins of the oracle's time-step and rate preparation (and its gradients).

- closed forms of softplus: log 2 at zero, softplus(v) - softplus(-v) = v,
  e^v for very negative v, numpy's logaddexp(0, v) for the per-head bias;
- the rate A = -exp(logA) and the retention bound 0 < exp(dt*A) <= 1
  ("Nemotron 3 Ultra: replaying a rounded state", section "The Mamba state
  update", theorem retention_bounds);
- the clamp ("Nemotron Kernels: From Inference To Backpropagation", section
  "From Classical State Space To A Selective Mamba State"): outputs inside the
  closed interval, zero gradient where saturated, the gradient passing at the
  exact boundary (the declared convention);
- central finite differences of the preparation alone and of the preparation
  composed with the oracle's scan, so that d raw, d bias and d logA are checked
  against the derivative of a loss through the whole forward;
- the softplus threshold branch: above 20 the float32 value of the
  mathematical softplus is the input itself, so the branch changes nothing in
  float32 (reading recorded with the oracle).
"""
import numpy as np
import pytest

from oracle import oracle

INF = float("inf")


def test_softplus_closed_forms():
    dt, _ = oracle.dt_prep(np.zeros((1, 1)), np.zeros(1), np.zeros(1))
    assert dt[0, 0] == pytest.approx(np.log(2.0), rel=1e-15)
    v = np.linspace(-30.0, 30.0, 121)
    pos, _ = oracle.dt_prep(v[:, None], np.zeros(1), np.zeros(1))
    neg, _ = oracle.dt_prep(-v[:, None], np.zeros(1), np.zeros(1))
    assert np.allclose(pos[:, 0] - neg[:, 0], v, rtol=0, atol=1e-13)
    tiny, _ = oracle.dt_prep(np.array([[-40.0]]), np.zeros(1), np.zeros(1))
    assert tiny[0, 0] == pytest.approx(np.exp(-40.0), rel=1e-15)
    # the bias is per head (last axis) and enters before the softplus
    r = np.random.default_rng(3)
    bias = r.normal(0.0, 3.0, 7)
    raw = r.normal(0.0, 2.0, (4, 7))
    dt, _ = oracle.dt_prep(raw, bias, np.zeros(7))
    assert np.allclose(dt, np.logaddexp(0.0, raw + bias[None, :]), rtol=1e-14, atol=0)


def test_rate_and_retention_bound():
    r = np.random.default_rng(4)
    logA = np.concatenate([r.uniform(-30.0, 30.0, 40), [0.0, np.log(16.0)]])
    raw = r.uniform(-50.0, 50.0, (64, logA.size))
    bias = r.normal(0.0, 1.0, logA.size)
    dt, A = oracle.dt_prep(raw, bias, logA)
    assert np.all(A < 0)
    assert np.allclose(np.log(-A), logA, rtol=0, atol=1e-14)
    assert A[-2] == -1.0 and A[-1] == pytest.approx(-16.0, rel=1e-15)
    assert np.all(dt > 0)
    z = dt * A[None, :]  # the retention is exp(z): in (0, 1] exactly when z <= 0 is finite
    assert np.all(np.isfinite(z)) and np.all(z <= 0.0)
    a = np.exp(z[z > -700.0])
    assert np.all(a > 0) and np.all(a <= 1.0)


def test_clamp_interval_and_boundary_convention():
    lo, hi = 0.05, 0.3
    r = np.random.default_rng(5)
    raw = r.normal(-2.0, 0.8, (400, 3))
    bias = np.array([0.0, 0.4, -0.4])
    dt, _ = oracle.dt_prep(raw, bias, np.zeros(3), lo, hi)
    sp = np.logaddexp(0.0, raw + bias)
    assert np.all(dt >= np.float32(lo)) and np.all(dt <= np.float32(hi))
    low, high = sp < np.float32(lo), sp > np.float32(hi)
    assert low.sum() > 20 and high.sum() > 20  # both ends are exercised
    assert np.all(dt[low] == np.float32(lo)) and np.all(dt[high] == np.float32(hi))
    ddt = r.standard_normal(raw.shape)
    d_raw, d_bias, _ = oracle.dt_prep_bwd(raw, bias, np.zeros(3), ddt, np.zeros(3), lo, hi)
    assert np.all(d_raw[low | high] == 0.0)
    mid = ~(low | high)
    sig = 1.0 / (1.0 + np.exp(-(raw + bias)))
    assert np.allclose(d_raw[mid], (ddt * sig)[mid], rtol=1e-14, atol=0)
    assert np.allclose(d_bias, d_raw.sum(axis=0), rtol=1e-13, atol=0)
    # exactly on either end: float32(softplus(24)) == 24 and float32(softplus(21)) == 21,
    # so these sit on the interval's ends and keep their gradient; 24.5 is outside
    raw_b = np.array([[24.0], [21.0], [24.5], [20.5]])
    dt_b, _ = oracle.dt_prep(raw_b, np.zeros(1), np.zeros(1), 21.0, 24.0)
    assert list(dt_b[:, 0]) == pytest.approx([24.0, 21.0, 24.0, 21.0], abs=1e-9)
    g, _, _ = oracle.dt_prep_bwd(raw_b, np.zeros(1), np.zeros(1), np.ones((4, 1)), np.zeros(1),
                                 21.0, 24.0)
    assert g[0, 0] == pytest.approx(1.0, abs=1e-9) and g[1, 0] == pytest.approx(1.0, abs=1e-9)
    assert g[2, 0] == 0.0 and g[3, 0] == 0.0


def test_threshold_branch_changes_nothing_in_float32():
    x = np.float32(20.0) + np.arange(0, 200000, dtype=np.float32) * np.float32(3e-4)
    dt, _ = oracle.dt_prep(x.astype(np.float64)[:, None], np.zeros(1), np.zeros(1))
    assert np.array_equal(dt[:, 0].astype(np.float32), x)
    g, _, _ = oracle.dt_prep_bwd(x.astype(np.float64)[:, None], np.zeros(1), np.zeros(1),
                                 np.ones((x.size, 1)), np.zeros(1))
    assert np.all(g[:, 0].astype(np.float32) == np.float32(1.0))


def test_gradients_of_the_preparation_by_finite_differences():
    lo, hi = 0.05, 0.3
    r = np.random.default_rng(6)
    rows, H = 9, 4
    raw = r.normal(-2.0, 0.8, (rows, H))
    bias = r.normal(0.0, 0.3, H)
    logA = r.uniform(0.0, np.log(16.0), H)
    w = r.standard_normal((rows, H))
    u = r.standard_normal(H)

    def loss(rw, b, la):
        dt, A = oracle.dt_prep(rw, b, la, lo, hi)
        return float(np.sum(w * dt) + np.sum(u * A))

    d_raw, d_bias, d_logA = oracle.dt_prep_bwd(raw, bias, logA, w, u, lo, hi)
    eps = 1e-6
    sp = np.logaddexp(0.0, raw + bias)
    far = (np.abs(sp - lo) > 1e-4) & (np.abs(sp - hi) > 1e-4)
    assert far.all()  # no finite-difference step crosses an end of the interval
    for i in range(rows):
        for h in range(H):
            e = np.zeros_like(raw)
            e[i, h] = eps
            fd = (loss(raw + e, bias, logA) - loss(raw - e, bias, logA)) / (2 * eps)
            assert fd == pytest.approx(d_raw[i, h], rel=1e-7, abs=1e-9)
    for h in range(H):
        e = np.zeros(H)
        e[h] = eps
        fd = (loss(raw, bias + e, logA) - loss(raw, bias - e, logA)) / (2 * eps)
        assert fd == pytest.approx(d_bias[h], rel=1e-7, abs=1e-9)
        fd = (loss(raw, bias, logA + e) - loss(raw, bias, logA - e)) / (2 * eps)
        assert fd == pytest.approx(d_logA[h], rel=1e-7, abs=1e-9)


@pytest.mark.parametrize("lo,hi", [(0.0, INF), (0.06, 0.25)])
def test_chain_through_the_scan_by_finite_differences(lo, hi):
    """d bias and d logA of L = sum dy * y, where the scan's dt and A come from the
    preparation: the oracle's reverse sweep gives ddt and dA, the preparation's
    backward carries them to the parameters."""
    b, t, h, p, n, g = 2, 6, 4, 3, 4, 2
    r = np.random.default_rng(7)
    x = r.standard_normal((b, t, h, p))
    B = r.standard_normal((b, t, g, n)) / 2
    C = r.standard_normal((b, t, g, n)) / 2
    D = r.standard_normal(h)
    dy = r.standard_normal((b, t, h, p))
    raw = r.normal(-2.0, 0.8, (b, t, h))
    bias = r.normal(0.0, 0.3, h)
    logA = r.uniform(0.0, np.log(8.0), h)

    def loss(rw, bi, la):
        dt, A = oracle.dt_prep(rw, bi, la, lo, hi)
        return float(np.sum(dy * oracle.fwd(x, B, C, dt, A, D)["y"]))

    dt, A = oracle.dt_prep(raw, bias, logA, lo, hi)
    gr = oracle.bwd(x, B, C, dt, A, D, dy)
    d_raw, d_bias, d_logA = oracle.dt_prep_bwd(raw, bias, logA, gr["ddt"], gr["dA"], lo, hi)
    sp = np.logaddexp(0.0, raw + bias)
    assert np.all((np.abs(sp - lo) > 1e-4) & (np.abs(sp - hi) > 1e-4))
    eps = 1e-6
    for k in range(h):
        e = np.zeros(h)
        e[k] = eps
        fd = (loss(raw, bias + e, logA) - loss(raw, bias - e, logA)) / (2 * eps)
        assert fd == pytest.approx(d_bias[k], rel=1e-6, abs=1e-8)
        fd = (loss(raw, bias, logA + e) - loss(raw, bias, logA - e)) / (2 * eps)
        assert fd == pytest.approx(d_logA[k], rel=1e-6, abs=1e-8)
    for idx in [(0, 0, 0), (1, 5, 3), (0, 3, 2), (1, 2, 1)]:
        e = np.zeros_like(raw)
        e[idx] = eps
        fd = (loss(raw + e, bias, logA) - loss(raw - e, bias, logA)) / (2 * eps)
        assert fd == pytest.approx(d_raw[idx], rel=1e-6, abs=1e-8)
