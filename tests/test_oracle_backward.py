"""Pins of the oracle's reverse sweep.

- central finite differences (fp64) of L = sum dy*y + sum dh_final*h_T with
  respect to every input, in the spirit of the gradient check of
  "Reverse-mode automatic differentiation" (OneModel docs), section 6 "Checks"
  (L = sum W*f(x) with a fixed pseudo-random W);
- hand-derived closed forms for a single token;
- group symmetry: identical heads in one group give dB, dC equal to the number
  of heads times one head's ("Nemotron Kernels: From Inference To
  Backpropagation", Kernel 1 backward: shared B/C receive the sum over the
  group's heads and channels).
"""
import numpy as np
import pytest

from oracle import oracle


def _problem(b, t, h, p, n, g, seed):
    r = np.random.default_rng(seed)
    return dict(
        x=r.standard_normal((b, t, h, p)),
        B=r.standard_normal((b, t, g, n)) / np.sqrt(n),
        C=r.standard_normal((b, t, g, n)) / np.sqrt(n),
        dt=np.log1p(np.exp(r.normal(-1.0, 0.5, (b, t, h)))),
        A=-np.exp(r.uniform(0, np.log(4), h)),
        D=r.standard_normal(h),
    ), r


def _loss(pr, h0, dy, dhf):
    out = oracle.fwd(**pr, h0=h0)
    return float(np.sum(dy * out["y"]) + np.sum(dhf * out["h_final"]))


@pytest.mark.parametrize("shape", [(1, 5, 2, 3, 4, 1), (2, 7, 4, 2, 3, 2)])
def test_finite_differences(shape):
    b, t, h, p, n, g = shape
    pr, r = _problem(*shape, seed=sum(shape))
    h0 = r.standard_normal((b, h, p, n))
    dy = r.standard_normal((b, t, h, p))
    dhf = r.standard_normal((b, h, p, n))
    grads = oracle.bwd(**pr, dy=dy, h0=h0, dh_final=dhf)
    eps = 1e-6
    named = dict(pr, h0=h0)
    gmap = {"x": "dx", "B": "dB", "C": "dC", "dt": "ddt", "A": "dA", "D": "dD", "h0": "dh0"}
    for name, gname in gmap.items():
        arr = named[name]
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            plus = {k: v.copy() for k, v in named.items()}
            minus = {k: v.copy() for k, v in named.items()}
            plus[name][idx] += eps
            minus[name][idx] -= eps
            hp = plus.pop("h0")
            hm = minus.pop("h0")
            fd[idx] = (_loss(plus, hp, dy, dhf) - _loss(minus, hm, dy, dhf)) / (2 * eps)
        an = grads[gname]
        scaled = np.max(np.abs(an - fd)) / np.max(np.abs(fd))
        assert scaled < 1e-7, (name, scaled)


def test_single_token_closed_forms():
    P, N = 3, 4
    r = np.random.default_rng(5)
    x, B, C = r.standard_normal(P), r.standard_normal(N), r.standard_normal(N)
    dtv, Av, Dv = 0.4, -0.9, 0.3
    h0 = r.standard_normal((P, N))
    dy = r.standard_normal(P)
    g = oracle.bwd(x.reshape(1, 1, 1, P), B.reshape(1, 1, 1, N), C.reshape(1, 1, 1, N),
                   np.array([[[dtv]]]), np.array([Av]), np.array([Dv]), dy.reshape(1, 1, 1, P),
                   h0=h0[None, None])
    a = np.exp(dtv * Av)
    h1 = a * h0 + dtv * np.outer(x, B)
    np.testing.assert_allclose(g["dx"].reshape(P), dy * (dtv * (C @ B) + Dv), rtol=1e-13)
    np.testing.assert_allclose(g["dB"].reshape(N), dtv * C * (dy @ x), rtol=1e-13)
    np.testing.assert_allclose(g["dC"].reshape(N), dy @ h1, rtol=1e-13)
    ddt = ((dy[:, None] * C[None, :] * np.outer(x, B)).sum()
           + (dy[:, None] * C[None, :] * h0).sum() * a * Av)
    np.testing.assert_allclose(g["ddt"].reshape(()), ddt, rtol=1e-13)
    np.testing.assert_allclose(g["dA"][0], (dy[:, None] * C[None, :] * h0).sum() * a * dtv,
                               rtol=1e-13)
    np.testing.assert_allclose(g["dD"][0], dy @ x, rtol=1e-13)
    np.testing.assert_allclose(g["dh0"][0, 0], a * np.outer(dy, C), rtol=1e-13)


def test_group_sum_of_identical_heads():
    r = np.random.default_rng(8)
    T, P, N, hpg = 6, 2, 3, 4
    one = dict(x=r.standard_normal((1, T, 1, P)), B=r.standard_normal((1, T, 1, N)),
               C=r.standard_normal((1, T, 1, N)), dt=np.full((1, T, 1), 0.3),
               A=np.array([-0.5]), D=np.array([0.2]))
    dy1 = r.standard_normal((1, T, 1, P))
    g1 = oracle.bwd(**one, dy=dy1)
    many = dict(x=np.repeat(one["x"], hpg, axis=2), B=one["B"], C=one["C"],
                dt=np.repeat(one["dt"], hpg, axis=2), A=np.repeat(one["A"], hpg),
                D=np.repeat(one["D"], hpg))
    gm = oracle.bwd(**many, dy=np.repeat(dy1, hpg, axis=2))
    np.testing.assert_allclose(gm["dB"], hpg * g1["dB"], rtol=1e-12)
    np.testing.assert_allclose(gm["dC"], hpg * g1["dC"], rtol=1e-12)
    for hh in range(hpg):
        np.testing.assert_allclose(gm["dx"][:, :, hh], g1["dx"][:, :, 0], rtol=1e-12)


def test_segment_recompute_matches_short_run():
    """T above the 256-token segment: gradients of the first tokens must not
    depend on how the reverse sweep keeps its states (compare T=300 run against
    the FD-pinned algorithm on a truncated problem with the tail's influence
    carried by dh_final)."""
    pr, r = _problem(1, 300, 2, 2, 3, 1, seed=77)
    dy = r.standard_normal((1, 300, 2, 2))
    full = oracle.bwd(**pr, dy=dy)
    # split at token 256: gradient into the state after token 255 from the tail
    head = {k: (v[:, :256] if k in ("x", "B", "C", "dt") else v) for k, v in pr.items()}
    tail = {k: (v[:, 256:] if k in ("x", "B", "C", "dt") else v) for k, v in pr.items()}
    mid = oracle.fwd(**head)["h_final"]
    gt = oracle.bwd(**tail, dy=dy[:, 256:], h0=mid)
    gh = oracle.bwd(**head, dy=dy[:, :256], dh_final=gt["dh0"])
    np.testing.assert_allclose(full["dx"][:, :256], gh["dx"], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(full["ddt"][:, 256:], gt["ddt"], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(full["dA"], gh["dA"] + gt["dA"], rtol=1e-11)
