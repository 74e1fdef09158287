"""Pins of the oracle's forward recurrence against things other than itself.

- the pages' worked SSM.step example (golden/ssm_step_example.json);
- the geometric-series closed form for constant inputs;
- P = N = 1 reduces to a first-order IIR filter: scipy.signal.lfilter;
- the group map g(h) = h // (H/G): a head reads only its own group's B and C;
- chunk_states[c] is the state after exactly c*L tokens (brute-force prefix runs);
- "full-sequence scan and repeated one-token decode agree" (Nemotron Kernels:
  From Inference To Backpropagation, Kernel 1, prefill/decode paragraph);
- the retention exp(dt*A) of every generated input lies in (0, 1]
  (Nemotron 3 Ultra: replaying a rounded state, "The Mamba state update").
"""
import json
import os

import numpy as np
import pytest
import scipy.signal
import torch

from backward_mamba_ssd_amd import inputs
from oracle import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def _rand_problem(b=2, t=9, h=4, p=3, n=5, g=2, seed=0):
    r = np.random.default_rng(seed)
    return dict(
        x=r.standard_normal((b, t, h, p)),
        B=r.standard_normal((b, t, g, n)) / np.sqrt(n),
        C=r.standard_normal((b, t, g, n)) / np.sqrt(n),
        dt=np.log1p(np.exp(r.normal(-2, 0.5, (b, t, h)))),
        A=-np.exp(r.uniform(0, np.log(16), h)),
        D=r.standard_normal(h),
    )


def test_worked_step_example():
    gold = json.load(open(os.path.join(GOLD, "ssm_step_example.json")))
    x = np.array(gold["value"]).reshape(1, 1, 1, 1)
    B = np.array(gold["write"]).reshape(1, 1, 1, 2)
    C = np.array(gold["read"]).reshape(1, 1, 1, 2)
    dt = np.ones((1, 1, 1))
    A = np.zeros(1)  # retention exp(1*0) = 1
    D = np.zeros(1)
    h0 = np.array(gold["state"]).reshape(1, 1, 1, 2)
    out = oracle.fwd(x, B, C, dt, A, D, h0=h0)
    assert out["y"].reshape(-1).tolist() == gold["output"]
    # reading the state before the update would have given 10
    assert out["h_final"].reshape(-1).tolist() == [12.0, 0.0]


@pytest.mark.parametrize("a_is_one", [False, True])
def test_constant_input_closed_form(a_is_one):
    P, N, T = 3, 4, 40
    r = np.random.default_rng(7)
    xv = r.standard_normal(P)
    Bv = r.standard_normal(N)
    Cv = r.standard_normal(N)
    dtv = 0.3
    Av = 0.0 if a_is_one else -0.7
    Dv = 0.4
    h0 = r.standard_normal((P, N))
    x = np.broadcast_to(xv, (1, T, 1, P))
    B = np.broadcast_to(Bv, (1, T, 1, N))
    C = np.broadcast_to(Cv, (1, T, 1, N))
    dt = np.full((1, T, 1), dtv)
    out = oracle.fwd(x, B, C, dt, np.array([Av]), np.array([Dv]), h0=h0[None, None])
    a = np.exp(dtv * Av)
    W = dtv * np.outer(xv, Bv)
    for i in range(T):
        k = i + 1
        geo = k if a_is_one else (1 - a ** k) / (1 - a)
        h_i = a ** k * h0 + W * geo
        y_i = h_i @ Cv + Dv * xv
        np.testing.assert_allclose(out["y"][0, i, 0], y_i, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out["h_final"][0, 0], h_i, rtol=1e-12, atol=1e-12)


def test_scalar_state_is_first_order_iir_filter():
    T = 300
    r = np.random.default_rng(11)
    x = r.standard_normal(T)
    dtv, Av, Bv, Cv, Dv = 0.17, -1.3, 0.8, -1.7, 0.25
    a = np.exp(dtv * Av)
    ref = scipy.signal.lfilter([Cv * Bv * dtv], [1.0, -a], x) + Dv * x
    out = oracle.fwd(x.reshape(1, T, 1, 1), np.full((1, T, 1, 1), Bv), np.full((1, T, 1, 1), Cv),
                     np.full((1, T, 1), dtv), np.array([Av]), np.array([Dv]))
    np.testing.assert_allclose(out["y"].reshape(-1), ref, rtol=1e-12, atol=1e-12)


def test_group_map_contiguous_blocks():
    pr = _rand_problem(b=1, t=6, h=6, p=2, n=3, g=3, seed=3)  # 2 heads per group
    base = oracle.fwd(**pr)["y"]
    for g in range(3):
        pert = {k: v.copy() for k, v in pr.items()}
        pert["B"][:, :, g] += 1.0
        pert["C"][:, :, g] -= 0.5
        y = oracle.fwd(**pert)["y"]
        changed = [not np.array_equal(y[:, :, hh], base[:, :, hh]) for hh in range(6)]
        assert changed == [hh // 2 == g for hh in range(6)]


@pytest.mark.parametrize("L", [1, 3, 4, 9, 20])
def test_chunk_states_are_prefix_states(L):
    pr = _rand_problem(b=2, t=9, seed=5)
    h0 = rng.standard_normal((2, 4, 3, 5))
    out = oracle.fwd(**pr, h0=h0, chunk=L, want_chunk_states=True)
    cs = out["chunk_states"]
    nc = (9 + L - 1) // L
    assert cs.shape[2] == nc
    np.testing.assert_array_equal(cs[:, :, 0], h0)
    for c in range(1, nc):
        sub = {k: (v[:, : c * L] if k in ("x", "B", "C", "dt") else v) for k, v in pr.items()}
        pref = oracle.fwd(**sub, h0=h0)["h_final"]
        np.testing.assert_array_equal(cs[:, :, c], pref)


def test_prefill_equals_repeated_decode():
    pr = _rand_problem(b=2, t=11, seed=9)
    h0 = rng.standard_normal((2, 4, 3, 5))
    out = oracle.fwd(**pr, h0=h0)
    state = h0.copy()
    for t in range(11):
        y = oracle.decode_step(state, pr["x"][:, t], pr["B"][:, t], pr["C"][:, t], pr["dt"][:, t],
                               pr["A"], pr["D"])
        np.testing.assert_array_equal(y, out["y"][:, t])
    np.testing.assert_array_equal(state, out["h_final"])


def test_generated_retention_in_unit_interval():
    for name in ("tiny_f32", "prefill_b4_t4096"):
        w = inputs.WORKLOADS[name]
        dt = inputs.draw("dt", (2, 64, w.nheads), w.seed)
        A = inputs.draw("A", (w.nheads,), w.seed)
        a = torch.exp(dt.double() * A.double())
        assert bool((dt > 0).all()) and bool((A < 0).all())
        assert bool((a > 0).all()) and bool((a <= 1).all())


def test_linear_in_inputs_with_zero_state():
    """With h0 = 0 and fixed dt, B, C, the map x -> y is linear (superposition)."""
    pr = _rand_problem(seed=21)
    x2 = np.random.default_rng(22).standard_normal(pr["x"].shape)
    y1 = oracle.fwd(**pr)["y"]
    y2 = oracle.fwd(**{**pr, "x": x2})["y"]
    y12 = oracle.fwd(**{**pr, "x": 2.0 * pr["x"] - 3.0 * x2})["y"]
    np.testing.assert_allclose(y12, 2.0 * y1 - 3.0 * y2, rtol=1e-12, atol=1e-12)
