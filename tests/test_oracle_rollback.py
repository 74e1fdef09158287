"""Pins of the oracle's draft snapshots and rollback ("Nemotron 3 Ultra:
replaying a rounded state", section "Rolling back rejected draft tokens").

The page proves three laws for any deterministic transition; each is checked
here against the oracle's own prefill run (the sequential recurrence in C,
reached through a different entry than the one-step update the snapshots use):
- the restored snapshot is exactly the state after running the accepted prefix
  (restore_eq_prefix), for every accepted length including 0 (the initial state
  is part of the stack) and the whole draft;
- continuing from the restored state reproduces the committed run: the final
  state and all outputs of prefix + continuation (run_after_restore);
- selecting a row of the stacked snapshots is that prefix's state
  (snapshots_unstack), per sequence with different accepted lengths.
Also: rejected draft inputs influence neither the restored state nor the
accepted outputs (the page: they contribute no recurrent state or outputs).
All comparisons are bit-exact: the same fp64 arithmetic in the same order.
"""
import numpy as np

from oracle import oracle

rng = np.random.default_rng(1234)


def _problem(b=3, t=6, h=4, p=3, n=5, g=2, seed=0):
    r = np.random.default_rng(seed)
    return {
        "x": r.standard_normal((b, t, h, p)),
        "B": r.standard_normal((b, t, g, n)) / np.sqrt(n),
        "C": r.standard_normal((b, t, g, n)) / np.sqrt(n),
        "dt": np.log1p(np.exp(r.normal(-2.0, 0.5, (b, t, h)))),
        "A": -np.exp(r.uniform(0.0, np.log(16.0), h)),
        "D": r.standard_normal(h),
    }, r.standard_normal((b, h, p, n))


def test_snapshot_zero_is_the_initial_state_and_last_the_full_draft():
    pr, s0 = _problem(seed=1)
    snaps, y = oracle.draft_snapshots(s0, **pr)
    assert snaps.shape == (7,) + s0.shape
    np.testing.assert_array_equal(snaps[0], s0)
    full = oracle.fwd(**pr, h0=s0)
    np.testing.assert_array_equal(snaps[-1], full["h_final"])
    np.testing.assert_array_equal(y, full["y"])
    np.testing.assert_array_equal(oracle.rollback(snaps, [0, 0, 0]), s0)
    np.testing.assert_array_equal(oracle.rollback(snaps, [6, 6, 6]), full["h_final"])


def test_restore_equals_running_the_accepted_prefix():
    pr, s0 = _problem(seed=2)
    snaps, _ = oracle.draft_snapshots(s0, **pr)
    for acc in ([0, 1, 2], [3, 5, 6], [6, 0, 4], [1, 1, 1]):
        got = oracle.rollback(snaps, acc)
        for b, a in enumerate(acc):
            sub = {k: (v[b:b + 1, :a] if k in ("x", "B", "C", "dt") else v) for k, v in pr.items()}
            want = oracle.fwd(**sub, h0=s0[b:b + 1])["h_final"][0] if a > 0 else s0[b]
            np.testing.assert_array_equal(got[b], want)


def test_run_after_restore_preserves_the_committed_run():
    pr, s0 = _problem(seed=3)
    cont, _ = _problem(t=4, seed=4)
    cont = {k: cont[k] for k in ("x", "B", "C", "dt")}
    snaps, ydraft = oracle.draft_snapshots(s0, **pr)
    a = 2  # every sequence accepts two draft tokens
    restored = oracle.rollback(snaps, [a] * 3)
    nxt = oracle.fwd(**cont, A=pr["A"], D=pr["D"], h0=restored)
    joined = {k: np.concatenate([pr[k][:, :a], cont[k]], axis=1) for k in ("x", "B", "C", "dt")}
    whole = oracle.fwd(**joined, A=pr["A"], D=pr["D"], h0=s0)
    np.testing.assert_array_equal(nxt["h_final"], whole["h_final"])
    np.testing.assert_array_equal(np.concatenate([ydraft[:, :a], nxt["y"]], axis=1), whole["y"])


def test_rejected_inputs_leave_no_trace():
    pr, s0 = _problem(seed=5)
    acc = [1, 3, 4]
    snaps, y = oracle.draft_snapshots(s0, **pr)
    pert = {k: v.copy() for k, v in pr.items()}
    for b, a in enumerate(acc):  # change every rejected token's inputs
        for k in ("x", "B", "C"):
            pert[k][b, a:] += 1.0
        pert["dt"][b, a:] *= 2.0
    snaps2, y2 = oracle.draft_snapshots(s0, **pert)
    np.testing.assert_array_equal(oracle.rollback(snaps, acc), oracle.rollback(snaps2, acc))
    for b, a in enumerate(acc):
        np.testing.assert_array_equal(y[b, :a], y2[b, :a])
        assert not np.array_equal(snaps[-1][b], snaps2[-1][b])  # the rejected tail did change


def test_empty_draft_is_the_initial_state():
    pr, s0 = _problem(t=0, seed=6)
    snaps, y = oracle.draft_snapshots(s0, **pr)
    assert snaps.shape[0] == 1 and y.shape[1] == 0
    np.testing.assert_array_equal(oracle.rollback(snaps, [0, 0, 0]), s0)
