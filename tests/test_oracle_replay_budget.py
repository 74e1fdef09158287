"""Pins of replay, the checkpoint error budget, the drift identities and the
storage counts, all from "Nemotron 3 Ultra: replaying a rounded state":

- "Recovering the state by replay": the s' = s + u example (10, 2, -3 -> 9;
  then 4 -> 13) and the identity that exact replay of the retained inputs from
  a saved state reproduces the live state and every output bit for bit;
- "An error budget for checkpoint writes": budgets 0.1 then 0.125, and the
  at-most-one-delta-per-write bound for 0 <= L <= 1;
- "Fewer writes can leave a larger error": the integer-grid cancellation
  example (-2 versus -3);
- "The Mamba state update": update(S) - update(T) = a (S - T);
- "From state error to output error": the read bound e * sum|C| and the
  +-10 example giving 0.2;
- "Stochastic rounding and the mean state": averaging an ensemble commutes with
  the affine update (update_mean);
- "Counting the state and attention cache": 8 MiB, 384 MiB, 24 GiB, 6144 B per
  token, crossovers 65,536 and 32,768 tokens;
- "Losing small gradient contributions in BF16": 256 + 1 in bf16 is 256.
"""
import json
import os
from fractions import Fraction

import numpy as np
import torch

from oracle import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    return json.load(open(os.path.join(GOLD, name)))


def _problem(b, t, h, p, n, g, seed):
    r = np.random.default_rng(seed)
    return dict(
        x=r.standard_normal((b, t, h, p)),
        B=r.standard_normal((b, t, g, n)) / np.sqrt(n),
        C=r.standard_normal((b, t, g, n)) / np.sqrt(n),
        dt=np.log1p(np.exp(r.normal(-2, 0.5, (b, t, h)))),
        A=-np.exp(r.uniform(0, np.log(16), h)),
        D=r.standard_normal(h),
    ), r


def test_replay_additive_example():
    g = _gold("replay_additive.json")
    observed, final = oracle.replay_additive(g["checkpoint"], g["pending"], g["suffix"])
    assert observed == g["observed"] and final == g["final"]
    _, from_observed = oracle.replay_additive(observed, [], g["suffix"])
    assert from_observed == final
    # the same example through the SSM oracle: P = N = 1, retention 1, B = dt = 1
    u = np.array(g["pending"] + g["suffix"], np.float64)
    T = len(u)
    out = oracle.fwd(u.reshape(1, T, 1, 1), np.ones((1, T, 1, 1)), np.ones((1, T, 1, 1)),
                     np.ones((1, T, 1)), np.zeros(1), np.zeros(1),
                     h0=np.full((1, 1, 1, 1), float(g["checkpoint"])))
    assert out["y"][0, len(g["pending"]) - 1, 0, 0] == g["observed"]
    assert out["h_final"].item() == g["final"]


def test_exact_replay_reproduces_live_bit_for_bit():
    pr, r = _problem(2, 40, 4, 3, 5, 2, seed=31)
    L = 8
    live = oracle.fwd(**pr, chunk=L, want_chunk_states=True)
    cs = live["chunk_states"]
    for j in range(cs.shape[2]):
        rep = oracle.replay(cs[:, :, j], pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"],
                            t0=j * L, r=L)
        nxt = cs[:, :, j + 1] if j + 1 < cs.shape[2] else live["h_final"]
        assert np.array_equal(rep["h_final"], nxt)
        assert np.array_equal(rep["y"], live["y"][:, j * L:(j + 1) * L])


def test_checkpoint_budget_example_and_linear_bound():
    g = _gold("checkpoint_budget.json")
    got = oracle.checkpoint_budget(Fraction(g["L"]), Fraction(g["delta"]), Fraction(g["E0"]),
                                   g["chunk_lengths"])
    assert got == [Fraction(v) for v in g["budgets"]]
    r = np.random.default_rng(0)
    for _ in range(200):
        L = Fraction(int(r.integers(0, 9)), 8)
        d = Fraction(int(r.integers(0, 20)), 10)
        e0 = Fraction(int(r.integers(0, 20)), 10)
        chunks = [int(c) for c in r.integers(0, 5, int(r.integers(1, 6)))]
        b = oracle.checkpoint_budget(L, d, e0, chunks)
        assert b[-1] <= e0 + len(chunks) * d


def test_fewer_writes_can_increase_error():
    g = _gold("grid_cancellation.json")
    u = [Fraction(v) for v in g["inputs"]]
    per_token = oracle.grid_schedule_run(g["a"], 0, [[v] for v in u])
    pairs = oracle.grid_schedule_run(g["a"], 0, [u[:2], u[2:]])
    exact = Fraction(g["exact"])
    assert per_token == g["per_token_final"] and pairs == g["pairs_final"]
    assert abs(per_token - exact) == Fraction(g["per_token_error"])
    assert abs(pairs - exact) == Fraction(g["pairs_error"])


def test_difference_identity_and_nonexpansive():
    pr, r = _problem(2, 1, 4, 3, 5, 2, seed=41)
    S = r.standard_normal((2, 4, 3, 5))
    T_ = r.standard_normal((2, 4, 3, 5))
    s1, s2 = S.copy(), T_.copy()
    args = [pr[k][:, 0] for k in ("x", "B", "C", "dt")] + [pr["A"], pr["D"]]
    oracle.decode_step(s1, *args)
    oracle.decode_step(s2, *args)
    a = np.exp(pr["dt"][:, 0] * pr["A"][None, :])  # [b, h]
    np.testing.assert_allclose(s1 - s2, a[:, :, None, None] * (S - T_), rtol=1e-12, atol=1e-14)
    assert np.max(np.abs(s1 - s2)) <= np.max(np.abs(S - T_))


def test_read_error_bound_and_example():
    g = _gold("read_error_example.json")
    C = np.array(g["read"])
    e = np.array(g["state_error"])
    assert abs(C @ e - g["output_difference"]) < 1e-15
    assert abs(np.max(np.abs(e)) * np.sum(np.abs(C)) - g["bound"]) < 1e-15
    # through the oracle: two states differing by e, same token, y differs by C . (a e)
    x = np.zeros((1, 1, 1, 1))
    B = np.zeros((1, 1, 1, 2))
    out1 = oracle.fwd(x, B, C.reshape(1, 1, 1, 2), np.ones((1, 1, 1)), np.zeros(1), np.zeros(1),
                      h0=np.zeros((1, 1, 1, 2)))
    out2 = oracle.fwd(x, B, C.reshape(1, 1, 1, 2), np.ones((1, 1, 1)), np.zeros(1), np.zeros(1),
                      h0=e.reshape(1, 1, 1, 2))
    assert abs(abs(out2["y"].item() - out1["y"].item()) - g["output_difference"]) < 1e-15


def test_update_commutes_with_ensemble_mean():
    pr, r = _problem(1, 1, 2, 3, 4, 1, seed=51)
    ens = r.standard_normal((6, 1, 2, 3, 4))
    args = [pr[k][:, 0] for k in ("x", "B", "C", "dt")] + [pr["A"], pr["D"]]
    upd = []
    for k in range(6):
        s = ens[k].copy()
        oracle.decode_step(s, *args)
        upd.append(s)
    m = ens.mean(0).copy()
    oracle.decode_step(m, *args)
    np.testing.assert_allclose(np.mean(upd, 0), m, rtol=1e-12, atol=1e-14)


def test_sr16_checkpoint_drift_contracts_by_retention():
    """Replay from an SR16 checkpoint: the difference to the live state is the
    checkpoint's rounding error times the product of retentions."""
    pr, r = _problem(1, 30, 2, 3, 4, 1, seed=61)
    h0 = (r.standard_normal((1, 2, 3, 4)) * 5).astype(np.float32)
    bits = oracle.sr16(h0, seed=3, ckpt=0)
    h16 = oracle.half_bits_to_double(bits)
    d0 = h16 - h0.astype(np.float64)
    live = oracle.fwd(**pr, h0=h0.astype(np.float64))["h_final"]
    rep = oracle.fwd(**pr, h0=h16)["h_final"]
    prod = np.exp((pr["dt"][0] * pr["A"][None, :]).sum(0))  # [h]
    np.testing.assert_allclose(rep - live, prod[None, :, None, None] * d0, rtol=1e-9,
                               atol=1e-15)


def test_storage_counts():
    g = _gold("storage_counts.json")
    blk = oracle.state_bytes(1, g["heads"], g["value_dim"], g["state_dim"], 4)
    assert g["heads"] * g["value_dim"] * g["state_dim"] == g["entries_per_block"]
    assert blk == g["fp32_bytes_per_block"] == 8 * 2 ** 20
    allb = oracle.state_bytes(g["mamba_blocks"], g["heads"], g["value_dim"], g["state_dim"], 4)
    assert allb == g["fp32_bytes_all_blocks"] == 384 * 2 ** 20
    assert g["sequences"] * allb == g["fp32_bytes_64_sequences"] == 24 * 2 ** 30
    per_tok = oracle.kv_bytes(g["attention_blocks"], 1, g["kv_heads"], g["kv_width"],
                              g["kv_bytes_per_entry"])
    assert per_tok == g["kv_bytes_per_token"]
    for bytes_per, key in ((4, "crossover_tokens_fp32_state"), (2, "crossover_tokens_fp16_state")):
        state = oracle.state_bytes(g["mamba_blocks"], g["heads"], g["value_dim"], g["state_dim"],
                                   bytes_per)
        t = g[key]
        kv = lambda n: oracle.kv_bytes(g["attention_blocks"], n, g["kv_heads"], g["kv_width"], 1)
        assert kv(t) == state and kv(t + 1) > state and kv(t - 1) < state


def test_bf16_accumulation_example():
    g = _gold("bf16_accumulation.json")
    s = torch.tensor(g["running_sum"], dtype=torch.bfloat16)
    c = torch.tensor(g["contribution"], dtype=torch.bfloat16)
    assert float(s + c) == g["bf16_result"]
    assert float(torch.tensor(257.0).to(torch.bfloat16)) == g["bf16_result"]  # RNE cast
    assert float(s.float() + c.float()) == g["fp32_result"]
