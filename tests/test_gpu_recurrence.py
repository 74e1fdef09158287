"""GPU parity of the token-serial kernels against the fp64 oracle.

Tolerances: 1e-5 scaled error where the whole computation is fp32 on identical
inputs (states, fp32 outputs and gradients); 2e-2 for bf16-stored outputs;
bit-exact for SR16 bits and for replay against repeated decode.
"""
import numpy as np
import pytest
import torch

from backward_mamba_ssd_amd import inputs
from oracle import oracle
from tests.parity import assert_close, to_np

pytestmark = pytest.mark.gpu

dev = torch.device("cuda:0")


@pytest.fixture(scope="module")
def ssm():
    from backward_mamba_ssd_amd import ssm as m
    return m


def _decode_inputs(b, h, p, n, g, dtype, seed, steps):
    td = inputs.torch_dtype(dtype)
    return {
        "state": inputs.draw("h0", (b, h, p, n), seed, dev),
        "A": inputs.draw("A", (h,), seed, dev),
        "D": inputs.draw("D", (h,), seed, dev),
        "x": inputs.draw("x", (steps, b, h, p), seed, dev, td),
        "B": inputs.draw("B", (steps, b, g, n), seed, dev, td, dstate=n),
        "C": inputs.draw("C", (steps, b, g, n), seed, dev, td, dstate=n),
        "dt": inputs.draw("dt", (steps, b, h), seed, dev),
    }


@pytest.mark.parametrize("shape,dtype", [((3, 16, 64, 128, 2), "bf16"), ((2, 3, 8, 16, 1), "f32"),
                                         ((2, 4, 32, 64, 2), "bf16"), ((1, 2, 5, 32, 2), "f32")])
def test_decode_matches_oracle(ssm, shape, dtype):
    b, h, p, n, g = shape
    steps = 5
    pr = _decode_inputs(b, h, p, n, g, dtype, 11, steps)
    st = pr["state"].clone()
    ref_state = to_np(pr["state"]).copy()
    ytol = 2e-2 if dtype == "bf16" else 1e-5
    for k in range(steps):
        y = ssm.ssm_decode_step(st, pr["x"][k], pr["B"][k], pr["C"][k], pr["dt"][k], pr["A"],
                                pr["D"])
        ry = oracle.decode_step(ref_state, pr["x"][k], pr["B"][k], pr["C"][k], pr["dt"][k],
                                pr["A"], pr["D"])
        torch.cuda.synchronize()
        assert_close(f"y step {k}", y, ry, ytol)
    assert_close("state", st, ref_state, 1e-5)


def _sr16_bracket(v64, M, seed, step):
    """SR16 bits of every float32 value within 1e-6*M of the fp64 values v64:
    the lowest and highest (SR16 is monotone in the value for a fixed entropy
    word), from the oracle's rounding of the two ends of that interval."""
    d = 1e-6 * M + 1e-38
    lo = oracle.sr16(np.float32(v64 - d), seed, step)
    hi = oracle.sr16(np.float32(v64 + d), seed, step)
    return lo, hi


@pytest.mark.parametrize("shape,dtype,seed,step", [((3, 16, 64, 128, 2), "bf16", 2, 0),
                                                   ((2, 4, 32, 64, 2), "f32", 3, 7),
                                                   ((1, 3, 5, 32, 1), "bf16", 5, 2 ** 40 + 3)])
def test_decode_sr16_state_cache(ssm, shape, dtype, seed, step):
    """Decode on a binary16 state cache ("Nemotron 3 Ultra: replaying a rounded
    state", introduction): the stored bits are the SR16 rounding, keyed by
    (seed, step, flat element index), of the one-step update of the widened
    state.  Checked against the oracle's fp64 step: where every float32 value
    within 1e-6 of the fp64 one rounds to the same bits those bits must be
    stored; elsewhere the stored value must lie between the two possible
    roundings.  The rounding error, in units of the binary16 spacing, must
    average to zero; y equals the float32 decode of the widened state."""
    b, h, p, n, g = shape
    pr = _decode_inputs(b, h, p, n, g, dtype, 100 + seed, 1)
    s16 = inputs.draw("h0", (b, h, p, n), 100 + seed).half()
    bits0 = s16.view(torch.int16).to(dev)
    wide = oracle.half_bits_to_double(s16.view(torch.int16).numpy().view(np.uint16))
    x, B, C, dt = pr["x"][0], pr["B"][0], pr["C"][0], pr["dt"][0]

    bits = bits0.clone()
    y = ssm.ssm_decode_step_sr16(bits, x, B, C, dt, pr["A"], pr["D"], seed, step)
    st32 = s16.float().to(dev)
    y32 = ssm.ssm_decode_step(st32, x, B, C, dt, pr["A"], pr["D"])
    again = bits0.clone()
    ssm.ssm_decode_step_sr16(again, x, B, C, dt, pr["A"], pr["D"], seed, step)
    other = bits0.clone()
    ssm.ssm_decode_step_sr16(other, x, B, C, dt, pr["A"], pr["D"], seed, step + 1)
    torch.cuda.synchronize()
    assert torch.equal(y, y32)
    assert torch.equal(bits, again)

    ref = wide.copy()
    ry = oracle.decode_step(ref, x, B, C, dt, pr["A"], pr["D"])
    assert_close("y", y, ry, 2e-2 if dtype == "bf16" else 1e-5)
    got = bits.cpu().numpy().view(np.uint16)
    M = np.abs(wide) + np.abs(to_np(x)[..., None] * to_np(B).repeat(h // g, axis=1)[:, :, None, :]
                              * to_np(dt)[..., None, None])
    lo, hi = _sr16_bracket(ref, M, seed, step)
    fixed = lo == hi
    print(f"  decided by the oracle: {fixed.mean():.4f} of {fixed.size}", flush=True)
    assert fixed.mean() > 0.95
    assert np.array_equal(got[fixed], lo[fixed]), int(np.sum(got[fixed] != lo[fixed]))
    gv, lv, hv = (oracle.half_bits_to_double(a) for a in (got, lo, hi))
    assert np.all((gv >= lv) & (gv <= hv))
    # unbiased: the signed rounding error averages to zero in binary16 spacings
    spacing = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -14))) - 10)
    z = (gv - ref) / spacing
    assert np.all(np.abs(z) <= 1.0 + 1e-3)
    if z.size > 100000:
        assert abs(z.mean()) < 5e-3, z.mean()
    # a different step key changes some rounding choices
    assert not torch.equal(bits, other)


def _seq_problem(b, t, h, p, n, g, dtype, seed, h0="randn"):
    return inputs.make_problem(b, t, h, p, n, g, dtype, seed, dev, h0=h0, dh_final=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_replay_equals_repeated_decode_bitwise(ssm, dtype):
    b, t, h, p, n, g = 2, 24, 8, 64, 128, 2
    pr = _seq_problem(b, t, h, p, n, g, dtype, 21)
    y_rep = torch.zeros_like(pr["x"])
    out = ssm.ssm_replay(pr["h0"], pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], 3, 17,
                         y=y_rep)
    st = pr["h0"].clone()
    for k in range(3, 20):
        y = ssm.ssm_decode_step(st, pr["x"][:, k].contiguous(), pr["B"][:, k].contiguous(),
                                pr["C"][:, k].contiguous(), pr["dt"][:, k].contiguous(), pr["A"],
                                pr["D"])
        assert torch.equal(y, y_rep[:, k]), k
    torch.cuda.synchronize()
    assert torch.equal(st, out["state"])


def test_replay_matches_oracle(ssm):
    b, t, h, p, n, g = 2, 40, 8, 64, 128, 4
    pr = _seq_problem(b, t, h, p, n, g, "bf16", 31)
    y = torch.zeros_like(pr["x"])
    out = ssm.ssm_replay(pr["h0"], pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], 7, 30,
                         y=y)
    ref = oracle.replay(pr["h0"], pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], 7, 30)
    torch.cuda.synchronize()
    assert_close("state", out["state"], ref["h_final"], 1e-5)
    assert_close("y", y[:, 7:37], ref["y"], 2e-2)


def test_exact_replay_reproduces_checkpoints(ssm):
    """Live run with checkpoints every 16 tokens; replay from each fp32 checkpoint
    reproduces the next one bit for bit (TorchLean page, "Recovering the state
    by replay")."""
    b, t, h, p, n, g, L = 2, 64, 4, 64, 128, 2, 16
    pr = _seq_problem(b, t, h, p, n, g, "bf16", 41)
    ck = [pr["h0"].clone()]
    for j in range(t // L):
        ck.append(ssm.ssm_replay(ck[-1], pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"],
                                 j * L, L)["state"])
    for j in range(t // L):
        again = ssm.ssm_replay(ck[j], pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"],
                               j * L, L)["state"]
        assert torch.equal(again, ck[j + 1])
    whole = ssm.ssm_replay(ck[0], pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], 0, t)
    assert torch.equal(whole["state"], ck[-1])


@pytest.mark.parametrize("shape", [(11, 100, 4, 70), (16, 256, 8, 16), (2, 8, 2, 0)])
def test_replay_from_binary16_checkpoint(ssm, shape):
    """Replay from SR16 bits equals replay from the same values widened to float32, state
    and y bit for bit (the two checkpoint types take different load paths into the same
    update; TorchLean page, "Recovering the state by replay").  1100 and 4096 (batch, head)
    pairs fill the GPU more than once, 70 tokens need a second retention refresh, r = 0
    returns the widened checkpoint."""
    b, h, g, r = shape
    t = r + 5
    pr = _seq_problem(b, t, h, 64, 128, g, "bf16", 61)
    bits = ssm.ssm_checkpoint_sr16(pr["h0"] * 3.0, 9, 1, 0)
    wide = bits.view(torch.float16).float()
    y_bits, y_wide = torch.zeros_like(pr["x"]), torch.zeros_like(pr["x"])
    got = ssm.ssm_replay(bits, pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], 2, r,
                         y=y_bits)["state"]
    want = ssm.ssm_replay(wide, pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], 2, r,
                          y=y_wide)["state"]
    alone = ssm.ssm_replay(bits, pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], 2, r)["state"]
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    assert torch.equal(alone, want)
    assert torch.equal(y_bits, y_wide)
    if r == 0:
        assert torch.equal(got, wide)


def test_sr16_bits_match_oracle(ssm):
    r = np.random.default_rng(5)
    vals = np.concatenate([
        (r.standard_normal(200000) * 10.0 ** r.integers(-9, 6, 200000)),
        r.uniform(-7e-8, 7e-8, 5000),
        [0.0, -0.0, np.inf, -np.inf, np.nan, 65504.0, 65519.0, 65520.0, 65535.9, 65536.0, 1e30,
         -65512.0, 2.0 ** -25, 2.0 ** -24, 1023.5 * 2.0 ** -24, 2047.5, 1.0 + 2.0 ** -12,
         1e-40, -1e-45, 6.1e-5],
    ]).astype(np.float32)
    for seed, ck, off in ((0, 0, 0), (12345, 7, 1000), (2 ** 63 + 5, 15, 3)):
        v = torch.from_numpy(vals).to(dev)
        got = ssm.ssm_checkpoint_sr16(v, seed, ck, off)
        torch.cuda.synchronize()
        want = oracle.sr16(vals, seed, ck, off)
        g = got.cpu().numpy().view(np.uint16)
        assert np.array_equal(g, want), int(np.sum(g != want))
    # values in the binary16 normal range only, so whole waves take the short form of the
    # rule: binade edges, the top binade's carry into infinity, both signs
    edges = np.array([2.0 ** e * (1.0 + f) for e in range(-14, 16)
                      for f in (0.0, 2.0 ** -11, 0.5, 1.0 - 2.0 ** -11, 1.0 - 2.0 ** -23)])
    normal = np.concatenate([
        np.tile(np.concatenate([edges, -edges, [65504.0, 65519.0, 65520.0, 65535.99, -65530.0]]),
                200),
        r.choice([-1.0, 1.0], 300000) * 2.0 ** r.uniform(-14, 16, 300000),
    ]).astype(np.float32)
    normal = normal[(np.abs(normal) >= 2.0 ** -14) & (np.abs(normal) < 65536.0)]
    for seed, ck, off in ((3, 1, 0), (2 ** 40 + 1, 9, 12345)):
        got = ssm.ssm_checkpoint_sr16(torch.from_numpy(normal).to(dev), seed, ck, off)
        torch.cuda.synchronize()
        want = oracle.sr16(normal, seed, ck, off)
        g = got.cpu().numpy().view(np.uint16)
        assert np.array_equal(g, want), int(np.sum(g != want))
    # ragged length and a non-multiple-of-8 offset into a larger state
    v = torch.from_numpy(vals[:1003]).to(dev)
    got = ssm.ssm_checkpoint_sr16(v, 99, 2, 17).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, oracle.sr16(vals[:1003], 99, 2, 17))


def test_sr16_replay_drift(ssm):
    """Replay from the SR16 checkpoint in lockstep with the live copy: drift is the
    rounding error carried by the product of retentions (difference identity,
    TorchLean page "The Mamba state update"), within fp32 noise."""
    b, t, h, p, n, g = 2, 64, 4, 64, 128, 2
    pr = _seq_problem(b, t, h, p, n, g, "bf16", 51)
    live0 = pr["h0"] * 4.0
    bits = ssm.ssm_checkpoint_sr16(live0, 5, 0, 0)
    out = ssm.ssm_replay(bits, pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], 0, t,
                         live=live0)
    live = ssm.ssm_replay(live0, pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], 0, t)
    torch.cuda.synchronize()
    d_end = (out["state"] - live["state"]).abs()
    assert abs(float(out["drift_max"][-1]) - float(d_end.max())) == 0.0
    np.testing.assert_allclose(float(out["drift_mean"][-1]), float(d_end.double().mean()),
                               rtol=1e-5)
    d0 = (bits.view(torch.float16).double() - live0.double())
    prod = torch.exp((pr["dt"][0].double() * pr["A"].double()[None, :]).sum(0))  # b = 0 only
    pred = prod[:, None, None] * d0[0]
    err = (out["state"][0].double() - live["state"][0].double()) - pred
    ulp = float(torch.finfo(torch.float32).eps) * float(live["state"].abs().max())
    assert float(err.abs().max()) <= 4 * t * ulp
    dm = out["drift_max"].cpu().numpy()
    assert np.all(dm[1:] <= dm[:-1] + 4 * ulp)  # nonexpansive up to fp32 noise


@pytest.mark.parametrize("L", [8, 16, 32, 64])
def test_tiny_f32_forward(ssm, L):
    w = inputs.WORKLOADS["tiny_f32"]
    pr = inputs.make_workload_problem(w, dev)
    y, hf, cs = ssm.ssm_fwd_chunked(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"],
                                    chunk=L)
    ref = oracle.fwd(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], chunk=L,
                     want_chunk_states=True)
    torch.cuda.synchronize()
    assert_close("y", y, ref["y"], 1e-5)
    assert_close("h_final", hf, ref["h_final"], 1e-5)
    assert_close("chunk_states", cs[:, :, 1:], ref["chunk_states"][:, :, 1:], 1e-5)


@pytest.mark.parametrize("L,h0,dhf", [(8, "zero", False), (16, "randn", True), (64, "zero", True),
                                      (32, "randn", False)])
def test_tiny_f32_backward(ssm, L, h0, dhf):
    w = inputs.WORKLOADS["tiny_f32"]
    pr = inputs.make_problem(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, "f32",
                             w.seed, dev, h0=h0, dh_final=dhf)
    _, _, cs = ssm.ssm_fwd_chunked(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"],
                                   h0=pr["h0"], chunk=L)
    g = ssm.ssm_bwd(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], cs, pr["dy"],
                    dh_final=pr["dh_final"], chunk=L)
    ref = oracle.bwd(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], pr["dy"],
                     h0=pr["h0"], dh_final=pr["dh_final"])
    torch.cuda.synchronize()
    for k in ("dx", "dB", "dC", "ddt", "dA", "dD", "dh0"):
        assert_close(k, g[k], ref[k], 1e-5)


def test_f32_multihead_groups_ragged(ssm):
    b, t, h, p, n, g, L = 2, 45, 6, 8, 16, 3, 16
    pr = inputs.make_problem(b, t, h, p, n, g, "f32", 61, dev, h0="randn", dh_final=True)
    y, hf, cs = ssm.ssm_fwd_chunked(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"],
                                    h0=pr["h0"], chunk=L)
    gr = ssm.ssm_bwd(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], cs, pr["dy"],
                     dh_final=pr["dh_final"], chunk=L)
    ref = oracle.fwd(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], h0=pr["h0"])
    rg = oracle.bwd(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], pr["dy"],
                    h0=pr["h0"], dh_final=pr["dh_final"])
    torch.cuda.synchronize()
    assert_close("y", y, ref["y"], 1e-5)
    assert_close("h_final", hf, ref["h_final"], 1e-5)
    for k in ("dx", "dB", "dC", "ddt", "dA", "dD", "dh0"):
        assert_close(k, gr[k], rg[k], 1e-5)


def test_zero_length_sequence(ssm):
    b, h, p, n, g = 2, 4, 8, 16, 2
    pr = inputs.make_problem(b, 0, h, p, n, g, "f32", 71, dev, h0="randn", dh_final=True)
    y, hf, cs = ssm.ssm_fwd_chunked(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"],
                                    h0=pr["h0"], chunk=16)
    gr = ssm.ssm_bwd(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], cs, pr["dy"],
                     dh_final=pr["dh_final"], chunk=16)
    torch.cuda.synchronize()
    assert torch.equal(hf, pr["h0"])
    assert torch.equal(gr["dh0"], pr["dh_final"])
    assert float(gr["dA"].abs().max()) == 0.0 and float(gr["dD"].abs().max()) == 0.0
