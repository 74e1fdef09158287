"""GPU parity of the speculative draft snapshots and the rollback
(ssm_draft_snapshots, ssm_rollback) against the fp64 oracle
("Nemotron 3 Ultra: replaying a rounded state", section "Rolling back rejected
draft tokens").

- every snapshot slot against the oracle's snapshot stack: 1e-5 scaled error
  (float32 state on identical inputs); draft outputs at 1e-5 (fp32) or 2e-2
  (bf16 storage);
- slot k equals the state after k ssm_decode_step calls, bit for bit (the same
  step arithmetic);
- the rollback is a copy: bit-exact against the selected slots, per sequence with
  different accepted counts (0 = the initial state, Dr = the whole draft), also
  in place into slot 0; and within 1e-5 of the oracle's restore;
- an accepted count out of range raises the error flag and leaves that
  sequence's output untouched (the kernel checks it; nothing faults);
- the serving shape: 64 sequences x 256 heads x [64, 128], a 4-token draft.
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


def _draft_problem(b, dr, h, p, n, g, dtype, seed):
    pr = inputs.make_problem(b, dr, h, p, n, g, dtype, seed=seed, device=dev, with_dy=False)
    pr["state0"] = inputs.draw("h0", (b, h, p, n), seed, dev)
    return pr


@pytest.mark.parametrize("shape,dtype", [((3, 5, 16, 64, 128, 2), "bf16"),
                                         ((2, 3, 4, 8, 16, 1), "f32"),
                                         ((4, 1, 8, 32, 64, 4), "bf16")])
def test_draft_snapshots_and_rollback(ssm, shape, dtype):
    b, dr, h, p, n, g = shape
    pr = _draft_problem(b, dr, h, p, n, g, dtype, 7100 + dr)
    args = [pr[k] for k in ("x", "B", "C", "dt", "A", "D")]
    snaps, y = ssm.ssm_draft_snapshots(pr["state0"], *args)
    # the same tokens through repeated decode calls
    st = pr["state0"].clone()
    dec = [st.clone()]
    for k in range(dr):
        ssm.ssm_decode_step(st, pr["x"][:, k].contiguous(), pr["B"][:, k].contiguous(),
                            pr["C"][:, k].contiguous(), pr["dt"][:, k].contiguous(), pr["A"],
                            pr["D"])
        dec.append(st.clone())
    accepted = [(3 * i) % (dr + 1) for i in range(b)]
    accepted[0] = 0
    accepted[-1] = dr
    acc_t = torch.tensor(accepted, dtype=torch.int32, device=dev)
    out = ssm.ssm_rollback(snaps, acc_t)
    torch.cuda.synchronize()
    rs, ry = oracle.draft_snapshots(pr["state0"], *args)
    for k in range(dr + 1):
        assert torch.equal(snaps[k], dec[k]), f"slot {k} differs from {k} decode steps"
        assert_close(f"slot {k}", snaps[k], rs[k], 1e-5)
    assert_close("y", y, ry, 2e-2 if dtype == "bf16" else 1e-5)
    for i, a in enumerate(accepted):
        assert torch.equal(out[i], snaps[a, i])
    assert_close("rollback", out, oracle.rollback(rs, accepted), 1e-5)
    # in place into slot 0: the next draft starts from the accepted prefix's state
    want = out.clone()
    ssm.ssm_rollback(snaps, acc_t, state_out=snaps[0])
    torch.cuda.synchronize()
    assert torch.equal(snaps[0], want)


def test_rollback_out_of_range_sets_the_flag(ssm):
    b, dr, h, p, n, g = 3, 2, 4, 16, 32, 2
    pr = _draft_problem(b, dr, h, p, n, g, "f32", 7200)
    snaps, _ = ssm.ssm_draft_snapshots(pr["state0"], *[pr[k] for k in ("x", "B", "C", "dt", "A", "D")],
                                       y=False)
    out = torch.full((b, h, p, n), 7.0, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    acc = torch.tensor([1, dr + 1, -1], dtype=torch.int32, device=dev)
    ssm.ssm_rollback(snaps, acc, state_out=out, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 1
    assert torch.equal(out[0], snaps[1, 0])
    assert bool((out[1] == 7.0).all()) and bool((out[2] == 7.0).all())
    err.zero_()
    ssm.ssm_rollback(snaps, torch.tensor([0, 2, 1], dtype=torch.int32, device=dev), state_out=out,
                     err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0


def test_serving_shape_draft_of_four(ssm):
    # one layer of the decode workload's shape: 64 sequences x 256 heads x [64, 128]
    w = inputs.WORKLOADS["decode_s64_l48"]
    b, dr = w.batch, 4
    pr = _draft_problem(b, dr, w.nheads, w.headdim, w.dstate, w.ngroups, "bf16", 7300)
    args = [pr[k] for k in ("x", "B", "C", "dt", "A", "D")]
    snaps, y = ssm.ssm_draft_snapshots(pr["state0"], *args)
    acc = torch.tensor([i % (dr + 1) for i in range(b)], dtype=torch.int32, device=dev)
    out = ssm.ssm_rollback(snaps, acc)
    torch.cuda.synchronize()
    rs, ry = oracle.draft_snapshots(pr["state0"], *args)
    for k in range(dr + 1):
        assert_close(f"slot {k}", snaps[k], rs[k], 1e-5)
    assert_close("y", y, ry, 2e-2)
    assert_close("rollback", out, oracle.rollback(rs, acc.cpu().numpy()), 1e-5)
