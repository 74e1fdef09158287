"""ssm_bwd_noalloc (the backward over the library's own scratch, for callers that
cannot allocate) against ssm_bwd: the same kernels on the same inputs, so every output
must match bit for bit.  Three calls in a row on one GPU, each smaller than the one
before: one 4096-token sequence at 256 heads x 64 x 128 with chunk 256 (the size the
scratch is stated for), a ragged bf16 problem (also checked against the oracle at the
bf16 tolerance), and a float32 problem on the exact-fp32 kernels (1e-5).  A problem
past the scratch is refused with SSM_ERR_WORKSPACE and writes nothing."""
import pytest
import torch

from backward_mamba_ssd_amd import inputs
from oracle import oracle
from tests.parity import assert_close

pytestmark = pytest.mark.gpu
dev = torch.device("cuda:0")
KEYS = ("dx", "dB", "dC", "ddt", "dA", "dD", "dh0")


@pytest.fixture(scope="module")
def ssm():
    from backward_mamba_ssd_amd import ssm as m
    return m


def _outputs(pr):
    b, t, h, p = pr["x"].shape
    g, n = pr["B"].shape[2], pr["B"].shape[3]
    f32 = dict(dtype=torch.float32, device=dev)
    return {"dx": torch.full_like(pr["x"], 7.0), "dB": torch.full((b, t, g, n), 7.0, **f32),
            "dC": torch.full((b, t, g, n), 7.0, **f32), "ddt": torch.full((b, t, h), 7.0, **f32),
            "dA": torch.full((h,), 7.0, **f32), "dD": torch.full((h,), 7.0, **f32),
            "dh0": torch.full((b, h, p, n), 7.0, **f32)}


CASES = [  # (batch, seqlen, heads, headdim, dstate, groups, chunk, dtype)
    (1, 4096, 256, 64, 128, 8, 256, "bf16"),
    (2, 700, 8, 64, 128, 2, 192, "bf16"),
    (1, 64, 2, 8, 16, 1, 16, "f32"),
]


def test_noalloc_matches_ssm_bwd_on_successive_calls(ssm):
    for i, (b, t, h, p, n, g, L, dt) in enumerate(CASES):
        print(f"no-alloc call {i}: batch {b} T {t} heads {h} P {p} N {n} groups {g} chunk {L} "
              f"{dt}", flush=True)
        pr = inputs.make_problem(b, t, h, p, n, g, dt, 900 + i, dev, h0="randn", dh_final=True)
        dims = ssm.dims_of(pr["x"], pr["B"], L)
        code = ssm.SSM_BF16 if dt == "bf16" else ssm.SSM_F32
        assert ssm.ssm_workspace_bytes(dims, code, ssm.SSM_WS_BWD) <= ssm.NOALLOC_SCRATCH_BYTES
        _, _, cs = ssm.ssm_fwd_chunked(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"],
                                       h0=pr["h0"], chunk=L)
        args = (pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], cs, pr["dy"])
        want = ssm.ssm_bwd(*args, dh_final=pr["dh_final"], chunk=L)
        got = ssm.ssm_bwd_noalloc(*args, _outputs(pr), dh_final=pr["dh_final"], chunk=L)
        torch.cuda.synchronize()
        for k in KEYS:
            assert torch.equal(got[k], want[k]), (i, k)
        if i > 0:  # small enough for the oracle here
            ref = oracle.bwd(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], pr["dy"],
                             h0=pr["h0"], dh_final=pr["dh_final"])
            tol = 2e-2 if dt == "bf16" else 1e-5
            for k in KEYS:
                assert_close(k, got[k], ref[k], tol)


def test_noalloc_refuses_a_problem_past_its_scratch(ssm):
    b, t, h, p, n, g, L = 2, 4096, 256, 64, 128, 8, 256  # two sequences: twice the scratch
    pr = inputs.make_problem(b, t, h, p, n, g, "bf16", 950, dev)
    dims = ssm.dims_of(pr["x"], pr["B"], L)
    assert ssm.ssm_workspace_bytes(dims, ssm.SSM_BF16, ssm.SSM_WS_BWD) > ssm.NOALLOC_SCRATCH_BYTES
    cs = torch.zeros((b, h, t // L, p, n), dtype=torch.float32, device=dev)
    out = _outputs(pr)
    with pytest.raises(ssm.SsmError) as ei:
        ssm.ssm_bwd_noalloc(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], cs, pr["dy"],
                            out, chunk=L)
    assert ei.value.status == 6  # SSM_ERR_WORKSPACE
    torch.cuda.synchronize()
    for k in KEYS:
        assert bool((out[k] == 7.0).all()), k  # nothing written
