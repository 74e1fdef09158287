"""GPU parity of the chunked MFMA forward (bf16 x/B/C, headdim 64, dstate 128).

Tolerance 2e-2 scaled error (bf16 MFMA operands, fp32 accumulation) on y,
h_final and chunk_states.  Sizes span several 64-token blocks, partial chunks
and ragged tails; the full prefill workload (batch 4, 256 heads, T = 4096,
chunk 256) is checked on whole (batch, group) units, which the oracle computes
exactly on their own since groups never interact.  Every chunked case asserts
that the MFMA kernels serve it.  The ends of the retention range
exp(dt*A) in (0, 1] ("Nemotron 3 Ultra: replaying a rounded state", section
"The Mamba state update") are covered too: a retention of 1 to float32
precision over T = 4096 (the state sums every write), a retention that
underflows to 0 within a token (dt*A <= -30: only the newest write survives),
and an initial state 10^4 times the writes.
"""
import numpy as np
import pytest
import torch

from backward_mamba_ssd_amd import inputs
from oracle import oracle
from tests.parity import assert_close

pytestmark = pytest.mark.gpu
dev = torch.device("cuda:0")


@pytest.fixture(scope="module")
def ssm():
    from backward_mamba_ssd_amd import ssm as m
    return m


def _assert_mfma(ssm, pr, L):
    assert ssm.ssm_uses_mfma_path(ssm.dims_of(pr["x"], pr["B"], L), ssm.SSM_BF16)


@pytest.mark.parametrize("t,L,h0", [(64, 64, "zero"), (200, 64, "randn"), (320, 128, "zero"),
                                    (513, 256, "randn"), (37, 64, "randn"), (1000, 192, "zero")])
def test_forward_matches_oracle(ssm, t, L, h0):
    b, h, p, n, g = 2, 8, 64, 128, 2
    pr = inputs.make_problem(b, t, h, p, n, g, "bf16", 100 + t, dev, h0=h0)
    _assert_mfma(ssm, pr, L)
    y, hf, cs = ssm.ssm_fwd_chunked(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"],
                                    h0=pr["h0"], chunk=L)
    ref = oracle.fwd(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], h0=pr["h0"],
                     chunk=L, want_chunk_states=True)
    torch.cuda.synchronize()
    assert_close("y", y, ref["y"], 2e-2)
    assert_close("h_final", hf, ref["h_final"], 2e-2)
    assert_close("chunk_states", cs, ref["chunk_states"], 2e-2)


def test_chunk_size_only_moves_the_saved_states(ssm):
    b, t, h, p, n, g = 1, 512, 4, 64, 128, 1
    pr = inputs.make_problem(b, t, h, p, n, g, "bf16", 7, dev)
    for L in (64, 128, 256):
        _assert_mfma(ssm, pr, L)
    outs = {L: ssm.ssm_fwd_chunked(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"],
                                   chunk=L) for L in (64, 128, 256)}
    for L in (128, 256):
        assert torch.equal(outs[L][0], outs[64][0])
        assert torch.equal(outs[L][1], outs[64][1])
        assert torch.equal(outs[L][2], outs[64][2][:, :, ::L // 64])


def test_prefill_equals_repeated_decode(ssm):
    """Nemotron Kernels: From Inference To Backpropagation, Kernel 1: the
    full-sequence scan and repeated one-token decode must agree."""
    b, t, h, p, n, g = 2, 96, 4, 64, 128, 2
    pr = inputs.make_problem(b, t, h, p, n, g, "bf16", 9, dev, h0="randn")
    _assert_mfma(ssm, pr, 64)
    y, hf, _ = ssm.ssm_fwd_chunked(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"],
                                   h0=pr["h0"], chunk=64)
    st = pr["h0"].clone()
    ys = []
    for k in range(t):
        ys.append(ssm.ssm_decode_step(st, pr["x"][:, k].contiguous(), pr["B"][:, k].contiguous(),
                                      pr["C"][:, k].contiguous(), pr["dt"][:, k].contiguous(),
                                      pr["A"], pr["D"]))
    torch.cuda.synchronize()
    assert_close("y vs decode", y, torch.stack(ys, 1), 2e-2)
    assert_close("h_final vs decode", hf, st, 2e-2)


def test_full_prefill_workload_sampled_groups(ssm):
    w = inputs.WORKLOADS["prefill_b4_t4096"]
    pr = inputs.make_workload_problem(w, dev, with_dy=False)
    _assert_mfma(ssm, pr, w.chunk)
    y, hf, cs = ssm.ssm_fwd_chunked(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"],
                                    chunk=w.chunk)
    torch.cuda.synchronize()
    hpg = w.nheads // w.ngroups
    for (bb, gg) in ((0, 0), (3, 7), (1, 4)):
        hs = slice(gg * hpg, (gg + 1) * hpg)
        print(f"group b={bb} g={gg}", flush=True)
        ref = oracle.fwd(pr["x"][bb:bb + 1, :, hs], pr["B"][bb:bb + 1, :, gg:gg + 1],
                         pr["C"][bb:bb + 1, :, gg:gg + 1], pr["dt"][bb:bb + 1, :, hs],
                         pr["A"][hs], pr["D"][hs], chunk=w.chunk, want_chunk_states=True)
        assert_close("y", y[bb:bb + 1, :, hs], ref["y"], 2e-2)
        assert_close("h_final", hf[bb:bb + 1, hs], ref["h_final"], 2e-2)
        assert_close("chunk_states", cs[bb:bb + 1, hs], ref["chunk_states"], 2e-2)


def retention_extreme(pr, case):
    """Move a seeded problem to one end of the retention range (in place, on the device).
    unit: A = -exp(-20) per head, so dt*A ~ -3e-10 and exp(dt*A) rounds to 1 in float32;
    underflow: dt in [1, 2] and A in [-60, -30], so dt*A <= -30 on every token;
    big_h0: the initial state scaled by 10^4 against writes of order dt*|x||B|."""
    if case == "unit":
        pr["A"] = torch.full_like(pr["A"], -float(np.exp(-20.0)))
    elif case == "underflow":
        pr["dt"] = 1.0 + torch.rand(pr["dt"].shape, generator=torch.Generator(dev).manual_seed(3),
                                    device=dev)
        pr["A"] = -30.0 - 30.0 * torch.rand(pr["A"].shape,
                                            generator=torch.Generator(dev).manual_seed(4),
                                            device=dev)
    elif case == "big_h0":
        pr["h0"] = pr["h0"] * 1e4
    return pr


@pytest.mark.parametrize("case", ["unit", "underflow", "big_h0"])
def test_forward_at_the_ends_of_the_retention_range(ssm, case):
    b, t, h, p, n, g, L = 1, 4096, 8, 64, 128, 2, 256
    pr = inputs.make_problem(b, t, h, p, n, g, "bf16", 60, dev, h0="randn")
    pr = retention_extreme(pr, case)
    _assert_mfma(ssm, pr, L)
    y, hf, cs = ssm.ssm_fwd_chunked(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"],
                                    h0=pr["h0"], chunk=L)
    ref = oracle.fwd(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], h0=pr["h0"],
                     chunk=L, want_chunk_states=True)
    torch.cuda.synchronize()
    assert_close("y", y, ref["y"], 2e-2)
    assert_close("h_final", hf, ref["h_final"], 2e-2)
    assert_close("chunk_states", cs, ref["chunk_states"], 2e-2)


def test_inference_form_equals_training_form(ssm):
    """Leaving out the saved chunk states (inference) or the final state changes no other
    output: y and h_final are bit-identical to the call that saves everything."""
    b, t, h, p, n, g = 2, 333, 8, 64, 128, 2
    pr = inputs.make_problem(b, t, h, p, n, g, "bf16", 21, dev, h0="randn")
    _assert_mfma(ssm, pr, 128)
    args = (pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"])
    y, hf, cs = ssm.ssm_fwd_chunked(*args, h0=pr["h0"], chunk=128)
    y1, hf1, cs1 = ssm.ssm_fwd_chunked(*args, h0=pr["h0"], chunk=128, chunk_states=None)
    y2, hf2, cs2 = ssm.ssm_fwd_chunked(*args, h0=pr["h0"], chunk=128, chunk_states=None,
                                       h_final=None)
    torch.cuda.synchronize()
    assert cs1 is None and cs2 is None and hf2 is None
    assert torch.equal(y1, y) and torch.equal(y2, y)
    assert torch.equal(hf1, hf)
