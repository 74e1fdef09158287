"""GPU parity of the chunked MFMA backward (bf16 x/B/C/dy, headdim 64, dstate 128).

Tolerance 2e-2 scaled error on dx, dB, dC, ddt, dA, dD, dh0 (bf16 MFMA
operands, fp32 accumulation, fp64 final dA/dD sums).  Small problems span
several 64-token blocks, partial chunks and ragged tails; the full prefill
workload (batch 4, 256 heads, T = 4096) is checked on one whole group over all
batches (so dA/dD of its heads are complete); each batch of a 256-head problem run
alone matches the batched run bit for bit (the two runs take the 4-wave and the
8-wave form of the reverse pass); the long-context workload
(T = 131,072, 512 saved chunk states per head) is checked over the full length
on one whole group (its group-summed dB and dC, and every per-head gradient)
and on two heads of other groups (outputs and saved states), with every oracle
input a seeded input; and the ends of the retention range are covered.
Every chunked case asserts that the MFMA kernels serve it.
"""
import numpy as np
import pytest
import torch

from backward_mamba_ssd_amd import inputs
from oracle import oracle
from tests.parity import assert_close

pytestmark = pytest.mark.gpu
dev = torch.device("cuda:0")
GRADS = ("dx", "dB", "dC", "ddt", "dA", "dD", "dh0")


@pytest.fixture(scope="module")
def ssm():
    from backward_mamba_ssd_amd import ssm as m
    return m


def _run(ssm, pr, L):
    y, hf, cs = ssm.ssm_fwd_chunked(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"],
                                    h0=pr["h0"], chunk=L)
    g = ssm.ssm_bwd(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], cs, pr["dy"],
                    dh_final=pr["dh_final"], chunk=L)
    return y, hf, cs, g


@pytest.mark.parametrize("t,L,h0,dhf", [(64, 64, "zero", False), (200, 64, "randn", True),
                                        (320, 128, "zero", True), (513, 256, "randn", False),
                                        (37, 64, "randn", True), (700, 192, "zero", True)])
def test_backward_matches_oracle(ssm, t, L, h0, dhf):
    b, h, p, n, g = 2, 8, 64, 128, 2
    pr = inputs.make_problem(b, t, h, p, n, g, "bf16", 300 + t, dev, h0=h0, dh_final=dhf)
    assert ssm.ssm_uses_mfma_path(ssm.dims_of(pr["x"], pr["B"], L), ssm.SSM_BF16)
    _, _, _, gr = _run(ssm, pr, L)
    ref = oracle.bwd(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], pr["dy"],
                     h0=pr["h0"], dh_final=pr["dh_final"])
    torch.cuda.synchronize()
    for k in GRADS:
        assert_close(k, gr[k], ref[k], 2e-2)


@pytest.mark.parametrize("t,h,g,L", [(600, 8, 2, 512), (200, 128, 1, 128)])
def test_shapes_outside_the_mfma_backward(ssm, t, h, g, L):
    # chunk 512 or 128 heads in one group: the MFMA forward saves the chunk states and
    # the exact-fp32 sequential backward takes over; same entry points, same tolerance
    b, p, n = 1, 64, 128
    pr = inputs.make_problem(b, t, h, p, n, g, "bf16", 700 + h, dev, h0="randn", dh_final=True)
    assert not ssm.ssm_uses_mfma_path(ssm.dims_of(pr["x"], pr["B"], L), ssm.SSM_BF16)
    _, _, _, gr = _run(ssm, pr, L)
    ref = oracle.bwd(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], pr["dy"],
                     h0=pr["h0"], dh_final=pr["dh_final"])
    torch.cuda.synchronize()
    for k in GRADS:
        assert_close(k, gr[k], ref[k], 2e-2)


def test_backward_deterministic(ssm):
    b, t, h, p, n, g, L = 2, 300, 8, 64, 128, 2, 128
    pr = inputs.make_problem(b, t, h, p, n, g, "bf16", 5, dev, h0="randn", dh_final=True)
    assert ssm.ssm_uses_mfma_path(ssm.dims_of(pr["x"], pr["B"], L), ssm.SSM_BF16)
    _, _, _, g1 = _run(ssm, pr, L)
    _, _, _, g2 = _run(ssm, pr, L)
    torch.cuda.synchronize()
    for k in GRADS:
        assert torch.equal(g1[k], g2[k]), k


@pytest.mark.parametrize("t,L", [(320, 128), (64, 64), (130, 64), (200, 256)])
def test_batch_slices_are_independent(ssm, t, L):
    # Every (batch, head) is computed by its own workgroups, so each batch run alone gives
    # the same bits as the batched run.  With 256 heads the batch-4 forward and reverse
    # pass fill an MI355X two and four deep and take their batch forms, while a batch of 1
    # takes the small-grid forms: this also checks that the forms agree bit for bit.  The
    # shapes cover the small-grid reverse pass's edges: a walk that is not a whole number
    # of its three-block passes (5, 3 and 4 blocks are padded by 1, 0 and 2 steps), one
    # block, a chunk end at every block (chunk 64), several chunk ends and ragged last
    # chunks.  (dA and dD sum over the batch, so only their batch-summed values are
    # compared, at tolerance.)
    b, h, p, n, g = 4, 256, 64, 128, 8
    pr = inputs.make_problem(b, t, h, p, n, g, "bf16", 41 + t, dev, h0="randn", dh_final=True)
    assert ssm.ssm_uses_mfma_path(ssm.dims_of(pr["x"], pr["B"], L), ssm.SSM_BF16)
    y, hf, cs, gr = _run(ssm, pr, L)
    dA = torch.zeros_like(gr["dA"], dtype=torch.float64)
    dD = torch.zeros_like(dA)
    for i in range(b):
        one = {k: (v[i:i + 1].contiguous() if (v is not None and v.dim() > 1) else v)
               for k, v in pr.items()}
        y1, hf1, cs1, g1 = _run(ssm, one, L)
        torch.cuda.synchronize()
        assert torch.equal(y1, y[i:i + 1]) and torch.equal(cs1, cs[i:i + 1]), i
        for k in ("dx", "dB", "dC", "ddt", "dh0"):
            assert torch.equal(g1[k], gr[k][i:i + 1]), (k, i)
        dA += g1["dA"].double()
        dD += g1["dD"].double()
    assert_close("dA over batch", gr["dA"], dA, 1e-5)
    assert_close("dD over batch", gr["dD"], dD, 1e-5)


def test_full_prefill_workload_one_group(ssm):
    w = inputs.WORKLOADS["prefill_b4_t4096"]
    pr = inputs.make_workload_problem(w, dev)
    assert ssm.ssm_uses_mfma_path(ssm.dims_of(pr["x"], pr["B"], w.chunk), ssm.SSM_BF16)
    _, _, _, gr = _run(ssm, pr, w.chunk)
    torch.cuda.synchronize()
    hpg = w.nheads // w.ngroups
    gg = 5
    hs = slice(gg * hpg, (gg + 1) * hpg)
    print(f"oracle backward: all batches, group {gg} ({hpg} heads)", flush=True)
    ref = oracle.bwd(pr["x"][:, :, hs], pr["B"][:, :, gg:gg + 1], pr["C"][:, :, gg:gg + 1],
                     pr["dt"][:, :, hs], pr["A"][hs], pr["D"][hs], pr["dy"][:, :, hs])
    assert_close("dx", gr["dx"][:, :, hs], ref["dx"], 2e-2)
    assert_close("dB", gr["dB"][:, :, gg:gg + 1], ref["dB"], 2e-2)
    assert_close("dC", gr["dC"][:, :, gg:gg + 1], ref["dC"], 2e-2)
    assert_close("ddt", gr["ddt"][:, :, hs], ref["ddt"], 2e-2)
    assert_close("dA", gr["dA"][hs], ref["dA"], 2e-2)
    assert_close("dD", gr["dD"][hs], ref["dD"], 2e-2)
    assert_close("dh0", gr["dh0"][:, hs], ref["dh0"], 2e-2)


def _one_head_groups(pr, heads, groups):
    """The listed heads as one-head groups: x, dt, dy, A, D of those heads and, for each,
    the B and C of the group that owns it.  The oracle's backward runs independent groups
    on separate host threads; summing the one-head groups' dB/dC over the heads of a group
    in ascending order adds exactly the per-head terms the oracle's own group sum adds,
    in the same order."""
    hs = list(heads)
    return dict(x=pr["x"][:, :, hs], B=pr["B"][:, :, list(groups)], C=pr["C"][:, :, list(groups)],
                dt=pr["dt"][:, :, hs], A=pr["A"][hs], D=pr["D"][hs])


def test_long_context_workload(ssm):
    w = inputs.WORKLOADS["long_b1_t131072"]
    pr = inputs.make_workload_problem(w, dev)
    assert ssm.ssm_uses_mfma_path(ssm.dims_of(pr["x"], pr["B"], w.chunk), ssm.SSM_BF16)
    y, hf, cs, gr = _run(ssm, pr, w.chunk)
    torch.cuda.synchronize()
    assert cs.shape[2] == w.seqlen // w.chunk == 512
    hpg = w.nheads // w.ngroups
    # Every oracle input below is a seeded input; no GPU output enters an oracle call.
    # (1) two heads of other groups over the whole sequence: y, the 512 saved states
    heads = (0, 131)
    sub = _one_head_groups(pr, heads, [h // hpg for h in heads])
    print(f"oracle long heads {heads}: forward", flush=True)
    rf = oracle.fwd(**sub, chunk=w.chunk, want_chunk_states=True)
    for i, h in enumerate(heads):
        assert_close(f"y head {h}", y[:, :, h:h + 1], rf["y"][:, :, i:i + 1], 2e-2)
        assert_close(f"chunk_states head {h}", cs[:, h:h + 1], rf["chunk_states"][:, i:i + 1],
                     2e-2)
    # (2) one whole group over the whole sequence: the group-summed dB and dC, and every
    #     per-head gradient of its 32 heads
    gg = 6
    hs = range(gg * hpg, (gg + 1) * hpg)
    sub = _one_head_groups(pr, hs, [gg] * hpg)
    print(f"oracle long group {gg}: backward over {w.seqlen} tokens", flush=True)
    rb = oracle.bwd(**sub, dy=pr["dy"][:, :, list(hs)])
    dB = np.zeros(rb["dB"][:, :, 0].shape)
    dC = np.zeros_like(dB)
    for k in range(hpg):  # the group sum, heads ascending
        dB += rb["dB"][:, :, k]
        dC += rb["dC"][:, :, k]
    hsl = slice(gg * hpg, (gg + 1) * hpg)
    assert_close("dB group", gr["dB"][:, :, gg], dB, 2e-2)
    assert_close("dC group", gr["dC"][:, :, gg], dC, 2e-2)
    for k, got in (("dx", gr["dx"][:, :, hsl]), ("ddt", gr["ddt"][:, :, hsl]),
                   ("dA", gr["dA"][hsl]), ("dD", gr["dD"][hsl]), ("dh0", gr["dh0"][:, hsl])):
        assert_close(k, got, rb[k], 2e-2)
    del rb
    print(f"oracle long group {gg}: forward", flush=True)
    rf = oracle.fwd(**sub, chunk=w.chunk, want_chunk_states=True)
    assert_close("y group", y[:, :, hsl], rf["y"], 2e-2)
    assert_close("h_final group", hf[:, hsl], rf["h_final"], 2e-2)
    assert_close("chunk_states group", cs[:, hsl], rf["chunk_states"], 2e-2)


@pytest.mark.parametrize("case", ["unit", "underflow", "big_h0"])
def test_backward_at_the_ends_of_the_retention_range(ssm, case):
    # retention 1 to float32 precision over T = 4096, retention underflowing within a
    # token, and a large initial state (see test_gpu_ssd_fwd.retention_extreme)
    from tests.test_gpu_ssd_fwd import retention_extreme
    b, t, h, p, n, g, L = 1, 4096, 8, 64, 128, 2, 256
    pr = inputs.make_problem(b, t, h, p, n, g, "bf16", 61, dev, h0="randn", dh_final=True)
    pr = retention_extreme(pr, case)
    assert ssm.ssm_uses_mfma_path(ssm.dims_of(pr["x"], pr["B"], L), ssm.SSM_BF16)
    _, _, _, gr = _run(ssm, pr, L)
    ref = oracle.bwd(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], pr["dy"],
                     h0=pr["h0"], dh_final=pr["dh_final"])
    torch.cuda.synchronize()
    for k in GRADS:
        assert_close(k, gr[k], ref[k], 2e-2)


def test_sixty_four_heads_per_group(ssm):
    # the widest group the MFMA backward takes: 64 heads share B and C, so the per-block
    # kernel's head loop and its per-head A, D reads span a whole wave
    b, t, h, p, n, g, L = 1, 200, 64, 64, 128, 1, 128
    pr = inputs.make_problem(b, t, h, p, n, g, "bf16", 77, dev, h0="randn", dh_final=True)
    assert ssm.ssm_uses_mfma_path(ssm.dims_of(pr["x"], pr["B"], L), ssm.SSM_BF16)
    _, _, _, gr = _run(ssm, pr, L)
    ref = oracle.bwd(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], pr["dy"],
                     h0=pr["h0"], dh_final=pr["dh_final"])
    torch.cuda.synchronize()
    for k in GRADS:
        assert_close(k, gr[k], ref[k], 2e-2)


def test_no_tokens_at_the_mfma_shape(ssm):
    # T = 0 at the MFMA head shape: the final state is the initial state, dh0 is
    # dh_final, and the parameter gradients are zero
    b, h, p, n, g = 2, 8, 64, 128, 2
    pr = inputs.make_problem(b, 0, h, p, n, g, "bf16", 78, dev, h0="randn", dh_final=True)
    y, hf, cs, gr = _run(ssm, pr, 256)
    torch.cuda.synchronize()
    assert y.numel() == 0 and cs.numel() == 0
    assert torch.equal(hf, pr["h0"])
    assert torch.equal(gr["dh0"], pr["dh_final"])
    assert float(gr["dA"].abs().max()) == 0.0 and float(gr["dD"].abs().max()) == 0.0


def test_grids_that_are_not_a_multiple_of_the_xcd_count(ssm):
    # 3 sequences x 6 heads in 3 groups: 18 forward and reverse-pass workgroups and 27
    # per-block workgroups, none a multiple of 8, so the workgroup ids are used as they come
    b, t, h, p, n, g, L = 3, 130, 6, 64, 128, 3, 64
    pr = inputs.make_problem(b, t, h, p, n, g, "bf16", 79, dev, h0="randn", dh_final=True)
    assert ssm.ssm_uses_mfma_path(ssm.dims_of(pr["x"], pr["B"], L), ssm.SSM_BF16)
    y, hf, cs, gr = _run(ssm, pr, L)
    rf = oracle.fwd(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], h0=pr["h0"], chunk=L,
                    want_chunk_states=True)
    rb = oracle.bwd(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], pr["dy"],
                    h0=pr["h0"], dh_final=pr["dh_final"])
    torch.cuda.synchronize()
    assert_close("y", y, rf["y"], 2e-2)
    assert_close("h_final", hf, rf["h_final"], 2e-2)
    assert_close("chunk_states", cs, rf["chunk_states"], 2e-2)
    for k in GRADS:
        assert_close(k, gr[k], rb[k], 2e-2)
