"""Host-only checks of the Python binding's argument validation (no GPU needed).

The C boundary receives raw pointers and cannot see a tensor's strides, dtype or
allocation size, so the binding checks every tensor against the call's dims
before any pointer reaches the library: a strided view, a wrong dtype, a wrong
shape or a tensor on another device raises ValueError (TypeError for a
non-tensor) and nothing is called.  Every case here fails that validation, so
CPU tensors are fine: the last check of every wrapper is that the tensors live
on a GPU.
"""
import pytest
import torch

ssm = pytest.importorskip("backward_mamba_ssd_amd.ssm")


def problem(b=2, t=8, h=4, p=64, n=128, g=2, dtype=torch.bfloat16):
    return {
        "x": torch.zeros((b, t, h, p), dtype=dtype),
        "B": torch.zeros((b, t, g, n), dtype=dtype),
        "C": torch.zeros((b, t, g, n), dtype=dtype),
        "dt": torch.ones((b, t, h)),
        "A": -torch.ones(h),
        "D": torch.zeros(h),
        "dy": torch.zeros((b, t, h, p), dtype=dtype),
    }


def fwd(pr, **kw):
    return ssm.ssm_fwd_chunked(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], **kw)


def bwd(pr, cs, **kw):
    return ssm.ssm_bwd(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], cs, pr["dy"], **kw)


def test_well_formed_host_tensors_are_refused_for_not_being_on_a_gpu():
    pr = problem()
    with pytest.raises(ValueError, match="GPU"):
        fwd(pr, chunk=64)


@pytest.mark.parametrize("what", ["strided_x", "B_dtype", "C_shape", "dt_dtype", "A_shape",
                                  "D_dtype", "y_shape", "h0_shape", "cs_shape"])
def test_fwd_rejects_malformed_tensors(what):
    pr = problem()
    kw = {"chunk": 4}
    if what == "strided_x":
        big = torch.zeros((2, 8, 8, 64), dtype=torch.bfloat16)
        pr["x"] = big[:, :, ::2]  # a strided view: same shape, not contiguous
    elif what == "B_dtype":
        pr["B"] = pr["B"].float()
    elif what == "C_shape":
        pr["C"] = torch.zeros((2, 8, 2, 64), dtype=torch.bfloat16)
    elif what == "dt_dtype":
        pr["dt"] = pr["dt"].double()
    elif what == "A_shape":
        pr["A"] = -torch.ones(3)
    elif what == "D_dtype":
        pr["D"] = pr["D"].to(torch.bfloat16)
    elif what == "y_shape":
        kw["y"] = torch.zeros((2, 8, 4, 32), dtype=torch.bfloat16)
    elif what == "h0_shape":
        kw["h0"] = torch.zeros((2, 4, 64, 64))
    elif what == "cs_shape":
        kw["chunk_states"] = torch.zeros((2, 4, 1, 64, 128))  # chunk 4 needs 2 chunks
    with pytest.raises(ValueError) as ei:
        fwd(pr, **kw)
    assert "GPU" not in str(ei.value)


def test_fwd_rejects_a_non_tensor_and_a_bad_chunk():
    pr = problem()
    with pytest.raises(TypeError):
        ssm.ssm_fwd_chunked(pr["x"], [1, 2], pr["C"], pr["dt"], pr["A"], pr["D"])
    with pytest.raises(ValueError):
        fwd(pr, chunk=0)


def test_bwd_rejects_chunk_states_saved_with_another_chunk():
    pr = problem(t=256)
    cs = torch.zeros((2, 4, 1, 64, 128))  # one chunk: saved with chunk 256
    with pytest.raises(ValueError, match="chunk_states"):
        bwd(pr, cs, chunk=64)  # chunk 64 reads 4 chunk states per head


@pytest.mark.parametrize("what", ["dy_dtype", "dh_final_shape", "out_dB_dtype", "out_dx_strided",
                                  "workspace_dtype"])
def test_bwd_rejects_malformed_tensors(what):
    pr = problem()
    cs = torch.zeros((2, 4, 2, 64, 128))
    kw = {"chunk": 4}
    if what == "dy_dtype":
        pr["dy"] = pr["dy"].float()
    elif what == "dh_final_shape":
        kw["dh_final"] = torch.zeros((2, 4, 128, 64))
    elif what in ("out_dB_dtype", "out_dx_strided"):
        out = {"dx": torch.zeros((2, 8, 4, 64), dtype=torch.bfloat16),
               "dB": torch.zeros((2, 8, 2, 128)), "dC": torch.zeros((2, 8, 2, 128)),
               "ddt": torch.zeros((2, 8, 4)), "dA": torch.zeros(4), "dD": torch.zeros(4),
               "dh0": None}
        if what == "out_dB_dtype":
            out["dB"] = out["dB"].to(torch.bfloat16)
        else:
            out["dx"] = torch.zeros((2, 8, 4, 128), dtype=torch.bfloat16)[..., ::2]
        kw["out"] = out
    elif what == "workspace_dtype":
        kw["workspace"] = torch.zeros(1 << 20, dtype=torch.float32)
    with pytest.raises(ValueError) as ei:
        bwd(pr, cs, **kw)
    assert "GPU" not in str(ei.value)


def test_decode_and_replay_reject_malformed_tensors():
    b, h, p, n, g = 2, 4, 64, 128, 2
    st = torch.zeros((b, h, p, n))
    x = torch.zeros((b, h, p), dtype=torch.bfloat16)
    Bv = torch.zeros((b, g, n), dtype=torch.bfloat16)
    dt, A, D = torch.ones((b, h)), -torch.ones(h), torch.zeros(h)
    with pytest.raises(ValueError, match="state"):
        ssm.ssm_decode_step(st.transpose(2, 3), x, Bv, Bv, dt, A, D)
    with pytest.raises(ValueError, match="C"):
        ssm.ssm_decode_step(st, x, Bv, Bv.float(), dt, A, D)
    with pytest.raises(ValueError, match="state16"):
        ssm.ssm_decode_step_sr16(st, x, Bv, Bv, dt, A, D, 1, 0)
    with pytest.raises(ValueError, match="GPU"):
        ssm.ssm_decode_step(st, x, Bv, Bv, dt, A, D)
    pr = problem()
    with pytest.raises(ValueError, match="ckpt"):
        ssm.ssm_replay(torch.zeros((2, 4, 64, 64)), pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"],
                       pr["D"], 0, 4)
    with pytest.raises(ValueError, match="live"):
        ssm.ssm_replay(torch.zeros((2, 4, 64, 128)), pr["x"], pr["B"], pr["C"], pr["dt"],
                       pr["A"], pr["D"], 0, 4, live=torch.zeros((2, 4, 64, 128), dtype=torch.half))
    with pytest.raises(ValueError, match="out"):
        ssm.ssm_checkpoint_sr16(st, 1, 0, out=torch.zeros((b, h, p, n), dtype=torch.int32))


def test_other_wrappers_reject_malformed_tensors():
    raw = torch.zeros((2, 8, 4))
    with pytest.raises(ValueError, match="dt_bias"):
        ssm.ssm_dt_prep(raw, torch.zeros(5), torch.zeros(4))
    with pytest.raises(ValueError, match="ddt"):
        ssm.ssm_dt_prep_bwd(raw, torch.zeros(4), torch.zeros(4), torch.zeros((2, 8, 5)),
                            torch.zeros(4))
    snaps = torch.zeros((3, 2, 4, 64, 128))
    with pytest.raises(ValueError, match="accepted"):
        ssm.ssm_rollback(snaps, torch.zeros(2, dtype=torch.int64))
    u = torch.zeros((2, 8, 16), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="conv_init"):
        ssm.ssm_conv1d_silu(u, torch.zeros((16, 4)), torch.zeros(16),
                            conv_init=torch.zeros((2, 4, 16), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="dout"):
        ssm.ssm_conv1d_silu_bwd(u, torch.zeros((16, 4)), torch.zeros(16),
                                torch.zeros((2, 8, 16)))
    with pytest.raises(ValueError, match="z"):
        ssm.ssm_gated_rmsnorm(torch.zeros((4, 16)), torch.zeros((4, 8)), torch.ones(16), 2)
    pr = problem()
    with pytest.raises(ValueError, match="snapshots"):
        ssm.ssm_draft_snapshots(None, pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"],
                                snapshots=torch.zeros((8, 2, 4, 64, 128)))
