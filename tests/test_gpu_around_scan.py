"""GPU parity of the stages around the scan against the fp64 oracle:
ssm_conv1d_silu(_bwd) (short causal depthwise convolution + SiLU) and
ssm_gated_rmsnorm(_bwd) (SiLU-gated group RMSNorm); "Nemotron Kernels: From
Inference To Backpropagation", Kernel 1 "Forward And Inference".

Tolerances (scaled error): 1e-5 for float32 storage and for the float32
parameter gradients (identical inputs, float32 arithmetic); 2e-2 for values
stored in bf16.  Shapes: ragged channel and token counts, widths 1..8, tokens
fewer than the window, no tokens, continuation through the carried samples
(decode is seqlen 1), groups of 8..8192 channels, and the prefill layer's full
size (batch 4 x 4096 tokens; 18,432 convolution channels = 256 heads x 64 +
2 x 8 groups x 128; 16,384 normalised channels in 8 groups) compared on
sampled channels / rows, with the parameter gradients over all of them.
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


def _conv_inputs(b, t, c, k, dtype, seed, init=True):
    td = inputs.torch_dtype(dtype)
    return {
        "u": inputs.draw("conv_u", (b, t, c), seed, dev, td),
        "w": inputs.draw("conv_w", (c, k), seed, dev),
        "bias": inputs.draw("conv_b", (c,), seed, dev),
        "init": inputs.draw("conv_init", (b, k - 1, c), seed, dev, td) if init else None,
        "dout": inputs.draw("dout", (b, t, c), seed, dev, td),
    }


def _check_conv(ssm, pr, dtype):
    tol = 2e-2 if dtype == "bf16" else 1e-5
    out, fin = ssm.ssm_conv1d_silu(pr["u"], pr["w"], pr["bias"], pr["init"])
    g = ssm.ssm_conv1d_silu_bwd(pr["u"], pr["w"], pr["bias"], pr["dout"], pr["init"])
    torch.cuda.synchronize()
    ro, rf = oracle.conv1d_silu(pr["u"], pr["w"], pr["bias"], pr["init"])
    rg = oracle.conv1d_silu_bwd(pr["u"], pr["w"], pr["bias"], pr["dout"], pr["init"])
    assert_close("out", out, ro, tol)
    assert np.array_equal(to_np(fin), rf)  # the carried samples are copies
    assert_close("du", g["du"], rg["du"], tol)
    assert_close("dw", g["dw"], rg["dw"], 1e-5)
    assert_close("dbias", g["dbias"], rg["dbias"], 1e-5)
    if pr["init"] is not None:
        assert_close("dconv_init", g["dconv_init"], rg["dinit"], tol)
    return out, fin


@pytest.mark.parametrize("b,t,c,k,dtype,init", [
    (2, 77, 36, 4, "f32", True), (3, 300, 64, 3, "bf16", False), (1, 1, 8, 4, "f32", True),
    (2, 5, 16, 8, "f32", True), (2, 600, 20, 1, "bf16", False), (1, 513, 1028, 4, "bf16", True),
    (2, 2, 12, 6, "f32", True)])
def test_conv1d_silu_matches_oracle(ssm, b, t, c, k, dtype, init):
    _check_conv(ssm, _conv_inputs(b, t, c, k, dtype, 8000 + t + k, init), dtype)


def test_conv1d_continuation_and_decode(ssm):
    # the carried samples make split runs (and one-token decode steps) equal the whole run
    pr = _conv_inputs(2, 40, 32, 4, "f32", 8100)
    whole, fin = ssm.ssm_conv1d_silu(pr["u"], pr["w"], pr["bias"], pr["init"])
    o1, f1 = ssm.ssm_conv1d_silu(pr["u"][:, :30].contiguous(), pr["w"], pr["bias"], pr["init"])
    parts, st = [o1], f1
    for t in range(30, 40):
        o, st = ssm.ssm_conv1d_silu(pr["u"][:, t:t + 1].contiguous(), pr["w"], pr["bias"], st)
        parts.append(o)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(parts, dim=1), whole)
    assert torch.equal(st, fin)


def test_conv1d_no_tokens(ssm):
    pr = _conv_inputs(2, 0, 16, 4, "f32", 8200)
    _, fin = ssm.ssm_conv1d_silu(pr["u"], pr["w"], pr["bias"], pr["init"])
    g = ssm.ssm_conv1d_silu_bwd(pr["u"], pr["w"], pr["bias"], pr["dout"], pr["init"])
    torch.cuda.synchronize()
    assert torch.equal(fin, pr["init"])
    assert bool((g["dw"] == 0).all()) and bool((g["dbias"] == 0).all())
    assert bool((g["dconv_init"] == 0).all())


def test_conv1d_prefill_layer_full_size(ssm):
    b, t, c, k = 4, 4096, 256 * 64 + 2 * 8 * 128, 4
    pr = _conv_inputs(b, t, c, k, "bf16", 8300, init=False)
    out, _ = ssm.ssm_conv1d_silu(pr["u"], pr["w"], pr["bias"])
    g = ssm.ssm_conv1d_silu_bwd(pr["u"], pr["w"], pr["bias"], pr["dout"], want_dinit=False)
    torch.cuda.synchronize()
    # channels are independent: the oracle on a sampled set of channels is exact for them
    cols = torch.arange(3, c, 61, device=dev)
    sub = {kk: (v[..., cols].contiguous() if kk in ("u", "dout") else v) for kk, v in pr.items()}
    sub["w"] = pr["w"][cols].contiguous()
    sub["bias"] = pr["bias"][cols].contiguous()
    ro, _ = oracle.conv1d_silu(sub["u"], sub["w"], sub["bias"])
    rg = oracle.conv1d_silu_bwd(sub["u"], sub["w"], sub["bias"], sub["dout"])
    assert_close("out", out[..., cols], ro, 2e-2)
    assert_close("du", g["du"][..., cols], rg["du"], 2e-2)
    assert_close("dw", g["dw"][cols], rg["dw"], 1e-5)
    assert_close("dbias", g["dbias"][cols], rg["dbias"], 1e-5)


def _norm_inputs(rows, c, dtype, seed):
    td = inputs.torch_dtype(dtype)
    return {"y": inputs.draw("conv_u", (rows, c), seed, dev, td),
            "z": inputs.draw("gate_z", (rows, c), seed, dev, td),
            "w": inputs.draw("norm_w", (c,), seed, dev),
            "dout": inputs.draw("dout", (rows, c), seed, dev, td)}


@pytest.mark.parametrize("rows,c,g,dtype", [(37, 64, 4, "f32"), (100, 2048, 1, "bf16"),
                                            (9, 16384, 2, "f32"), (70, 48, 2, "bf16"),
                                            (33, 6144, 1, "f32")])
def test_gated_rmsnorm_matches_oracle(ssm, rows, c, g, dtype):
    tol = 2e-2 if dtype == "bf16" else 1e-5
    pr = _norm_inputs(rows, c, dtype, 8400 + rows)
    out = ssm.ssm_gated_rmsnorm(pr["y"], pr["z"], pr["w"], g)
    gr = ssm.ssm_gated_rmsnorm_bwd(pr["y"], pr["z"], pr["w"], pr["dout"], g)
    torch.cuda.synchronize()
    assert_close("out", out, oracle.gated_rmsnorm(pr["y"], pr["z"], pr["w"], g), tol)
    rg = oracle.gated_rmsnorm_bwd(pr["y"], pr["z"], pr["w"], pr["dout"], g)
    assert_close("dy", gr["dy"], rg["dy"], tol)
    assert_close("dz", gr["dz"], rg["dz"], tol)
    assert_close("dw", gr["dw"], rg["dw"], 1e-5)


def test_gated_rmsnorm_no_rows(ssm):
    pr = _norm_inputs(0, 64, "f32", 8500)
    gr = ssm.ssm_gated_rmsnorm_bwd(pr["y"], pr["z"], pr["w"], pr["dout"], 4)
    torch.cuda.synchronize()
    assert bool((gr["dw"] == 0).all())


def test_gated_rmsnorm_prefill_layer_full_size(ssm):
    rows, c, g = 4 * 4096, 256 * 64, 8
    pr = _norm_inputs(rows, c, "bf16", 8600)
    out = ssm.ssm_gated_rmsnorm(pr["y"], pr["z"], pr["w"], g)
    gr = ssm.ssm_gated_rmsnorm_bwd(pr["y"], pr["z"], pr["w"], pr["dout"], g)
    torch.cuda.synchronize()
    sel = torch.arange(5, rows, 97, device=dev)  # rows are independent for out, dy, dz
    sub = {k: (v[sel].contiguous() if k != "w" else v) for k, v in pr.items()}
    assert_close("out", out[sel], oracle.gated_rmsnorm(sub["y"], sub["z"], sub["w"], g), 2e-2)
    rs = oracle.gated_rmsnorm_bwd(sub["y"], sub["z"], sub["w"], sub["dout"], g)
    assert_close("dy", gr["dy"][sel], rs["dy"], 2e-2)
    assert_close("dz", gr["dz"][sel], rs["dz"], 2e-2)
    rw = oracle.gated_rmsnorm_bwd(pr["y"], pr["z"], pr["w"], pr["dout"], g)["dw"]  # all rows
    assert_close("dw", gr["dw"], rw, 1e-5)
