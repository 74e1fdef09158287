"""Seeded synthetic inputs for the selective SSM recurrence.

This module only draws random numbers; it holds none of the recurrence's
arithmetic.  The same tensors feed the GPU library and (copied to the host) the
fp64 oracle, so both sides always see identical values.

Distributions (one recipe for every workload):
  time-step preparation inputs: dt_raw ~ N(0, 0.25), dt_bias ~ N(-2, 0.01) per
  head (so dt_raw + dt_bias matches the N(-2, 0.5) spread below), logA ~ U(0, ln 16);
  upstream ddt, dA ~ N(0, 1);
  stages around the scan: conv input, initial samples, gate z, upstream dout ~ N(0, 1);
  conv weights [channels, K] ~ N(0, 1/K), conv bias ~ N(0, 0.01), norm scale ~ N(1, 0.01);
  x ~ N(0, 1); B, C ~ N(0, 1/N); dt = softplus(N(-2, 0.5)) (positive, float32);
  A = -exp(U(0, ln 16)) per head (float32); D ~ N(0, 1) per head (float32);
  dy ~ N(0, 1); optional h0 / dh_final ~ N(0, 1) (float32).
x, B, C and dy are drawn in float32 and cast once to the storage dtype
(bf16 casts round to nearest even).  Each tensor has its own generator seeded
with ``seed + tensor_id`` so adding a tensor never changes the others.

The shapes and dtypes of the named workloads follow the Mamba-2 head shape of
Nemotron 3 Ultra (256 heads, 64 value channels, 128 state coordinates, 8
groups sharing B and C) from "Nemotron 3 Ultra: replaying a rounded state",
section "Counting the state and attention cache".
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

TENSOR_IDS = {"x": 1, "B": 2, "C": 3, "dt": 4, "A": 5, "D": 6, "dy": 7, "h0": 8,
              "dh_final": 9, "dt_raw": 10, "dt_bias": 11, "logA": 12, "ddt": 13, "dA": 14,
              "conv_u": 15, "conv_w": 16, "conv_b": 17, "conv_init": 18, "gate_z": 19,
              "norm_w": 20, "dout": 21}


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    dtype: str  # "f32" or "bf16": storage dtype of x, B, C, dy, y, dx
    seed: int
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    # tiny fp32 case the oracle finishes instantly (also run at chunk 8/16/32)
    "tiny_f32": Workload("tiny_f32", 1, 64, 1, 8, 16, 1, 64, "f32", 1000),
    # prefill forward+backward of one layer at the Ultra head shape
    "prefill_b4_t4096": Workload("prefill_b4_t4096", 4, 4096, 256, 64, 128, 8, 256, "bf16", 2000),
    # decode: 64 sequences x 48 layers, one token per step, 100 steps
    "decode_s64_l48": Workload("decode_s64_l48", 64, 1, 256, 64, 128, 8, 1, "bf16", 3000,
                               {"layers": 48, "steps": 100}),
    # checkpoint (SR16 every 1024 tokens) and replay
    "ckpt_replay_b16_t16384": Workload("ckpt_replay_b16_t16384", 16, 16384, 256, 64, 128, 8,
                                       1024, "bf16", 4000),
    # long-context training backward from 512 saved chunk states per head
    "long_b1_t131072": Workload("long_b1_t131072", 1, 131072, 256, 64, 128, 8, 256, "bf16", 5000),
}


def torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, seed, device):
    return torch.randn(shape, generator=_gen(device, seed), device=device, dtype=torch.float32)


def _rand(shape, seed, device):
    return torch.rand(shape, generator=_gen(device, seed), device=device, dtype=torch.float32)


def draw(name, shape, seed, device="cpu", dtype=torch.float32, dstate=None):
    """Draw one named tensor of the recipe."""
    s = seed + TENSOR_IDS[name]
    if name in ("x", "dy", "D", "h0", "dh_final"):
        v = _randn(shape, s, device)
    elif name in ("B", "C"):
        v = _randn(shape, s, device) * (1.0 / math.sqrt(dstate))
    elif name == "dt":
        v = torch.nn.functional.softplus(-2.0 + 0.5 * _randn(shape, s, device))
    elif name == "A":
        v = -torch.exp(_rand(shape, s, device) * math.log(16.0))
    elif name == "dt_raw":   # raw + bias ~ N(-2, ~0.5), the spread of the prepared dt above
        v = 0.5 * _randn(shape, s, device)
    elif name == "dt_bias":
        v = -2.0 + 0.1 * _randn(shape, s, device)
    elif name == "logA":     # A = -exp(logA) = -exp(U(0, ln 16)) as above
        v = _rand(shape, s, device) * math.log(16.0)
    elif name in ("ddt", "dA", "conv_u", "conv_init", "gate_z", "dout"):
        v = _randn(shape, s, device)
    elif name == "conv_w":   # [channels, K]: N(0, 1/K), a unit-gain filter on average
        v = _randn(shape, s, device) / math.sqrt(shape[-1])
    elif name == "conv_b":
        v = 0.1 * _randn(shape, s, device)
    elif name == "norm_w":
        v = 1.0 + 0.1 * _randn(shape, s, device)
    else:
        raise KeyError(name)
    return v.to(dtype).contiguous()


def make_problem(batch, seqlen, nheads, headdim, dstate, ngroups, dtype="bf16", seed=1000,
                 device="cpu", h0="zero", dh_final=False, with_dy=True):
    """Inputs of one prefill/backward problem, all on ``device``.

    Layouts: x, dy [batch, seqlen, nheads, headdim]; B, C [batch, seqlen, ngroups,
    dstate]; dt [batch, seqlen, nheads]; A, D [nheads]; h0, dh_final
    [batch, nheads, headdim, dstate] (h0 is None when ``h0 == "zero"``).
    """
    td = torch_dtype(dtype) if isinstance(dtype, str) else dtype
    b, t, h, p, n, g = batch, seqlen, nheads, headdim, dstate, ngroups
    out = {
        "x": draw("x", (b, t, h, p), seed, device, td),
        "B": draw("B", (b, t, g, n), seed, device, td, dstate=n),
        "C": draw("C", (b, t, g, n), seed, device, td, dstate=n),
        "dt": draw("dt", (b, t, h), seed, device),
        "A": draw("A", (h,), seed, device),
        "D": draw("D", (h,), seed, device),
        "h0": draw("h0", (b, h, p, n), seed, device) if h0 == "randn" else None,
    }
    if with_dy:
        out["dy"] = draw("dy", (b, t, h, p), seed, device, td)
    out["dh_final"] = draw("dh_final", (b, h, p, n), seed, device) if dh_final else None
    return out


def make_workload_problem(w: Workload, device="cpu", **kw):
    return make_problem(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups,
                        w.dtype, w.seed, device, **kw)


def make_decode_problem(nseq, nlayers, steps, nheads, headdim, dstate, ngroups, seed=3000,
                        device="cpu", dtype="bf16"):
    """Decode workload: per-layer states and per-step inputs drawn ahead.

    state [nlayers, nseq, nheads, headdim, dstate] f32 ~ N(0,1);
    A, D [nlayers, nheads]; x [steps, nlayers, nseq, nheads, headdim];
    B, C [steps, nlayers, nseq, ngroups, dstate]; dt [steps, nlayers, nseq, nheads].
    """
    td = torch_dtype(dtype)
    S, Lr, b, h, p, n, g = steps, nlayers, nseq, nheads, headdim, dstate, ngroups
    return {
        "state": draw("h0", (Lr, b, h, p, n), seed, device),
        "A": draw("A", (Lr, h), seed, device),
        "D": draw("D", (Lr, h), seed, device),
        "x": draw("x", (S, Lr, b, h, p), seed, device, td),
        "B": draw("B", (S, Lr, b, g, n), seed, device, td, dstate=n),
        "C": draw("C", (S, Lr, b, g, n), seed, device, td, dstate=n),
        "dt": draw("dt", (S, Lr, b, h), seed, device),
    }
