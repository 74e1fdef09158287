"""Benchmark: forward + backward of the chunked SSM recurrence on one MI355X.

A step is one pass of the whole training hot path over one batch: the chunked
forward (saving the chunk-boundary states) followed by the backward that
returns dx, dB, dC, ddt, dA, dD.  The workload is one Mamba-2 layer at the
Nemotron 3 Ultra head shape: batch 4, 256 heads, headdim 64, dstate 128,
8 groups, T = 4096, chunk 256, bf16 x/B/C/dy, fp32 state (seeded synthetic
inputs, see backward_mamba_ssd_amd.inputs).  Inputs are resident in HBM before
the timed region.  `value` is tokens/s = batch * T * steps / elapsed.

Also reported:
  roofline      the dominant kernel (largest mean duration, timed with HIP events
                on the stream it runs on) against the HBM roof, from the
                algorithmic bytes per launch;
  cpu_baseline  the fp64 oracle timed on this host on a bounded sample;
  secondary     decode state-update GB/s (64 sequences x 48 layers x
                [256,64,128] fp32 states, in place), SR16 checkpoint GB/s.

Prints exactly one JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
FP32_VALU_PEAK_TFLOPS = 157.3  # MI355X fp32 vector, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def fwd_bytes_per_token(w):
    """Algorithmic HBM bytes per token of the chunked forward (training mode):
    x read + y write (2 B each), B and C read (2 B), dt read (4 B), and the
    chunk-boundary state written once per chunk (4 B per state element)."""
    H, P, N, G, L = w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    return 2 * H * P + 2 * H * P + 2 * 2 * G * N + 4 * H + 4 * H * P * N / L


def bwd_method_bytes_per_token(w):
    """The method's algorithmic HBM bytes per token of the backward: x, dy read and dx
    written (2 B each), the saved chunk-boundary state read once (4 B per element per
    chunk), B and C read (2 B), dB and dC written (4 B), dt read and ddt written (4 B).
    145,408 B/token at 256 heads x 64 x 128, 8 groups, chunk 256."""
    H, P, N, G, L = w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    return 3 * 2 * H * P + 4 * H * P * N / L + 2 * 2 * G * N + 2 * 4 * G * N + 2 * 4 * H


def bwd_block_design_bytes_per_token(w):
    """Bytes per token the per-block backward kernel of this design moves: the method's
    backward bytes plus its read of the chunk-exit state gradients that the reverse
    pass leaves in the workspace (bf16, once per chunk)."""
    H, P, N, L = w.nheads, w.headdim, w.dstate, w.chunk
    return bwd_method_bytes_per_token(w) + 2 * H * P * N / L


def fwd_flops_per_token(w):
    """The method's MFMA-mapped flops of the chunked forward per token (causal halves
    counted once): group Gram L*N/hpg, intra-chunk output L*P, chunk state 2PN,
    off-diagonal output 2PN, per head (50,176 per token-head at the head shape above)."""
    H, P, N, G, L = w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    return H * (L * N / (H // G) + L * P + 2 * P * N + 2 * P * N)


def bwd_flops_per_token(w):
    """The method's flops of the backward per token: off-diagonal + reverse state pass
    4PN, intra-chunk 2LP + 3LN/hpg, chunk-state gradients 4PN, per head."""
    H, P, N, G, L = w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    return H * (4 * P * N + 2 * L * P + 3 * L * N / (H // G) + 4 * P * N)


def bwd_call_design_bytes_per_token(w):
    """Bytes per token the whole backward call of this design moves: the reverse state
    pass (dy and C read, chunk-exit state gradients written once per chunk in bf16) plus
    the per-block kernel (bwd_block_design_bytes_per_token).  The reverse pass reads dy,
    C and dt a second time, so this exceeds the method's bytes."""
    H, P, N, G, L = w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    return 2 * H * P + 2 * G * N + 4 * H + 2 * H * P * N / L + bwd_block_design_bytes_per_token(w)


def path_entry(flops, nbytes, ms, flop_peak_tflops=None):
    """flops, bytes, rates and the fraction of both roofs for one timed path."""
    sec = ms * 1e-3
    gbps = nbytes / sec / 1e9
    e = {"ms": round(ms, 4), "bytes": int(nbytes), "GBps": round(gbps, 1),
         "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}
    if flops:
        tf = flops / sec / 1e12
        peak = flop_peak_tflops or BF16_PEAK_TFLOPS
        e.update({"flops": float(flops), "TFLOPs": round(tf, 2), "flop_peak_TFLOPs": peak,
                  "flop_frac": round(tf / peak, 4)})
        e["bound"] = "hbm" if e["hbm_frac"] >= e["flop_frac"] else "flop"
    return e


# the files a kernel's code comes from (launch.hpp only declares host launchers; the
# chunked path's argument blocks live in ssd_common.hpp)
KERNEL_SOURCES = {
    "ssd_fwd_kernel": ("ssd_fwd.hip", "ssd_common.hpp", "common.hpp"),
    "ssd_bwd_block_kernel": ("ssd_bwd.hip", "ssd_common.hpp", "common.hpp"),
    "ssd_bwd_dstate_kernel": ("ssd_bwd.hip", "ssd_common.hpp", "common.hpp"),
}


def kernel_source_sha256(kernel):
    """sha256 over the HIP sources a kernel is built from (in a fixed order)."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "backward_mamba_ssd_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary
    profiles/<kernel>_<workload>_hbm_counters.md (FETCH_SIZE and WRITE_SIZE,
    each scaled by what the counter reads for a copy of known size), or None
    when there is no summary or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_source_sha256(kernel):
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def fwd_mfma_flops_per_token(w):
    """MFMA flops the forward kernel issues per token (64-token blocks, per head):
    Gram 10 causal 16x16 tiles x K=128, outputs 16 tiles x K=128 plus 6 steps of
    K=32 per 16-row slice, state update 32 tiles x K=64 (2 flops per MAC)."""
    per_block_macs = (10 * 16 * 16 * 128 + 16 * 16 * 16 * 128 + 4 * 6 * 16 * 16 * 32
                      + 32 * 16 * 16 * 64)
    return 2 * per_block_macs / 64 * w.nheads


def cpu_baseline(w, budget_s=30.0):
    """fp64 oracle (sequential recurrence + reverse sweep) on a bounded sample:
    4 batches x 4 groups (128 heads) x a token window, grown until the run takes
    a few seconds; reported as equivalent full-width tokens/s (tokens x heads
    fraction / seconds)."""
    import torch  # noqa: F401

    from backward_mamba_ssd_amd import inputs
    from oracle import oracle

    oracle.build(force=False)
    ngr = 4
    hpg = w.nheads // w.ngroups
    hs = ngr * hpg
    cores = oracle.num_threads()
    T = 128
    while True:
        pr = inputs.make_problem(w.batch, T, hs, w.headdim, w.dstate, ngr, "bf16", w.seed, "cpu")
        t0 = time.perf_counter()
        oracle.fwd(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"])
        oracle.bwd(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], pr["dy"])
        el = time.perf_counter() - t0
        if el > budget_s / 3 or T >= 16384:
            break
        T *= 2
    tok = w.batch * T * hs / w.nheads
    return {
        "value": tok / el,
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"batch {w.batch} x {ngr} of {w.ngroups} groups ({hs} of {w.nheads} heads) x "
                   f"{T} tokens, fp64 forward + reverse sweep, {el:.1f} s on {cores} threads; "
                   f"value counts batch*T*heads/{w.nheads} tokens"),
    }


def time_fwd_bwd(w, dev, steps, warmup):
    """Time `steps` fwd+bwd steps of workload w (inputs resident before timing).
    Returns per-step event means/medians and the wall-clock over the timed steps."""
    import statistics

    import torch

    from backward_mamba_ssd_amd import inputs, ssm

    pr = inputs.make_workload_problem(w, dev)
    dims = ssm.dims_of(pr["x"], pr["B"], w.chunk)
    b, t, h, p = pr["x"].shape
    g, n = pr["B"].shape[2], pr["B"].shape[3]
    nc = (t + w.chunk - 1) // w.chunk
    f32 = dict(dtype=torch.float32, device=dev)
    y = torch.empty_like(pr["x"])
    cs = torch.empty((b, h, nc, p, n), **f32)
    grads = {"dx": torch.empty_like(pr["x"]), "dB": torch.empty((b, t, g, n), **f32),
             "dC": torch.empty((b, t, g, n), **f32), "ddt": torch.empty((b, t, h), **f32),
             "dA": torch.empty((h,), **f32), "dD": torch.empty((h,), **f32), "dh0": None}
    ws = torch.empty(ssm.ssm_workspace_bytes(dims, ssm.SSM_BF16, ssm.SSM_WS_BWD),
                     dtype=torch.uint8, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        ssm.ssm_fwd_chunked(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], chunk=w.chunk,
                            h_final=None, chunk_states=cs, y=y)
        args = (pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], cs, pr["dy"])
        if ev is not None:
            ev[1].record()
            # the per-block kernel's own duration: the call records ev[2], ev[3] around it
            ssm.ssm_bwd_timed(*args, (ev[2], ev[3]), chunk=w.chunk, out=grads, workspace=ws)
            ev[4].record()
        else:
            ssm.ssm_bwd(*args, chunk=w.chunk, out=grads, workspace=ws)

    for _ in range(warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        step(evs[k])
    torch.cuda.synchronize()
    el = time.perf_counter() - t0

    def stat(i, j):
        v = [e[i].elapsed_time(e[j]) for e in evs]
        return sum(v) / len(v), statistics.median(v)

    r = {"tokens": b * t, "wall_s": el,
         "fwd": stat(0, 1), "blk": stat(2, 3), "bwd": stat(1, 4), "step": stat(0, 4)}
    del pr, y, cs, grads, ws
    torch.cuda.empty_cache()
    return r


def measured_peaks(dev):
    """Achievable rates on this GPU: a 1 GiB device-to-device copy (read + write bytes)
    and an 8192^3 bf16 matrix product (torch / hipBLASLt)."""
    import torch

    out = {}
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    out["copy_GBps"] = round(2 * src.numel() * 4 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del src, dst
    n = 8192
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    a = torch.randn((n, n), generator=g, device=dev).to(torch.bfloat16)
    bm = torch.randn((n, n), generator=g, device=dev).to(torch.bfloat16).contiguous()
    for _ in range(2):
        torch.mm(a, bm)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        torch.mm(a, bm)
    e1.record()
    torch.cuda.synchronize()
    out["bf16_gemm_TFLOPs"] = round(2 * n ** 3 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
    del a, bm
    torch.cuda.empty_cache()
    return out


def replay_sweep(dev):
    """Replay r tokens from SR16 checkpoints at the checkpoint workload's shape
    (16 sequences x 256 heads x [64,128]): bytes, GB/s and fp32-VALU fraction."""
    import torch

    from backward_mamba_ssd_amd import inputs, ssm

    w = inputs.WORKLOADS["ckpt_replay_b16_t16384"]
    rmax = 1024
    pr = inputs.make_problem(w.batch, rmax, w.nheads, w.headdim, w.dstate, w.ngroups, "bf16",
                             w.seed, dev, with_dy=False)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed + 99)
    live = torch.randn((w.batch, w.nheads, w.headdim, w.dstate), generator=g, device=dev)
    bits = ssm.ssm_checkpoint_sr16(live, 5, 0)
    out_state = torch.empty_like(live)
    heads = w.batch * w.nheads
    PN = w.headdim * w.dstate
    res = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for r in (1, 4, 16, 64, 256, 1024):
        ssm.ssm_replay(bits, pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], 0, r,
                       state_out=out_state)
        torch.cuda.synchronize()
        reps = 20 if r <= 64 else 5
        e0.record()
        for _ in range(reps):
            ssm.ssm_replay(bits, pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], 0, r,
                           state_out=out_state)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        nbytes = heads * (PN * (2 + 4) + r * (2 * w.headdim + 4 + 2 * 2 * w.dstate * w.ngroups
                                                  / w.nheads))
        flops = heads * 3 * PN * r
        res[f"r{r}"] = path_entry(flops, nbytes, ms, FP32_VALU_PEAK_TFLOPS)
    del pr, live, bits, out_state
    torch.cuda.empty_cache()
    return res


def dt_prep_rates(dev):
    """Time-step preparation at the prefill workload's [batch, T, heads]: forward
    (raw read, dt written: 8 B per element) and backward (raw and ddt read, d_raw
    written: 12 B per element; the per-head bias partials are not counted)."""
    import torch

    from backward_mamba_ssd_amd import inputs, ssm

    w = inputs.WORKLOADS["prefill_b4_t4096"]
    shp = (w.batch, w.seqlen, w.nheads)
    pr = {k: inputs.draw(k, s, w.seed, dev) for k, s in
          (("dt_raw", shp), ("dt_bias", (w.nheads,)), ("logA", (w.nheads,)), ("ddt", shp),
           ("dA", (w.nheads,)))}
    dt, A = ssm.ssm_dt_prep(pr["dt_raw"], pr["dt_bias"], pr["logA"], 0.0, float("inf"))
    g = ssm.ssm_dt_prep_bwd(pr["dt_raw"], pr["dt_bias"], pr["logA"], pr["ddt"], pr["dA"])
    dims = ssm.make_dims(*shp, 1, 1, 1, 1)
    ws = torch.empty(max(1, ssm.ssm_workspace_bytes(dims, ssm.SSM_F32, ssm.SSM_WS_DT_PREP_BWD)),
                     dtype=torch.uint8, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {}
    n = dt.numel()
    for name, fn, nbytes in (
            ("fwd", lambda: ssm.ssm_dt_prep(pr["dt_raw"], pr["dt_bias"], pr["logA"], 0.0,
                                            float("inf"), dt=dt, A=A), 8 * n),
            ("bwd", lambda: ssm.ssm_dt_prep_bwd(pr["dt_raw"], pr["dt_bias"], pr["logA"],
                                                pr["ddt"], pr["dA"], out=g, workspace=ws),
             12 * n)):
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(50):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = path_entry(0, nbytes, e0.elapsed_time(e1) / 50)
    del pr, dt, A, g, ws
    torch.cuda.empty_cache()
    return res


def draft_rollback_rates(dev, layers=8, ndraft=4):
    """Speculative draft with per-step snapshots and the rollback, at the decode
    workload's per-layer shape (64 sequences x 256 heads x [64, 128] fp32 states),
    `layers` layers, a draft of `ndraft` tokens.  Draft bytes per layer: slot 0 read,
    `ndraft` slots written, inputs and outputs; rollback: one state read + one written."""
    import torch

    from backward_mamba_ssd_amd import inputs, ssm

    w = inputs.WORKLOADS["decode_s64_l48"]
    b, h, p, n, g = w.batch, w.nheads, w.headdim, w.dstate, w.ngroups
    snaps = [torch.empty((ndraft + 1, b, h, p, n), dtype=torch.float32, device=dev)
             for _ in range(layers)]
    for l in range(layers):
        snaps[l][0].copy_(inputs.draw("h0", (b, h, p, n), w.seed + l, dev))
    pr = inputs.make_problem(b, ndraft, h, p, n, g, "bf16", w.seed, dev, with_dy=False)
    y = torch.empty_like(pr["x"])
    acc = torch.tensor([i % (ndraft + 1) for i in range(b)], dtype=torch.int32, device=dev)
    out = torch.empty((b, h, p, n), dtype=torch.float32, device=dev)
    args = [pr[k] for k in ("x", "B", "C", "dt", "A", "D")]
    state_b = b * h * p * n * 4
    io_b = ndraft * (b * h * (2 * p * 2 + 4) + b * g * 2 * 2 * n)
    res = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for name, fn, nbytes in (
            ("draft", lambda l: ssm.ssm_draft_snapshots(None, *args, y=y, snapshots=snaps[l]),
             (1 + ndraft) * state_b + io_b),
            ("rollback", lambda l: ssm.ssm_rollback(snaps[l], acc, state_out=out), 2 * state_b)):
        fn(0)
        torch.cuda.synchronize()
        e0.record()
        for rep in range(3):
            for l in range(layers):
                fn(l)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / (3 * layers)
        res[name] = path_entry(0, nbytes, ms)
    res["shape"] = f"{b} sequences x {h} heads x [{p},{n}], draft of {ndraft}, per layer call"
    del snaps, pr, y, out
    torch.cuda.empty_cache()
    return res


def around_scan_rates(dev):
    """The stages around the scan at the prefill layer's size (batch 4 x 4096 tokens):
    the causal conv1d + SiLU over 18,432 channels (256 heads x 64 + 2 x 8 groups x 128),
    4 taps, and the gated RMSNorm over 16,384 channels in 8 groups, bf16 storage.
    Bytes: conv forward u read + out written (4 B per element), backward u, dout read +
    du written (6 B); norm forward y, z read + out written (6 B), backward y, z, dout
    read + dy, dz written (10 B).  Parameter partials are not counted."""
    import torch

    from backward_mamba_ssd_amd import inputs, ssm

    b, t, k = 4, 4096, 4
    c = 256 * 64 + 2 * 8 * 128
    seed = 9000
    bf = torch.bfloat16
    u = inputs.draw("conv_u", (b, t, c), seed, dev, bf)
    w = inputs.draw("conv_w", (c, k), seed, dev)
    bias = inputs.draw("conv_b", (c,), seed, dev)
    dout = inputs.draw("dout", (b, t, c), seed, dev, bf)
    res = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out = torch.empty_like(u)
    n = u.numel()
    res["conv_fwd"] = path_entry(0, 4 * n, timed(lambda: ssm.ssm_conv1d_silu(u, w, bias, out=out,
                                                                               conv_final=None)))
    ws = torch.empty(ssm.lib().ssm_conv1d_silu_workspace_bytes(b, t, c, k), dtype=torch.uint8,
                     device=dev)
    res["conv_bwd"] = path_entry(0, 6 * n, timed(lambda: ssm.ssm_conv1d_silu_bwd(
        u, w, bias, dout, want_dinit=False, workspace=ws)))
    del u, dout, out, ws
    rows, cn, g = b * t, 256 * 64, 8
    y = inputs.draw("conv_u", (rows, cn), seed, dev, bf)
    z = inputs.draw("gate_z", (rows, cn), seed, dev, bf)
    nw = inputs.draw("norm_w", (cn,), seed, dev)
    do = inputs.draw("dout", (rows, cn), seed, dev, bf)
    o = torch.empty_like(y)
    m = y.numel()
    res["norm_fwd"] = path_entry(0, 6 * m, timed(lambda: ssm.ssm_gated_rmsnorm(y, z, nw, g, out=o)))
    ws = torch.empty(ssm.lib().ssm_gated_rmsnorm_workspace_bytes(rows, cn, g), dtype=torch.uint8,
                     device=dev)
    res["norm_bwd"] = path_entry(0, 10 * m, timed(lambda: ssm.ssm_gated_rmsnorm_bwd(
        y, z, nw, do, g, workspace=ws)))
    res["shape"] = (f"conv: batch {b} x {t} tokens x {c} channels, {k} taps; norm: {rows} rows x "
                    f"{cn} channels, {g} groups; bf16 storage")
    del y, z, do, o, ws
    torch.cuda.empty_cache()
    return res


def decode_rates(dev):
    """Decode on the full 64 x 48 x 100 workload (float32 state and FP16-SR state cache)
    and the SR16 checkpoint rate."""
    import torch

    from backward_mamba_ssd_amd import inputs, ssm

    out = {}
    w = inputs.WORKLOADS["decode_s64_l48"]
    layers, steps = w.extra["layers"], w.extra["steps"]
    log(f"decode: {w.batch} sequences x {layers} layers x {steps} steps")
    pr = inputs.make_decode_problem(w.batch, layers, steps, w.nheads, w.headdim, w.dstate,
                                    w.ngroups, w.seed, dev)
    y = torch.empty((layers, w.batch, w.nheads, w.headdim), dtype=torch.bfloat16, device=dev)
    for l in range(layers):  # warm-up: one step
        ssm.ssm_decode_step(pr["state"][l], pr["x"][0, l], pr["B"][0, l], pr["C"][0, l],
                            pr["dt"][0, l], pr["A"][l], pr["D"][l], y=y[l])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(steps):
        for l in range(layers):
            ssm.ssm_decode_step(pr["state"][l], pr["x"][s, l], pr["B"][s, l], pr["C"][s, l],
                                pr["dt"][s, l], pr["A"][l], pr["D"][l], y=y[l])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    PN = w.headdim * w.dstate
    per_call = (w.batch * w.nheads * (8 * PN + 2 * 2 * w.headdim + 4)
                + w.batch * w.ngroups * 2 * 2 * w.dstate)
    dec = path_entry(steps * layers * w.batch * w.nheads * 5 * PN, steps * layers * per_call, ms,
                     FP32_VALU_PEAK_TFLOPS)
    dec["ms_per_step_48_layers"] = round(ms / steps, 4)
    dec["tokens_per_s"] = round(w.batch * steps / (ms * 1e-3), 1)
    out["decode"] = dec
    # the same decode on a binary16 state cache, stochastically rounded on store
    s16 = torch.stack([pr["state"][l].half().view(torch.int16) for l in range(layers)])
    for l in range(layers):
        ssm.ssm_decode_step_sr16(s16[l], pr["x"][0, l], pr["B"][0, l], pr["C"][0, l],
                                 pr["dt"][0, l], pr["A"][l], pr["D"][l], 1, l, y=y[l])
    torch.cuda.synchronize()
    e0.record()
    for s in range(steps):
        for l in range(layers):
            ssm.ssm_decode_step_sr16(s16[l], pr["x"][s, l], pr["B"][s, l], pr["C"][s, l],
                                     pr["dt"][s, l], pr["A"][l], pr["D"][l], 1,
                                     (s + 1) * layers + l, y=y[l])
    e1.record()
    torch.cuda.synchronize()
    ms16 = e0.elapsed_time(e1)
    per_call16 = per_call - w.batch * w.nheads * 4 * PN
    d16 = path_entry(steps * layers * w.batch * w.nheads * 5 * PN, steps * layers * per_call16,
                     ms16, FP32_VALU_PEAK_TFLOPS)
    d16["ms_per_step_48_layers"] = round(ms16 / steps, 4)
    d16["tokens_per_s"] = round(w.batch * steps / (ms16 * 1e-3), 1)
    out["decode_sr16_state"] = d16
    del s16
    st = pr["state"][0]
    del pr
    bits = torch.empty(st.shape, dtype=torch.int16, device=dev)
    ssm.ssm_checkpoint_sr16(st, 1, 0, out=bits)
    torch.cuda.synchronize()
    e0.record()
    for k in range(20):
        ssm.ssm_checkpoint_sr16(st, 1, k, out=bits)
    e1.record()
    torch.cuda.synchronize()
    out["sr16"] = path_entry(0, st.numel() * 6, e0.elapsed_time(e1) / 20)
    del st, bits
    torch.cuda.empty_cache()
    return out


def long_context_rates(dev):
    """fwd+bwd on the T = 131,072 long-context workload (512 saved states per head)."""
    from backward_mamba_ssd_amd import inputs

    wl = inputs.WORKLOADS["long_b1_t131072"]
    log(f"long context: {wl.name}")
    r = time_fwd_bwd(wl, dev, steps=3, warmup=1)
    fb = fwd_flops_per_token(wl) + bwd_flops_per_token(wl)
    by = fwd_bytes_per_token(wl) + bwd_method_bytes_per_token(wl)
    lc = path_entry(fb * r["tokens"], by * r["tokens"], r["step"][1])
    lc["kernels_ms"] = {"ssd_fwd_kernel": round(r["fwd"][1], 4),
                        "ssm_bwd_call": round(r["bwd"][1], 4),
                        "ssd_bwd_block_kernel": round(r["blk"][1], 4)}
    lc["tokens_per_s"] = round(r["tokens"] * 3 / r["wall_s"], 1)
    lc["workload"] = wl.name
    return lc


def fwd_inference_rates(dev):
    """The chunked forward in inference form on the prefill workload: outputs and the
    final state only, no chunk-boundary states saved (70,656 B per token at the head
    shape: x, y, B, C, dt)."""
    import statistics

    import torch

    from backward_mamba_ssd_amd import inputs, ssm

    w = inputs.WORKLOADS["prefill_b4_t4096"]
    pr = inputs.make_workload_problem(w, dev, with_dy=False)
    b, t, h, p = pr["x"].shape
    n = pr["B"].shape[3]
    y = torch.empty_like(pr["x"])
    hf = torch.empty((b, h, p, n), dtype=torch.float32, device=dev)

    def run():
        ssm.ssm_fwd_chunked(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], chunk=w.chunk,
                            h_final=hf, chunk_states=None, y=y)

    for _ in range(10):  # also brings the clocks up when the section runs alone
        run()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(20)]
    for e0, e1 in ev:
        e0.record()
        run()
        e1.record()
    torch.cuda.synchronize()
    ms = statistics.median(e0.elapsed_time(e1) for e0, e1 in ev)
    H, P, N, G = w.nheads, w.headdim, w.dstate, w.ngroups
    nbytes = (2 * H * P + 2 * H * P + 2 * 2 * G * N + 4 * H) * b * t + 4 * b * H * P * N
    e = path_entry(fwd_flops_per_token(w) * b * t, nbytes, ms)
    e["tokens_per_s"] = round(b * t / (ms * 1e-3), 1)
    e["workload"] = w.name
    del pr, y, hf
    torch.cuda.empty_cache()
    return e


def copy_calibration(dev):
    """Three plain 1 GiB device-to-device copies: the known-size reference that scales
    the HBM byte counters (FETCH_SIZE, WRITE_SIZE) of a profiled run."""
    import torch

    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    n = src.numel() * 4
    del src, dst
    torch.cuda.empty_cache()
    return n


SECTIONS = {
    "fwd_inference": fwd_inference_rates,
    "decode": decode_rates,
    "dt_prep": dt_prep_rates,
    "draft_rollback": draft_rollback_rates,
    "around_scan": around_scan_rates,
    "replay_sr16_b16": replay_sweep,
    "long_context_fwd_bwd": long_context_rates,
}


def secondary(dev):
    """Every path besides the fwd+bwd step: decode, SR16, time-step preparation, drafts and
    rollback, the stages around the scan, the replay sweep and the long-context step."""
    out = {}
    for name, fn in SECTIONS.items():
        log(f"{name} ...")
        r = fn(dev)
        if name == "decode":
            out.update(r)
        else:
            out[name] = r
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_b4_t4096")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--section", choices=sorted(SECTIONS),
                    help="run only this secondary measurement and print its JSON (for profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy (3 times), the known-size "
                         "reference for scaling HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(sharding is design-only); rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from backward_mamba_ssd_amd import inputs

    dev = torch.device("cuda:0")
    if args.section:
        out = {"section": args.section, "result": SECTIONS[args.section](dev)}
        if args.copy_calibration:
            out["copy_calibration_bytes"] = copy_calibration(dev)
        print(json.dumps(out), flush=True)
        return
    w = inputs.WORKLOADS[args.workload]
    log(f"workload {w.name}: batch {w.batch} T {w.seqlen} heads {w.nheads} P {w.headdim} "
        f"N {w.dstate} groups {w.ngroups} chunk {w.chunk}")
    K = args.steps
    r = time_fwd_bwd(w, dev, K, args.warmup)
    tokens = r["tokens"]
    el = r["wall_s"]
    fwd_ms, blk_ms, bwd_ms = r["fwd"][0], r["blk"][0], r["bwd"][0]
    value = tokens * K / el
    log(f"step {el / K * 1e3:.3f} ms: forward kernel {fwd_ms:.3f} ms, backward call {bwd_ms:.3f} ms "
        f"(per-block kernel {blk_ms:.3f} ms)")

    # per kernel: (mean ms, the method's algorithmic bytes per launch, this design's bytes)
    kernels = {
        "ssd_fwd_kernel": (fwd_ms, fwd_bytes_per_token(w) * tokens, fwd_bytes_per_token(w) * tokens),
        "ssd_bwd_block_kernel": (blk_ms, bwd_method_bytes_per_token(w) * tokens,
                                 bwd_block_design_bytes_per_token(w) * tokens),
    }
    dom = max(kernels, key=lambda k: kernels[k][0])
    ms, nbytes, dbytes = kernels[dom]
    achieved = nbytes / (ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(dom, w.name),
                "kernel": dom, "mean_ms": round(ms, 4), "bytes_per_launch": int(nbytes),
                "design_bytes_per_launch": int(dbytes)}
    ff, bf = fwd_flops_per_token(w) * tokens, bwd_flops_per_token(w) * tokens
    fb, bb = fwd_bytes_per_token(w) * tokens, bwd_method_bytes_per_token(w) * tokens
    paths = {
        "fwd_chunked": path_entry(ff, fb, r["fwd"][1]),
        "bwd_call": path_entry(bf, bb, r["bwd"][1]),
        "fwd_bwd_step": path_entry(ff + bf, fb + bb, r["step"][1]),
    }
    paths["bwd_call"]["design_bytes"] = int(bwd_call_design_bytes_per_token(w) * tokens)
    paths["bwd_call"]["design_over_method_bytes"] = round(
        bwd_call_design_bytes_per_token(w) / bwd_method_bytes_per_token(w), 3)
    res = {
        "metric": "SSM fwd+bwd tokens/s at 256h x 64 x 128",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(el / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; x,B,C,dy bf16; dt,A,D fp32)",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "nheads": w.nheads,
                   "headdim": w.headdim, "dstate": w.dstate, "ngroups": w.ngroups,
                   "chunk": w.chunk},
        "roofline": roofline,
        "kernels_ms": {"ssd_fwd_kernel": round(fwd_ms, 4), "ssm_bwd_call": round(bwd_ms, 4),
                       "ssd_bwd_block_kernel": round(blk_ms, 4)},
        "kernels_median_ms": {"ssd_fwd_kernel": round(r["fwd"][1], 4),
                              "ssm_bwd_call": round(r["bwd"][1], 4),
                              "ssd_bwd_block_kernel": round(r["blk"][1], 4)},
        "paths": paths,
        "fwd_mfma_frac": round(fwd_mfma_flops_per_token(w) * tokens / (fwd_ms * 1e-3)
                               / (BF16_PEAK_TFLOPS * 1e12), 4),
    }
    if not args.no_secondary:
        pk = measured_peaks(dev)
        res["measured_peaks"] = pk
        roofline["measured_peak"] = pk["copy_GBps"]
        roofline["frac_of_measured"] = round(achieved / pk["copy_GBps"], 4)
        res["secondary"] = secondary(dev)
        torch.cuda.empty_cache()
    if args.copy_calibration:
        res["copy_calibration_bytes"] = copy_calibration(dev)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
