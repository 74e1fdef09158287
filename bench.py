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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def fwd_bytes_per_token(w):
    """Algorithmic HBM bytes per token of the chunked forward (training mode):
    x read + y write (2 B each), B and C read (2 B), dt read (4 B), and the
    chunk-boundary state written once per chunk (4 B per state element)."""
    H, P, N, G, L = w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    return 2 * H * P + 2 * H * P + 2 * 2 * G * N + 4 * H + 4 * H * P * N / L


def bwd_block_bytes_per_token(w):
    """Algorithmic HBM bytes per token of the per-block backward kernel:
    x, dy read and dx written (2 B each), the chunk-boundary state and the
    chunk-exit state gradient read once per chunk (4 B per element), B and C
    read (2 B), dB and dC written (4 B), dt read and ddt written (4 B)."""
    H, P, N, G, L = w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    return (3 * 2 * H * P + 2 * 4 * H * P * N / L + 2 * 2 * G * N + 2 * 4 * G * N + 2 * 4 * H)


KERNEL_SOURCES = {
    "ssd_fwd_kernel": ("ssd_fwd.hip", "ssd_common.hpp", "common.hpp", "launch.hpp"),
    "ssd_bwd_block_kernel": ("ssd_bwd.hip", "ssd_common.hpp", "common.hpp", "launch.hpp"),
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


def cpu_baseline(w, budget_s=20.0):
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


def secondary(dev):
    """Decode (full 64 x 48 x 100 workload) and SR16 rates."""
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
    gbps = steps * layers * per_call / (ms * 1e-3) / 1e9
    out["decode_state_update_GBps"] = round(gbps, 1)
    out["decode_hbm_frac"] = round(gbps / HBM_PEAK_GBPS, 4)
    out["decode_ms_per_step_48_layers"] = round(ms / steps, 4)
    out["decode_tokens_per_s"] = round(w.batch * steps / (ms * 1e-3), 1)
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
    ms = e0.elapsed_time(e1) / 20
    out["sr16_GBps"] = round(st.numel() * 6 / (ms * 1e-3) / 1e9, 1)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_b4_t4096")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy (3 times), the known-size "
                         "reference for scaling HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(sharding is design-only); rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from backward_mamba_ssd_amd import inputs, ssm

    dev = torch.device("cuda:0")
    w = inputs.WORKLOADS[args.workload]
    log(f"workload {w.name}: batch {w.batch} T {w.seqlen} heads {w.nheads} P {w.headdim} "
        f"N {w.dstate} groups {w.ngroups} chunk {w.chunk}")
    pr = inputs.make_workload_problem(w, dev)
    dims = ssm.dims_of(pr["x"], pr["B"], w.chunk)
    assert ssm.ssm_uses_mfma_path(dims, ssm.SSM_BF16)
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
        if ev is not None:
            ev[1].record()
            ssm.ssm_profile_next_bwd_block(ev[2], ev[3])
        ssm.ssm_bwd(pr["x"], pr["B"], pr["C"], pr["dt"], pr["A"], pr["D"], cs, pr["dy"],
                    chunk=w.chunk, out=grads, workspace=ws)
        if ev is not None:
            ev[4].record()

    for _ in range(args.warmup):
        step()
    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        step(evs[k])
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / K
    blk_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / K
    bwd_ms = sum(e[1].elapsed_time(e[4]) for e in evs) / K
    tokens = b * t
    value = tokens * K / el
    log(f"step {el / K * 1e3:.3f} ms: forward kernel {fwd_ms:.3f} ms, backward call {bwd_ms:.3f} ms "
        f"(per-block kernel {blk_ms:.3f} ms)")

    kernels = {
        "ssd_fwd_kernel": (fwd_ms, fwd_bytes_per_token(w) * tokens),
        "ssd_bwd_block_kernel": (blk_ms, bwd_block_bytes_per_token(w) * tokens),
    }
    dom = max(kernels, key=lambda k: kernels[k][0])
    ms, nbytes = kernels[dom]
    achieved = nbytes / (ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(dom, w.name),
                "kernel": dom, "mean_ms": round(ms, 4), "bytes_per_launch": int(nbytes)}
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
        "config": {"workload": w.name, "batch": b, "seqlen": t, "nheads": h, "headdim": p,
                   "dstate": n, "ngroups": g, "chunk": w.chunk},
        "roofline": roofline,
        "kernels_ms": {"ssd_fwd_kernel": round(fwd_ms, 4), "ssm_bwd_call": round(bwd_ms, 4),
                       "ssd_bwd_block_kernel": round(blk_ms, 4)},
        "fwd_mfma_frac": round(fwd_mfma_flops_per_token(w) * tokens / (fwd_ms * 1e-3)
                               / (BF16_PEAK_TFLOPS * 1e12), 4),
    }
    del pr, y, cs, grads, ws
    torch.cuda.empty_cache()
    if not args.no_secondary:
        res["secondary"] = secondary(dev)
        torch.cuda.empty_cache()
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = src.numel() * 4
        del src, dst
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
