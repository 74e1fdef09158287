"""fp64 CPU oracle for the Mamba-2 selective SSM recurrence -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The GPU product path never touches it and
it shares no code with the HIP library.

The heavy loops live in ``ssm_oracle.c`` (plain sequential C, fp64, OpenMP over
independent (batch, head) or (batch, group) units); this file compiles it with
gcc, marshals numpy arrays, and holds the few scalar helpers that the pages
state as small examples:

* ``checkpoint_budget`` -- "Nemotron 3 Ultra: replaying a rounded state",
  section "An error budget for checkpoint writes": after each checkpoint write
  the allowance is the previous one shrunk by L**n (n tokens since the last
  write) plus one write allowance delta.
* ``grid_schedule_run`` -- same page, section "Fewer writes can leave a larger
  error": the scalar update s' = a*s + u with round-half-even writes onto the
  integer grid at the end of every chunk of the schedule.
* ``state_bytes`` / ``kv_bytes`` -- same page, section "Counting the state and
  attention cache": payload counts of the recurrent state and of the KV cache.
* ``replay_additive`` -- same page, section "Recovering the state by replay":
  the s' = s + u example of replaying the pending buffer from a checkpoint.

``draft_snapshots`` / ``rollback`` -- same page, section "Rolling back rejected
draft tokens": a snapshot after every draft step with the initial state first,
and the restore that selects the snapshot after the accepted prefix.

``conv1d_silu`` / ``gated_rmsnorm`` (and their ``_bwd``) wrap the C versions of
the stages around the scan: the short causal depthwise convolution with SiLU,
and the SiLU-gated RMSNorm over groups of channels.

``dt_prep`` / ``dt_prep_bwd`` wrap the C preparation of the time step
(softplus of raw + bias, clamped to a closed interval) and of the per-head rate
A = -exp(logA), with their gradients.

Parity of every function here is pinned by ``tests/test_oracle_*.py`` against
closed forms, a textbook filter (scipy.signal.lfilter), central finite
differences, brute force, and the pages' worked values under ``tests/golden``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from fractions import Fraction

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile ssm_oracle.c with gcc (fp64, no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
            i64, vp, u64 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_uint64
            lib.oracle_fwd.argtypes = [i64] * 7 + [vp] * 10
            lib.oracle_fwd.restype = None
            lib.oracle_bwd.argtypes = [i64] * 6 + [vp] * 16
            lib.oracle_bwd.restype = None
            lib.oracle_decode_step.argtypes = [i64] * 5 + [vp] * 8
            lib.oracle_decode_step.restype = None
            lib.oracle_splitmix64_output.argtypes = [u64, u64]
            lib.oracle_splitmix64_output.restype = u64
            lib.oracle_hash32.argtypes = [u64, u64, u64]
            lib.oracle_hash32.restype = ctypes.c_uint32
            lib.oracle_sr16_one.argtypes = [ctypes.c_float, ctypes.c_uint32]
            lib.oracle_sr16_one.restype = ctypes.c_uint16
            lib.oracle_sr16.argtypes = [vp, vp, i64, u64, u64, u64]
            lib.oracle_sr16.restype = None
            lib.oracle_half_to_double_array.argtypes = [vp, vp, i64]
            lib.oracle_half_to_double_array.restype = None
            f32 = ctypes.c_float
            lib.oracle_dt_prep.argtypes = [i64, i64, vp, vp, vp, f32, f32, vp, vp]
            lib.oracle_dt_prep.restype = None
            lib.oracle_dt_prep_bwd.argtypes = [i64, i64, vp, vp, vp, f32, f32, vp, vp, vp, vp, vp]
            lib.oracle_dt_prep_bwd.restype = None
            lib.oracle_conv1d_silu.argtypes = [i64] * 4 + [vp] * 6
            lib.oracle_conv1d_silu.restype = None
            lib.oracle_conv1d_silu_bwd.argtypes = [i64] * 4 + [vp] * 9
            lib.oracle_conv1d_silu_bwd.restype = None
            f64 = ctypes.c_double
            lib.oracle_gated_rmsnorm.argtypes = [i64] * 3 + [vp] * 3 + [f64, vp]
            lib.oracle_gated_rmsnorm.restype = None
            lib.oracle_gated_rmsnorm_bwd.argtypes = [i64] * 3 + [vp] * 3 + [f64] + [vp] * 4
            lib.oracle_gated_rmsnorm_bwd.restype = None
            lib.oracle_num_threads.argtypes = []
            lib.oracle_num_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _f32(a):
    """Contiguous float32 numpy array (the SR16 rule reads float32 values)."""
    if hasattr(a, "detach"):  # torch tensor: bf16 -> f32 is exact
        a = a.detach().to("cpu").float().contiguous().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _f64(a):
    """Exact widening to a contiguous float64 numpy array (bf16/fp16/fp32 in)."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor: bf16 -> f64 is exact
        a = a.detach().to("cpu").double().contiguous().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def fwd(x, B, C, dt, A, D, h0=None, chunk=None, want_chunk_states=False):
    """Sequential forward.  x [Bsz,T,H,P], B/C [Bsz,T,G,N], dt [Bsz,T,H], A/D [H].

    Returns dict with y [Bsz,T,H,P], h_final [Bsz,H,P,N] and, when
    ``want_chunk_states``, chunk_states [Bsz,H,nc,P,N] (state entering each
    chunk of ``chunk`` tokens).  All float64.
    """
    x, B, C, dt, A, D = (_f64(v) for v in (x, B, C, dt, A, D))
    h0 = _f64(h0)
    Bsz, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    L = int(chunk) if chunk else T
    assert L >= 1 and H % G == 0
    nc = (T + L - 1) // L
    y = np.empty((Bsz, T, H, P), np.float64)
    hf = np.empty((Bsz, H, P, N), np.float64)
    cs = np.empty((Bsz, H, nc, P, N), np.float64) if want_chunk_states else None
    _load().oracle_fwd(Bsz, T, H, P, N, G, L, _p(x), _p(B), _p(C), _p(dt), _p(A), _p(D),
                       _p(h0), _p(y), _p(hf), _p(cs))
    out = {"y": y, "h_final": hf}
    if want_chunk_states:
        out["chunk_states"] = cs
    return out


def bwd(x, B, C, dt, A, D, dy, h0=None, dh_final=None):
    """Reverse sweep; returns dict dx, dB, dC, ddt, dA, dD, dh0 (float64)."""
    x, B, C, dt, A, D, dy = (_f64(v) for v in (x, B, C, dt, A, D, dy))
    h0, dh_final = _f64(h0), _f64(dh_final)
    Bsz, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    out = {
        "dx": np.empty((Bsz, T, H, P), np.float64),
        "dB": np.empty((Bsz, T, G, N), np.float64),
        "dC": np.empty((Bsz, T, G, N), np.float64),
        "ddt": np.empty((Bsz, T, H), np.float64),
        "dA": np.empty((H,), np.float64),
        "dD": np.empty((H,), np.float64),
        "dh0": np.empty((Bsz, H, P, N), np.float64),
    }
    _load().oracle_bwd(Bsz, T, H, P, N, G, _p(x), _p(B), _p(C), _p(dt), _p(A), _p(D),
                       _p(h0), _p(dy), _p(dh_final), _p(out["dx"]), _p(out["dB"]),
                       _p(out["dC"]), _p(out["ddt"]), _p(out["dA"]), _p(out["dD"]),
                       _p(out["dh0"]))
    return out


def decode_step(state, x, B, C, dt, A, D):
    """One token on a float64 state [Bsz,H,P,N] (updated in place); returns y [Bsz,H,P]."""
    assert state.dtype == np.float64 and state.flags["C_CONTIGUOUS"]
    x, B, C, dt, A, D = (_f64(v) for v in (x, B, C, dt, A, D))
    Bsz, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    y = np.empty((Bsz, H, P), np.float64)
    _load().oracle_decode_step(Bsz, H, P, N, G, _p(state), _p(x), _p(B), _p(C), _p(dt),
                               _p(A), _p(D), _p(y))
    return y


def replay(ckpt, x, B, C, dt, A, D, t0, r):
    """Run r tokens (t0 .. t0+r-1 of full-length inputs) from a saved state.

    This is the forward from a given state: the retained prepared inputs are
    applied again in order ("Recovering the state by replay").  Returns dict
    with y [Bsz,r,H,P] and h_final [Bsz,H,P,N].
    """
    sl = slice(t0, t0 + r)
    return fwd(_f64(x)[:, sl], _f64(B)[:, sl], _f64(C)[:, sl], _f64(dt)[:, sl], A, D,
               h0=ckpt)


# ----------------------------------------------------------------------------
# speculative drafts and rollback ("Nemotron 3 Ultra: replaying a rounded state",
# section "Rolling back rejected draft tokens")
# ----------------------------------------------------------------------------

def draft_snapshots(state0, x, B, C, dt, A, D):
    """The snapshot stack of a draft of Dr tokens: slot 0 is the initial state (the
    page includes it, so rejecting the whole draft selects it) and slot k the state
    after the first k draft tokens, each token taken by the one-step update.
    x [Bsz,Dr,H,P], B/C [Bsz,Dr,G,N], dt [Bsz,Dr,H]; returns (snapshots
    [Dr+1,Bsz,H,P,N], y [Bsz,Dr,H,P]), float64."""
    s = np.array(_f64(state0), dtype=np.float64, order="C", copy=True)
    x, B, C, dt = (_f64(v) for v in (x, B, C, dt))
    Bsz, Dr, H, P = x.shape
    snaps = np.empty((Dr + 1,) + s.shape, np.float64)
    y = np.empty((Bsz, Dr, H, P), np.float64)
    snaps[0] = s
    for k in range(Dr):
        y[:, k] = decode_step(s, np.ascontiguousarray(x[:, k]), np.ascontiguousarray(B[:, k]),
                              np.ascontiguousarray(C[:, k]), np.ascontiguousarray(dt[:, k]), A, D)
        snaps[k + 1] = s
    return snaps, y


def rollback(snapshots, accepted):
    """The state to continue from after verification: for sequence b, the stored
    snapshot after its accepted[b] draft tokens (the page's restore)."""
    snapshots = _f64(snapshots)
    return np.stack([snapshots[int(a), b] for b, a in enumerate(accepted)])


# ----------------------------------------------------------------------------
# the stages around the scan ("Nemotron Kernels...", Kernel 1 "Forward And
# Inference": causal Conv1D + SiLU before the scan, gated group RMSNorm after it)
# ----------------------------------------------------------------------------

def conv1d_silu(u, w, bias, init=None):
    """SiLU of the short causal depthwise convolution.  u [Bsz,T,C], w [C,K],
    bias [C], init [Bsz,K-1,C] or None (zeros).  Returns (out [Bsz,T,C],
    final [Bsz,K-1,C]: the last K-1 samples, the next call's init)."""
    u, w, bias, init = _f64(u), _f64(w), _f64(bias), _f64(init)
    Bsz, T, C = u.shape
    K = w.shape[1]
    out = np.empty((Bsz, T, C), np.float64)
    fin = np.empty((Bsz, K - 1, C), np.float64)
    _load().oracle_conv1d_silu(Bsz, T, C, K, _p(u), _p(w), _p(bias), _p(init), _p(out), _p(fin))
    return out, fin


def conv1d_silu_bwd(u, w, bias, dout, init=None):
    """Gradients of sum(dout * out): dict du [Bsz,T,C], dw [C,K], dbias [C],
    dinit [Bsz,K-1,C]."""
    u, w, bias, init, dout = _f64(u), _f64(w), _f64(bias), _f64(init), _f64(dout)
    Bsz, T, C = u.shape
    K = w.shape[1]
    g = {"du": np.empty((Bsz, T, C)), "dw": np.empty((C, K)), "dbias": np.empty(C),
         "dinit": np.empty((Bsz, K - 1, C))}
    _load().oracle_conv1d_silu_bwd(Bsz, T, C, K, _p(u), _p(w), _p(bias), _p(init), _p(dout),
                                   _p(g["du"]), _p(g["dw"]), _p(g["dbias"]), _p(g["dinit"]))
    return g


def gated_rmsnorm(y, z, w, ngroups, eps=1e-5):
    """out = g / rms_group(g) * w with g = y * SiLU(z), groups of C/ngroups
    consecutive channels.  y, z [..., C], w [C]."""
    y, z, w = _f64(y), _f64(z), _f64(w)
    C = y.shape[-1]
    rows = y.size // C if C else 0
    out = np.empty(y.shape, np.float64)
    _load().oracle_gated_rmsnorm(rows, C, ngroups, _p(y), _p(z), _p(w), float(eps), _p(out))
    return out


def gated_rmsnorm_bwd(y, z, w, dout, ngroups, eps=1e-5):
    """Gradients of sum(dout * out): dict dy, dz [..., C], dw [C]."""
    y, z, w, dout = _f64(y), _f64(z), _f64(w), _f64(dout)
    C = y.shape[-1]
    rows = y.size // C if C else 0
    g = {"dy": np.empty(y.shape), "dz": np.empty(y.shape), "dw": np.empty(C)}
    _load().oracle_gated_rmsnorm_bwd(rows, C, ngroups, _p(y), _p(z), _p(w), float(eps), _p(dout),
                                     _p(g["dy"]), _p(g["dz"]), _p(g["dw"]))
    return g


# ----------------------------------------------------------------------------
# time-step and rate preparation ("Nemotron Kernels...", section "From Classical
# State Space To A Selective Mamba State"; TorchLean page, "The Mamba state update")
# ----------------------------------------------------------------------------

def dt_prep(raw, bias, logA, lo=0.0, hi=float("inf")):
    """dt = clamp(softplus(raw + bias[h]), lo, hi) [..., H] and A = -exp(logA) [H]."""
    raw = _f64(raw)
    H = raw.shape[-1]
    rows = raw.size // H if H else 0
    dt = np.empty(raw.shape, np.float64)
    A = np.empty(H, np.float64)
    _load().oracle_dt_prep(rows, H, _p(raw), _p(_f64(bias)), _p(_f64(logA)), ctypes.c_float(lo),
                           ctypes.c_float(hi), _p(dt), _p(A))
    return dt, A


def dt_prep_bwd(raw, bias, logA, ddt, dA, lo=0.0, hi=float("inf")):
    """Gradients (d_raw [..., H], d_bias [H], d_logA [H]) from ddt and dA."""
    raw = _f64(raw)
    H = raw.shape[-1]
    rows = raw.size // H if H else 0
    d_raw = np.empty(raw.shape, np.float64)
    d_bias = np.empty(H, np.float64)
    d_logA = np.empty(H, np.float64)
    _load().oracle_dt_prep_bwd(rows, H, _p(raw), _p(_f64(bias)), _p(_f64(logA)),
                               ctypes.c_float(lo), ctypes.c_float(hi), _p(_f64(ddt)),
                               _p(_f64(dA)), _p(d_raw), _p(d_bias), _p(d_logA))
    return d_raw, d_bias, d_logA


# ----------------------------------------------------------------------------
# counter-based entropy and stochastic rounding to binary16
# ----------------------------------------------------------------------------

def splitmix64_output(seed: int, k: int) -> int:
    return int(_load().oracle_splitmix64_output(seed & (2**64 - 1), k & (2**64 - 1)))


def hash32(seed: int, ckpt: int, elem: int) -> int:
    return int(_load().oracle_hash32(seed & (2**64 - 1), ckpt, elem))


def sr16_one(v: float, u: int) -> int:
    return int(_load().oracle_sr16_one(ctypes.c_float(v), ctypes.c_uint32(u)))


def sr16(v, seed: int, ckpt: int, elem_offset: int = 0):
    """SR16 bits (uint16 array, same shape) of float32 values v."""
    v = _f32(v)
    out = np.empty(v.shape, np.uint16)
    _load().oracle_sr16(_p(v), _p(out), v.size, seed & (2**64 - 1), ckpt, elem_offset)
    return out


def half_bits_to_double(bits):
    bits = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    out = np.empty(bits.shape, np.float64)
    _load().oracle_half_to_double_array(_p(bits), _p(out), bits.size)
    return out


# ----------------------------------------------------------------------------
# scalar helpers from the TorchLean page's small examples (exact rationals)
# ----------------------------------------------------------------------------

def checkpoint_budget(L, delta, e0, chunk_lengths):
    """Worst-case allowance after each checkpoint write: E <- L**n * E + delta."""
    e = Fraction(e0)
    out = []
    for n in chunk_lengths:
        e = Fraction(L) ** n * e + Fraction(delta)
        out.append(e)
    return out


def _round_half_even(v: Fraction) -> Fraction:
    fl = v.numerator // v.denominator
    rem = v - fl
    if rem > Fraction(1, 2):
        return Fraction(fl + 1)
    if rem < Fraction(1, 2):
        return Fraction(fl)
    return Fraction(fl if fl % 2 == 0 else fl + 1)


def grid_schedule_run(a, s0, chunks):
    """s' = a*s + u over each chunk, then a nearest-even write onto the integers."""
    s = Fraction(s0)
    for chunk in chunks:
        for u in chunk:
            s = Fraction(a) * s + Fraction(u)
        s = _round_half_even(s)
    return s


def replay_additive(checkpoint, pending, suffix=()):
    """Replay for the transition s' = s + u: the observed state, then the suffix."""
    s = checkpoint
    for u in pending:
        s = s + u
    observed = s
    for u in suffix:
        s = s + u
    return observed, s


def state_bytes(blocks, heads, value_dim, state_dim, bytes_per_entry):
    return blocks * heads * value_dim * state_dim * bytes_per_entry


def kv_bytes(attn_blocks, tokens, kv_heads, width, bytes_per_entry):
    """Keys and values (two tensors) for every attention block and token."""
    return attn_blocks * tokens * 2 * kv_heads * width * bytes_per_entry
