"""ctypes binding of the C-ABI library ``libssm_mi355x.so`` (see include/ssm.h).

The functions carry the C names.  They only marshal arguments: read shapes off
torch tensors, allocate outputs and workspace with torch on the tensors'
device, pass raw device pointers and the current HIP stream, and raise
``SsmError`` on a non-zero status.  Every step of the computation runs in the
library's gfx950 kernels; there is no other code path.  If the library is not
built the import of this module fails loudly.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssm_mi355x.so")

SSM_F32, SSM_BF16, SSM_F16 = 0, 1, 2
SSM_WS_FWD, SSM_WS_BWD, SSM_WS_REPLAY, SSM_WS_DT_PREP_BWD = 0, 1, 2, 3
NOALLOC_SCRATCH_BYTES = 65 << 20  # SSM_NOALLOC_SCRATCH_BYTES: the scratch of ssm_bwd_noalloc
_SIZE_MAX = ctypes.c_size_t(-1).value

EXPORTS = ("ssm_fwd_chunked", "ssm_bwd", "ssm_bwd_timed", "ssm_bwd_noalloc", "ssm_decode_step",
           "ssm_decode_step_sr16", "ssm_checkpoint_sr16", "ssm_replay", "ssm_draft_snapshots",
           "ssm_rollback", "ssm_conv1d_silu", "ssm_conv1d_silu_bwd",
           "ssm_conv1d_silu_workspace_bytes", "ssm_gated_rmsnorm", "ssm_gated_rmsnorm_bwd",
           "ssm_gated_rmsnorm_workspace_bytes", "ssm_dt_prep", "ssm_dt_prep_bwd",
           "ssm_workspace_bytes", "ssm_status_string", "ssm_uses_mfma_path")


class ssm_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("batch", "seqlen", "nheads", "headdim", "dstate", "ngroups", "chunk")]


class SsmError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i64, u64, i32 = (ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64, ctypes.c_uint64,
                             ctypes.c_int)
    D = ctypes.POINTER(ssm_dims)
    f32 = ctypes.c_float
    lib.ssm_status_string.argtypes = [i32]
    lib.ssm_status_string.restype = ctypes.c_char_p
    lib.ssm_workspace_bytes.argtypes = [D, i32, i32, i64]
    lib.ssm_workspace_bytes.restype = sz
    lib.ssm_uses_mfma_path.argtypes = [D, i32]
    lib.ssm_uses_mfma_path.restype = i32
    lib.ssm_fwd_chunked.argtypes = [D, i32] + [vp] * 10 + [vp, sz, vp]
    lib.ssm_fwd_chunked.restype = i32
    lib.ssm_bwd.argtypes = [D, i32] + [vp] * 16 + [vp, sz, vp]
    lib.ssm_bwd.restype = i32
    lib.ssm_bwd_timed.argtypes = [D, i32] + [vp] * 16 + [vp, sz, vp, vp]
    lib.ssm_bwd_timed.restype = i32
    lib.ssm_bwd_noalloc.argtypes = [D, i32] + [vp] * 16 + [vp]
    lib.ssm_bwd_noalloc.restype = i32
    lib.ssm_decode_step.argtypes = [D, i32] + [vp] * 8 + [vp]
    lib.ssm_decode_step.restype = i32
    lib.ssm_decode_step_sr16.argtypes = [D, i32] + [vp] * 8 + [u64, u64, vp]
    lib.ssm_decode_step_sr16.restype = i32
    lib.ssm_checkpoint_sr16.argtypes = [vp, vp, u64, u64, u64, u64, vp]
    lib.ssm_checkpoint_sr16.restype = i32
    lib.ssm_replay.argtypes = ([D, i32, vp, i32, vp] + [vp] * 6 + [i64, i64] + [vp] * 4
                               + [vp, sz, vp])
    lib.ssm_replay.restype = i32
    lib.ssm_conv1d_silu.argtypes = [i64] * 4 + [i32] + [vp] * 7
    lib.ssm_conv1d_silu.restype = i32
    lib.ssm_conv1d_silu_workspace_bytes.argtypes = [i64] * 4
    lib.ssm_conv1d_silu_workspace_bytes.restype = sz
    lib.ssm_conv1d_silu_bwd.argtypes = [i64] * 4 + [i32] + [vp] * 10 + [sz, vp]
    lib.ssm_conv1d_silu_bwd.restype = i32
    lib.ssm_gated_rmsnorm.argtypes = [i64] * 3 + [i32] + [vp] * 3 + [f32, vp, vp]
    lib.ssm_gated_rmsnorm.restype = i32
    lib.ssm_gated_rmsnorm_workspace_bytes.argtypes = [i64] * 3
    lib.ssm_gated_rmsnorm_workspace_bytes.restype = sz
    lib.ssm_gated_rmsnorm_bwd.argtypes = [i64] * 3 + [i32] + [vp] * 3 + [f32] + [vp] * 5 + [sz, vp]
    lib.ssm_gated_rmsnorm_bwd.restype = i32
    lib.ssm_draft_snapshots.argtypes = [D, i32] + [vp] * 8 + [vp]
    lib.ssm_draft_snapshots.restype = i32
    lib.ssm_rollback.argtypes = [D, vp, vp, vp, vp, vp]
    lib.ssm_rollback.restype = i32
    lib.ssm_dt_prep.argtypes = [D, vp, vp, vp, f32, f32, vp, vp, vp]
    lib.ssm_dt_prep.restype = i32
    lib.ssm_dt_prep_bwd.argtypes = [D, vp, vp, vp, f32, f32, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ssm_dt_prep_bwd.restype = i32
    return lib


_lib = _load()


def lib():
    return _lib


def status_string(status: int) -> str:
    return _lib.ssm_status_string(int(status)).decode()


def _check(status, where):
    if status != 0:
        raise SsmError(status, where)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t or None
    return t.data_ptr() or None


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dtype_code(t):
    if t.dtype == torch.float32:
        return SSM_F32
    if t.dtype == torch.bfloat16:
        return SSM_BF16
    raise TypeError(f"unsupported storage dtype {t.dtype}")


def make_dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk=1):
    return ssm_dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk)


def dims_of(x, B, chunk):
    b, t, h, p = x.shape
    g, n = B.shape[2], B.shape[3]
    return make_dims(b, t, h, p, n, g, chunk)


def ssm_workspace_bytes(dims, dtype_code, which, r=0):
    v = _lib.ssm_workspace_bytes(ctypes.byref(dims), int(dtype_code), int(which), int(r))
    if v == _SIZE_MAX:
        raise SsmError(3, "ssm_workspace_bytes")
    return int(v)


def ssm_uses_mfma_path(dims, dtype_code):
    return bool(_lib.ssm_uses_mfma_path(ctypes.byref(dims), int(dtype_code)))


_STORAGE = (torch.float32, torch.bfloat16)


def _arg(name, t, shape, dtypes, device=None):
    """Check one tensor argument before its pointer reaches the library: a torch
    tensor of one of ``dtypes``, exactly ``shape``, contiguous (the kernels index
    dense row-major memory) and on ``device`` when given.  Raises ValueError (or
    TypeError for a non-tensor) so that no kernel ever sees a buffer smaller or
    laid out differently than the call's dims say."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected one of {tuple(dtypes)}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    return t


def _opt(name, t, shape, dtypes, device=None):
    return None if t is None else _arg(name, t, shape, dtypes, device)


def _on_gpu(dev):
    if dev.type != "cuda":
        raise ValueError(f"tensors are on {dev}; the library runs on a GPU device")
    return dev


def _int(name, v, lo):
    if isinstance(v, bool) or not isinstance(v, int) or v < lo:
        raise ValueError(f"{name}: expected an int >= {lo}, got {v!r}")
    return v


def _seq_inputs(x, B, C, dt, A, D):
    """x [b,t,h,p] (f32|bf16), B, C [b,t,g,n] of x's dtype, dt [b,t,h] f32, A, D [h]
    f32, all on x's device.  Returns (b, t, h, p, g, n, device)."""
    for name, t in (("x", x), ("B", B)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if x.dim() != 4:
        raise ValueError("x: expected a 4-d tensor [batch, seqlen, nheads, headdim]")
    _arg("x", x, x.shape, _STORAGE)
    b, t, h, p = x.shape
    if B.dim() != 4:
        raise ValueError("B: expected a 4-d tensor [batch, seqlen, ngroups, dstate]")
    g, n = B.shape[2], B.shape[3]
    dev = x.device
    _arg("B", B, (b, t, g, n), (x.dtype,), dev)
    _arg("C", C, (b, t, g, n), (x.dtype,), dev)
    _arg("dt", dt, (b, t, h), (torch.float32,), dev)
    _arg("A", A, (h,), (torch.float32,), dev)
    _arg("D", D, (h,), (torch.float32,), dev)
    return b, t, h, p, g, n, dev


def _check_ws(ws, device):
    """A caller's workspace: a flat contiguous uint8 tensor on the call's device."""
    if ws is not None:
        _arg("workspace", ws, (ws.numel(),), (torch.uint8,), device)


def _workspace(nbytes, device, ws):
    if nbytes == 0:
        return None, 0
    if ws is not None and ws.numel() >= nbytes:
        return ws, int(ws.numel())
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def ssm_fwd_chunked(x, B, C, dt, A, D, h0=None, chunk=256, h_final=True, chunk_states=True,
                    y=None, workspace=None, stream=None):
    """Chunked prefill forward.  Returns (y, h_final or None, chunk_states or None)."""
    b, t, h, p, g, n, dev = _seq_inputs(x, B, C, dt, A, D)
    _int("chunk", chunk, 1)
    nc = (t + chunk - 1) // chunk
    f32 = (torch.float32,)
    _opt("h0", h0, (b, h, p, n), f32, dev)
    _opt("y", y, x.shape, (x.dtype,), dev)
    if isinstance(h_final, torch.Tensor):
        _arg("h_final", h_final, (b, h, p, n), f32, dev)
    if isinstance(chunk_states, torch.Tensor):
        _arg("chunk_states", chunk_states, (b, h, nc, p, n), f32, dev)
    _check_ws(workspace, dev)
    _on_gpu(dev)
    dims = make_dims(b, t, h, p, n, g, chunk)
    code = _dtype_code(x)
    if y is None:
        y = torch.empty_like(x)
    hf = (torch.empty((b, h, p, n), dtype=torch.float32, device=dev) if h_final is True
          else (h_final if isinstance(h_final, torch.Tensor) else None))
    cs = (torch.empty((b, h, nc, p, n), dtype=torch.float32, device=dev) if chunk_states is True
          else (chunk_states if isinstance(chunk_states, torch.Tensor) else None))
    ws, wsb = _workspace(ssm_workspace_bytes(dims, code, SSM_WS_FWD), dev, workspace)
    st = _lib.ssm_fwd_chunked(ctypes.byref(dims), code, _ptr(x), _ptr(B), _ptr(C), _ptr(dt),
                              _ptr(A), _ptr(D), _ptr(h0), _ptr(y), _ptr(hf), _ptr(cs), _ptr(ws),
                              wsb, _stream(stream))
    _check(st, "ssm_fwd_chunked")
    return y, hf, cs


def _bwd_prepare(x, B, C, dt, A, D, chunk_states, dy, dh_final, chunk, dh0, out, workspace,
                 need_workspace=True):
    b, t, h, p, g, n, dev = _seq_inputs(x, B, C, dt, A, D)
    _int("chunk", chunk, 1)
    nc = (t + chunk - 1) // chunk
    f32 = (torch.float32,)
    _arg("chunk_states", chunk_states, (b, h, nc, p, n), f32, dev)
    _arg("dy", dy, x.shape, (x.dtype,), dev)
    _opt("dh_final", dh_final, (b, h, p, n), f32, dev)
    if out is not None:
        _arg("dx", out["dx"], x.shape, (x.dtype,), dev)
        for k in ("dB", "dC"):
            _arg(k, out[k], (b, t, g, n), f32, dev)
        _arg("ddt", out["ddt"], (b, t, h), f32, dev)
        for k in ("dA", "dD"):
            _arg(k, out[k], (h,), f32, dev)
        _opt("dh0", out.get("dh0"), (b, h, p, n), f32, dev)
    _check_ws(workspace, dev)
    _on_gpu(dev)
    dims = make_dims(b, t, h, p, n, g, chunk)
    code = _dtype_code(x)
    if out is None:
        fo = dict(dtype=torch.float32, device=dev)
        out = {
            "dx": torch.empty_like(x),
            "dB": torch.empty((b, t, g, n), **fo),
            "dC": torch.empty((b, t, g, n), **fo),
            "ddt": torch.empty((b, t, h), **fo),
            "dA": torch.empty((h,), **fo),
            "dD": torch.empty((h,), **fo),
            "dh0": torch.empty((b, h, p, n), **fo) if dh0 else None,
        }
    ws, wsb = (_workspace(ssm_workspace_bytes(dims, code, SSM_WS_BWD), dev, workspace)
               if need_workspace else (None, 0))
    args = [ctypes.byref(dims), code, _ptr(x), _ptr(B), _ptr(C), _ptr(dt), _ptr(A), _ptr(D),
            _ptr(chunk_states), _ptr(dy), _ptr(dh_final), _ptr(out["dx"]), _ptr(out["dB"]),
            _ptr(out["dC"]), _ptr(out["ddt"]), _ptr(out["dA"]), _ptr(out["dD"]),
            _ptr(out.get("dh0")), _ptr(ws), wsb]
    return out, args


def ssm_bwd(x, B, C, dt, A, D, chunk_states, dy, dh_final=None, chunk=256, dh0=True, out=None,
            workspace=None, stream=None):
    """Backward.  Returns dict dx, dB, dC, ddt, dA, dD, dh0 (dh0 None if not asked)."""
    out, args = _bwd_prepare(x, B, C, dt, A, D, chunk_states, dy, dh_final, chunk, dh0, out,
                             workspace)
    _check(_lib.ssm_bwd(*args, _stream(stream)), "ssm_bwd")
    return out


def ssm_bwd_timed(x, B, C, dt, A, D, chunk_states, dy, block_events, dh_final=None, chunk=256,
                  dh0=True, out=None, workspace=None, stream=None):
    """ssm_bwd that records the two torch.cuda.Event objects ``block_events`` around
    its per-block kernel (on the call's stream).  Returns the gradient dict."""
    if len(block_events) != 2:
        raise ValueError("block_events: two torch.cuda.Event objects")
    out, args = _bwd_prepare(x, B, C, dt, A, D, chunk_states, dy, dh_final, chunk, dh0, out,
                             workspace)
    handles = []
    for ev in block_events:
        ev.record()  # creates the underlying hipEvent_t; the call records it again
        handles.append(ev.cuda_event)
    evs = (ctypes.c_void_p * 2)(*handles)
    _check(_lib.ssm_bwd_timed(*args, evs, _stream(stream)), "ssm_bwd_timed")
    return out


def ssm_bwd_noalloc(x, B, C, dt, A, D, chunk_states, dy, out, dh_final=None, chunk=256,
                    stream=None):
    """ssm_bwd over the library's own scratch: the caller passes every output in ``out``
    (dx, dB, dC, ddt, dA, dD and optionally dh0) and nothing is allocated.  Returns ``out``."""
    if out is None:
        raise ValueError("out: the no-allocation backward writes into caller-provided outputs")
    _, args = _bwd_prepare(x, B, C, dt, A, D, chunk_states, dy, dh_final, chunk, False, out,
                           None, need_workspace=False)
    _check(_lib.ssm_bwd_noalloc(*args[:-2], _stream(stream)), "ssm_bwd_noalloc")
    return out


def ssm_decode_step(state, x, B, C, dt, A, D, y=None, stream=None):
    """In-place one-token update of state [b,h,p,n]; returns y [b,h,p]."""
    if not isinstance(state, torch.Tensor) or state.dim() != 4:
        raise ValueError("state: expected a 4-d tensor [batch, nheads, headdim, dstate]")
    _arg("state", state, state.shape, (torch.float32,))
    return _decode(state, x, B, C, dt, A, D, y, stream, None, None)


def _decode(state, x, B, C, dt, A, D, y, stream, seed, step):
    b, h, p, n = state.shape
    dev = state.device
    if not isinstance(B, torch.Tensor) or B.dim() != 3:
        raise ValueError("B: expected a 3-d tensor [batch, ngroups, dstate]")
    g = B.shape[1]
    _arg("x", x, (b, h, p), _STORAGE, dev)
    _arg("B", B, (b, g, n), (x.dtype,), dev)
    _arg("C", C, (b, g, n), (x.dtype,), dev)
    _arg("dt", dt, (b, h), (torch.float32,), dev)
    _arg("A", A, (h,), (torch.float32,), dev)
    _arg("D", D, (h,), (torch.float32,), dev)
    _opt("y", y, (b, h, p), (x.dtype,), dev)
    _on_gpu(dev)
    dims = make_dims(b, 1, h, p, n, g, 1)
    code = _dtype_code(x)
    if y is None:
        y = torch.empty_like(x)
    if seed is None:
        st = _lib.ssm_decode_step(ctypes.byref(dims), code, _ptr(state), _ptr(x), _ptr(B),
                                  _ptr(C), _ptr(dt), _ptr(A), _ptr(D), _ptr(y), _stream(stream))
        _check(st, "ssm_decode_step")
    else:
        st = _lib.ssm_decode_step_sr16(ctypes.byref(dims), code, _ptr(state), _ptr(x), _ptr(B),
                                       _ptr(C), _ptr(dt), _ptr(A), _ptr(D), _ptr(y),
                                       seed & (2**64 - 1), int(step) & (2**64 - 1),
                                       _stream(stream))
        _check(st, "ssm_decode_step_sr16")
    return y


def ssm_decode_step_sr16(state16, x, B, C, dt, A, D, seed, step, y=None, stream=None):
    """In-place one-token update of a binary16 state cache [b,h,p,n] (int16 tensor
    holding the bits), stochastically rounded under (seed, step); returns y [b,h,p]."""
    if not isinstance(state16, torch.Tensor) or state16.dim() != 4:
        raise ValueError("state16: expected a 4-d tensor [batch, nheads, headdim, dstate]")
    _arg("state16", state16, state16.shape, (torch.int16, torch.float16))
    return _decode(state16, x, B, C, dt, A, D, y, stream, int(seed), step)


def ssm_checkpoint_sr16(state, seed, ckpt_index, elem_offset=0, out=None, stream=None):
    """SR16 bits of a float32 state (returned as an int16 tensor holding the bits)."""
    if not isinstance(state, torch.Tensor):
        raise TypeError("state: expected a torch.Tensor")
    _arg("state", state, state.shape, (torch.float32,))
    _opt("out", out, state.shape, (torch.int16, torch.float16), state.device)
    if state.numel() > 0:
        _on_gpu(state.device)
    if out is None:
        out = torch.empty(state.shape, dtype=torch.int16, device=state.device)
    st = _lib.ssm_checkpoint_sr16(_ptr(state), _ptr(out), state.numel(), seed & (2**64 - 1),
                                  int(ckpt_index), int(elem_offset), _stream(stream))
    _check(st, "ssm_checkpoint_sr16")
    return out


def ssm_replay(ckpt, x, B, C, dt, A, D, t0, r, state_out=None, y=None, live=None,
               workspace=None, stream=None):
    """Replay tokens t0..t0+r-1 from ckpt (float32 state, or int16 SR16 bits).

    Returns dict with state (float32), and when ``live`` is given drift_max and
    drift_mean [r].  ``y`` (full-length output tensor) is written if given.
    """
    b, t, h, p, g, n, dev = _seq_inputs(x, B, C, dt, A, D)
    _arg("ckpt", ckpt, (b, h, p, n), (torch.float32, torch.int16, torch.float16), dev)
    _opt("state_out", state_out, (b, h, p, n), (torch.float32,), dev)
    _opt("y", y, x.shape, (x.dtype,), dev)
    _opt("live", live, (b, h, p, n), (torch.float32,), dev)
    _int("t0", t0, 0)
    _int("r", r, 0)
    _check_ws(workspace, dev)
    _on_gpu(dev)
    dims = make_dims(b, t, h, p, n, g, 1)
    code = _dtype_code(x)
    ck_code = SSM_F32 if ckpt.dtype == torch.float32 else SSM_F16
    if state_out is None:
        state_out = torch.empty((b, h, p, n), dtype=torch.float32, device=dev)
    dmax = dmean = None
    ws, wsb = None, 0
    if live is not None and r > 0:
        dmax = torch.empty(r, dtype=torch.float32, device=dev)
        dmean = torch.empty(r, dtype=torch.float32, device=dev)
        ws, wsb = _workspace(ssm_workspace_bytes(dims, code, SSM_WS_REPLAY, r), dev, workspace)
    st = _lib.ssm_replay(ctypes.byref(dims), code, _ptr(ckpt), ck_code, _ptr(state_out), _ptr(x),
                         _ptr(B), _ptr(C), _ptr(dt), _ptr(A), _ptr(D), int(t0), int(r), _ptr(y),
                         _ptr(live), _ptr(dmax), _ptr(dmean), _ptr(ws), wsb, _stream(stream))
    _check(st, "ssm_replay")
    return {"state": state_out, "drift_max": dmax, "drift_mean": dmean}


def _dt_prep_dims(dt_raw, dt_bias, logA):
    if not isinstance(dt_raw, torch.Tensor) or dt_raw.dim() != 3:
        raise ValueError("dt_raw: expected a 3-d tensor [batch, seqlen, nheads]")
    _arg("dt_raw", dt_raw, dt_raw.shape, (torch.float32,))
    b, t, h = dt_raw.shape
    dev = dt_raw.device
    _arg("dt_bias", dt_bias, (h,), (torch.float32,), dev)
    _arg("logA", logA, (h,), (torch.float32,), dev)
    return make_dims(b, t, h, 1, 1, 1, 1), dev


def ssm_dt_prep(dt_raw, dt_bias, logA, dt_lo=0.0, dt_hi=float("inf"), dt=None, A=None,
                stream=None):
    """dt = clamp(softplus(dt_raw + dt_bias[h]), dt_lo, dt_hi) and A = -exp(logA).
    Returns (dt [batch, seqlen, nheads], A [nheads]), float32."""
    dims, dev = _dt_prep_dims(dt_raw, dt_bias, logA)
    _opt("dt", dt, dt_raw.shape, (torch.float32,), dev)
    _opt("A", A, logA.shape, (torch.float32,), dev)
    _on_gpu(dev)
    if dt is None:
        dt = torch.empty_like(dt_raw)
    if A is None:
        A = torch.empty_like(logA)
    st = _lib.ssm_dt_prep(ctypes.byref(dims), _ptr(dt_raw), _ptr(dt_bias), _ptr(logA),
                          float(dt_lo), float(dt_hi), _ptr(dt), _ptr(A), _stream(stream))
    _check(st, "ssm_dt_prep")
    return dt, A


def ssm_dt_prep_bwd(dt_raw, dt_bias, logA, ddt, dA, dt_lo=0.0, dt_hi=float("inf"), out=None,
                    workspace=None, stream=None):
    """Gradients through ssm_dt_prep: dict d_raw, d_bias, d_logA (float32)."""
    dims, dev = _dt_prep_dims(dt_raw, dt_bias, logA)
    f32 = (torch.float32,)
    _arg("ddt", ddt, dt_raw.shape, f32, dev)
    _arg("dA", dA, logA.shape, f32, dev)
    if out is not None:
        _arg("d_raw", out["d_raw"], dt_raw.shape, f32, dev)
        _arg("d_bias", out["d_bias"], logA.shape, f32, dev)
        _arg("d_logA", out["d_logA"], logA.shape, f32, dev)
    _check_ws(workspace, dev)
    _on_gpu(dev)
    if out is None:
        out = {"d_raw": torch.empty_like(dt_raw), "d_bias": torch.empty_like(dt_bias),
               "d_logA": torch.empty_like(logA)}
    ws, wsb = _workspace(ssm_workspace_bytes(dims, SSM_F32, SSM_WS_DT_PREP_BWD), dev, workspace)
    st = _lib.ssm_dt_prep_bwd(ctypes.byref(dims), _ptr(dt_raw), _ptr(dt_bias), _ptr(logA),
                              float(dt_lo), float(dt_hi), _ptr(ddt), _ptr(dA), _ptr(out["d_raw"]),
                              _ptr(out["d_bias"]), _ptr(out["d_logA"]), _ptr(ws), wsb,
                              _stream(stream))
    _check(st, "ssm_dt_prep_bwd")
    return out


def ssm_draft_snapshots(state0, x, B, C, dt, A, D, y=True, snapshots=None, stream=None):
    """Draft Dr tokens (x [batch, Dr, H, P], ...) from state0 [batch, H, P, N] with a
    snapshot after every step.  Returns (snapshots [Dr+1, batch, H, P, N] float32 with
    slot 0 = state0, y [batch, Dr, H, P] or None)."""
    b, dr, h, p, g, n, dev = _seq_inputs(x, B, C, dt, A, D)
    f32 = (torch.float32,)
    _opt("snapshots", snapshots, (dr + 1, b, h, p, n), f32, dev)
    if snapshots is None:
        _arg("state0", state0, (b, h, p, n), f32, dev)
    if isinstance(y, torch.Tensor):
        _arg("y", y, x.shape, (x.dtype,), dev)
    _on_gpu(dev)
    dims = make_dims(b, dr, h, p, n, g, 1)
    if snapshots is None:
        snapshots = torch.empty((dr + 1, b, h, p, n), dtype=torch.float32, device=dev)
        snapshots[0].copy_(state0)
    yt = torch.empty_like(x) if y is True else (y if isinstance(y, torch.Tensor) else None)
    st = _lib.ssm_draft_snapshots(ctypes.byref(dims), _dtype_code(x), _ptr(snapshots), _ptr(x),
                                  _ptr(B), _ptr(C), _ptr(dt), _ptr(A), _ptr(D), _ptr(yt),
                                  _stream(stream))
    _check(st, "ssm_draft_snapshots")
    return snapshots, yt


def ssm_rollback(snapshots, accepted, state_out=None, err=None, stream=None):
    """state_out[b] = snapshots[accepted[b], b]; accepted is a device int32 [batch]."""
    if not isinstance(snapshots, torch.Tensor) or snapshots.dim() != 5:
        raise ValueError("snapshots: expected a 5-d tensor [Dr+1, batch, H, P, N]")
    _arg("snapshots", snapshots, snapshots.shape, (torch.float32,))
    s1, b, h, p, n = snapshots.shape
    dev = snapshots.device
    _arg("accepted", accepted, (b,), (torch.int32,), dev)
    if state_out is not None:
        # one of the snapshot slots (a view of the stack) or a separate [b,h,p,n] buffer
        _arg("state_out", state_out, (b, h, p, n), (torch.float32,), dev)
    if err is not None:
        _arg("err", err, err.shape, (torch.int32,), dev)
        if err.numel() < 1:
            raise ValueError("err: needs one int32 element")
    _on_gpu(dev)
    dims = make_dims(b, s1 - 1, h, p, n, 1, 1)
    if state_out is None:
        state_out = torch.empty((b, h, p, n), dtype=torch.float32, device=dev)
    st = _lib.ssm_rollback(ctypes.byref(dims), _ptr(snapshots), _ptr(accepted), _ptr(state_out),
                           _ptr(err), _stream(stream))
    _check(st, "ssm_rollback")
    return state_out


def _conv_args(u, w, bias, conv_init):
    if not isinstance(u, torch.Tensor) or u.dim() != 3:
        raise ValueError("u: expected a 3-d tensor [batch, seqlen, channels]")
    _arg("u", u, u.shape, _STORAGE)
    b, t, c = u.shape
    dev = u.device
    if not isinstance(w, torch.Tensor) or w.dim() != 2:
        raise ValueError("w: expected a 2-d tensor [channels, width]")
    k = w.shape[1]
    _arg("w", w, (c, k), (torch.float32,), dev)
    _arg("bias", bias, (c,), (torch.float32,), dev)
    _opt("conv_init", conv_init, (b, k - 1, c), (u.dtype,), dev)
    return b, t, c, k, dev


def ssm_conv1d_silu(u, w, bias, conv_init=None, out=None, conv_final=True, stream=None):
    """SiLU of the short causal depthwise convolution.  u [batch, T, C] (fp32 or
    bf16), w [C, K], bias [C] float32, conv_init [batch, K-1, C] or None.
    Returns (out [batch, T, C], conv_final [batch, K-1, C] or None)."""
    b, t, c, k, dev = _conv_args(u, w, bias, conv_init)
    _opt("out", out, u.shape, (u.dtype,), dev)
    if isinstance(conv_final, torch.Tensor):
        _arg("conv_final", conv_final, (b, k - 1, c), (u.dtype,), dev)
    _on_gpu(dev)
    if out is None:
        out = torch.empty_like(u)
    fin = (torch.empty((b, k - 1, c), dtype=u.dtype, device=dev) if conv_final is True
           else (conv_final if isinstance(conv_final, torch.Tensor) else None))
    st = _lib.ssm_conv1d_silu(b, t, c, k, _dtype_code(u), _ptr(u), _ptr(w), _ptr(bias),
                              _ptr(conv_init), _ptr(out), _ptr(fin), _stream(stream))
    _check(st, "ssm_conv1d_silu")
    return out, fin


def ssm_conv1d_silu_bwd(u, w, bias, dout, conv_init=None, want_dinit=True, workspace=None,
                        stream=None):
    """Gradients of sum(dout * out): dict du, dw, dbias, dconv_init."""
    b, t, c, k, dev = _conv_args(u, w, bias, conv_init)
    _arg("dout", dout, u.shape, (u.dtype,), dev)
    _check_ws(workspace, dev)
    _on_gpu(dev)
    g = {"du": torch.empty_like(u), "dw": torch.empty_like(w), "dbias": torch.empty_like(bias),
         "dconv_init": (torch.empty((b, k - 1, c), dtype=u.dtype, device=dev)
                        if want_dinit else None)}
    need = _lib.ssm_conv1d_silu_workspace_bytes(b, t, c, k)
    if need == _SIZE_MAX:
        raise SsmError(2, "ssm_conv1d_silu_workspace_bytes")
    ws, wsb = _workspace(int(need), dev, workspace)
    st = _lib.ssm_conv1d_silu_bwd(b, t, c, k, _dtype_code(u), _ptr(u), _ptr(w), _ptr(bias),
                                  _ptr(conv_init), _ptr(dout), _ptr(g["du"]), _ptr(g["dw"]),
                                  _ptr(g["dbias"]), _ptr(g["dconv_init"]), _ptr(ws), wsb,
                                  _stream(stream))
    _check(st, "ssm_conv1d_silu_bwd")
    return g


def _norm_args(y, z, w):
    if not isinstance(y, torch.Tensor) or y.dim() < 1:
        raise ValueError("y: expected a tensor [..., channels]")
    _arg("y", y, y.shape, _STORAGE)
    dev = y.device
    c = y.shape[-1]
    _arg("z", z, y.shape, (y.dtype,), dev)
    _arg("w", w, (c,), (torch.float32,), dev)
    rows = y.numel() // c if c else 0
    return rows, c, dev


def ssm_gated_rmsnorm(y, z, w, ngroups, eps=1e-5, out=None, stream=None):
    """out = y*SiLU(z) / rms over groups of C/ngroups channels * w.  y, z [..., C]."""
    rows, c, dev = _norm_args(y, z, w)
    _opt("out", out, y.shape, (y.dtype,), dev)
    _on_gpu(dev)
    if out is None:
        out = torch.empty_like(y)
    st = _lib.ssm_gated_rmsnorm(rows, c, ngroups, _dtype_code(y), _ptr(y), _ptr(z), _ptr(w),
                                float(eps), _ptr(out), _stream(stream))
    _check(st, "ssm_gated_rmsnorm")
    return out


def ssm_gated_rmsnorm_bwd(y, z, w, dout, ngroups, eps=1e-5, workspace=None, stream=None):
    """Gradients of sum(dout * out): dict dy, dz, dw."""
    rows, c, dev = _norm_args(y, z, w)
    _arg("dout", dout, y.shape, (y.dtype,), dev)
    _check_ws(workspace, dev)
    _on_gpu(dev)
    g = {"dy": torch.empty_like(y), "dz": torch.empty_like(z), "dw": torch.empty_like(w)}
    need = _lib.ssm_gated_rmsnorm_workspace_bytes(rows, c, ngroups)
    if need == _SIZE_MAX:
        raise SsmError(2, "ssm_gated_rmsnorm_workspace_bytes")
    ws, wsb = _workspace(int(need), dev, workspace)
    st = _lib.ssm_gated_rmsnorm_bwd(rows, c, ngroups, _dtype_code(y), _ptr(y), _ptr(z), _ptr(w),
                                    float(eps), _ptr(dout), _ptr(g["dy"]), _ptr(g["dz"]),
                                    _ptr(g["dw"]), _ptr(ws), wsb, _stream(stream))
    _check(st, "ssm_gated_rmsnorm_bwd")
    return g
