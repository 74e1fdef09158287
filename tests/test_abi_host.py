"""Host-only checks of the C-ABI library (no GPU needed, nothing enqueued).

- the built library loads and exports every function declared in include/ssm.h;
- invalid calls are rejected with the documented status before any work
  ("Reverse-mode automatic differentiation" (OneModel docs), section 2: errors
  are detected before any work) -- every case here fails validation, so no
  kernel is ever launched;
- workspace sizing and the MFMA-path predicate are pure host logic.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm.h")

ssm = pytest.importorskip("backward_mamba_ssd_amd.ssm")

OK, NULL, DIMS, UNSUP, DTYPE, ALIGN, WS, HIP = range(8)
FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced (validation fails first)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("ssm_fwd_chunked", "ssm_decode_step", "ssm_bwd", "ssm_checkpoint_sr16",
              "ssm_replay"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(ssm.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(ssm.EXPORTS) == set(declared_functions())


def test_status_strings():
    for code in range(8):
        assert ssm.status_string(code).startswith("SSM_")


def dims(**kw):
    base = dict(batch=2, seqlen=100, nheads=4, headdim=64, dstate=128, ngroups=2, chunk=64)
    base.update(kw)
    return ssm.make_dims(**base)


def fwd(d, dtype=ssm.SSM_BF16, x=FAKE, B=FAKE, C=FAKE, dt=FAKE, A=FAKE, D=FAKE, h0=None, y=FAKE,
        hf=None, cs=None):
    L = ssm.lib()
    dp = ctypes.byref(d) if d is not None else None
    return L.ssm_fwd_chunked(dp, dtype, x, B, C, dt, A, D, h0, y, hf, cs, None, 0, None)


def bwd(d, ws=None, wsb=0, **over):
    L = ssm.lib()
    a = dict(x=FAKE, B=FAKE, C=FAKE, dt=FAKE, A=FAKE, D=FAKE, cs=FAKE, dy=FAKE, dhf=None, dx=FAKE,
             dB=FAKE, dC=FAKE, ddt=FAKE, dA=FAKE, dD=FAKE, dh0=None)
    a.update(over)
    return L.ssm_bwd(ctypes.byref(d), ssm.SSM_BF16, a["x"], a["B"], a["C"], a["dt"], a["A"],
                     a["D"], a["cs"], a["dy"], a["dhf"], a["dx"], a["dB"], a["dC"], a["ddt"],
                     a["dA"], a["dD"], a["dh0"], ws, wsb, None)


def test_fwd_validation():
    assert fwd(None) == NULL
    assert fwd(dims(nheads=6, ngroups=4)) == DIMS
    assert fwd(dims(chunk=0)) == DIMS
    assert fwd(dims(headdim=0)) == DIMS
    assert fwd(dims(batch=-1)) == DIMS
    assert fwd(dims(), dtype=7) == DTYPE
    assert fwd(dims(dstate=100)) == UNSUP
    assert fwd(dims(), x=None) == NULL
    assert fwd(dims(), y=FAKE + 1) == ALIGN
    assert fwd(dims(), h0=FAKE + 8) == ALIGN
    assert fwd(dims(), A=None) == NULL


def test_bwd_validation():
    d = dims()
    need = ssm.ssm_workspace_bytes(d, ssm.SSM_BF16, ssm.SSM_WS_BWD)
    assert need > 0
    assert bwd(d) == WS
    assert bwd(d, ws=FAKE, wsb=need - 1) == WS
    assert bwd(d, ws=FAKE, wsb=need, cs=None) == NULL
    assert bwd(d, ws=FAKE + 8, wsb=need) == ALIGN
    assert bwd(dims(nheads=3, ngroups=2), ws=FAKE, wsb=need) == DIMS


def test_timed_backward_validation():
    # same validation as ssm_bwd; the event array is required, and both handles too
    L = ssm.lib()
    d = dims()
    need = ssm.ssm_workspace_bytes(d, ssm.SSM_BF16, ssm.SSM_WS_BWD)
    a = [FAKE] * 7 + [FAKE, None] + [FAKE] * 6 + [None]  # x..chunk_states, dy, dh_final, dx..dD, dh0

    def timed(dd, ev, ws=FAKE, wsb=need):
        return L.ssm_bwd_timed(ctypes.byref(dd), ssm.SSM_BF16, *a, ws, wsb, ev, None)

    assert timed(d, None) == NULL
    null_pair = (ctypes.c_void_p * 2)(None, None)
    assert timed(d, null_pair) == NULL
    assert timed(dims(nheads=3, ngroups=2), null_pair) == DIMS  # dims are checked first
    assert timed(d, null_pair, ws=None) == WS


def test_decode_replay_sr16_validation():
    L = ssm.lib()
    d = dims(seqlen=1)
    args = [FAKE] * 8
    assert L.ssm_decode_step(ctypes.byref(d), ssm.SSM_BF16, None, *args[1:], None) == NULL
    assert L.ssm_decode_step(ctypes.byref(dims(dstate=48)), ssm.SSM_BF16, *args, None) == UNSUP
    sr = L.ssm_decode_step_sr16
    assert sr(ctypes.byref(d), ssm.SSM_BF16, None, *args[1:], 0, 0, None) == NULL
    assert sr(ctypes.byref(d), ssm.SSM_BF16, FAKE + 2, *args[1:], 0, 0, None) == ALIGN
    assert sr(ctypes.byref(d), 7, *args, 0, 0, None) == DTYPE
    assert sr(ctypes.byref(dims(dstate=48)), ssm.SSM_BF16, *args, 0, 0, None) == UNSUP
    assert sr(ctypes.byref(dims(batch=0)), ssm.SSM_BF16, None, None, None, None, None, FAKE,
              FAKE, None, 0, 0, None) == OK
    assert L.ssm_checkpoint_sr16(None, FAKE, 10, 0, 0, 0, None) == NULL
    assert L.ssm_checkpoint_sr16(FAKE, FAKE + 1, 10, 0, 0, 0, None) == ALIGN
    assert L.ssm_checkpoint_sr16(FAKE, FAKE + 16, 10, 0, 0, 0, None) == DIMS  # aliasing
    assert L.ssm_checkpoint_sr16(None, None, 0, 0, 0, 0, None) == OK  # empty: no-op
    rd = dims(seqlen=50)
    common = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE]

    def rep(t0, r, live=None, dm=None, dn=None, ws=None, wsb=0, ckd=ssm.SSM_F32):
        return L.ssm_replay(ctypes.byref(rd), ssm.SSM_BF16, FAKE, ckd, FAKE, *common, t0, r, None,
                            live, dm, dn, ws, wsb, None)

    assert rep(40, 11) == DIMS
    assert rep(-1, 5) == DIMS
    assert rep(0, 5, ckd=ssm.SSM_BF16) == DTYPE
    assert rep(0, 5, live=FAKE) == NULL
    assert rep(0, 5, live=FAKE, dm=FAKE, dn=FAKE) == WS
    need = ssm.ssm_workspace_bytes(rd, ssm.SSM_BF16, ssm.SSM_WS_REPLAY, 5)
    assert need >= 2 * 5 * (2 * 4 * 4) * 4  # two [r][batch*heads*4] float arrays


def test_empty_batch_is_a_noop():
    # batch 0: valid, nothing to do, returns OK without touching any pointer
    assert fwd(dims(batch=0), x=None, B=None, C=None, dt=None, y=None) == OK


def test_workspace_and_path_predicates():
    d = dims(batch=4, seqlen=4096, nheads=256, ngroups=8, chunk=256)
    assert ssm.ssm_workspace_bytes(d, ssm.SSM_BF16, ssm.SSM_WS_FWD) == 0
    assert ssm.ssm_workspace_bytes(d, ssm.SSM_BF16, ssm.SSM_WS_BWD) > 0
    with pytest.raises(ssm.SsmError):
        ssm.ssm_workspace_bytes(dims(dstate=48), ssm.SSM_BF16, ssm.SSM_WS_FWD)
    assert not ssm.ssm_uses_mfma_path(dims(headdim=8, dstate=16), ssm.SSM_F32)
    assert not ssm.ssm_uses_mfma_path(d, ssm.SSM_F32)
    assert ssm.ssm_uses_mfma_path(d, ssm.SSM_BF16)
    # the MFMA backward needs chunk <= 256 and at most 64 heads per group
    assert not ssm.ssm_uses_mfma_path(dims(batch=4, seqlen=4096, nheads=256, ngroups=8, chunk=512),
                                      ssm.SSM_BF16)
    assert not ssm.ssm_uses_mfma_path(dims(batch=1, seqlen=256, nheads=128, ngroups=1, chunk=256),
                                      ssm.SSM_BF16)
    assert not ssm.ssm_uses_mfma_path(dims(batch=1, seqlen=256, nheads=8, ngroups=1, chunk=96),
                                      ssm.SSM_BF16)


def prep_dims(batch=2, seqlen=100, nheads=256):
    return ssm.make_dims(batch, seqlen, nheads, 1, 1, 1, 1)


def test_dt_prep_rejects_bad_calls_before_any_work():
    L = ssm.lib()
    d = prep_dims()
    inf, nan = float("inf"), float("nan")

    def prep(dd, raw=FAKE, bias=FAKE, logA=FAKE, lo=0.0, hi=inf, dt=FAKE, A=FAKE):
        return L.ssm_dt_prep(ctypes.byref(dd) if dd is not None else None, raw, bias, logA, lo,
                             hi, dt, A, None)

    assert prep(None) == NULL
    assert prep(d, lo=0.2, hi=0.1) == DIMS          # empty interval
    assert prep(d, lo=nan) == DIMS and prep(d, hi=nan) == DIMS
    assert prep(prep_dims(nheads=0)) == DIMS
    assert prep(prep_dims(batch=-1)) == DIMS
    assert prep(d, raw=None) == NULL and prep(d, A=None) == NULL and prep(d, logA=None) == NULL
    assert prep(d, dt=FAKE + 2) == ALIGN

    def prep_bwd(dd, ws=None, wsb=0, **over):
        a = dict(raw=FAKE, bias=FAKE, logA=FAKE, lo=0.0, hi=inf, ddt=FAKE, dA=FAKE, d_raw=FAKE,
                 d_bias=FAKE, d_logA=FAKE)
        a.update(over)
        return L.ssm_dt_prep_bwd(ctypes.byref(dd), a["raw"], a["bias"], a["logA"], a["lo"],
                                 a["hi"], a["ddt"], a["dA"], a["d_raw"], a["d_bias"],
                                 a["d_logA"], ws, wsb, None)

    need = ssm.ssm_workspace_bytes(d, ssm.SSM_F32, ssm.SSM_WS_DT_PREP_BWD)
    # 200 rows -> 13 row tiles of 16, one fp64 partial per (tile, head), rounded to 256 B
    assert need == 13 * 256 * 8
    assert prep_bwd(d) == WS
    assert prep_bwd(d, ws=FAKE, wsb=need - 1) == WS
    assert prep_bwd(d, ws=FAKE, wsb=need, lo=1.0, hi=0.5) == DIMS
    assert prep_bwd(d, ws=FAKE, wsb=need, dA=None) == NULL
    assert prep_bwd(d, ws=FAKE, wsb=need, ddt=None) == NULL
    assert prep_bwd(d, ws=FAKE + 4, wsb=need) == ALIGN
    assert prep_bwd(d, ws=FAKE, wsb=need, d_bias=FAKE + 1) == ALIGN
    # no rows: the per-row pointers may be NULL (the call still writes d_bias = 0, d_logA)
    assert ssm.ssm_workspace_bytes(prep_dims(seqlen=0), ssm.SSM_F32, ssm.SSM_WS_DT_PREP_BWD) == 0


def test_draft_and_rollback_reject_bad_calls_before_any_work():
    L = ssm.lib()
    d = dims(batch=3, seqlen=4, nheads=4, headdim=64, dstate=128, ngroups=2)

    def draft(dd, snaps=FAKE, x=FAKE, B=FAKE, C=FAKE, dt=FAKE, A=FAKE, D=FAKE, y=None,
              dtype=ssm.SSM_BF16):
        return L.ssm_draft_snapshots(ctypes.byref(dd), dtype, snaps, x, B, C, dt, A, D, y, None)

    assert draft(d, snaps=None) == NULL
    assert draft(d, x=None) == NULL
    assert draft(d, A=None) == NULL
    assert draft(d, snaps=FAKE + 4) == ALIGN
    assert draft(d, dtype=9) == DTYPE
    assert draft(dims(dstate=100)) == UNSUP

    def rb(dd, snaps=FAKE, acc=FAKE, out=FAKE + (1 << 30), err=None):
        return L.ssm_rollback(ctypes.byref(dd), snaps, acc, out, err, None)

    assert rb(d, snaps=None) == NULL and rb(d, acc=None) == NULL and rb(d, out=None) == NULL
    assert rb(d, out=FAKE + (1 << 30) + 8) == ALIGN
    assert rb(d, acc=FAKE + 2) == ALIGN
    assert rb(d, err=FAKE + 1) == ALIGN
    assert rb(dims(batch=70000, seqlen=4)) == DIMS
    slot = 3 * 4 * 64 * 128 * 4
    assert rb(d, out=FAKE + slot // 2) == DIMS          # straddles two slots
    assert rb(d, out=FAKE - slot // 2) == DIMS          # overlaps slot 0 from below
    assert rb(dims(batch=0)) == OK                        # nothing to do


def test_conv_and_norm_reject_bad_calls_before_any_work():
    L = ssm.lib()
    B16, F32 = ssm.SSM_BF16, ssm.SSM_F32

    def conv(b=2, t=10, c=16, k=4, dtype=B16, u=FAKE, w=FAKE, bias=FAKE, init=None,
             out=FAKE + (1 << 30), fin=None):
        return L.ssm_conv1d_silu(b, t, c, k, dtype, u, w, bias, init, out, fin, None)

    assert conv(dtype=7) == DTYPE
    assert conv(k=0) == DIMS and conv(k=9) == DIMS and conv(c=6) == DIMS and conv(b=70000) == DIMS
    assert conv(u=None) == NULL and conv(w=None) == NULL and conv(bias=None) == NULL
    assert conv(out=FAKE + 8) == ALIGN and conv(bias=FAKE + 4) == ALIGN
    assert conv(out=FAKE + 64) == DIMS  # overlaps the input
    need = L.ssm_conv1d_silu_workspace_bytes(2, 600, 16, 4)
    assert need == 2 * 3 * 5 * 16 * 8  # 3 tiles of 256 tokens, K + 1 partial rows
    assert L.ssm_conv1d_silu_workspace_bytes(2, 600, 16, 9) == ctypes.c_size_t(-1).value

    def conv_bwd(ws=None, wsb=0, **kw):
        a = dict(u=FAKE, w=FAKE, bias=FAKE, init=None, dout=FAKE + (2 << 30), du=FAKE + (1 << 30),
                 dw=FAKE, dbias=FAKE, dinit=None)
        a.update(kw)
        return L.ssm_conv1d_silu_bwd(2, 600, 16, 4, B16, a["u"], a["w"], a["bias"], a["init"],
                                     a["dout"], a["du"], a["dw"], a["dbias"], a["dinit"], ws, wsb,
                                     None)

    assert conv_bwd() == WS and conv_bwd(ws=FAKE, wsb=need - 8) == WS
    assert conv_bwd(ws=FAKE, wsb=need, dw=None) == NULL
    assert conv_bwd(ws=FAKE, wsb=need, du=FAKE) == DIMS  # du overlaps u

    def norm(rows=8, c=64, g=4, eps=1e-5, dtype=F32, y=FAKE, z=FAKE, w=FAKE, out=FAKE):
        return L.ssm_gated_rmsnorm(rows, c, g, dtype, y, z, w, eps, out, None)

    assert norm(c=60) == DIMS          # 60 / 4 = 15 channels per group, not a multiple of 8
    assert norm(c=64, g=3) == DIMS     # groups do not divide the channels
    assert norm(c=2 * 8200, g=2) == DIMS  # group wider than 8192
    assert norm(eps=-1.0) == DIMS and norm(eps=float("nan")) == DIMS and norm(eps=float("inf")) == DIMS
    assert norm(y=None) == NULL and norm(w=None) == NULL
    assert norm(out=FAKE + 4) == ALIGN
    nneed = L.ssm_gated_rmsnorm_workspace_bytes(100, 64, 4)
    assert nneed == 4 * 64 * 8  # 4 tiles of 32 rows
    assert L.ssm_gated_rmsnorm_bwd(100, 64, 4, F32, FAKE, FAKE, FAKE, 1e-5, FAKE, FAKE, FAKE,
                                   FAKE, None, 0, None) == WS
