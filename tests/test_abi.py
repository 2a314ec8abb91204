"""CPU tests of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments synchronously, before any HIP call
(so these run without a GPU)."""
import ctypes
import os
import re

import pytest

from selective_state_space_56_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

INVALID, UNSUPPORTED = 1, 2
FAKE = 0x7F0000000000  # never dereferenced: every case below fails validation first


def declared_functions():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(mamba_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.LIB_PATH):
        from selective_state_space_56_amd.build import build
        build()
    return bd.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == {"mamba_scan_workspace_size", "mamba_scan_fwd", "mamba_scan_fwd_init",
                          "mamba_state_update", "mamba_status_string", "mamba_last_error",
                          "mamba_conv1d_fwd", "mamba_conv1d_update", "mamba_scan_bwd",
                          "mamba_scan_bwd_workspace_size", "mamba_ssd_fwd",
                          "mamba_ssd_workspace_size", "mamba_scan_fwd_strided",
                          "mamba_scan_workspace_size_strided", "mamba_state_update_strided",
                          "mamba_scan_fwd_noalloc"}
    for n in names:
        assert hasattr(lib, n), f"{n} declared in the header but not exported"


def test_status_strings(lib):
    assert lib.mamba_status_string(0) == b"MAMBA_OK"
    assert lib.mamba_status_string(1) == b"MAMBA_ERR_INVALID_ARG"
    assert lib.mamba_status_string(2) == b"MAMBA_ERR_UNSUPPORTED"
    assert lib.mamba_status_string(3) == b"MAMBA_ERR_HIP"
    assert lib.mamba_status_string(99) == b"MAMBA_ERR_UNKNOWN"


def P(k):
    """Distinct fake device addresses, 4 KiB apart (aligned, non-overlapping
    for the tiny sizes used here)."""
    return ctypes.c_void_p(FAKE + 0x100000 * k)


def scan(lib, desc, x=1, delta=2, A=3, B=4, C=5, D=6, z=7, bias=8, out=9, last=10, ws=None,
         ws_bytes=0):
    args = [x, delta, A, B, C, D, z, bias, out, last]
    ptrs = [None if a is None else (P(a) if isinstance(a, int) else a) for a in args]
    w = None if ws is None else (P(ws) if isinstance(ws, int) else ws)
    return lib.mamba_scan_fwd(None if desc is None else ctypes.byref(desc), *ptrs, w,
                              ctypes.c_size_t(ws_bytes), None)


def scan_init(lib, desc, h0, out=9, last=10, ws=None, ws_bytes=0):
    args = [1, 2, 3, 4, 5, 6, 7, 8, h0, out, last]
    ptrs = [None if a is None else (P(a) if isinstance(a, int) else a) for a in args]
    w = None if ws is None else (P(ws) if isinstance(ws, int) else ws)
    return lib.mamba_scan_fwd_init(ctypes.byref(desc), *ptrs, w, ctypes.c_size_t(ws_bytes), None)


def test_scan_init_validates_h0(lib):
    d = D_()
    assert scan_init(lib, d, h0=9) == INVALID               # h0 == out
    assert "h0 overlaps" in err(lib)
    assert scan_init(lib, d, h0=10) == INVALID              # h0 == last_state
    assert "h0 overlaps" in err(lib)
    odd = ctypes.c_void_p(FAKE + 0x100000 * 12 + 2)
    assert scan_init(lib, d, h0=odd) == INVALID
    assert "aligned" in err(lib)
    dw = D_(batch=1, seqlen=64, dim=16, flags=4)
    need = lib.mamba_scan_workspace_size(ctypes.byref(dw))
    assert scan_init(lib, dw, h0=20, ws=20, ws_bytes=need) == INVALID   # h0 == workspace
    assert "h0 overlaps" in err(lib)
    # the common checks run as for mamba_scan_fwd, under this entry point's name
    assert lib.mamba_scan_fwd_init(None, *([None] * 12), ctypes.c_size_t(0), None) == INVALID
    assert "mamba_scan_fwd_init: desc is NULL" in err(lib)


def upd(lib, desc, state=11, x=1, delta=2, A=3, B=4, C=5, D=6, z=7, bias=8, out=9):
    args = [state, x, delta, A, B, C, D, z, bias, out]
    ptrs = [None if a is None else (P(a) if isinstance(a, int) else a) for a in args]
    return lib.mamba_state_update(None if desc is None else ctypes.byref(desc), *ptrs, None)


def D_(batch=2, seqlen=8, dim=16, dstate=16, io=1, flags=0):
    return bd.Desc(batch, seqlen, dim, dstate, io, flags)


def err(lib):
    return lib.mamba_last_error().decode()


def test_scan_rejects_bad_descriptors(lib):
    assert scan(lib, None) == INVALID
    assert "desc is NULL" in err(lib)
    assert scan(lib, D_(batch=-1)) == INVALID
    assert scan(lib, D_(seqlen=-3)) == INVALID
    assert scan(lib, D_(dim=-2)) == INVALID
    assert scan(lib, D_(io=7)) == INVALID
    assert scan(lib, D_(dstate=0)) == INVALID
    for n in (3, 5, 32, 64):
        assert scan(lib, D_(dstate=n)) == UNSUPPORTED
        assert "dstate" in err(lib)
    assert scan(lib, D_(flags=1 << 18)) == INVALID
    assert scan(lib, D_(batch=1 << 20, dim=1 << 20)) == UNSUPPORTED


@pytest.mark.parametrize("missing", ["x", "delta", "A", "B", "C", "out"])
def test_scan_rejects_null_required(lib, missing):
    assert scan(lib, D_(), **{missing: None}) == INVALID
    assert missing in err(lib)


def test_scan_rejects_overlap_and_alignment(lib):
    assert scan(lib, D_(), out=1) == INVALID               # out == x
    assert "out overlaps x" in err(lib)
    assert scan(lib, D_(), last=4) == INVALID              # last_state == B
    assert scan(lib, D_(), last=9) == INVALID              # last_state == out
    odd = ctypes.c_void_p(FAKE + 0x100000 + 1)
    assert scan(lib, D_(), x=odd) == INVALID
    assert "aligned" in err(lib)
    odd4 = ctypes.c_void_p(FAKE + 0x100000 * 3 + 2)
    assert scan(lib, D_(), A=odd4) == INVALID


def test_scan_workspace_contract(lib):
    # forcing 4 time segments needs a workspace; passing none or too little fails
    d = D_(batch=1, seqlen=64, dim=16, flags=4)
    need = lib.mamba_scan_workspace_size(ctypes.byref(d))
    assert need >= 3 * 16 * 17 * 4 and need % 256 == 0
    assert scan(lib, d) == INVALID
    assert "workspace" in err(lib)
    assert scan(lib, d, ws=20, ws_bytes=need - 1) == INVALID
    mis = ctypes.c_void_p(FAKE + 0x100000 * 20 + 64)
    assert scan(lib, d, ws=mis, ws_bytes=need) == INVALID
    assert scan(lib, d, ws=1, ws_bytes=need) == INVALID   # workspace overlaps x
    # small problems need none; invalid descriptors report 0
    assert lib.mamba_scan_workspace_size(ctypes.byref(D_(batch=128, seqlen=256, dim=4096))) == 0
    assert lib.mamba_scan_workspace_size(ctypes.byref(D_(dstate=3))) == 0
    assert lib.mamba_scan_workspace_size(None) == 0


def test_workspace_size_is_deterministic(lib):
    for shape in [(1, 131072, 5120), (2, 2048, 1536), (8, 2048, 5120), (1, 256, 64)]:
        d = D_(batch=shape[0], seqlen=shape[1], dim=shape[2])
        a = lib.mamba_scan_workspace_size(ctypes.byref(d))
        b = lib.mamba_scan_workspace_size(ctypes.byref(d))
        assert a == b and a % 256 == 0


def test_scan_empty_problems_are_noops(lib):
    # no rows: nothing to do, no pointer needed, no HIP call
    assert scan(lib, D_(batch=0), x=None, delta=None, A=None, B=None, C=None, out=None) == 0
    assert scan(lib, D_(dim=0), x=None, delta=None, A=None, B=None, C=None, out=None) == 0
    # zero-length sequence without a final state: nothing to write
    assert scan(lib, D_(seqlen=0), x=None, delta=None, A=None, B=None, C=None, out=None,
                last=None) == 0
    assert err(lib) == ""


def test_state_update_validation(lib):
    assert upd(lib, None) == INVALID
    assert upd(lib, D_(seqlen=2)) == INVALID
    assert "seqlen must be 1" in err(lib)
    assert upd(lib, D_(seqlen=1, flags=1)) == INVALID
    assert upd(lib, D_(seqlen=1, dstate=12)) == UNSUPPORTED
    for missing in ["state", "x", "delta", "A", "B", "C", "out"]:
        assert upd(lib, D_(seqlen=1), **{missing: None}) == INVALID, missing
        assert missing in err(lib)
    assert upd(lib, D_(seqlen=1), out=11) == INVALID       # out == state
    assert upd(lib, D_(seqlen=1), state=1) == INVALID      # state == x
    mis = ctypes.c_void_p(FAKE + 0x100000 * 11 + 8)        # 8-byte aligned only
    assert upd(lib, D_(seqlen=1), state=mis) == INVALID
    assert "16-byte" in err(lib)
    assert upd(lib, D_(batch=0, seqlen=1), state=None, x=None, delta=None, A=None, B=None,
               C=None, out=None) == 0


def CD(batch=2, seqlen=8, dim=16, width=4, io=1, flags=0):
    return bd.ConvDesc(batch, seqlen, dim, width, io, flags)


def conv(lib, desc, xin=1, weight=2, bias=3, sin=4, out=5, sout=6):
    args = [xin, weight, bias, sin, out, sout]
    ptrs = [None if a is None else (P(a) if isinstance(a, int) else a) for a in args]
    return lib.mamba_conv1d_fwd(None if desc is None else ctypes.byref(desc), *ptrs, None)


def conv_upd(lib, desc, state=4, xin=1, weight=2, bias=3, out=5):
    args = [state, xin, weight, bias, out]
    ptrs = [None if a is None else (P(a) if isinstance(a, int) else a) for a in args]
    return lib.mamba_conv1d_update(None if desc is None else ctypes.byref(desc), *ptrs, None)


def test_conv_validation(lib):
    assert conv(lib, None) == INVALID
    assert conv(lib, CD(width=0)) == INVALID
    assert conv(lib, CD(width=5)) == UNSUPPORTED
    assert "width" in err(lib)
    assert conv(lib, CD(io=3)) == INVALID
    assert conv(lib, CD(flags=1)) == INVALID
    assert conv(lib, CD(batch=-1)) == INVALID
    for missing in ("xin", "weight", "out"):
        kw = {missing: None}
        assert conv(lib, CD(), **kw) == INVALID, missing
        assert missing in err(lib)
    assert conv(lib, CD(), out=1) == INVALID                 # out == xin
    assert "out overlaps xin" in err(lib)
    assert conv(lib, CD(), sout=4) == INVALID                # state_out == state_in
    assert "state_out overlaps state_in" in err(lib)
    assert conv(lib, CD(), sout=5) == INVALID                # state_out == out
    assert conv(lib, CD(), out=ctypes.c_void_p(FAKE + 0x100000 * 5 + 1)) == INVALID
    assert "aligned" in err(lib)
    assert conv(lib, CD(), weight=ctypes.c_void_p(FAKE + 0x100000 * 2 + 2)) == INVALID
    # nothing to do: no rows
    assert conv(lib, CD(batch=0), xin=None, weight=None, out=None) == 0


def test_conv_update_validation(lib):
    assert conv_upd(lib, CD(seqlen=2)) == INVALID
    assert "seqlen must be 1" in err(lib)
    assert conv_upd(lib, CD(seqlen=1, width=7)) == UNSUPPORTED
    for missing in ("state", "xin", "weight", "out"):
        assert conv_upd(lib, CD(seqlen=1), **{missing: None}) == INVALID, missing
        assert missing in err(lib)
    assert conv_upd(lib, CD(seqlen=1), out=4) == INVALID     # out == state
    assert conv_upd(lib, CD(seqlen=1), state=1) == INVALID   # state == xin
    assert "state overlaps xin" in err(lib)


BWD_ARGS = ["x", "delta", "A", "B", "C", "D", "z", "bias", "h0", "dout", "dlast", "dx", "ddelta",
            "dA", "dB", "dC", "dD", "dz", "dbias", "dh0"]


def bwd(lib, desc, ws=None, ws_bytes=0, **over):
    """mamba_scan_bwd with every pointer a distinct fake address (argument k
    at P(k + 1)) unless overridden (None = NULL)."""
    ptrs = []
    for k, name in enumerate(BWD_ARGS):
        v = over.get(name, k + 1)
        ptrs.append(None if v is None else (P(v) if isinstance(v, int) else v))
    w = None if ws is None else (P(ws) if isinstance(ws, int) else ws)
    return lib.mamba_scan_bwd(None if desc is None else ctypes.byref(desc), *ptrs, w,
                              ctypes.c_size_t(ws_bytes), None)


def test_scan_bwd_validation(lib):
    d = D_(batch=1, seqlen=64, dim=16, flags=2)
    need = lib.mamba_scan_bwd_workspace_size(ctypes.byref(d))
    assert need > 0 and need % 256 == 0
    assert lib.mamba_scan_bwd_workspace_size(None) == 0
    assert lib.mamba_scan_bwd_workspace_size(ctypes.byref(D_(dstate=3))) == 0
    assert lib.mamba_scan_bwd_workspace_size(ctypes.byref(D_(flags=1 << 16))) == 0
    assert bwd(lib, None) == INVALID
    assert "mamba_scan_bwd: desc is NULL" in err(lib)
    assert bwd(lib, D_(dstate=32), ws=40, ws_bytes=need) == UNSUPPORTED
    assert bwd(lib, D_(flags=1 << 20), ws=40, ws_bytes=need) == INVALID
    # one state checkpoint (batch * dim * dstate * 4 bytes) must stay below 2^31
    big = D_(batch=6554, seqlen=8, dim=5120)
    assert lib.mamba_scan_bwd_workspace_size(ctypes.byref(big)) == 0
    assert bwd(lib, big, ws=40, ws_bytes=need) == UNSUPPORTED
    assert "below 2^31" in err(lib)
    assert lib.mamba_scan_bwd_workspace_size(ctypes.byref(D_(batch=6553, seqlen=8, dim=5120))) > 0
    for name in ["x", "delta", "A", "B", "C", "dout", "dx", "ddelta", "dA", "dB", "dC"]:
        assert bwd(lib, d, ws=40, ws_bytes=need, **{name: None}) == INVALID, name
        assert f"{name} is NULL" in err(lib)
    assert bwd(lib, d, ws=None, ws_bytes=need) == INVALID          # workspace missing
    assert "workspace" in err(lib)
    assert bwd(lib, d, ws=40, ws_bytes=need - 256) == INVALID      # too small
    assert "needed" in err(lib)
    assert bwd(lib, d, ws=ctypes.c_void_p(FAKE + 0x100000 * 40 + 64), ws_bytes=need) == INVALID
    assert "256-byte aligned" in err(lib)
    # outputs must not overlap inputs, each other or the workspace
    assert bwd(lib, d, ws=40, ws_bytes=need, dx=1) == INVALID
    assert "dx overlaps x" in err(lib)
    assert bwd(lib, d, ws=40, ws_bytes=need, dB=12) == INVALID
    assert "overlaps" in err(lib)
    assert bwd(lib, d, ws=40, ws_bytes=need, dh0=40) == INVALID
    assert "dh0 overlaps workspace" in err(lib)
    assert bwd(lib, d, ws=40, ws_bytes=need, dA=10) == INVALID      # dA == dout
    odd = ctypes.c_void_p(FAKE + 0x100000 * 30 + 1)
    assert bwd(lib, d, ws=40, ws_bytes=need, ddelta=odd) == INVALID
    assert "aligned" in err(lib)
    odd4 = ctypes.c_void_p(FAKE + 0x100000 * 30 + 2)
    assert bwd(lib, d, ws=40, ws_bytes=need, dC=odd4) == INVALID
    assert "aligned" in err(lib)
    # without a gate dz is ignored, so it may alias anything
    assert bwd(lib, d, ws=None, ws_bytes=0, z=None, dz=1) == INVALID
    assert "workspace" in err(lib)
    # nothing to do for dim == 0; dA is required otherwise, even with no steps
    assert bwd(lib, D_(dim=0), **{k: None for k in BWD_ARGS}) == 0
    assert bwd(lib, D_(seqlen=0), dA=None) == INVALID


ZOH = 1 << 16


def test_zoh_flag_validation(lib):
    """MAMBA_SCAN_ZOH is accepted by the forward entry points, other high bits
    are not; the decode call accepts ZOH but no segment bits; the backward of
    the ZOH mode is reported unsupported."""
    d = D_(batch=1, seqlen=64, dim=16)
    dz_ = D_(batch=1, seqlen=64, dim=16, flags=ZOH)
    assert lib.mamba_scan_workspace_size(ctypes.byref(dz_)) == lib.mamba_scan_workspace_size(ctypes.byref(d))
    assert lib.mamba_scan_workspace_size(ctypes.byref(D_(flags=1 << 18))) == 0
    assert scan(lib, D_(flags=1 << 18)) == INVALID
    assert "unknown flag bits" in err(lib)
    assert upd(lib, D_(seqlen=1, flags=ZOH | 3)) == INVALID
    assert "MAMBA_SCAN_ZOH" in err(lib)
    assert lib.mamba_scan_bwd_workspace_size(ctypes.byref(dz_)) == 0
    need = lib.mamba_scan_bwd_workspace_size(ctypes.byref(d))
    assert bwd(lib, dz_, ws=40, ws_bytes=need) == UNSUPPORTED
    assert "ZOH" in err(lib)


def test_groups_validation(lib):
    """ngroups must divide dim; the full-sequence entry points need whole
    256-channel tiles per group; decode takes any divisor."""
    bad = D_(batch=1, seqlen=8, dim=640)
    bad.ngroups = 3                                   # 640 % 3 != 0
    assert scan(lib, bad) == INVALID
    assert "not a multiple of ngroups" in err(lib)
    part = D_(batch=1, seqlen=8, dim=640)
    part.ngroups = 2                                  # 320 channels per group
    assert scan(lib, part) == UNSUPPORTED
    assert "multiple of 256" in err(lib)
    assert lib.mamba_scan_workspace_size(ctypes.byref(part)) == 0
    assert lib.mamba_scan_bwd_workspace_size(ctypes.byref(part)) == 0
    assert bwd(lib, part, ws=40, ws_bytes=1 << 20) == UNSUPPORTED
    neg = D_(batch=1, seqlen=8, dim=512)
    neg.ngroups = -1
    assert scan(lib, neg) == INVALID
    dec = D_(batch=1, seqlen=1, dim=640)
    dec.ngroups = 3
    assert upd(lib, dec) == INVALID                   # still must divide dim
    ok = D_(batch=1, seqlen=64, dim=512)
    ok.ngroups = 2
    one = D_(batch=1, seqlen=64, dim=512)
    assert lib.mamba_scan_workspace_size(ctypes.byref(ok)) == lib.mamba_scan_workspace_size(ctypes.byref(one))


def ssd(lib, desc, ws=None, ws_bytes=0, **over):
    names = ["x", "dt", "A", "B", "C", "D", "dt_bias", "h0", "out", "last_state"]
    ptrs = []
    for k, name in enumerate(names):
        v = over.get(name, k + 1)
        ptrs.append(None if v is None else (P(v) if isinstance(v, int) else v))
    w = None if ws is None else (P(ws) if isinstance(ws, int) else ws)
    return lib.mamba_ssd_fwd(None if desc is None else ctypes.byref(desc), *ptrs, w,
                             ctypes.c_size_t(ws_bytes), None)


def test_ssd_validation(lib):
    S = lambda **kw: bd.SsdDesc(*[kw.get(k, v) for k, v in
                                  [("batch", 1), ("seqlen", 64), ("nheads", 4), ("headdim", 64),
                                   ("dstate", 128), ("ngroups", 1), ("io", 1), ("flags", 0)]])
    d = S()
    need = lib.mamba_ssd_workspace_size(ctypes.byref(d))
    assert need > 0 and need % 256 == 0
    assert ssd(lib, None) == INVALID
    assert ssd(lib, S(headdim=32), ws=40, ws_bytes=need) == UNSUPPORTED
    assert ssd(lib, S(dstate=64), ws=40, ws_bytes=need) == UNSUPPORTED
    assert ssd(lib, S(io=0), ws=40, ws_bytes=need) == UNSUPPORTED
    assert ssd(lib, S(ngroups=3), ws=40, ws_bytes=need) == INVALID
    assert ssd(lib, S(flags=1), ws=40, ws_bytes=need) == INVALID
    for name in ["x", "dt", "A", "B", "C", "out"]:
        assert ssd(lib, d, ws=40, ws_bytes=need, **{name: None}) == INVALID, name
    assert ssd(lib, d, ws=40, ws_bytes=need - 256) == INVALID
    assert ssd(lib, d, ws=40, ws_bytes=need, out=1) == INVALID          # out == x
    assert "overlaps" in err(lib)
    odd = ctypes.c_void_p(FAKE + 0x100000 * 30 + 8)
    assert ssd(lib, d, ws=40, ws_bytes=need, B=odd) == INVALID          # B needs 16 bytes
    assert "aligned" in err(lib)
    assert lib.mamba_ssd_workspace_size(ctypes.byref(S(headdim=32))) == 0


def ST(**kw):
    return bd.Strides(*(kw.get(k, 0) for k in ("x", "delta", "z", "out", "bc")))


def scan_strided(lib, desc, strides, x=1, delta=2, A=3, B=4, C=5, D=6, z=7, bias=8, h0=None, out=9,
                 last=10, ws=None, ws_bytes=0):
    args = [x, delta, A, B, C, D, z, bias, h0, out, last]
    ptrs = [None if a is None else (P(a) if isinstance(a, int) else a) for a in args]
    w = None if ws is None else (P(ws) if isinstance(ws, int) else ws)
    return lib.mamba_scan_fwd_strided(ctypes.byref(desc), None if strides is None else ctypes.byref(strides),
                                      *ptrs, w, ctypes.c_size_t(ws_bytes), None)


def upd_strided(lib, desc, strides, state=11, x=1, delta=2, A=3, B=4, C=5, D=6, z=7, bias=8, out=9):
    args = [state, x, delta, A, B, C, D, z, bias, out]
    ptrs = [None if a is None else (P(a) if isinstance(a, int) else a) for a in args]
    return lib.mamba_state_update_strided(ctypes.byref(desc), ctypes.byref(strides), *ptrs, None)


def test_strided_validation(lib):
    d = D_()                                                # dim 16, N 16, bf16
    assert scan_strided(lib, d, ST(x=15)) == INVALID        # below the row length
    assert "x stride 15" in err(lib)
    assert scan_strided(lib, d, ST(z=8)) == INVALID
    assert scan_strided(lib, d, ST(bc=8)) == INVALID        # B/C rows hold G * N = 16
    assert "bc stride" in err(lib)
    assert scan_strided(lib, d, ST(out=1 << 27)) == UNSUPPORTED
    assert scan_strided(lib, d, ST(bc=17)) == INVALID       # bf16 B/C rows must stay 4-byte aligned
    assert "B/C rows" in err(lib)
    # out's rows interleaved with x's: the spans overlap
    base = FAKE + 0x100000 * 20
    assert scan_strided(lib, d, ST(x=32, out=32), x=ctypes.c_void_p(base),
                        out=ctypes.c_void_p(base + 32)) == INVALID
    assert "out overlaps x" in err(lib)
    # an input wider than its rows reaches further: last_state right after x's first rows
    assert scan_strided(lib, d, ST(x=4096), x=ctypes.c_void_p(base),
                        last=ctypes.c_void_p(base + 64 * 1024)) == INVALID
    assert "last_state overlaps x" in err(lib)
    # the common checks run under this entry point's name
    assert scan_strided(lib, D_(dstate=5), None) == UNSUPPORTED
    assert "mamba_scan_fwd_strided" in err(lib)


def test_strided_workspace_size(lib):
    long = D_(batch=64, seqlen=1 << 18, dim=4096)   # enough channel tiles for one or two segments
    plain = lib.mamba_scan_workspace_size(ctypes.byref(long))
    assert lib.mamba_scan_workspace_size_strided(ctypes.byref(long), None) == plain
    assert lib.mamba_scan_workspace_size_strided(ctypes.byref(long), ctypes.byref(ST())) == plain
    # wider rows keep every in-segment offset within 31 bits with more segments
    assert lib.mamba_scan_workspace_size_strided(ctypes.byref(long), ctypes.byref(ST(x=65536))) > plain
    assert lib.mamba_scan_workspace_size_strided(ctypes.byref(long), ctypes.byref(ST(x=5))) == 0


SPLIT = 1 << 17


def test_split_flag_validation(lib):
    """MAMBA_SCAN_SPLIT_STATES forces the state-split kernel: it needs no
    workspace, takes dstate 16 and the first-order weight only, and excludes a
    forced number of segments; the decode and backward calls reject it."""
    assert lib.mamba_scan_workspace_size(ctypes.byref(D_(batch=1, seqlen=64, dim=16, flags=SPLIT))) == 0
    assert lib.mamba_scan_workspace_size(ctypes.byref(D_(dstate=8, flags=SPLIT))) == 0
    assert scan(lib, D_(dstate=8, flags=SPLIT)) == UNSUPPORTED
    assert "MAMBA_SCAN_SPLIT_STATES" in err(lib)
    assert scan(lib, D_(flags=SPLIT | ZOH)) == UNSUPPORTED
    assert scan(lib, D_(flags=SPLIT | 3)) == INVALID
    assert "exclude" in err(lib)
    assert upd(lib, D_(seqlen=1, flags=SPLIT)) == INVALID
    assert bwd(lib, D_(batch=1, seqlen=64, dim=16, flags=SPLIT), ws=40, ws_bytes=1 << 20) == INVALID
    # rows so wide that 9 steps of them pass 2^31 bytes: not for the split kernel
    assert scan_strided(lib, D_(flags=SPLIT), ST(x=1 << 27)) == UNSUPPORTED


def test_split_is_opt_in(lib):
    """The segmented kernel is the default (it cuts a long sequence over few
    rows into segments and asks for a workspace); the flag switches to the
    state-split kernel, which asks for none."""
    ws = lambda **k: lib.mamba_scan_workspace_size(ctypes.byref(D_(**k)))
    for shape in (dict(batch=8, seqlen=2048, dim=5120), dict(batch=1, seqlen=2048, dim=5120)):
        assert ws(**shape) > 0
        assert ws(**shape, flags=SPLIT) == 0


def test_state_update_strided_validation(lib):
    d = D_(seqlen=1)
    assert upd_strided(lib, d, ST(delta=3)) == INVALID
    assert "delta stride" in err(lib)
    assert upd_strided(lib, d, ST(bc=15)) == INVALID
    assert upd_strided(lib, D_(seqlen=2), ST()) == INVALID
    assert "mamba_state_update_strided" in err(lib)
    base = FAKE + 0x100000 * 20
    assert upd_strided(lib, d, ST(x=64, out=64), x=ctypes.c_void_p(base),
                       out=ctypes.c_void_p(base + 64)) == INVALID
    assert "out overlaps x" in err(lib)


def scan_noalloc(lib, desc, h0=None, out=9, last=10):
    args = [1, 2, 3, 4, 5, 6, 7, 8, h0, out, last]
    ptrs = [None if a is None else (P(a) if isinstance(a, int) else a) for a in args]
    return lib.mamba_scan_fwd_noalloc(ctypes.byref(desc), *ptrs, None)


def test_scan_noalloc_validation(lib):
    """The allocation-free scan validates like mamba_scan_fwd_init, and a
    segment plan larger than its fixed scratch array is refused (before any
    HIP call) with the sizes in the message."""
    d = D_()
    assert scan_noalloc(lib, d, h0=9) == INVALID               # h0 == out
    assert scan_noalloc(lib, d, out=None) == INVALID           # out missing
    assert scan_noalloc(lib, D_(flags=1 << 20)) == INVALID     # unknown flag bit
    big = D_(batch=4, seqlen=100000, dim=5120, flags=4000)     # 4000 forced segments
    assert lib.mamba_scan_workspace_size(ctypes.byref(big)) > (48 << 20)
    assert scan_noalloc(lib, big) == UNSUPPORTED
    msg = lib.mamba_last_error().decode()
    assert "scratch" in msg and str(48 << 20) in msg, msg
    assert lib.mamba_scan_fwd_noalloc(None, *[P(k) for k in range(1, 12)], None) == INVALID
