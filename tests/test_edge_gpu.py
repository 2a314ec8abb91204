"""GPU parity in the regimes where a step size is large or an input vanishes,
on every kernel that advances the state: the default scan (whose S4D-Real
tiles keep the state divided by Delta * x), the state-split scan, the
one-token update and the backward. The pages build selection on exactly
these regimes ("Mamba and selective state spaces, from first principles",
"Discretisation: zero-order hold": a large step wipes the state; "Selection":
a large step at a document boundary resets it), and a zero input is the case
where the rescaled state leans on its floor for Delta * x. Inputs come from
workloads.make_edge_inputs (bias up to 20, isolated Delta_raw spikes of
10..20, runs of exact zeros across chunk and segment edges, subnormal and
1e-30 inputs). Every output is compared in full with the fp64 oracle.

Also here: the one-segment plan ignores whatever workspace the caller passes
(no stale tile flags), and two properties of the recurrence checked on the
kernel itself ("State space models and Mamba", "One system, two views"): y
is linear in x when Delta, B, C are fixed and there is no gate, and the D
term adds exactly D * x."""
import ctypes
import os

import numpy as np
import pytest
import torch

from gpu_common import TOL, norm_err, plain_rel_err, to_dev
from selective_state_space_56_amd import binding, scan_bwd, scan_fwd, state_update
from selective_state_space_56_amd.workloads import (WORKLOADS, make_bwd_grads, make_edge_inputs,
                                                    make_scan_inputs, make_trained_A,
                                                    to_f64_numpy)

pytestmark = pytest.mark.gpu

NT = max(1, min(16, len(os.sched_getaffinity(0))))


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def _f(t):
    return None if t is None else to_f64_numpy(t)


def _edge_workload(io, L=600, dim=512, batch=2):
    return WORKLOADS["mamba130m_layer"].with_shape(name="edge", batch=batch, seqlen=L, dim=dim,
                                                   io=io)


def _oracle(orc, inp):
    return orc.scan(_f(inp["x"]), _f(inp["delta"]), _f(inp["A"]), _f(inp["B"]), _f(inp["C"]),
                    D=_f(inp["D"]), z=_f(inp["z"]), delta_bias=_f(inp["delta_bias"]), nthreads=NT)


def _compare(label, io, y, h, ry, rh):
    tol = TOL[io]
    ey, eh = norm_err(_f(y), ry), norm_err(_f(h), rh)
    py, ph = plain_rel_err(_f(y), ry), plain_rel_err(_f(h), rh)
    py3 = plain_rel_err(_f(y), ry, floor=1e-3)
    _say(f"{label}: err(y)={ey:.3e} err(state)={eh:.3e} plain rel (|r|>=rms) y={py:.3e} "
         f"state={ph:.3e} (|r|>=1e-3 rms) y={py3:.3e} tol={tol:g}")
    assert np.all(np.isfinite(_f(y))) and np.all(np.isfinite(_f(h)))
    assert ey <= tol, f"y error {ey} > {tol}"
    assert eh <= tol, f"state error {eh} > {tol}"
    if io == "f32":
        assert py <= tol, f"plain y error {py} > {tol}"
        assert ph <= tol, f"plain state error {ph} > {tol}"


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("segments", [0, 1, 5, 12])
def test_edge_scan_default(orc, dev, io, segments):
    w = _edge_workload(io)
    _say(f"case edge scan default {io} seg={segments}")
    inp = to_dev(make_edge_inputs(w, seed=31), dev)
    out, last = scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                         z=inp["z"], delta_bias=inp["delta_bias"], segments=segments)
    torch.cuda.synchronize()
    ry, rh = _oracle(orc, inp)
    _compare(f"edge scan {io} seg={segments}", io, out, last, ry, rh)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_edge_scan_split(orc, dev, io):
    w = _edge_workload(io)
    _say(f"case edge scan split {io}")
    inp = to_dev(make_edge_inputs(w, seed=32), dev)
    out, last = scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                         z=inp["z"], delta_bias=inp["delta_bias"], split_states=True)
    torch.cuda.synchronize()
    ry, rh = _oracle(orc, inp)
    _compare(f"edge split {io}", io, out, last, ry, rh)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_edge_general_A(orc, dev, io):
    """The same regimes on the per-state exponential path (trained-like A)."""
    w = _edge_workload(io)
    _say(f"case edge scan general A {io}")
    inp = make_edge_inputs(w, seed=33)
    inp["A"] = make_trained_A(w, seed=33)
    inp = to_dev(inp, dev)
    out, last = scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                         z=inp["z"], delta_bias=inp["delta_bias"], segments=5)
    torch.cuda.synchronize()
    ry, rh = _oracle(orc, inp)
    _compare(f"edge general A {io}", io, out, last, ry, rh)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_edge_decode(orc, dev, io):
    """The whole edge sequence one token at a time from a zero state: every
    step's y and the final state against the oracle's scan (the decode step is
    the scan's step)."""
    w = _edge_workload(io, dim=320)
    _say(f"case edge decode {io}")
    inp = to_dev(make_edge_inputs(w, seed=34), dev)
    state = torch.zeros((w.batch, w.dim, w.dstate), device=dev)
    ys = []
    for t in range(w.seqlen):
        tok = {k: inp[k][:, t].contiguous() for k in ("x", "delta", "z", "B", "C")}
        ys.append(state_update(state, tok["x"], tok["delta"], inp["A"], tok["B"], tok["C"],
                               D=inp["D"], z=tok["z"], delta_bias=inp["delta_bias"]))
    torch.cuda.synchronize()
    ry, rh = _oracle(orc, inp)
    _compare(f"edge decode {io}", io, torch.stack(ys, dim=1), state, ry, rh)


KEYS = [("dx", "dx"), ("ddelta", "ddelta"), ("dz", "dz"), ("dA", "dA"), ("dB", "dB"),
        ("dC", "dC"), ("dD", "dD"), ("ddelta_bias", "dbias"), ("dh0", "dh0")]


@pytest.mark.parametrize("io,segments", [("f32", 0), ("f32", 1), ("f32", 5), ("bf16", 0),
                                         ("bf16", 5)])
def test_edge_bwd(orc, dev, io, segments):
    """Every gradient in the edge regimes against the oracle's reverse pass."""
    w = _edge_workload(io)
    _say(f"case edge bwd {io} seg={segments}")
    inp = to_dev(make_edge_inputs(w, seed=35), dev)
    gr = to_dev(make_bwd_grads(w, seed=35), dev)
    g = scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], gr["dout"], D=inp["D"],
                 z=inp["z"], delta_bias=inp["delta_bias"], dlast=gr["dlast"], segments=segments)
    torch.cuda.synchronize()
    ref = orc.scan_bwd(_f(inp["x"]), _f(inp["delta"]), _f(inp["A"]), _f(inp["B"]), _f(inp["C"]),
                       _f(gr["dout"]), D=_f(inp["D"]), z=_f(inp["z"]),
                       delta_bias=_f(inp["delta_bias"]), dlast=_f(gr["dlast"]), nthreads=NT)
    errs = {k: norm_err(_f(g[k]), ref[rk]) for k, rk in KEYS}
    _say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()) + f" tol={TOL[io]:g}")
    for k, _ in KEYS:
        assert np.all(np.isfinite(_f(g[k]))), k
    bad = {k: v for k, v in errs.items() if not v <= TOL[io]}
    assert not bad, f"gradients off: {bad}"


@pytest.mark.parametrize("fill", [0xFF, 0x00])
def test_one_segment_ignores_workspace(orc, dev, fill):
    """A plan of one time segment needs no workspace; a buffer passed anyway,
    whatever it holds, must not steer the kernels (a stale nonzero word once
    sent general-A tiles down the S4D-Real path). Called through the C ABI
    with a filled buffer, short sequences (one segment by the library's own
    plan), trained-like A and the S4D-Real A."""
    lib = binding.load_library()
    for general in (True, False):
        w = WORKLOADS["mamba130m_layer"].with_shape(name="ws1", batch=3, seqlen=64, dim=600,
                                                    io="f32")
        inp = make_scan_inputs(w, seed=36)
        if general:
            inp["A"] = make_trained_A(w, seed=36)
        inp = to_dev(inp, dev)
        d = binding.Desc(w.batch, w.seqlen, w.dim, w.dstate, binding.MAMBA_F32, 0, 1)
        assert lib.mamba_scan_workspace_size(ctypes.byref(d)) == 0
        ws = torch.full((1 << 16,), fill, dtype=torch.uint8, device=dev)
        out = torch.empty((w.batch, w.seqlen, w.dim), dtype=torch.float32, device=dev)
        last = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device=dev)
        p = binding._ptr
        st = lib.mamba_scan_fwd(ctypes.byref(d), p(inp["x"]), p(inp["delta"]), p(inp["A"]),
                                p(inp["B"]), p(inp["C"]), p(inp["D"]), p(inp["z"]),
                                p(inp["delta_bias"]), p(out), p(last), p(ws),
                                ctypes.c_size_t(ws.numel()), binding._stream(dev))
        assert st == binding.MAMBA_OK, lib.mamba_last_error()
        torch.cuda.synchronize()
        assert torch.all(ws == fill), "the library wrote into a workspace it does not need"
        ry, rh = _oracle(orc, inp)
        _compare(f"one segment, workspace 0x{fill:02x}, general={general}", "f32", out, last, ry,
                 rh)


def test_linear_in_x(dev):
    """With Delta_raw, B, C fixed and no gate, y is linear in x: y(x1 + 2 x2)
    = y(x1) + 2 y(x2), and so is the final state; checked on the kernel's own
    outputs (fp32 io, S4D-Real and trained-like A, with segments)."""
    w = WORKLOADS["mamba130m_layer"].with_shape(name="lin", batch=2, seqlen=700, dim=384,
                                                io="f32")
    a = to_dev(make_scan_inputs(w, seed=37), dev)
    b = to_dev(make_scan_inputs(w, seed=38), dev)
    for general in (False, True):
        A = to_dev({"A": make_trained_A(w, seed=37)}, dev)["A"] if general else a["A"]
        outs = []
        for xx in (a["x"], b["x"], a["x"] + 2.0 * b["x"]):
            y, h = scan_fwd(xx, a["delta"], A, a["B"], a["C"], D=a["D"],
                            delta_bias=a["delta_bias"], segments=4)
            outs.append((_f(y), _f(h)))
        torch.cuda.synchronize()
        ly = outs[0][0] + 2.0 * outs[1][0]
        lh = outs[0][1] + 2.0 * outs[1][1]
        ey, eh = norm_err(outs[2][0], ly), norm_err(outs[2][1], lh)
        _say(f"linearity general={general}: err(y)={ey:.2e} err(state)={eh:.2e}")
        assert ey <= TOL["f32"] and eh <= TOL["f32"]


def test_d_term_additive(dev):
    """The direct term adds D * x to y before the gate: y(D) / silu(z) -
    y(no D) / silu(z) = D * x, the state is unchanged (bitwise); without the
    gate the difference is D * x directly."""
    w = WORKLOADS["mamba130m_layer"].with_shape(name="dadd", batch=2, seqlen=500, dim=320,
                                                io="f32")
    i = to_dev(make_scan_inputs(w, seed=39), dev)
    yD, hD = scan_fwd(i["x"], i["delta"], i["A"], i["B"], i["C"], D=i["D"],
                      delta_bias=i["delta_bias"])
    y0, h0 = scan_fwd(i["x"], i["delta"], i["A"], i["B"], i["C"], delta_bias=i["delta_bias"])
    torch.cuda.synchronize()
    assert torch.equal(hD, h0)
    dx = _f(i["D"])[None, None, :] * _f(i["x"])
    e = norm_err(_f(yD) - _f(y0), dx)
    _say(f"D additivity (no gate): err={e:.2e}")
    assert e <= 1e-5
    yg, _ = scan_fwd(i["x"], i["delta"], i["A"], i["B"], i["C"], D=i["D"], z=i["z"],
                     delta_bias=i["delta_bias"])
    y0g, _ = scan_fwd(i["x"], i["delta"], i["A"], i["B"], i["C"], z=i["z"],
                      delta_bias=i["delta_bias"])
    torch.cuda.synchronize()
    zz = _f(i["z"])
    gate = zz / (1.0 + np.exp(-zz))
    e = norm_err(_f(yg) - _f(y0g), dx * gate)
    _say(f"D additivity (gated): err={e:.2e}")
    assert e <= 1e-5
