"""A seeded sweep over problem shapes and options, forward and backward,
against the fp64 oracle: batch 1-4, sequence lengths from 1 to 700 steps,
channel counts from 1 to 600 (partial channel tiles, odd counts that take the
register-staged copies), every supported state size, fp32 and bf16 io,
forced and automatic time segments, with and without the gate, D, the bias,
an initial state and the final-state gradient, S4D-Real and trained-like A.
The cases are drawn once from a fixed seed, so every run checks the same
ones; each prints its configuration before it runs."""
import os

import numpy as np
import pytest
import torch

from gpu_common import TOL, gpu_scan, norm_err, oracle_scan, to_dev
from selective_state_space_56_amd import scan_bwd
from selective_state_space_56_amd.workloads import (WORKLOADS, make_bwd_grads, make_scan_inputs,
                                                    make_trained_A, to_f64_numpy)

pytestmark = pytest.mark.gpu

NT = max(1, min(16, len(os.sched_getaffinity(0))))


def _draw(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        cases.append(dict(
            batch=int(rng.integers(1, 5)),
            seqlen=int(rng.choice([1, 9] + [int(rng.integers(2, 700)) for _ in range(4)])),
            dim=int(rng.choice([1, 63, 256] + [int(rng.integers(2, 600)) for _ in range(3)])),
            dstate=int(rng.choice([1, 2, 4, 8, 16])),
            io=str(rng.choice(["f32", "bf16"])),
            segments=int(rng.choice([0, 1, int(rng.integers(2, 24))])),
            gate=bool(rng.integers(0, 2)),
            with_D=bool(rng.integers(0, 2)),
            with_bias=bool(rng.integers(0, 2)),
            h0=bool(rng.integers(0, 2)),
            trained=bool(rng.integers(0, 2)),
            seed=int(rng.integers(0, 1 << 20)),
        ))
    return cases


FWD_CASES = _draw(32, 5150)
BWD_CASES = _draw(20, 7341)


def _label(c):
    return (f"{c['batch']}x{c['seqlen']}x{c['dim']}-N{c['dstate']}-{c['io']}-seg{c['segments']}"
            f"-g{int(c['gate'])}D{int(c['with_D'])}b{int(c['with_bias'])}h{int(c['h0'])}"
            f"t{int(c['trained'])}")


def _setup(c, dev):
    w = WORKLOADS["mamba130m_layer"].with_shape(name="sweep", batch=c["batch"], seqlen=c["seqlen"],
                                                dim=c["dim"], dstate=c["dstate"], io=c["io"],
                                                gate=c["gate"])
    inp = to_dev(make_scan_inputs(w, seed=c["seed"]), dev)
    if c["trained"]:
        inp["A"] = make_trained_A(w, seed=c["seed"] + 1).to(dev)
    h0 = None
    if c["h0"]:
        g = torch.Generator().manual_seed(c["seed"] + 2)
        h0 = torch.randn((c["batch"], c["dim"], c["dstate"]), generator=g).to(dev)
    return w, inp, h0


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


@pytest.mark.parametrize("c", FWD_CASES, ids=_label)
def test_sweep_forward(orc, dev, c):
    print(f"case sweep forward {_label(c)}", flush=True)
    w, inp, h0 = _setup(c, dev)
    kw = dict(with_D=c["with_D"], with_z=c["gate"], with_bias=c["with_bias"], h0=h0)
    out, last = gpu_scan(inp, segments=c["segments"], **kw)
    ref_y, ref_h = oracle_scan(orc, inp, nthreads=NT, **kw)
    ey = norm_err(to_f64_numpy(out), ref_y)
    eh = norm_err(to_f64_numpy(last), ref_h)
    print(f"  err(y)={ey:.2e} err(state)={eh:.2e} tol={TOL[w.io]:g}", flush=True)
    assert ey <= TOL[w.io] and eh <= TOL[w.io], (ey, eh)


def _f(t):
    return None if t is None else to_f64_numpy(t)


@pytest.mark.parametrize("c", BWD_CASES, ids=_label)
def test_sweep_backward(orc, dev, c):
    print(f"case sweep backward {_label(c)}", flush=True)
    w, inp, h0 = _setup(c, dev)
    gr = to_dev(make_bwd_grads(w, seed=c["seed"] + 3), dev)
    D = inp["D"] if c["with_D"] else None
    bias = inp["delta_bias"] if c["with_bias"] else None
    z = inp["z"]
    dlast = gr["dlast"] if c["h0"] else None   # the two optional state ends together
    g = scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], gr["dout"], D=D, z=z,
                 delta_bias=bias, h0=h0, dlast=dlast, segments=c["segments"])
    torch.cuda.synchronize()
    ref = orc.scan_bwd(_f(inp["x"]), _f(inp["delta"]), _f(inp["A"]), _f(inp["B"]), _f(inp["C"]),
                       _f(gr["dout"]), D=_f(D), z=_f(z), delta_bias=_f(bias), h0=_f(h0),
                       dlast=_f(dlast), nthreads=NT)
    errs = {}
    for k, rk in [("dx", "dx"), ("ddelta", "ddelta"), ("dz", "dz"), ("dA", "dA"), ("dB", "dB"),
                  ("dC", "dC"), ("dD", "dD"), ("ddelta_bias", "dbias"), ("dh0", "dh0")]:
        if k == "dz" and z is None:
            assert g["dz"] is None
            continue
        errs[k] = norm_err(to_f64_numpy(g[k]), ref[rk])
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()) + f" tol={TOL[w.io]:g}",
          flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL[w.io]}
    assert not bad, f"gradients off: {bad}"
