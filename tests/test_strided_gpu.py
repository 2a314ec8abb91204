"""GPU parity of the strided entry points (mamba_scan_fwd_strided,
mamba_state_update_strided, through the C ABI): token tensors that are column
slices of wider row-major tensors, as they come out of the block's input
projection (x and z as the two halves of one row) and of the projection that
produces B and C per token. The arithmetic does not depend on the layout, so
the results must equal, bit for bit, those of the contiguous entry points on
copies of the same values; one case is also compared with the oracle. The
columns of a strided output's rows that lie outside the output must be left
untouched."""
import os

import pytest
import torch

from gpu_common import TOL, norm_err, to_dev
from selective_state_space_56_amd import scan_fwd, state_update
from selective_state_space_56_amd.workloads import (WORKLOADS, make_decode_state, make_decode_token,
                                                    make_grouped_bc, make_params, make_scan_inputs,
                                                    to_f64_numpy)

pytestmark = pytest.mark.gpu

NT = max(1, min(16, len(os.sched_getaffinity(0))))
SENTINEL = -1234.5


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def _embed(parts, extra_front, extra_back):
    """One buffer whose rows hold `extra_front` filler columns, then each
    tensor of `parts` (same leading shape) side by side, then `extra_back`
    filler columns; returns the views of the parts inside it."""
    lead = parts[0].shape[:-1]
    width = extra_front + sum(p.shape[-1] for p in parts) + extra_back
    buf = torch.full(lead + (width,), SENTINEL, dtype=parts[0].dtype, device=parts[0].device)
    views, at = [], extra_front
    for p in parts:
        buf[..., at:at + p.shape[-1]] = p
        views.append(buf[..., at:at + p.shape[-1]])
        at += p.shape[-1]
    return buf, views


@pytest.mark.parametrize("io,dim,front,back,segments,h0", [
    ("bf16", 512, 0, 0, 0, False),     # xz split of one row: 16-byte rows, direct LDS copies
    ("bf16", 512, 2, 0, 3, True),      # rows 4-byte aligned only; three segments and h0
    ("bf16", 384, 1, 0, 0, False),     # rows 2-byte aligned: register-staged copies
    ("f32", 256, 1, 3, 2, False),      # fp32 io, 4-byte rows
])
def test_scan_strided_equals_contiguous(dev, io, dim, front, back, segments, h0):
    w = WORKLOADS["mamba130m_layer"].with_shape(name="strided", batch=2, seqlen=300, dim=dim, io=io)
    inp = to_dev(make_scan_inputs(w, seed=dim + front), dev)
    N = w.dstate
    h0t = torch.randn((w.batch, dim, N), generator=torch.Generator().manual_seed(4)).to(dev) if h0 else None
    _say(f"case strided scan {io} dim={dim} front={front} back={back} seg={segments} h0={h0}")
    ref_y, ref_h = scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"], z=inp["z"],
                            delta_bias=inp["delta_bias"], h0=h0t, segments=segments)
    # x and z share rows (the input projection's two halves); B and C are
    # slices of a wider per-token row; delta has filler around it; out is
    # written into the middle of wider rows
    _, (x, z) = _embed([inp["x"], inp["z"]], front, back)
    _, (delta,) = _embed([inp["delta"]], front, back + 8)
    _, (B, C) = _embed([inp["B"], inp["C"]], 2 * front + 6, back)
    obuf, (out,) = _embed([torch.zeros_like(inp["x"])], front, 64)
    y, hN = scan_fwd(x, delta, inp["A"], B, C, D=inp["D"], z=z, delta_bias=inp["delta_bias"], h0=h0t,
                     out=out, segments=segments)
    torch.cuda.synchronize()
    assert y.data_ptr() == out.data_ptr()
    assert torch.equal(y, ref_y), (y.float() - ref_y.float()).abs().max().item()
    assert torch.equal(hN, ref_h)
    # only the output's own columns were written
    keep = torch.ones(obuf.shape[-1], dtype=torch.bool, device=dev)
    keep[front:front + dim] = False
    assert bool((obuf[..., keep] == SENTINEL).all())


def test_scan_strided_vs_oracle(orc, dev):
    w = WORKLOADS["mamba130m_layer"].with_shape(name="strided", batch=2, seqlen=260, dim=256)
    inp = to_dev(make_scan_inputs(w, seed=3), dev)
    _, (x, z) = _embed([inp["x"], inp["z"]], 0, 0)
    _, (B, C) = _embed([inp["B"], inp["C"]], 8, 0)
    y, hN = scan_fwd(x, inp["delta"], inp["A"], B, C, D=inp["D"], z=z, delta_bias=inp["delta_bias"])
    torch.cuda.synchronize()
    f = {k: None if v is None else to_f64_numpy(v) for k, v in inp.items()}
    ry, rh = orc.scan(f["x"], f["delta"], f["A"], f["B"], f["C"], D=f["D"], z=f["z"],
                      delta_bias=f["delta_bias"], nthreads=NT)
    ey, eh = norm_err(to_f64_numpy(y), ry), norm_err(to_f64_numpy(hN), rh)
    _say(f"strided scan vs oracle: err(y)={ey:.2e} err(state)={eh:.2e}")
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


def test_scan_strided_groups(dev):
    """B and C of two channel groups as (batch, L, G, N) slices of wider rows."""
    w = WORKLOADS["mamba130m_layer"].with_shape(name="strided", batch=2, seqlen=200, dim=512)
    inp = to_dev(make_scan_inputs(w, seed=5), dev)
    Bg, Cg = make_grouped_bc(w, 2, device=dev, seed=1)
    ref_y, ref_h = scan_fwd(inp["x"], inp["delta"], inp["A"], Bg, Cg, D=inp["D"], z=inp["z"],
                            delta_bias=inp["delta_bias"])
    _, (Bf, Cf) = _embed([Bg.flatten(-2), Cg.flatten(-2)], 10, 2)
    B, C = Bf.unflatten(-1, (2, w.dstate)), Cf.unflatten(-1, (2, w.dstate))
    y, hN = scan_fwd(inp["x"], inp["delta"], inp["A"], B, C, D=inp["D"], z=inp["z"],
                     delta_bias=inp["delta_bias"])
    torch.cuda.synchronize()
    assert torch.equal(y, ref_y) and torch.equal(hN, ref_h)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_state_update_strided_equals_contiguous(dev, io):
    wd = WORKLOADS["decode_4096"].with_shape(name="strided_decode", batch=40, dim=320, io=io)
    params = make_params(wd, device=dev)
    s_ref = make_decode_state(wd, device=dev)
    s_str = s_ref.clone()
    for step in range(3):
        t = make_decode_token(wd, step, device=dev)
        _say(f"case strided decode {io} step {step}")
        y_ref = state_update(s_ref, t["x"], t["delta"], params["A"], t["B"], t["C"], D=params["D"],
                             z=t["z"], delta_bias=params["delta_bias"])
        _, (x, z) = _embed([t["x"], t["z"]], 0, 0)
        _, (delta,) = _embed([t["delta"]], 3, 1)
        _, (B, C) = _embed([t["B"], t["C"]], 6, 0)
        obuf, (out,) = _embed([torch.zeros_like(t["x"])], 2, 5)
        y = state_update(s_str, x, delta, params["A"], B, C, D=params["D"], z=z,
                         delta_bias=params["delta_bias"], out=out)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(s_str, s_ref)
        keep = torch.ones(obuf.shape[-1], dtype=torch.bool, device=dev)
        keep[2:2 + wd.dim] = False
        assert bool((obuf[..., keep] == SENTINEL).all())
