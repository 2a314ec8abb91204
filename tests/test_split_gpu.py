"""GPU parity of the state-split scan kernel (MAMBA_SCAN_SPLIT_STATES: the 16
states of each (batch, channel) row on four lanes, the whole sequence in one
pass) against the fp64 oracle, forced through the flag at sizes the oracle
finishes in seconds: lengths around the 8-step chunk and ragged tails, partial
64-channel tiles and a single channel, the general and mixed decay paths, h0,
channel groups, strided tensors and absent optional arguments; the full-size
2.8B layer on sampled channels; and its agreement with the segmented kernel."""
import os

import numpy as np
import pytest
import torch

from gpu_common import BlockedErr, TOL, norm_err, oracle_scan, to_dev
from selective_state_space_56_amd import scan_fwd
from selective_state_space_56_amd.workloads import (WORKLOADS, make_decode_state, make_grouped_bc,
                                                    make_scan_inputs, make_trained_A,
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


def _split(inp, with_D=True, with_z=True, with_bias=True, h0=None, **kw):
    out, last = scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"],
                         D=inp["D"] if with_D else None, z=inp["z"] if with_z else None,
                         delta_bias=inp["delta_bias"] if with_bias else None, h0=h0,
                         split_states=True, **kw)
    torch.cuda.synchronize()
    return out, last


def _check(orc, w, inp, tol=None, **kw):
    tol = TOL[w.io] if tol is None else tol
    out, last = _split(inp, **kw)
    ry, rh = oracle_scan(orc, inp, nthreads=NT, **kw)
    ey, eh = norm_err(to_f64_numpy(out), ry), norm_err(to_f64_numpy(last), rh)
    _say(f"split {w.name} {w.batch}x{w.seqlen}x{w.dim} {w.io}: err(y)={ey:.3e} "
         f"err(state)={eh:.3e} tol={tol:g}")
    assert ey <= tol and eh <= tol
    return out, last


@pytest.mark.parametrize("batch,L,dim,io", [
    (2, 300, 200, "bf16"),    # ragged tail (300 = 37 chunks + 4), partial tile
    (1, 1, 64, "f32"),        # one step: one partial chunk
    (1, 7, 65, "f32"),        # one partial chunk, one channel in the second tile
    (3, 8, 1, "f32"),         # exactly one chunk, one channel
    (2, 9, 130, "bf16"),      # one step past a chunk
    (1, 17, 64, "f32"),
    (2, 1001, 300, "bf16"),
    (1, 4096, 64, "f32"),     # long: fp32 tolerance over 512 chunks
])
def test_split_shapes(orc, dev, batch, L, dim, io):
    w = WORKLOADS["mamba130m_layer"].with_shape(name="split", batch=batch, seqlen=L, dim=dim, io=io)
    inp = to_dev(make_scan_inputs(w, seed=L + dim), dev)
    _check(orc, w, inp)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_split_general_A(orc, dev, io):
    w = WORKLOADS["mamba130m_layer"].with_shape(name="split_generalA", batch=2, seqlen=600, dim=300,
                                                 io=io)
    inp = make_scan_inputs(w, seed=11)
    inp["A"] = make_trained_A(w, seed=11)
    _check(orc, w, to_dev(inp, dev))


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_split_mixed_tiles(orc, dev, io):
    """64-channel tiles: tile 0 has one general channel (17), tile 1
    (64..127) is all general, the rest keep the S4D-Real shape except the last
    channel of the partial last tile."""
    w = WORKLOADS["mamba130m_layer"].with_shape(name="split_mixed", batch=2, seqlen=500, dim=780,
                                                 io=io)
    inp = make_scan_inputs(w, seed=12)
    inp["A"] = make_trained_A(w, seed=12, channels=[17] + list(range(64, 128)) + [779])
    _check(orc, w, to_dev(inp, dev))


@pytest.mark.parametrize("io,general", [("f32", False), ("bf16", False), ("f32", True)])
def test_split_initial_state(orc, dev, io, general):
    w = WORKLOADS["mamba130m_layer"].with_shape(name="split_h0", batch=2, seqlen=301, dim=300, io=io)
    inp = make_scan_inputs(w, seed=21)
    if general:
        inp["A"] = make_trained_A(w, seed=21)
    inp = to_dev(inp, dev)
    h0 = make_decode_state(w, device=dev, seed=21)
    _check(orc, w, inp, h0=h0)


def test_split_optional_arguments_absent(orc, dev):
    w = WORKLOADS["mamba130m_layer"].with_shape(name="split_bare", batch=2, seqlen=203, dim=130)
    inp = to_dev(make_scan_inputs(w, seed=4), dev)
    _check(orc, w, inp, with_D=False, with_z=False, with_bias=False)
    out, last = scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"], z=inp["z"],
                         delta_bias=inp["delta_bias"], return_last_state=False, split_states=True)
    ref, _ = _split(inp)
    torch.cuda.synchronize()
    assert last is None and torch.equal(out, ref)


@pytest.mark.parametrize("G,io", [(2, "bf16"), (4, "f32")])
def test_split_groups(orc, dev, G, io):
    """B and C per group of channels (dim / G channels each)."""
    w = WORKLOADS["mamba130m_layer"].with_shape(name="split_groups", batch=2, seqlen=260,
                                                 dim=256 * G, io=io)
    inp = to_dev(make_scan_inputs(w, seed=6), dev)
    Bg, Cg = make_grouped_bc(w, G, device=dev, seed=6)
    inp["B"], inp["C"] = Bg, Cg
    out, last = _split(inp)
    f = {k: None if v is None else to_f64_numpy(v) for k, v in inp.items()}
    ry, rh = orc.scan(f["x"], f["delta"], f["A"], f["B"], f["C"], D=f["D"], z=f["z"],
                      delta_bias=f["delta_bias"], nthreads=NT)
    ey, eh = norm_err(to_f64_numpy(out), ry), norm_err(to_f64_numpy(last), rh)
    _say(f"split groups G={G} {io}: err(y)={ey:.3e} err(state)={eh:.3e}")
    assert ey <= TOL[io] and eh <= TOL[io]


def test_split_strided_equals_contiguous(dev):
    """x and z as the two halves of one row, B and C slices of a wider row,
    the output inside wider rows: bit-identical to the contiguous call, and
    the output rows' other columns untouched."""
    w = WORKLOADS["mamba130m_layer"].with_shape(name="split_strided", batch=2, seqlen=300, dim=256)
    inp = to_dev(make_scan_inputs(w, seed=8), dev)
    ref_y, ref_h = _split(inp)
    dim, N = w.dim, w.dstate
    xz = torch.cat([inp["x"], inp["z"]], dim=-1)
    x, z = xz[..., :dim], xz[..., dim:]
    bc = torch.cat([torch.zeros_like(inp["B"][..., :2]), inp["B"], inp["C"]], dim=-1)
    B, C = bc[..., 2:2 + N], bc[..., 2 + N:]
    obuf = torch.full((w.batch, w.seqlen, dim + 70), SENTINEL, dtype=inp["x"].dtype, device=dev)
    out = obuf[..., 5:5 + dim]
    y, h = scan_fwd(x, inp["delta"], inp["A"], B, C, D=inp["D"], z=z, delta_bias=inp["delta_bias"],
                    out=out, split_states=True)
    torch.cuda.synchronize()
    assert torch.equal(y, ref_y) and torch.equal(h, ref_h)
    keep = torch.ones(obuf.shape[-1], dtype=torch.bool, device=dev)
    keep[5:5 + dim] = False
    assert bool((obuf[..., keep] == SENTINEL).all())


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_split_agrees_with_segmented(dev, io):
    """The two kernels compute the same recurrence in different orders: their
    outputs agree to the io precision and their final states closely."""
    w = WORKLOADS["mamba130m_layer"].with_shape(name="split_vs_seg", batch=2, seqlen=2048, dim=512,
                                                 io=io)
    inp = to_dev(make_scan_inputs(w, seed=5), dev)
    ys, hs = _split(inp)
    for segments in (1, 8):
        yg, hg = scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                          z=inp["z"], delta_bias=inp["delta_bias"], segments=segments)
        torch.cuda.synchronize()
        ey = norm_err(to_f64_numpy(ys), to_f64_numpy(yg))
        eh = norm_err(to_f64_numpy(hs), to_f64_numpy(hg))
        _say(f"split vs segmented ({segments}) {io}: y {ey:.2e} state {eh:.2e}")
        assert ey <= (1e-2 if io == "bf16" else 1e-5) and eh <= 1e-4


@pytest.mark.parametrize("general", [False, True])
def test_split_full_size(orc, dev, general):
    """8 x 2048 x 5120 bf16 (the Mamba-2.8B layer), every output compared with
    the oracle run on blocks of 1024 channels (rows are independent)."""
    w = WORKLOADS["mamba2p8b_prefill"]
    _say(f"case split {w.name} general={general} (full size, every channel)")
    inp = make_scan_inputs(w, device=dev)
    if general:
        inp["A"] = make_trained_A(w, device=dev)
    out, last = _split(inp)
    ey, eh = BlockedErr(), BlockedErr()
    for c0 in range(0, w.dim, 1024):
        ch = np.arange(c0, min(w.dim, c0 + 1024))
        ry, rh = oracle_scan(orc, inp, channels=ch, nthreads=NT)
        ey.add(out[:, :, c0:c0 + len(ch)], ry)
        eh.add(last[:, c0:c0 + len(ch)], rh)
    e_y, e_h = ey.err(), eh.err()
    _say(f"split full size: err(y)={e_y:.3e} err(state)={e_h:.3e}")
    assert e_y <= TOL["bf16"] and e_h <= TOL["bf16"]


def test_split_run_twice_bitwise(dev):
    w = WORKLOADS["mamba130m_layer"].with_shape(name="split_det", batch=2, seqlen=1024, dim=512)
    inp = to_dev(make_scan_inputs(w, seed=9), dev)
    o1, l1 = _split(inp)
    o2, l2 = _split(inp)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_split_empty_sequence(dev):
    """L = 0 with the flag: nothing to scan; the final state is h0, or zeros."""
    w = WORKLOADS["mamba130m_layer"].with_shape(name="split_empty", batch=2, seqlen=0, dim=70)
    inp = to_dev(make_scan_inputs(w, seed=2), dev)
    h0 = make_decode_state(w, device=dev, seed=2)
    out, last = _split(inp, h0=h0)
    assert out.shape == (2, 0, 70) and torch.equal(last, h0)
    last0 = torch.full((2, 70, 16), 7.0, device=dev)
    scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"], z=inp["z"],
             delta_bias=inp["delta_bias"], last_state=last0, split_states=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(last0).item() == 0


def test_split_rejects_unsupported(dev):
    w = WORKLOADS["mamba130m_layer"].with_shape(name="split_bad", batch=1, seqlen=16, dim=64, dstate=8)
    inp = to_dev(make_scan_inputs(w, seed=1), dev)
    with pytest.raises(RuntimeError, match="MAMBA_SCAN_SPLIT_STATES"):
        _split(inp)
