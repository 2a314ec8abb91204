"""GPU parity of the causal convolution + SiLU front-end (mamba_conv1d_fwd,
mamba_conv1d_update, through the C ABI) against the fp64 oracle on the same
seeded inputs. The returned state holds raw inputs, so it must match exactly;
outputs are compared with the error metric of gpu_common."""
import os

import numpy as np
import pytest
import torch

from gpu_common import TOL, norm_err
from selective_state_space_56_amd import conv1d_fwd, conv1d_update
from selective_state_space_56_amd.workloads import WORKLOADS, make_conv_inputs, to_f64_numpy

pytestmark = pytest.mark.gpu

NT = max(1, min(16, len(os.sched_getaffinity(0))))


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def _wl(batch, L, dim, io):
    return WORKLOADS["mamba130m_layer"].with_shape(name="conv", batch=batch, seqlen=L, dim=dim, io=io)


def _check(orc, w, inp, width, with_bias=True, with_state=True, channels=None):
    bias = inp["bias"] if with_bias else None
    sin = inp["state"] if with_state else None
    out, sout = conv1d_fwd(inp["xin"], inp["weight"], bias, sin)
    torch.cuda.synchronize()
    xin = to_f64_numpy(inp["xin"])
    wt = to_f64_numpy(inp["weight"])
    b64 = None if bias is None else to_f64_numpy(bias)
    s64 = None if sin is None else to_f64_numpy(sin)
    got = to_f64_numpy(out)
    got_s = to_f64_numpy(sout) if sout is not None else None
    if channels is not None:
        xin, wt = xin[:, :, channels], wt[channels]
        b64 = None if b64 is None else b64[channels]
        s64 = None if s64 is None else s64[:, channels]
        got = got[:, :, channels]
        got_s = None if got_s is None else got_s[:, channels]
    ref, ref_s = orc.conv1d(xin, wt, b64, s64, nthreads=NT)
    e = norm_err(got, ref)
    _say(f"conv {w.batch}x{w.seqlen}x{w.dim} W={width} {w.io} bias={with_bias} "
         f"state={with_state}: err={e:.3e}")
    assert e <= TOL[w.io], e
    if got_s is not None:
        assert np.array_equal(got_s, ref_s), "state_out must hold the exact inputs"
    return out, sout


@pytest.mark.parametrize("batch,L,dim,width,io", [
    (2, 300, 256, 4, "bf16"),     # 8-byte channel groups (4 bf16)
    (2, 150, 20, 4, "bf16"),      # 4-channel groups, rows not whole 16-byte pieces
    (1, 97, 132, 3, "bf16"),      # 4-channel groups, partial last workgroup
    (2, 300, 256, 4, "f32"),      # 16-byte channel groups (4 fp32)
    (3, 65, 37, 4, "bf16"),       # odd channel count: one channel per thread
    (1, 129, 40, 3, "f32"),
    (2, 70, 48, 2, "bf16"),
    (2, 50, 24, 1, "f32"),        # no state
    (2, 2, 64, 4, "bf16"),        # shorter than the window
    (1, 1, 16, 4, "f32"),
])
def test_conv_vs_oracle(orc, dev, batch, L, dim, width, io):
    w = _wl(batch, L, dim, io)
    inp = {k: v.to(dev) for k, v in make_conv_inputs(w, width, seed=batch + L + dim).items()}
    _check(orc, w, inp, width)
    _check(orc, w, inp, width, with_bias=False, with_state=False)


def test_conv_empty_sequence_keeps_state(dev):
    w = _wl(2, 0, 64, "bf16")
    inp = {k: v.to(dev) for k, v in make_conv_inputs(w, 4, seed=3).items()}
    out, sout = conv1d_fwd(inp["xin"], inp["weight"], inp["bias"], inp["state"])
    torch.cuda.synchronize()
    assert out.shape == (2, 0, 64) and torch.equal(sout, inp["state"])


def test_conv_in_pieces(dev):
    """Pieces chained through the state give the one-call output bitwise (each
    output depends only on the same four inputs, the taps and the bias)."""
    w = _wl(2, 700, 512, "bf16")
    inp = {k: v.to(dev) for k, v in make_conv_inputs(w, 4, seed=9).items()}
    whole, s_whole = conv1d_fwd(inp["xin"], inp["weight"], inp["bias"], inp["state"])
    outs, st = [], inp["state"]
    for a, b in [(0, 1), (1, 3), (3, 130), (130, 700)]:
        o, st = conv1d_fwd(inp["xin"][:, a:b].contiguous(), inp["weight"], inp["bias"], st.clone())
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, dim=1), whole)
    assert torch.equal(st, s_whole)


@pytest.mark.parametrize("width,io,dim", [(4, "bf16", 512), (4, "f32", 37), (3, "bf16", 40),
                                          (1, "f32", 64)])
def test_conv_update_vs_oracle(orc, dev, width, io, dim):
    """Six decode tokens against the oracle's shift-register update, then the
    same tokens through the sequence form reproduce outputs and state."""
    w = _wl(3, 6, dim, io)
    inp = {k: v.to(dev) for k, v in make_conv_inputs(w, width, seed=17).items()}
    st = inp["state"].clone()
    ref_st = to_f64_numpy(inp["state"])
    wt, b64 = to_f64_numpy(inp["weight"]), to_f64_numpy(inp["bias"])
    outs = []
    for t in range(6):
        x_t = inp["xin"][:, t].contiguous()
        o = conv1d_update(st, x_t, inp["weight"], inp["bias"])
        ref_o, ref_st = orc.conv1d_update(ref_st, to_f64_numpy(x_t), wt, b64)
        torch.cuda.synchronize()
        assert norm_err(to_f64_numpy(o), ref_o) <= TOL[io]
        outs.append(o)
    assert np.array_equal(to_f64_numpy(st), ref_st)
    seq, s_seq = conv1d_fwd(inp["xin"], inp["weight"], inp["bias"], inp["state"])
    torch.cuda.synchronize()
    assert torch.equal(torch.stack(outs, dim=1), seq)
    assert torch.equal(st, s_seq)


def test_conv_full_size(orc, dev):
    """The Mamba-2.8B-shaped prefill input (8 x 2048 x 5120, bf16) as the
    bench launches it, every output and the whole state compared."""
    w = WORKLOADS["mamba2p8b_prefill"]
    _say("case conv full size")
    inp = make_conv_inputs(w, 4, device=dev)
    _check(orc, w, inp, 4)
