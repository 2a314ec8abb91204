"""Seeded synthetic inputs shaped like the pages' workloads.

This module is the one piece shared by the HIP path's callers (tests, bench)
and the oracle's callers: it draws random tensors and holds none of the
method's arithmetic (no softplus, no exponentials, no recurrence). The shapes
come from the models the pages discuss: Mamba-2.8B has width 2,560, 5,120 inner
channels and N = 16 states ("Mamba and selective state spaces, from first
principles", "The Mamba block"); A starts as the S4D-Real diagonal
A_n = -(n + 1) (same page, "A state space model").

Distributions, drawn in float32 from one seeded ``torch.Generator`` in the
order x, Delta_raw, bias, B, C, D, z, then rounded to bfloat16 (round to
nearest even) where the workload stores bf16:
  x ~ N(0, 1); Delta_raw ~ N(0, s^2); bias ~ U(log(e^lo - 1), log(e^hi - 1))
  (uniform in bias space, so softplus(bias) spans [lo, hi]); B, C ~ N(0, 1)
  shared by all channels of a batch row; D = 1 or U(0.5, 1.5); z ~ N(0, 1).
Decode workloads add an fp32 initial state h0 ~ N(0, 1) and one token per
sequence per step.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int          # tokens per scan call (1 for decode)
    dim: int             # D_inner channels
    dstate: int          # N
    io: str              # "f32" or "bf16": storage of x, Delta_raw, z, B, C, y
    gate: bool           # z present (y * silu(z))
    d_skip: str          # "one" (D = 1) or "uniform" (D ~ U(0.5, 1.5))
    delta_lo: float      # softplus(bias) range
    delta_hi: float
    delta_std: float     # std of Delta_raw
    decode_steps: int = 0

    @property
    def elem_steps(self) -> int:
        steps = self.decode_steps if self.decode_steps else self.seqlen
        return self.batch * steps * self.dim

    @property
    def torch_io(self):
        return torch.float32 if self.io == "f32" else torch.bfloat16

    def with_shape(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    # tiny fp32 correctness case
    "tiny_fp32": Workload("tiny_fp32", 1, 256, 64, 16, "f32", False, "one", 0.001, 0.1, 0.5),
    # Mamba-130M-shaped layer (width 768, expand 2)
    "mamba130m_layer": Workload("mamba130m_layer", 2, 2048, 1536, 16, "bf16", True, "uniform",
                                0.001, 0.1, 0.5),
    # Mamba-2.8B-shaped prefill layer (width 2560, expand 2): the headline workload
    "mamba2p8b_prefill": Workload("mamba2p8b_prefill", 8, 2048, 5120, 16, "bf16", True, "uniform",
                                  0.001, 0.1, 0.5),
    # long context at 2.8B width, small Delta so the state persists
    "long_context_131k": Workload("long_context_131k", 1, 131072, 5120, 16, "bf16", True, "uniform",
                                  0.0005, 0.01, 0.5),
    # batched one-token decode against a resident fp32 state, 64 steps
    "decode_4096": Workload("decode_4096", 4096, 1, 5120, 16, "bf16", True, "uniform",
                            0.001, 0.1, 1.0, decode_steps=64),
}


def bias_range(w: Workload):
    """Endpoints of the uniform bias draw: the bias values whose softplus is
    delta_lo and delta_hi (inverse of log(1 + e^b), used only to place the
    draw's endpoints)."""
    return math.log(math.expm1(w.delta_lo)), math.log(math.expm1(w.delta_hi))


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def make_params(w: Workload, device="cpu", seed=0):
    """Per-channel parameters A (dim, N), D (dim,), bias (dim,), all fp32.
    Drawn from their own generator so that decode steps and scans share them."""
    g = _gen(device, seed + 7919)
    lo, hi = bias_range(w)
    bias = torch.rand(w.dim, generator=g, device=device) * (hi - lo) + lo
    if w.d_skip == "one":
        D = torch.ones(w.dim, device=device)
    else:
        D = torch.rand(w.dim, generator=g, device=device) + 0.5
    A = -torch.arange(1, w.dstate + 1, dtype=torch.float32, device=device).repeat(w.dim, 1)
    return {"A": A.contiguous(), "D": D, "delta_bias": bias}


def make_trained_A(w: Workload, device="cpu", seed=0, spread=0.5, channels=None):
    """A as it looks after training moved it off the S4D-Real start:
    A[d, n] = -(n + 1) * f, f log-normal with log-std `spread`, drawn per
    (channel, state) from its own seeded generator, so that no such channel
    keeps the A[d, n] = (n + 1) A[d, 0] shape. With `channels` (indices), only
    those channels are changed and the others keep -(n + 1)."""
    g = _gen(device, seed + 31337)
    base = -torch.arange(1, w.dstate + 1, dtype=torch.float32, device=device).repeat(w.dim, 1)
    f = torch.exp(spread * torch.randn((w.dim, w.dstate), generator=g, device=device))
    A = base * f
    if channels is not None:
        keep = torch.ones(w.dim, dtype=torch.bool, device=device)
        keep[torch.as_tensor(channels, device=device)] = False
        A[keep] = base[keep]
    return A.contiguous()


def make_conv_params(w: Workload, width=4, device="cpu", seed=0):
    """Depthwise convolution taps (dim, width) and bias (dim,), fp32, drawn
    uniform in [-1/sqrt(width), 1/sqrt(width)] (the usual initialisation of a
    convolution whose fan-in is its width), from their own generator."""
    g = _gen(device, seed + 271828)
    k = 1.0 / math.sqrt(width)
    weight = (torch.rand((w.dim, width), generator=g, device=device) * 2 - 1) * k
    bias = (torch.rand(w.dim, generator=g, device=device) * 2 - 1) * k
    return {"weight": weight.contiguous(), "bias": bias}


def make_conv_inputs(w: Workload, width=4, device="cpu", seed=0):
    """The convolution's input xin ~ N(0, 1) (batch, L, dim) and a state
    (batch, dim, width - 1) ~ N(0, 1) holding earlier inputs, in the io
    dtype, plus make_conv_params()."""
    g = _gen(device, seed + 161803)
    xin = torch.randn((w.batch, w.seqlen, w.dim), generator=g, device=device)
    state = torch.randn((w.batch, w.dim, width - 1), generator=g, device=device)
    out = {"xin": xin.to(w.torch_io), "state": state.to(w.torch_io)}
    out.update(make_conv_params(w, width, device, seed))
    return out


def make_scan_inputs(w: Workload, device="cpu", seed=0):
    """x, delta (Delta_raw), z: (batch, L, dim); B, C: (batch, L, N) in the
    workload's io dtype; plus make_params(). z is None without a gate."""
    g = _gen(device, seed)
    shp = (w.batch, w.seqlen, w.dim)
    x = torch.randn(shp, generator=g, device=device)
    delta = torch.randn(shp, generator=g, device=device) * w.delta_std
    B = torch.randn((w.batch, w.seqlen, w.dstate), generator=g, device=device)
    C = torch.randn((w.batch, w.seqlen, w.dstate), generator=g, device=device)
    z = torch.randn(shp, generator=g, device=device) if w.gate else None
    io = w.torch_io
    out = {"x": x.to(io), "delta": delta.to(io), "B": B.to(io), "C": C.to(io),
           "z": None if z is None else z.to(io)}
    out.update(make_params(w, device, seed))
    return out


def make_decode_state(w: Workload, device="cpu", seed=0):
    """Initial fp32 state h0 ~ N(0, 1), (batch, dim, N)."""
    g = _gen(device, seed + 104729)
    return torch.randn((w.batch, w.dim, w.dstate), generator=g, device=device)


def make_decode_token(w: Workload, step: int, device="cpu", seed=0):
    """One token per sequence for decode step ``step``: x, delta, z: (batch, dim);
    B, C: (batch, N), in the io dtype."""
    g = _gen(device, seed * 1000003 + 17 * step + 1)
    shp = (w.batch, w.dim)
    x = torch.randn(shp, generator=g, device=device)
    delta = torch.randn(shp, generator=g, device=device) * w.delta_std
    B = torch.randn((w.batch, w.dstate), generator=g, device=device)
    C = torch.randn((w.batch, w.dstate), generator=g, device=device)
    z = torch.randn(shp, generator=g, device=device) if w.gate else None
    io = w.torch_io
    return {"x": x.to(io), "delta": delta.to(io), "B": B.to(io), "C": C.to(io),
            "z": None if z is None else z.to(io)}


def make_grouped_bc(w: Workload, ngroups: int, device="cpu", seed=0, decode=False):
    """B and C ~ N(0, 1) for ngroups groups of channels: (batch, L, G, N), or
    (batch, G, N) for one decode token, in the io dtype."""
    g = _gen(device, seed * 31337 + 11)
    shp = (w.batch, ngroups, w.dstate) if decode else (w.batch, w.seqlen, ngroups, w.dstate)
    B = torch.randn(shp, generator=g, device=device).to(w.torch_io)
    C = torch.randn(shp, generator=g, device=device).to(w.torch_io)
    return B, C


@dataclass(frozen=True)
class SsdWorkload:
    """A Mamba-2 SSD layer: nheads heads of headdim channels, dstate states,
    B and C in ngroups groups of heads."""
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int = 64
    dstate: int = 128
    ngroups: int = 1
    delta_lo: float = 0.001   # softplus(dt_bias) range
    delta_hi: float = 0.1
    delta_std: float = 0.5    # std of dt

    @property
    def elem_steps(self) -> int:
        return self.batch * self.seqlen * self.nheads * self.headdim

    def with_shape(self, **kw) -> "SsdWorkload":
        d = dict(self.__dict__)
        d.update(kw)
        return SsdWorkload(**d)


SSD_WORKLOADS = {
    # the Mamba-2 2.7B layer's heads (80 x 64 channels, N = 128, one B/C group)
    # at the headline batch and length
    "mamba2_2p7b_layer": SsdWorkload("mamba2_2p7b_layer", 8, 2048, 80),
}


def make_ssd_inputs(w: SsdWorkload, device="cpu", seed=0):
    """x ~ N(0, 1) (batch, L, H, P); dt ~ N(0, s^2) (batch, L, H); B, C ~ N(0, 1)
    (batch, L, G, N), all bf16; per head: dt_bias uniform in bias space between
    softplus^-1(lo) and softplus^-1(hi), A = -exp(U(log 1, log 16)), D ~
    U(0.5, 1.5), fp32."""
    g = _gen(device, seed)
    x = torch.randn((w.batch, w.seqlen, w.nheads, w.headdim), generator=g, device=device)
    dt = torch.randn((w.batch, w.seqlen, w.nheads), generator=g, device=device) * w.delta_std
    B = torch.randn((w.batch, w.seqlen, w.ngroups, w.dstate), generator=g, device=device)
    C = torch.randn((w.batch, w.seqlen, w.ngroups, w.dstate), generator=g, device=device)
    gp = _gen("cpu", seed + 7)
    lo, hi = math.log(math.expm1(w.delta_lo)), math.log(math.expm1(w.delta_hi))
    dt_bias = lo + (hi - lo) * torch.rand(w.nheads, generator=gp)
    A = -torch.exp(torch.rand(w.nheads, generator=gp) * math.log(16.0))
    D = 0.5 + torch.rand(w.nheads, generator=gp)
    bf = torch.bfloat16
    return {"x": x.to(bf), "dt": dt.to(bf), "B": B.to(bf), "C": C.to(bf),
            "A": A.to(device), "D": D.to(device), "dt_bias": dt_bias.to(device)}


def make_bwd_grads(w: Workload, device="cpu", seed=0):
    """Incoming gradients for the backward pass: dout ~ N(0, 1) (batch, L, dim)
    in the io dtype, and dlast ~ N(0, 1) (batch, dim, N) fp32 for the final
    state."""
    g = _gen(device, seed * 7919 + 3)
    dout = torch.randn((w.batch, w.seqlen, w.dim), generator=g, device=device).to(w.torch_io)
    dlast = torch.randn((w.batch, w.dim, w.dstate), generator=g, device=device)
    return {"dout": dout, "dlast": dlast}


def to_f64_numpy(t):
    """Exact widening of a (possibly bf16) tensor to a float64 numpy array."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()


# Steps at which make_edge_inputs places runs of exact zeros in x: each run is
# at least 16 steps long, and together they cross the 8-step chunk edges and
# the segment edges of 1, 4, 5 and 12 time segments at L = 600 (56, 112, 120,
# 152, 168, 240, 304, 456, 480), plus one run that ends the sequence.
EDGE_ZERO_RUNS = ((50, 70), (104, 130), (145, 175), (230, 262), (296, 312), (450, 500), (584, 600))


def make_edge_inputs(w: Workload, device="cpu", seed=0):
    """make_scan_inputs() moved into the regimes where a step size is large or
    an input vanishes ("Mamba and selective state spaces, from first
    principles", "Discretisation: zero-order hold": a large step wipes the
    state; "Selection": a large step at a document boundary resets it):

      channels d % 4 == 1: bias ~ U(3, 8) (every step large);
      channels d % 4 == 2: bias ~ U(8, 20) (state wiped at every step);
      channels d % 4 == 3: Delta_raw raised by U(10, 20) at about 2 % of the
                           steps (isolated resets), bias unchanged;
      channels d % 3 == 0: x exactly 0 on the runs EDGE_ZERO_RUNS;
      channels d % 3 == 1: x = +-1e-39 (subnormal in fp32 and bf16) on steps
                           300..339 and +-1e-30 on steps 340..359;
      every channel:       x exactly 0 on steps 576..591.

    Values are placed, never computed from the method; rounding to the io
    dtype happens after placement, as in make_scan_inputs()."""
    base = make_scan_inputs(w.with_shape(io="f32"), device=device, seed=seed)
    g = _gen(device, seed + 424242)
    x = base["x"].clone()
    delta = base["delta"].clone()
    bias = base["delta_bias"].clone()
    L, dim = w.seqlen, w.dim
    ch = torch.arange(dim, device=device)
    m1, m2, m3 = ch % 4 == 1, ch % 4 == 2, ch % 4 == 3
    bias[m1] = 3.0 + 5.0 * torch.rand(int(m1.sum()), generator=g, device=device)
    bias[m2] = 8.0 + 12.0 * torch.rand(int(m2.sum()), generator=g, device=device)
    spikes = torch.rand((w.batch, L, dim), generator=g, device=device) < 0.02
    lift = 10.0 + 10.0 * torch.rand((w.batch, L, dim), generator=g, device=device)
    delta = torch.where(spikes & m3, delta + lift, delta)
    z0 = ch % 3 == 0
    for a, b in EDGE_ZERO_RUNS:
        a, b = min(a, L), min(b, L)
        x[:, a:b, z0] = 0.0
    tiny = ch % 3 == 1
    sign = torch.where(torch.rand((w.batch, L, dim), generator=g, device=device) < 0.5, -1.0, 1.0)
    for (a, b), mag in (((300, 340), 1e-39), ((340, 360), 1e-30)):
        a, b = min(a, L), min(b, L)
        x[:, a:b, tiny] = (sign[:, a:b] * mag)[:, :, tiny]
    x[:, min(576, L):min(592, L), :] = 0.0
    io = w.torch_io
    out = {"x": x.to(io), "delta": delta.to(io), "B": base["B"].to(io), "C": base["C"].to(io),
           "z": None if base["z"] is None else base["z"].to(io),
           "A": base["A"], "D": base["D"], "delta_bias": bias}
    return out
