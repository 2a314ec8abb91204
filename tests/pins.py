"""Checks that pin the fp64 oracle to facts the pages and the mathematics fix.

Each ``pin_*`` function takes an ``oracle.Oracle`` handle and raises
``AssertionError`` when the oracle disagrees with the pinned fact. They are run
against the real oracle by ``test_oracle_pins.py`` and against deliberately
broken copies of the oracle source by ``test_oracle_mutants.py`` (every broken
copy must fail at least one pin).

No pin re-types the oracle's loop: expected values come from printed numbers,
closed forms (impulse responses, prefix sums, the gated-RNN form, a product of
decays written as one exponential of a sum), brute-force convolution sums, or
an affine-pair tree scan.
"""
from __future__ import annotations

import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(got, want, rtol, atol=0.0, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    if got.shape != want.shape:
        raise AssertionError(f"{what}: shape {got.shape} != {want.shape}")
    err = np.abs(got - want)
    lim = atol + rtol * np.abs(want)
    if not np.all(err <= lim):
        i = int(np.argmax(err - lim))
        raise AssertionError(f"{what}: max violation at flat {i}: got {got.flat[i]!r}, "
                             f"want {want.flat[i]!r}, err {err.flat[i]:.3e}")


def read_golden(name="worked_example.txt"):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split("=", 1)
            vals[k.strip()] = np.array([float(t) for t in v.split()])
    return vals


def _inv_softplus(v):
    """The Delta_raw whose softplus is v (v > 0): log(exp(v) - 1)."""
    return math.log(math.expm1(v))


def _sigmoid(v):
    return 1.0 / (1.0 + np.exp(-v))


# ---------------------------------------------------------------------------
# Values printed on the pages
# ---------------------------------------------------------------------------

def pin_worked_example(orc):
    """"State space models and Mamba", "A worked example": decay 0.8, input
    weight 0.5, input [2, 0, 3] -> states [1.0, 0.8, 2.14]; kernel
    [0.5, 0.4, 0.32]. Mapped onto S6 with one state: Delta = 1 (Delta_raw =
    softplus^-1(1)), A = ln 0.8 so exp(Delta A) = 0.8, B = 0.5 so the
    first-order Bbar = Delta B = 0.5, C = 1. The same numbers must come out
    with Delta = 2, A = ln(0.8)/2, B = 0.25 (Delta scales both A and B), and
    with the softplus argument moved from Delta_raw into the bias."""
    g = read_golden()
    a, b, c = float(g["decay"][0]), float(g["input_weight"][0]), float(g["readout"][0])
    u = g["inputs"].reshape(1, 3, 1)
    C = np.full((1, 3, 1), c)
    for Delta in (1.0, 2.0):
        A = np.array([[math.log(a) / Delta]])
        B = np.full((1, 3, 1), b / Delta)
        draw = np.full((1, 3, 1), _inv_softplus(Delta))
        y, h = orc.scan(u, draw, A, B, C)
        _close(y.ravel(), g["states"], 1e-12, 1e-14, f"worked example states (Delta={Delta})")
        _close(y.ravel(), g["printed_recurrent"], 1e-12, 1e-14, "printed recurrent tensor")
        _close(h.ravel(), g["states"][-1:], 1e-12, 0, "final state")
        # same Delta reached through the bias instead of Delta_raw
        y2, _ = orc.scan(u, np.zeros_like(draw), A, B, C,
                         delta_bias=np.array([_inv_softplus(Delta)]))
        _close(y2.ravel(), g["states"], 1e-12, 1e-14, "worked example via bias")
        # impulse input -> convolution kernel
        imp = np.array([1.0, 0.0, 0.0]).reshape(1, 3, 1)
        k, _ = orc.scan(imp, draw, A, B, C)
        _close(k.ravel(), g["kernel"], 1e-12, 1e-14, "worked example kernel")
        # the page's convolution sum for the third output
        kern = g["kernel"]
        conv3 = sum(kern[lag] * g["inputs"][2 - lag] for lag in range(3))
        _close(conv3, g["third_conv_output"][0], 1e-12, 0, "third conv output")
        _close(y.ravel()[2], conv3, 1e-12, 0, "recurrence == convolution")
        # K_0 = D + C Bbar
        yD, _ = orc.scan(u, draw, A, B, C, D=g["direct_term"])
        _close(yD.ravel(), g["outputs_with_direct_term"], 1e-12, 1e-14, "with D term")


# ---------------------------------------------------------------------------
# Special cases with closed forms
# ---------------------------------------------------------------------------

def pin_gated_rnn(orc):
    """"Mamba and selective state spaces, from first principles",
    "Discretisation: zero-order hold": with N = 1, A = -1, B = 1 and
    Delta = softplus(z_t) the recurrence is the gated RNN
    h_t = (1 - g_t) h_{t-1} + g_t x_t, g_t = sigmoid(z_t). That identity is
    exact under the zero-order-hold Bbar. Under the first-order Bbar the decay
    is still exactly 1 - sigmoid(z_t) = exp(-Delta_t) and the input weight is
    Delta_t itself."""
    rng = np.random.default_rng(11)
    L, dim = 50, 3
    zt = rng.normal(0, 2.0, size=(1, L, dim))
    x = rng.normal(0, 1.0, size=(1, L, dim))
    A = -np.ones((dim, 1))
    B = np.ones((1, L, 1))
    C = np.ones((1, L, 1))
    g = _sigmoid(zt)
    # gated RNN, written with the sigmoid (not with exp(-softplus))
    h = np.zeros(dim)
    want_zoh = np.zeros_like(x)
    for t in range(L):
        h = (1 - g[0, t]) * h + g[0, t] * x[0, t]
        want_zoh[0, t] = h
    y, last = orc.scan(x, zt, A, B, C, zoh=True)
    _close(y, want_zoh, 1e-12, 1e-14, "gated RNN (ZOH)")
    _close(last[0, :, 0], h, 1e-12, 1e-14, "gated RNN final state")
    # first-order Bbar: decay 1 - sigmoid(z), input weight log(1 + e^z)
    Delta = np.logaddexp(0.0, zt)
    h = np.zeros(dim)
    want_fo = np.zeros_like(x)
    for t in range(L):
        h = (1 - g[0, t]) * h + Delta[0, t] * x[0, t]
        want_fo[0, t] = h
    y, _ = orc.scan(x, zt, A, B, C)
    _close(y, want_fo, 1e-12, 1e-14, "gated RNN (first-order Bbar)")


def pin_lti_convolution(orc):
    """Constant Delta, B, C make the system time-invariant, so it is the causal
    convolution y = x * K with K_k = C Abar^k Bbar plus the direct term D x
    (erikxu.me notes, "State Space Models"; "Mamba and selective state
    spaces", "S4: fixed dynamics, so a convolution"; "State space models and
    Mamba", "One system, two views"). Brute-force O(L^2) sum, N = 16,
    per-channel A, several batches and channels."""
    rng = np.random.default_rng(12)
    batch, L, dim, N = 2, 40, 3, 16
    A = -rng.uniform(0.05, 2.0, size=(dim, N))
    c = rng.normal(-1.0, 0.7, size=(batch, dim))           # Delta_raw per (b, d)
    bias = rng.normal(0, 0.3, size=dim)
    Bv = rng.normal(size=(batch, N))
    Cv = rng.normal(size=(batch, N))
    D = rng.normal(size=dim)
    x = rng.normal(size=(batch, L, dim))
    draw = np.broadcast_to(c[:, None, :], (batch, L, dim)).copy()
    B = np.broadcast_to(Bv[:, None, :], (batch, L, N)).copy()
    C = np.broadcast_to(Cv[:, None, :], (batch, L, N)).copy()
    want = np.zeros_like(x)
    for b in range(batch):
        for d in range(dim):
            Delta = float(np.logaddexp(0.0, c[b, d] + bias[d]))
            abar = np.exp(Delta * A[d])
            K = np.array([np.sum(Cv[b] * abar ** k * Delta * Bv[b]) for k in range(L)])
            for t in range(L):
                want[b, t, d] = sum(K[k] * x[b, t - k, d] for k in range(t + 1)) + D[d] * x[b, t, d]
    y, _ = orc.scan(x, draw, A, B, C, D=D, delta_bias=bias)
    _close(y, want, 1e-11, 1e-13, "LTI convolution")


def pin_write_then_read(orc):
    """Selective (time-varying) case with a closed form. Write only at step
    t_w (B_{t_w} = beta e_n), read only at step t_r (C_{t_r} = gamma e_m).
    Then y_{t_r} = [n == m] gamma beta Delta_{t_w} x_{t_w}
    exp(A_n sum_{s=t_w+1..t_r} Delta_s): the decays of the steps in between
    multiply, and each step's decay uses that step's own Delta ("Mamba and
    selective state spaces", "Selection: B, C and Delta from the token" and
    "The hardware-aware scan"). Every other output is D x_t."""
    rng = np.random.default_rng(13)
    batch, L, dim, N = 2, 12, 3, 16
    A = -rng.uniform(0.1, 1.5, size=(dim, N))
    draw = rng.normal(0, 1.0, size=(batch, L, dim))
    x = rng.normal(size=(batch, L, dim))
    D = rng.normal(size=dim)
    Delta = np.logaddexp(0.0, draw)
    for (tw, tr, n, m) in [(2, 9, 5, 5), (2, 9, 5, 6), (4, 4, 0, 0), (0, 11, 15, 15), (7, 3, 1, 1)]:
        B = np.zeros((batch, L, N))
        C = np.zeros((batch, L, N))
        B[:, tw, n] = 1.7
        C[:, tr, m] = -0.6
        y, _ = orc.scan(x, draw, A, B, C, D=D)
        want = D[None, None, :] * x
        if n == m and tr >= tw:
            S = Delta[:, tw + 1:tr + 1, :].sum(axis=1)                 # (batch, dim)
            want[:, tr, :] += -0.6 * 1.7 * Delta[:, tw, :] * x[:, tw, :] * np.exp(A[None, :, n] * S)
        _close(y, want, 1e-12, 1e-14, f"write t={tw} n={n}, read t={tr} m={m}")


def pin_impulse_per_state(orc):
    """Impulse response of each state of the S4D-Real diagonal A_n = -(n+1)
    ("Mamba and selective state spaces", "A state space model"): input
    x = delta_0, B = C = e_n and constant Delta give
    y_t = Delta exp(-(n+1) Delta)^t."""
    L, N = 30, 16
    Delta = 0.37
    A = -(np.arange(N, dtype=np.float64) + 1.0)[None, :]
    x = np.zeros((1, L, 1))
    x[0, 0, 0] = 1.0
    draw = np.full((1, L, 1), _inv_softplus(Delta))
    t = np.arange(L)
    for n in (0, 3, 15):
        B = np.zeros((1, L, N))
        B[..., n] = 1.0
        y, last = orc.scan(x, draw, A, B, B.copy())
        _close(y.ravel(), Delta * np.exp(-(n + 1) * Delta) ** t, 1e-12, 1e-300, f"impulse n={n}")
        want_last = np.zeros(N)
        want_last[n] = Delta * math.exp(-(n + 1) * Delta * (L - 1))
        _close(last.ravel(), want_last, 1e-12, 1e-300, f"impulse final state n={n}")


def pin_degenerate_A(orc):
    """A = 0 gives Abar = 1, so the state is the prefix sum of Delta B x and the
    output is a read-out of cumulative sums. A very negative gives Abar = 0, a
    memoryless map y_t = (C_t . Delta_t B_t) x_t + D x_t ("Mamba and selective
    state spaces", "Discretisation": large Delta*|a| wipes the state, small
    keeps it). ZOH with A = 0 is rejected (division by A)."""
    rng = np.random.default_rng(14)
    batch, L, dim, N = 2, 25, 4, 16
    x = rng.normal(size=(batch, L, dim))
    draw = rng.normal(-1, 1, size=(batch, L, dim))
    B = rng.normal(size=(batch, L, N))
    C = rng.normal(size=(batch, L, N))
    D = rng.normal(size=dim)
    Delta = np.logaddexp(0.0, draw)
    # A = 0: prefix sums
    dBx = Delta[:, :, :, None] * B[:, :, None, :] * x[:, :, :, None]     # (b, t, d, n)
    H = np.cumsum(dBx, axis=1)
    want = np.einsum("btn,btdn->btd", C, H) + D * x
    y, last = orc.scan(x, draw, np.zeros((dim, N)), B, C, D=D)
    _close(y, want, 1e-11, 1e-12, "A = 0 prefix sum")
    _close(last, H[:, -1], 1e-11, 1e-12, "A = 0 final state")
    # A -> -inf: memoryless
    want = np.einsum("btn,btn->bt", C, B)[:, :, None] * Delta * x + D * x
    y, last = orc.scan(x, draw, np.full((dim, N), -1e6), B, C, D=D)
    _close(y, want, 1e-12, 1e-13, "A = -1e6 memoryless")
    try:
        orc.scan(x, draw, np.zeros((dim, N)), B, C, zoh=True)
    except ValueError:
        pass
    else:
        raise AssertionError("ZOH with A = 0 was not rejected")


def pin_zoh_small_A_limit(orc):
    """As A -> 0 the exact zero-order-hold Bbar = (exp(Delta A) - 1)/A B tends
    to the first-order Delta B ("Discretisation: zero-order hold": the
    first-order form is the leading term in Delta)."""
    rng = np.random.default_rng(15)
    batch, L, dim, N = 1, 20, 3, 16
    x = rng.normal(size=(batch, L, dim))
    draw = rng.normal(-1, 1, size=(batch, L, dim))
    B = rng.normal(size=(batch, L, N))
    C = rng.normal(size=(batch, L, N))
    # (exp(Delta A) - 1) / A = Delta (1 + Delta A / 2 + ...): with A = -1e-6 and
    # Delta < 3 the two forms differ by a relative 1.5e-6 at most, and the
    # fp64 cancellation in exp(Delta A) - 1 adds about 1e-10 / Delta.
    A = -1e-6 * np.ones((dim, N))
    y_zoh, _ = orc.scan(x, draw, A, B, C, zoh=True)
    y_fo, _ = orc.scan(x, draw, A, B, C)
    # outputs are sums of O(1) terms that may cancel, so the bound is absolute
    _close(y_zoh, y_fo, 0, 5e-6 * np.max(np.abs(y_fo)), "ZOH -> first order as A -> 0")
    # and they must differ at a finite A (so the test mode is really ZOH)
    A = -np.ones((dim, N))
    y_zoh, _ = orc.scan(x, draw, A, B, C, zoh=True)
    y_fo, _ = orc.scan(x, draw, A, B, C)
    if np.allclose(y_zoh, y_fo, rtol=1e-3):
        raise AssertionError("ZOH and first-order Bbar agree at A = -1")


# ---------------------------------------------------------------------------
# Structure: affine-pair scan, bounds, linearity, layout, decode == scan
# ---------------------------------------------------------------------------

def _tree_scan(pairs):
    """Inclusive scan of affine maps h -> a h + b by recursive halving with the
    combine (a1, b1) then (a2, b2) = (a2 a1, a2 b1 + b2) ("Mamba and selective
    state spaces", "The hardware-aware scan")."""
    n = len(pairs)
    if n == 1:
        return list(pairs)
    mid = n // 2
    left = _tree_scan(pairs[:mid])
    right = _tree_scan(pairs[mid:])
    a1, b1 = left[-1]
    return left + [(a2 * a1, a2 * b1 + b2) for (a2, b2) in right]


def pin_pair_scan(orc):
    """The oracle's sequential states equal an associative tree scan of the
    per-step affine pairs, for N = 16 and odd lengths."""
    rng = np.random.default_rng(16)
    batch, L, dim, N = 1, 37, 2, 16
    A = -rng.uniform(0.1, 3, size=(dim, N))
    x = rng.normal(size=(batch, L, dim))
    draw = rng.normal(-0.5, 1, size=(batch, L, dim))
    B = rng.normal(size=(batch, L, N))
    C = rng.normal(size=(batch, L, N))
    Delta = np.logaddexp(0.0, draw)
    y, last = orc.scan(x, draw, A, B, C)
    for d in range(dim):
        pairs = [(np.exp(Delta[0, t, d] * A[d]), Delta[0, t, d] * B[0, t] * x[0, t, d]) for t in range(L)]
        states = [bb for (_, bb) in _tree_scan(pairs)]          # h_t = b of the prefix (h_-1 = 0)
        want_y = np.array([np.dot(C[0, t], states[t]) for t in range(L)])
        _close(y[0, :, d], want_y, 1e-11, 1e-13, "tree scan outputs")
        _close(last[0, d], states[-1], 1e-11, 1e-13, "tree scan final state")


def pin_bounded(orc):
    """With A < 0 and Delta > 0 every Abar lies in (0, 1), so
    |h_{t,n}| <= sum_{s<=t} |Delta_s B_{s,n} x_s| ("Discretisation": each decay
    lies strictly between 0 and 1; "A state space model": the S4D-Real
    diagonal is stable)."""
    rng = np.random.default_rng(17)
    batch, L, dim, N = 2, 64, 5, 16
    A = -np.tile(np.arange(1, N + 1, dtype=np.float64), (dim, 1))
    x = rng.normal(size=(batch, L, dim))
    draw = rng.normal(0, 2, size=(batch, L, dim))
    B = rng.normal(size=(batch, L, N))
    C = rng.normal(size=(batch, L, N))
    Delta = np.logaddexp(0.0, draw)
    _, last = orc.scan(x, draw, A, B, C)
    bound = np.sum(np.abs(Delta[:, :, :, None] * B[:, :, None, :] * x[:, :, :, None]), axis=1)
    if not np.all(np.abs(last) <= bound * (1 + 1e-12)):
        raise AssertionError("state exceeds the sum-of-inputs bound")
    if not np.all(np.abs(last) > 0):
        raise AssertionError("state vanished although inputs are nonzero")


def pin_linearity_and_direct_term(orc):
    """Without the gate, and with Delta, B, C fixed, y is linear in x; setting D
    adds exactly D x ("State space models and Mamba", "One system, two views":
    D is a path from input to output that bypasses the state)."""
    rng = np.random.default_rng(18)
    batch, L, dim, N = 2, 30, 4, 16
    A = -rng.uniform(0.1, 2, size=(dim, N))
    x1 = rng.normal(size=(batch, L, dim))
    x2 = rng.normal(size=(batch, L, dim))
    draw = rng.normal(size=(batch, L, dim))
    B = rng.normal(size=(batch, L, N))
    C = rng.normal(size=(batch, L, N))
    D = rng.normal(size=dim)
    y1, h1 = orc.scan(x1, draw, A, B, C)
    y2, h2 = orc.scan(x2, draw, A, B, C)
    y12, h12 = orc.scan(x1 + 2 * x2, draw, A, B, C)
    _close(y12, y1 + 2 * y2, 1e-10, 1e-12, "linearity in x")
    _close(h12, h1 + 2 * h2, 1e-10, 1e-12, "state linearity in x")
    yD, _ = orc.scan(x1, draw, A, B, C, D=D)
    _close(yD - y1, D * x1, 1e-10, 1e-12, "direct term")


def pin_gate(orc):
    """The gate multiplies the whole SSM output, direct term included, by
    silu(z) = z sigmoid(z) ("Mamba and selective state spaces", "The Mamba
    block"). silu(0) = 0 and silu(z) -> z for large z."""
    rng = np.random.default_rng(19)
    batch, L, dim, N = 1, 20, 3, 16
    A = -rng.uniform(0.1, 2, size=(dim, N))
    x = rng.normal(size=(batch, L, dim))
    draw = rng.normal(size=(batch, L, dim))
    B = rng.normal(size=(batch, L, N))
    C = rng.normal(size=(batch, L, N))
    D = rng.normal(size=dim)
    z = rng.normal(0, 2, size=(batch, L, dim))
    y0, _ = orc.scan(x, draw, A, B, C, D=D)
    yz, _ = orc.scan(x, draw, A, B, C, D=D, z=z)
    _close(yz, y0 * z * _sigmoid(z), 1e-13, 1e-15, "gate = y * z * sigmoid(z)")
    y_zero, _ = orc.scan(x, draw, A, B, C, D=D, z=np.zeros_like(z))
    _close(y_zero, np.zeros_like(y0), 0, 0, "silu(0) = 0")
    y_big, _ = orc.scan(x, draw, A, B, C, D=D, z=np.full_like(z, 60.0))
    _close(y_big, 60.0 * y0, 1e-13, 1e-15, "silu(60) = 60")


def pin_rows_independent(orc):
    """Each (batch, channel) row is its own SSM; B and C belong to the batch
    row and are shared by all its channels; A, D and the bias belong to the
    channel (erikxu.me notes, "State Space Models", one SSM per dimension;
    "Mamba and selective state spaces", "Selection": B_t and C_t are N numbers
    per token). A multi-row call equals single-row calls on sliced inputs."""
    rng = np.random.default_rng(20)
    batch, L, dim, N = 3, 9, 5, 16
    A = -rng.uniform(0.1, 2, size=(dim, N))
    x = rng.normal(size=(batch, L, dim))
    draw = rng.normal(size=(batch, L, dim))
    B = rng.normal(size=(batch, L, N))
    C = rng.normal(size=(batch, L, N))
    D = rng.normal(size=dim)
    z = rng.normal(size=(batch, L, dim))
    bias = rng.normal(0, 0.5, size=dim)
    h0 = rng.normal(size=(batch, dim, N))
    y, last = orc.scan(x, draw, A, B, C, D=D, z=z, delta_bias=bias, h0=h0)
    for b in range(batch):
        for d in range(dim):
            sl = (slice(b, b + 1), slice(None), slice(d, d + 1))
            yy, hh = orc.scan(x[sl], draw[sl], A[d:d + 1], B[b:b + 1], C[b:b + 1], D=D[d:d + 1],
                              z=z[sl], delta_bias=bias[d:d + 1], h0=h0[b:b + 1, d:d + 1])
            _close(y[sl], yy, 0, 0, f"row ({b},{d}) output")
            _close(last[b, d], hh[0, 0], 0, 0, f"row ({b},{d}) final state")


def pin_initial_state(orc):
    """Unrolling from an initial state adds C Abar^t x_0 to the output
    ("State space models and Mamba", "One system, two views"): with a nonzero
    h0 the output is the zero-state output plus the read-out of the decayed
    initial state, C_t exp(A sum_{s<=t} Delta_s) h0."""
    rng = np.random.default_rng(21)
    batch, L, dim, N = 2, 15, 3, 16
    A = -rng.uniform(0.1, 2, size=(dim, N))
    x = rng.normal(size=(batch, L, dim))
    draw = rng.normal(-1, 1, size=(batch, L, dim))
    B = rng.normal(size=(batch, L, N))
    C = rng.normal(size=(batch, L, N))
    h0 = rng.normal(size=(batch, dim, N))
    Delta = np.logaddexp(0.0, draw)
    S = np.cumsum(Delta, axis=1)                                  # (b, t, d)
    decayed = np.exp(S[:, :, :, None] * A[None, None]) * h0[:, None]   # (b, t, d, n)
    y0, h_zero = orc.scan(x, draw, A, B, C)
    y, last = orc.scan(x, draw, A, B, C, h0=h0)
    _close(y - y0, np.einsum("btn,btdn->btd", C, decayed), 1e-10, 1e-12, "initial-state term")
    _close(last - h_zero, decayed[:, -1], 1e-10, 1e-12, "initial-state final")


def pin_decode_equals_scan(orc):
    """The one-token update is the scan's step: L updates from h = 0 equal
    the scan, and prefill(L) followed by one update equals prefill(L + 1)
    (erikxu.me notes, "State Space Models": constant work per new token from
    the carried state)."""
    rng = np.random.default_rng(22)
    batch, L, dim, N = 2, 10, 3, 16
    A = -rng.uniform(0.1, 2, size=(dim, N))
    x = rng.normal(size=(batch, L + 1, dim))
    draw = rng.normal(size=(batch, L + 1, dim))
    B = rng.normal(size=(batch, L + 1, N))
    C = rng.normal(size=(batch, L + 1, N))
    D = rng.normal(size=dim)
    z = rng.normal(size=(batch, L + 1, dim))
    bias = rng.normal(0, 0.5, size=dim)
    y_full, h_full = orc.scan(x, draw, A, B, C, D=D, z=z, delta_bias=bias)
    st = np.zeros((batch, dim, N))
    for t in range(L + 1):
        yt, st = orc.state_update(st, x[:, t], draw[:, t], A, B[:, t], C[:, t], D=D, z=z[:, t],
                                  delta_bias=bias)
        _close(yt, y_full[:, t], 1e-13, 1e-15, f"decode step {t}")
    _close(st, h_full, 1e-13, 1e-15, "decode final state")
    y_pre, h_pre = orc.scan(x[:, :L], draw[:, :L], A, B[:, :L], C[:, :L], D=D, z=z[:, :L],
                            delta_bias=bias)
    y1, h1 = orc.state_update(h_pre, x[:, L], draw[:, L], A, B[:, L], C[:, L], D=D, z=z[:, L],
                              delta_bias=bias)
    _close(y1, y_full[:, L], 1e-13, 1e-15, "prefill + decode")
    _close(h1, h_full, 1e-13, 1e-15, "prefill + decode state")


# ---------------------------------------------------------------------------
# Gradients (the backward pass)
# ---------------------------------------------------------------------------

def _bwd_problem(seed, batch=2, L=7, dim=3, N=4):
    rng = np.random.default_rng(seed)
    p = dict(x=rng.normal(size=(batch, L, dim)), delta=rng.normal(size=(batch, L, dim)),
             A=-rng.uniform(0.2, 2, (dim, N)), B=rng.normal(size=(batch, L, N)),
             C=rng.normal(size=(batch, L, N)), D=rng.normal(size=dim), z=rng.normal(size=(batch, L, dim)),
             delta_bias=rng.normal(0, .5, dim), h0=rng.normal(size=(batch, dim, N)))
    dout = rng.normal(size=(batch, L, dim))
    dlast = rng.normal(size=(batch, dim, N))
    return p, dout, dlast, rng


def pin_bwd_finite_differences(orc):
    """Every gradient agrees with central differences of the forward oracle:
    d/dtheta of sum(dout * y) + sum(dlast * last_state)."""
    _bwd_fd_check(orc, 41, gated=True)


def pin_bwd_finite_differences_bare(orc):
    """The same without gate, D, bias, initial state or final-state gradient;
    then also dz = 0, dD = sum dout x and dbias = sum ddelta."""
    _bwd_fd_check(orc, 43, gated=False)


def _bwd_fd_check(orc, seed, gated):
    p, dout, dlast, rng = _bwd_problem(seed)
    if not gated:
        for k in ("D", "z", "delta_bias", "h0"):
            p[k] = None
        dlast = None

    def loss(**kw):
        a = dict(p)
        a.update(kw)
        y, last = orc.scan(a["x"], a["delta"], a["A"], a["B"], a["C"], D=a["D"], z=a["z"],
                           delta_bias=a["delta_bias"], h0=a["h0"])
        return float((y * dout).sum() + (0.0 if dlast is None else (last * dlast).sum()))

    g = orc.scan_bwd(p["x"], p["delta"], p["A"], p["B"], p["C"], dout, D=p["D"], z=p["z"],
                     delta_bias=p["delta_bias"], h0=p["h0"], dlast=dlast)
    if not gated:
        _close(g["dz"], np.zeros_like(g["dz"]), 0, 0, "dz without a gate")
        _close(g["dD"], (dout * p["x"]).sum(axis=(0, 1)), 1e-13, 1e-14, "dD without a gate")
        _close(g["dbias"], g["ddelta"].sum(axis=(0, 1)), 1e-12, 1e-14, "dbias = sum ddelta")
    eps = 1e-6
    for name, gk in [("x", "dx"), ("delta", "ddelta"), ("A", "dA"), ("B", "dB"), ("C", "dC"),
                     ("D", "dD"), ("z", "dz"), ("delta_bias", "dbias"), ("h0", "dh0")]:
        arr = p[name]
        if arr is None:
            continue
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            hi, lo = arr.copy(), arr.copy()
            hi[idx] += eps
            lo[idx] -= eps
            fd = (loss(**{name: hi}) - loss(**{name: lo})) / (2 * eps)
            _close(g[gk][idx], fd, 1e-5, 1e-7, f"d{name}{idx}")


def pin_bwd_readout_only(orc):
    """With C = 0 and no final-state gradient nothing flows into the state:
    dA = dB = ddelta = dh0 = 0, dx = D ds, dD = sum ds x, dbias = 0, and
    dC = sum_d ds h (the states themselves, from the forward)."""
    p, dout, _, _ = _bwd_problem(42)
    C = np.zeros_like(p["C"])
    g = orc.scan_bwd(p["x"], p["delta"], p["A"], p["B"], C, dout, D=p["D"], z=p["z"],
                     delta_bias=p["delta_bias"], h0=p["h0"])
    ds = dout * _silu(p["z"])
    for k in ("dA", "dB", "ddelta", "dh0", "dbias"):
        _close(g[k], np.zeros_like(g[k]), 0, 0, k)
    _close(g["dx"], p["D"] * ds, 1e-14, 1e-15, "dx = D ds")
    _close(g["dD"], (ds * p["x"]).sum(axis=(0, 1)), 1e-13, 1e-14, "dD")
    # the states: scan with C = e_n reads state n out as y (no D, no gate)
    batch, L, dim = p["x"].shape
    N = p["A"].shape[1]
    want = np.zeros((batch, L, N))
    for n in range(N):
        e = np.zeros((batch, L, N))
        e[:, :, n] = 1.0
        h_n, _ = orc.scan(p["x"], p["delta"], p["A"], p["B"], e, delta_bias=p["delta_bias"],
                          h0=p["h0"])
        want[:, :, n] = (ds * h_n).sum(axis=2)
    _close(g["dC"], want, 1e-12, 1e-13, "dC")


def pin_groups_decompose(orc):
    """Channels in G groups, each group with its own B_t, C_t: the scan, the
    one-token update and every gradient equal G single-group problems on the
    channel slices (rows never mix; a group's B and C reach only its
    channels)."""
    rng = np.random.default_rng(51)
    batch, L, dim, N, G = 2, 9, 6, 4, 3
    per = dim // G
    x, delta, z = rng.normal(size=(3, batch, L, dim))
    A = -rng.uniform(0.2, 2, (dim, N))
    B = rng.normal(size=(batch, L, G, N))
    C = rng.normal(size=(batch, L, G, N))
    D = rng.normal(size=dim)
    bias = rng.normal(0, .5, dim)
    h0 = rng.normal(size=(batch, dim, N))
    dout = rng.normal(size=(batch, L, dim))
    dlast = rng.normal(size=(batch, dim, N))
    y, last = orc.scan(x, delta, A, B, C, D=D, z=z, delta_bias=bias, h0=h0)
    g = orc.scan_bwd(x, delta, A, B, C, dout, D=D, z=z, delta_bias=bias, h0=h0, dlast=dlast)
    st = h0.copy()
    ys_dec = []
    for t in range(3):
        o, st = orc.state_update(st, x[:, t], delta[:, t], A, B[:, t], C[:, t], D=D, z=z[:, t],
                                 delta_bias=bias)
        ys_dec.append(o)
    for k in range(G):
        sl = slice(k * per, (k + 1) * per)
        ys, ls = orc.scan(x[:, :, sl], delta[:, :, sl], A[sl], B[:, :, k], C[:, :, k], D=D[sl],
                          z=z[:, :, sl], delta_bias=bias[sl], h0=h0[:, sl])
        _close(y[:, :, sl], ys, 1e-15, 1e-15, f"group {k} y")
        _close(last[:, sl], ls, 1e-15, 1e-15, f"group {k} last state")
        gs = orc.scan_bwd(x[:, :, sl], delta[:, :, sl], A[sl], B[:, :, k], C[:, :, k], dout[:, :, sl],
                          D=D[sl], z=z[:, :, sl], delta_bias=bias[sl], h0=h0[:, sl],
                          dlast=dlast[:, sl])
        for key in ("dx", "ddelta", "dz"):
            _close(g[key][:, :, sl], gs[key], 1e-13, 1e-15, f"group {k} {key}")
        for key in ("dA", "dD", "dbias"):
            _close(g[key][sl], gs[key], 1e-13, 1e-15, f"group {k} {key}")
        _close(g["dh0"][:, sl], gs["dh0"], 1e-13, 1e-15, f"group {k} dh0")
        _close(g["dB"][:, :, k], gs["dB"], 1e-13, 1e-15, f"group {k} dB")
        _close(g["dC"][:, :, k], gs["dC"], 1e-13, 1e-15, f"group {k} dC")
        sts = h0[:, sl].copy()
        for t in range(3):
            o, sts = orc.state_update(sts, x[:, t, sl], delta[:, t, sl], A[sl], B[:, t, k],
                                      C[:, t, k], D=D[sl], z=z[:, t, sl], delta_bias=bias[sl])
            _close(ys_dec[t][:, sl], o, 1e-15, 1e-15, f"group {k} decode step {t}")
        _close(st[:, sl], sts, 1e-15, 1e-15, f"group {k} decode state")


BWD_PINS = [pin_bwd_finite_differences, pin_bwd_finite_differences_bare, pin_bwd_readout_only,
            pin_groups_decompose]


# ---------------------------------------------------------------------------
# Mamba-2 SSD (ai.thesatyajit.com, "Mamba and selective state spaces, from
# first principles", section "Mamba-2: state space duality")
# ---------------------------------------------------------------------------

def _ssd_problem(seed, batch=2, L=11, H=4, P=3, N=5, G=2):
    rng = np.random.default_rng(seed)
    return dict(x=rng.normal(size=(batch, L, H, P)), dt=rng.normal(size=(batch, L, H)),
                A=-rng.uniform(0.2, 2, H), B=rng.normal(size=(batch, L, G, N)),
                C=rng.normal(size=(batch, L, G, N)), D=rng.normal(size=H),
                dt_bias=rng.normal(0, .5, H), h0=rng.normal(size=(batch, H, N, P)))


def pin_ssd_is_s6_with_scalar_decay(orc):
    """SSD is the S6 layer whose states all decay at their head's rate: the S6
    oracle on H * P channels, with A[d, n] = A_h for every n, the head's
    Delta_raw, bias and D on each of its channels, and B, C in groups of
    heads, gives the same outputs and states (the S6 state h[d, n] of channel
    d = h * P + p is S[h][n, p])."""
    q = _ssd_problem(61)
    batch, L, H, P = q["x"].shape
    N = q["B"].shape[3]
    y, last = orc.ssd(q["x"], q["dt"], q["A"], q["B"], q["C"], D=q["D"], dt_bias=q["dt_bias"],
                      h0=q["h0"])
    rep = lambda v: np.repeat(v, P, axis=-1)
    y6, last6 = orc.scan(q["x"].reshape(batch, L, H * P), rep(q["dt"]),
                         np.repeat(q["A"], P)[:, None] * np.ones((1, N)), q["B"], q["C"],
                         D=rep(q["D"]), delta_bias=rep(q["dt_bias"]),
                         h0=q["h0"].transpose(0, 1, 3, 2).reshape(batch, H * P, N))
    _close(y.reshape(batch, L, H * P), y6, 1e-13, 1e-15, "SSD = S6 with scalar decay (y)")
    _close(last.transpose(0, 1, 3, 2).reshape(batch, H * P, N), last6, 1e-13, 1e-15,
           "SSD = S6 with scalar decay (state)")


def pin_ssd_dual_form(orc):
    """Unrolled, the layer is one masked matrix product (the duality): with C
    as queries, B as keys and Delta x as values, y = (L o C B^T)(Delta x) +
    D x, where L[t, s] = exp(A_h sum_{u=s+1..t} Delta_u) on and below the
    diagonal and 0 above it (a decay mask in place of the softmax)."""
    q = _ssd_problem(62)
    batch, L, H, P = q["x"].shape
    G = q["B"].shape[2]
    y, _ = orc.ssd(q["x"], q["dt"], q["A"], q["B"], q["C"], D=q["D"], dt_bias=q["dt_bias"])
    for b in range(batch):
        for h in range(H):
            g = h // (H // G)
            Dl = np.logaddexp(0.0, q["dt"][b, :, h] + q["dt_bias"][h])   # softplus
            cum = np.cumsum(Dl * q["A"][h])
            mask = np.tril(np.exp(cum[:, None] - cum[None, :]))
            scores = q["C"][b, :, g] @ q["B"][b, :, g].T
            want = (mask * scores) @ (Dl[:, None] * q["x"][b, :, h]) + q["D"][h] * q["x"][b, :, h]
            _close(y[b, :, h], want, 1e-12, 1e-14, f"SSD dual form b={b} h={h}")


SSD_PINS = [pin_ssd_is_s6_with_scalar_decay, pin_ssd_dual_form]


# ---------------------------------------------------------------------------
# Causal depthwise convolution + SiLU (the SSM branch's front-end:
# ai.thesatyajit.com, "The Mamba block"; erikxu.me notes, "Mamba")
# ---------------------------------------------------------------------------

def _silu(v):
    return v * _sigmoid(v)


def pin_conv_impulse(orc):
    """A unit impulse at t0 in one channel gives silu(bias + w[W-1-k]) at
    t0 + k for k < W and silu(bias) elsewhere: the current input meets the
    last tap, and the filter never looks ahead (causal)."""
    W, L, t0 = 4, 12, 5
    w = np.array([[0.5, -1.5, 2.0, 3.0], [0.25, 0.5, -0.75, 1.25]])
    bias = np.array([0.0, -0.3])
    x = np.zeros((1, L, 2))
    x[0, t0, 1] = 1.0
    out, _ = orc.conv1d(x, w, bias)
    want = np.full(L, _silu(bias[1]))
    for k in range(W):
        want[t0 + k] = _silu(bias[1] + w[1, W - 1 - k])
    _close(out[0, :, 1], want, 1e-15, 1e-15, "impulse, channel 1")
    _close(out[0, :, 0], np.zeros(L), 0, 0, "silent channel")


def pin_conv_matches_library_convolution(orc):
    """Per channel, the pre-activation is numpy's full discrete convolution of
    the input with the reversed taps, truncated to the first L outputs."""
    rng = np.random.default_rng(31)
    for W in (4, 3, 2, 1):
        x = rng.normal(size=(2, 37, 5))
        w = rng.normal(size=(5, W))
        bias = rng.normal(size=5)
        out, _ = orc.conv1d(x, w, bias)
        want = np.empty_like(out)
        for b in range(2):
            for d in range(5):
                pre = np.convolve(x[b, :, d], w[d, ::-1])[:37] + bias[d]
                want[b, :, d] = _silu(pre)
        _close(out, want, 1e-13, 1e-14, f"np.convolve, width {W}")


def pin_conv_pieces(orc):
    """A sequence convolved in pieces, each starting from the previous piece's
    state (its last W - 1 inputs), gives the one-piece result."""
    rng = np.random.default_rng(32)
    x = rng.normal(size=(2, 40, 6))
    w = rng.normal(size=(6, 4))
    bias = rng.normal(size=6)
    s0 = rng.normal(size=(2, 6, 3))
    whole, s_whole = orc.conv1d(x, w, bias, state_in=s0)
    outs, st = [], s0
    for a, b in [(0, 1), (1, 2), (2, 17), (17, 40)]:
        o, st = orc.conv1d(x[:, a:b], w, bias, state_in=st)
        outs.append(o)
    _close(np.concatenate(outs, axis=1), whole, 1e-14, 1e-15, "pieces")
    _close(st, s_whole, 0, 0, "final state")
    _close(s_whole, x[:, -3:].transpose(0, 2, 1), 0, 0, "state = last three inputs")


def pin_conv_short_sequence_state(orc):
    """With fewer than W - 1 new inputs the returned state still holds the
    last W - 1 inputs overall, oldest first: the older ones from the given
    state, then the new ones."""
    rng = np.random.default_rng(33)
    s0 = rng.normal(size=(1, 3, 3))
    x = rng.normal(size=(1, 2, 3))
    _, st = orc.conv1d(x, rng.normal(size=(3, 4)), state_in=s0)
    want = np.concatenate([s0, x.transpose(0, 2, 1)], axis=2)[:, :, -3:]
    _close(st, want, 0, 0, "short-sequence state")
    _, st0 = orc.conv1d(np.zeros((1, 0, 3)), rng.normal(size=(3, 4)), state_in=s0)
    _close(st0, s0, 0, 0, "empty sequence keeps the state")


def pin_conv_update_equals_conv(orc):
    """The one-token update (state shift register) applied L times gives the
    sequence convolution and its final state."""
    rng = np.random.default_rng(34)
    x = rng.normal(size=(3, 9, 4))
    w = rng.normal(size=(4, 4))
    bias = rng.normal(size=4)
    s0 = rng.normal(size=(3, 4, 3))
    whole, s_whole = orc.conv1d(x, w, bias, state_in=s0)
    st = s0
    for t in range(9):
        o, st = orc.conv1d_update(st, x[:, t], w, bias)
        _close(o, whole[:, t], 1e-14, 1e-15, f"update step {t}")
    _close(st, s_whole, 0, 0, "update final state")


CONV_PINS = [
    pin_conv_impulse,
    pin_conv_matches_library_convolution,
    pin_conv_pieces,
    pin_conv_short_sequence_state,
    pin_conv_update_equals_conv,
]


ALL_PINS = SSD_PINS + [
    pin_worked_example,
    pin_gated_rnn,
    pin_lti_convolution,
    pin_write_then_read,
    pin_impulse_per_state,
    pin_degenerate_A,
    pin_zoh_small_A_limit,
    pin_pair_scan,
    pin_bounded,
    pin_linearity_and_direct_term,
    pin_gate,
    pin_rows_independent,
    pin_initial_state,
    pin_decode_equals_scan,
] + CONV_PINS + BWD_PINS
