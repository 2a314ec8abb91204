"""CPU test: the pins are sharp enough to catch plausible mistakes in the oracle.

Each mutation below is a small, plausible slip (a dropped term, a wrong sign,
a wrong index, a transposed operand, an off-by-one in time). The test applies
it to a copy of ``oracle/ssm_oracle.c`` in a temporary directory, compiles the
copy, runs every pin against it in a child process (a mutant may index badly,
so it must not share this process), and requires at least one pin to fail
(a crash does not count: the pins themselves must reject the mutant).
The real oracle source is never modified.
"""
import json
import os
import subprocess
import sys
import textwrap

import pytest

from oracle.oracle import ORACLE_SRC, build_oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, exact text in ssm_oracle.c, replacement)
MUTATIONS = [
    ("softplus_pos_branch", "if (u > 0.0) return u + log1p(exp(-u));", "if (u > 0.0) return u;"),
    ("softplus_neg_branch", "return log1p(exp(u));", "return exp(u);"),
    ("euler_decay", "double abar = exp(Delta * A_d[n]);", "double abar = 1.0 + Delta * A_d[n];"),
    ("bbar_without_delta", "bbar = Delta * B_t[n];", "bbar = B_t[n];"),
    ("no_decay", "h[n] = abar * h[n] + bbar * x;", "h[n] = h[n] + bbar * x;"),
    ("readout_with_B", "y += C_t[n] * h[n];", "y += B_t[n] * h[n];"),
    ("drop_D", "if (D_d) y += (*D_d) * x;", ""),
    ("drop_gate", "if (z) y *= silu(*z);", ""),
    ("drop_bias", "double Delta = softplus(delta_raw + bias);", "double Delta = softplus(delta_raw);"),
    ("A_row_index", "A + d * dstate,\n                          B + j", "A + d,\n                          B + j"),
    ("nonzero_init", "h0[(b * dim + d) * dstate + n] : 0.0;", "h0[(b * dim + d) * dstate + n] : 1.0;"),
    ("BC_time_off_by_one", "int64_t j = ((b * seqlen + t) * ngroups + g) * dstate;",
     "int64_t j = ((b * seqlen + (t > 0 ? t - 1 : t)) * ngroups + g) * dstate;"),
    ("sigmoid_sign", "return v / (1.0 + exp(-v));", "return v / (1.0 + exp(v));"),
    ("readout_before_update", "h[n] = abar * h[n] + bbar * x;\n    y += C_t[n] * h[n];",
     "y += C_t[n] * h[n];\n    h[n] = abar * h[n] + bbar * x;"),
    ("gate_before_D", "if (D_d) y += (*D_d) * x;\n  if (z) y *= silu(*z);",
     "if (z) y *= silu(*z);\n  if (D_d) y += (*D_d) * x;"),
    ("zoh_sign", "bbar = (abar - 1.0) / A_d[n] * B_t[n];", "bbar = (1.0 - abar) / A_d[n] * B_t[n];"),
    ("decode_state_row", "out[i] = row_step(dstate, state + i * dstate",
     "out[i] = row_step(dstate, state + d * dstate"),
    ("decode_BC_swap", "B + j, C + j, D ? D + d : NULL,\n", "C + j, B + j, D ? D + d : NULL,\n"),
    ("last_state_layout", "last_state[(b * dim + d) * dstate + n] = h[n];",
     "last_state[(d * batch + b) * dstate + n] = h[n];"),
    ("x_layout", "int64_t i = (b * seqlen + t) * dim + d;   /* (b, t, d) */",
     "int64_t i = (t * batch + b) * dim + d;"),
    ("decay_uses_bias_free_delta", "double abar = exp(Delta * A_d[n]);",
     "double abar = exp(softplus(delta_raw) * A_d[n]);"),
    # backward pass
    ("bwd_no_adjoint_decay", "          lam[n] *= abar;\n", ""),
    ("bwd_dC_previous_state", "pC[j + n] += ds * hs[(t + 1) * N + n];", "pC[j + n] += ds * hs[t * N + n];"),
    ("bwd_dB_without_delta", "pB[j + n] += lam[n] * Dl * xt;", "pB[j + n] += lam[n] * xt;"),
    ("bwd_dA_without_abar", "dA_acc[n] += lam[n] * Dl * abar * hprev;", "dA_acc[n] += lam[n] * Dl * hprev;"),
    ("bwd_dx_without_D", "double dDl = 0.0, dxt = D ? D[d] * ds : 0.0;", "double dDl = 0.0, dxt = 0.0;"),
    ("bwd_softplus_grad_sign", "ddelta[i] = dDl * sigmoid(u);", "ddelta[i] = dDl * sigmoid(-u);"),
    ("scan_group_index", "int64_t j = ((b * seqlen + t) * ngroups + g) * dstate;",
     "int64_t j = ((b * seqlen + t) * ngroups + d % ngroups) * dstate;"),
    ("decode_group_index", "int64_t j = (b * ngroups + d / per_group) * dstate;",
     "int64_t j = (b * ngroups + d % ngroups) * dstate;"),
    ("bwd_group_index",
     "const int64_t i = (b * L + t) * dim + d, j = ((b * L + t) * G + d / per_group) * N;\n        const double u",
     "const int64_t i = (b * L + t) * dim + d, j = ((b * L + t) * G + d % G) * N;\n        const double u"),
    ("ssd_input_without_delta", "S[n * P + p] = a * S[n * P + p] + Delta * Bt[n] * xt[p];",
     "S[n * P + p] = a * S[n * P + p] + Bt[n] * xt[p];"),
    ("ssd_head_group", "const int64_t g = h / per_group;", "const int64_t g = h % G;"),
    ("ssd_readout_B", "y += Ct[n] * S[n * P + p];", "y += Bt[n] * S[n * P + p];"),
    ("ssd_decay_sign", "const double a = exp(Delta * A[h]);", "const double a = exp(-Delta * A[h]);"),
    ("bwd_dz_silu_grad", "dz[i] = dout[i] * s * sg * (1.0 + z[i] * (1.0 - sg));",
     "dz[i] = dout[i] * s * sg;"),
    ("bwd_dlast_dropped", "lam[n] = dlast ? dlast[(b * dim + d) * N + n] : 0.0;", "lam[n] = 0.0;"),
    ("bwd_ddelta_misses_input_term", "dDl += lam[n] * (A_d[n] * abar * hprev + xt * B[j + n]);",
     "dDl += lam[n] * (A_d[n] * abar * hprev);"),
    # causal convolution front-end
    ("conv_taps_reversed", "v += weight[d * width + j] *", "v += weight[d * width + (width - 1 - j)] *"),
    ("conv_drop_bias", "double v = bias ? bias[d] : 0.0;\n        for (int64_t j = 0; j < width; ++j)",
     "double v = 0.0;\n        for (int64_t j = 0; j < width; ++j)"),
    ("conv_no_silu", "out[(b * seqlen + t) * dim + d] = silu(v);", "out[(b * seqlen + t) * dim + d] = v;"),
    ("conv_state_out_offset", "conv_input(xin, state_in, seqlen, dim, width, b, d, seqlen - (width - 1) + j);",
     "conv_input(xin, state_in, seqlen, dim, width, b, d, seqlen - width + j);"),
    ("conv_state_in_reversed", "return state_in[(b * dim + d) * (width - 1) + (width - 1) + t];",
     "return state_in[(b * dim + d) * (width - 1) + (-1 - t)];"),
    ("conv_update_shift_direction", "for (int64_t j = 0; j + 1 < width - 1; ++j) s[j] = s[j + 1];",
     "for (int64_t j = width - 3; j >= 0; --j) s[j + 1] = s[j];"),
    ("conv_update_new_input_tap", "v += w[width - 1] * xin[b * dim + d];", "v += w[0] * xin[b * dim + d];"),
    ("conv_update_drops_bias", "double v = bias ? bias[d] : 0.0;\n      for (int64_t j = 0; j < width - 1; ++j)",
     "double v = 0.0;\n      for (int64_t j = 0; j < width - 1; ++j)"),
]

RUNNER = textwrap.dedent("""
    import json, sys
    sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
    from oracle.oracle import Oracle
    import pins
    orc = Oracle({lib!r})
    failed = []
    for p in pins.ALL_PINS:
        try:
            p(orc)
        except Exception as e:  # AssertionError, or a rejected call
            failed.append(p.__name__)
    print(json.dumps(failed))
""")


def test_mutation_list_applies_once():
    src = open(ORACLE_SRC).read()
    for name, old, new in MUTATIONS:
        assert src.count(old) == 1, f"mutation {name}: pattern occurs {src.count(old)} times"


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1
    mut_src = tmp_path / "ssm_oracle_mutant.c"
    mut_src.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    build_oracle(str(mut_src), str(lib))
    code = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=str(lib))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"mutant {name} crashed instead of failing a pin:\n{r.stderr[-2000:]}"
    failed = json.loads(r.stdout.strip().splitlines()[-1])
    assert failed, f"mutant {name} passed every pin"
