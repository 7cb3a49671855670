"""CPU-only pins of the fp64 oracle (no GPU involved).

The second half plants mistakes in copies of the oracle source (a dropped
term, a wrong sign, a transposed operand, an exclusive mask ...) and checks
that the pins catch every one of them.
"""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

import oracle
from tests import oracle_checks as oc


@pytest.mark.parametrize("check", oc.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, check):
    check(orc)


# (name, exact source text, replacement, the checks that must catch it)
MUTATIONS = [
    ("phi_drops_plus_one", "return x > 0.0 ? x + 1.0 : exp(x); }", "return x > 0.0 ? x + 0.0 : exp(x); }",
     [oc.check_phi, oc.check_forward_exact]),
    ("dphi_wrong_branch", "return x > 0.0 ? 1.0 : exp(x); }", "return x > 0.0 ? 1.0 : 1.0; }",
     [oc.check_backward_vs_quadratic, oc.check_backward_fd]),
    ("state_update_uses_query", "for (int64_t m = 0; m < M; ++m) S[d * M + m] += kh[d] * V[i * M + m];\n                Z[d] += kh[d];\n            }\n            /* readout */",
     "for (int64_t m = 0; m < M; ++m) S[d * M + m] += qh[d] * V[i * M + m];\n                Z[d] += kh[d];\n            }\n            /* readout */",
     [oc.check_forward_vs_brute, oc.check_invariants]),
    ("normalizer_counts_tokens", "                Z[d] += kh[d];\n            }\n            /* readout */",
     "                Z[d] += 1.0;\n            }\n            /* readout */",
     [oc.check_forward_vs_brute, oc.check_closed_forms]),
    ("exclusive_causal_mask", "            /* readout */\n            double dd = 0.0;",
     "            /* readout */\n            for (int64_t d = 0; d < D; ++d) { Z[d] -= kh[d]; for (int64_t m = 0; m < M; ++m) S[d * M + m] -= kh[d] * V[i * M + m]; }\n            double dd = 0.0;",
     [oc.check_forward_vs_brute, oc.check_closed_forms]),
    ("readout_transposed_index", "for (int64_t d = 0; d < D; ++d) n += qh[d] * S[d * M + m];\n                O[i * M + m] = n / dd;\n            }\n            if (den)",
     "for (int64_t d = 0; d < D; ++d) n += qh[d] * S[(d * M + m) % (D * M) == 0 ? 0 : (m * D + d) % (D * M)];\n                O[i * M + m] = n / dd;\n            }\n            if (den)",
     [oc.check_forward_vs_brute]),
    ("noncausal_drops_key_feature_map", "double kd = phi(K[j * D + d]);", "double kd = K[j * D + d];",
     [oc.check_forward_vs_brute, oc.check_invariants]),
    ("backward_drops_normalizer_term", "double acc = h[i] * Z[d];", "double acc = 0.0 * Z[d];",
     [oc.check_backward_vs_quadratic, oc.check_backward_identities]),
    ("backward_sign_of_h", "h[i] = -go / dd;", "h[i] = go / dd;",
     [oc.check_backward_vs_quadratic, oc.check_backward_fd]),
    ("backward_dv_uses_query", "for (int64_t d = 0; d < D; ++d) acc += S[d * M + m] * kh[d];",
     "for (int64_t d = 0; d < D; ++d) acc += S[d * M + m] * qh[d];",
     [oc.check_backward_vs_quadratic, oc.check_backward_autograd]),
    ("backward_reverse_sum_misses_u", "Z[d] += h[j] * qh[d];", "Z[d] += h[j] * kh[d];",
     [oc.check_backward_vs_quadratic, oc.check_backward_identities]),
    ("decode_normalizer_uses_key", "dd += phi(qq[d]) * ZZ[d];", "dd += phi(kk[d]) * ZZ[d];",
     [oc.check_decode]),
    ("forward_drops_initial_z",
     "if (Z_io) memcpy(Z, Z_io + bh * D, (size_t)D * sizeof(double));",
     "if (Z_io && N < 0) memcpy(Z, Z_io + bh * D, (size_t)D * sizeof(double));",
     [oc.check_initial_state]),
    ("noncausal_backward_drops_u",
     "                double acc = u[d];",
     "                double acc = 0.0 * u[d];",
     [oc.check_backward_noncausal]),
    ("noncausal_backward_h_sign",
     "            const double h = -go / dd;",
     "            const double h = go / dd;",
     [oc.check_backward_noncausal]),
    ("rff_sin_for_cos",
     "out[i * R + r] = scale * cos(a);",
     "out[i * R + r] = scale * sin(a);",
     [oc.check_rff_worked_example, oc.check_rff_estimates_rbf_kernel]),
    ("rff_omega_transposed",
     "for (int64_t d = 0; d < D; ++d) a += x[i * D + d] * omega[d * R + r];",
     "for (int64_t d = 0; d < D; ++d) a += x[i * D + d] * omega[(r % D) * R + d];",
     [oc.check_rff_worked_example, oc.check_rff_estimates_rbf_kernel]),
    ("rff_scale_1_over_r",
     "const double scale = sqrt(2.0 / (double)R);",
     "const double scale = 2.0 / (double)R;",
     [oc.check_rff_worked_example, oc.check_rff_estimates_rbf_kernel]),
    ("features_forward_reads_before_update",
     "for (int64_t m = 0; m < M; ++m) S[f * M + m] += K[i * F + f] * V[i * M + m];",
     "for (int64_t m = 0; m < M; ++m) S[f * M + m] += (i > 0) * K[(i - (i > 0)) * F + f] * V[(i - (i > 0)) * M + m];",
     [oc.check_forward_features]),
    ("poly2_diagonal_features_only",
     "pk[a * D + b] = K[i * D + a] * K[i * D + b];",
     "pk[a * D + b] = (a == b) * K[i * D + a] * K[i * D + b];",
     [oc.check_poly2]),
    ("poly2_query_features_from_keys",
     "pq[a * D + b] = Q[i * D + a] * Q[i * D + b];",
     "pq[a * D + b] = Q[i * D + a] * K[i * D + b];",
     [oc.check_poly2]),
    ("poly2_backward_drops_factor_two",
     "dQ[i * D + a] += e * 2.0 * dot * kj[a];",
     "dQ[i * D + a] += e * dot * kj[a];",
     [oc.check_poly2_backward]),
    ("poly2_backward_drops_output_term",
     "const double e = (gv - go) / den;",
     "const double e = (gv - 0.0 * go) / den;",
     [oc.check_poly2_backward]),
    ("poly2_backward_dv_unsquared",
     "for (int64_t m = 0; m < M; ++m) dV[j * M + m] += dot * dot * gi[m] / den;",
     "for (int64_t m = 0; m < M; ++m) dV[j * M + m] += dot * gi[m] / den;",
     [oc.check_poly2_backward]),
    ("poly2_backward_dk_uses_key",
     "dK[j * D + a] += e * 2.0 * dot * qi[a];",
     "dK[j * D + a] += e * 2.0 * dot * kj[a];",
     [oc.check_poly2_backward]),
    ("decode_reads_before_update_of_s",
     "for (int64_t m = 0; m < M; ++m) SS[d * M + m] += kd * vv[m];",
     "for (int64_t m = 0; m < M; ++m) SS[d * M + m] += kd * vv[m] * (m > 0);",
     [oc.check_decode]),
]


@pytest.fixture(scope="module")
def oracle_src():
    with open(os.path.join(os.path.dirname(oracle.__file__), "la_oracle.c")) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new,checks", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tmp_path, oracle_src, name, old, new, checks):
    assert oracle_src.count(old) == 1, f"mutation anchor for {name} not unique/present"
    src = tmp_path / f"{name}.c"
    src.write_text(oracle_src.replace(old, new))
    so = tmp_path / f"{name}.so"
    oracle.build(str(src), str(so))
    lib = oracle.load(str(so))
    caught = []
    for check in checks:
        try:
            check(lib)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"planted mistake {name} went unnoticed by {[c.__name__ for c in checks]}"


def test_oracle_builds_with_warnings_as_errors(tmp_path):
    src = os.path.join(os.path.dirname(oracle.__file__), "la_oracle.c")
    subprocess.run(["gcc", "-O2", "-Wall", "-Wextra", "-Werror", "-fopenmp", "-fsyntax-only", src], check=True)
