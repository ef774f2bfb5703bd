"""Sensitivity of the pins: each plausible mistake planted in a copy of the oracle
(on the CPU, never in the GPU path) must fail at least one pin."""
import os

import pytest

import oracle
from oracle_backward_pins import BACKWARD_PINS
from oracle_pins import PINS

# (name, text in l3_oracle.c, replacement)
MUTANTS = [
    ("score_index_shift", "acc += kr[c] * x[c];", "acc += kr[c] * x[(c + 1) % d_in];"),
    ("no_softmax_normalisation", "for (int64_t j = 0; j < d; ++j) s[j] /= z;", "(void)z;"),
    ("softmax_sign", "s[j] = exp(s[j] - mx);", "s[j] = exp(mx - s[j]);"),
    ("value_row_off_by_one", "const double *vr = WV + (a + j) * d_emb;",
     "const double *vr = WV + ((a + j + 1) % v_rows) * d_emb;"),
    ("drop_last_row", "const int64_t d = off[t + 1] - off[t];",
     "const int64_t d = off[t + 1] - off[t] > 1 ? off[t + 1] - off[t] - 1 : 1;"),
    ("w_up_transposed", "acc += wr[c] * o[c];", "acc += Wup[c * d_up + r] * o[c];"),
    ("unbiased_variance", "var /= (double)d_up;", "var /= (double)(d_up - 1);"),
    ("eps_outside_sqrt", "1.0 / sqrt(var + eps);", "1.0 / (sqrt(var) + eps);"),
    ("gamma_beta_swapped", "* inv * gamma[r] + beta[r];", "* inv * beta[r] + gamma[r];"),
    ("concat_order", "acc += wr[r] * y[r];", "acc += wr[d_in + r] * y[r];"),
    ("no_residual_term", "acc += wr[d_up + c] * x[c];", "(void)c;"),
    ("mean_not_subtracted", "var += (h[r] - mean) * (h[r] - mean);", "var += h[r] * h[r];"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    mutated = src.replace(old, new)
    if "v_rows" in new:
        mutated = mutated.replace("static void l3o_token(", "static int64_t v_rows = 1;\nstatic void l3o_token(", 1)
        mutated = mutated.replace("    int rc = l3o_check_offsets(off, vocab, v, k);",
                                  "    v_rows = v;\n    int rc = l3o_check_offsets(off, vocab, v, k);", 1)
    p = tmp_path / f"{name}.c"
    p.write_text(mutated)
    so = oracle.build(str(p), str(tmp_path / f"lib{name}.so"))
    lib = oracle.load(so)
    failed = []
    for pin in PINS:
        try:
            pin(lib)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"


# mistakes in the backward pass, each of which must fail a backward pin
BACKWARD_MUTANTS = [
    ("bwd_no_softmax_centering", "const double ds = p[j] * (dp[j] - pdp);",
     "const double ds = p[j] * dp[j];"),
    ("bwd_ln_no_mean_term", "dh[r] = rstd * (dy[r] * gamma[r] - mg - yh[r] * mgy);",
     "dh[r] = rstd * (dy[r] * gamma[r] - yh[r] * mgy);"),
    ("bwd_ln_no_projection_term", "dh[r] = rstd * (dy[r] * gamma[r] - mg - yh[r] * mgy);",
     "dh[r] = rstd * (dy[r] * gamma[r] - mg);"),
    ("bwd_w_up_transposed", "acc += Wup[r * d_emb + c] * dh[r];", "acc += Wup[c * d_up + r] * dh[r];"),
    ("bwd_dgamma_unnormalised", "dgamma[r] += dy[r] * yh[r];", "dgamma[r] += dy[r] * h[r];"),
    ("bwd_dx_no_attention_term", "dx[i * d_in + c] += ds * kr[c];", "(void)kr;"),
    ("bwd_dv_first_row_only", "double *gv = dWV + (a + j) * d_emb;", "double *gv = dWV + a * d_emb;"),
    ("bwd_dk_uses_dp", "gk[c] += ds * xi[c];", "gk[c] += dp[j] * xi[c];"),
    # the per-row magnitudes the GPU backward's tolerance is built from
    ("bwd_kmag_no_output_term", "if (kmag) kmag[a + j] += p[j] * (sqrt(vd) + od) * xmax;",
     "if (kmag) kmag[a + j] += p[j] * sqrt(vd) * xmax;"),
    ("bwd_kmag_no_p", "if (kmag) kmag[a + j] += p[j] * (sqrt(vd) + od) * xmax;",
     "if (kmag) kmag[a + j] += (sqrt(vd) + od) * xmax;"),
    ("bwd_kmag_l1", "od = sqrt(od);", "od = sqrt(od) * 2.0;"),
    ("bwd_vmag_first_row", "if (vmag) vmag[a + j] += p[j] * dmax;", "if (vmag) vmag[a] += p[j] * dmax;"),
]


@pytest.mark.parametrize("name,old,new", BACKWARD_MUTANTS, ids=[m[0] for m in BACKWARD_MUTANTS])
def test_backward_mutant_is_caught(tmp_path, name, old, new):
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    p = tmp_path / f"{name}.c"
    p.write_text(src.replace(old, new))
    lib = oracle.load(oracle.build(str(p), str(tmp_path / f"lib{name}.so")))
    failed = []
    for pin in BACKWARD_PINS:
        try:
            pin(lib)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every backward pin"
