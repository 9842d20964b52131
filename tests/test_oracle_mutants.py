"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of oracle/oracle.c (a flipped sign, a
dropped term, a wrong or transposed index, a missing step), builds it on the
CPU, and runs the pin suites (tests/test_oracle_tables.py and
tests/test_oracle_conv.py) against it in a subprocess.  The pins must fail for
every mutant, and pass for the unmodified source built the same way."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = [os.path.join(ROOT, "tests", "test_oracle_tables.py"), os.path.join(ROOT, "tests", "test_oracle_conv.py")]

MUTANTS = {
    "real_basis_sign": ("re[r][-m + l] = h;", "re[r][-m + l] = -h;"),
    "racah_sign_dropped": ("sum += ((k & 1) ? -1.0 : 1.0) / den;", "sum += 1.0 / den;"),
    "racah_prefactor": ("double pre1 = (2.0 * J + 1.0) *", "double pre1 = (2.0 * J + 2.0) *"),
    "real_imag_swapped": ("const double *src = ((l1 + l2 + l3) % 2 == 0) ? tre : tim;",
                          "const double *src = ((l1 + l2 + l3) % 2 == 0) ? tim : tre;"),
    "no_sign_canon": ("sign = src[i] > 0 ? 1.0 : -1.0;", "sign = 1.0;"),
    "conj_missing": ("double pi = -(a1r[i][a] * a2i[j][b] + a1i[i][a] * a2r[j][b]);",
                     "double pi = (a1r[i][a] * a2i[j][b] + a1i[i][a] * a2r[j][b]);"),
    "path_parity": ("out[4 * k + 3] = xpar[i] * ypar[j];", "out[4 * k + 3] = xpar[i];"),
    "fwd_y_index": ("double yv = Y[e * YD + q->yoff + q->m2[t]];\n                        o[",
                    "double yv = Y[e * YD + q->yoff + q->m3[t] % q->n2];\n                        o["),
    "fwd_w_transposed": ("double w = W[(e * P + p) * U + u];\n                    for (int t = 0; t < q->nnz; ++t) {\n                        double xv",
                         "double w = W[(e * U + u) * P + p];\n                    for (int t = 0; t < q->nnz; ++t) {\n                        double xv"),
    "gy_without_w": ("gy[q->yoff + q->m2[t]] += q->c[t] * xv * w * gv;", "gy[q->yoff + q->m2[t]] += q->c[t] * xv * gv;"),
    "gx_wrong_receiver": ("int64_t e = sperm[j], r = recv[e];", "int64_t e = sperm[j], r = src[e];"),
    "gw_wrong_g_index": ("double gv = g[r * OD + q->ooff + (int64_t)(u * q->ou) * q->n3 + q->m3[t]];\n                        acc +=",
                         "double gv = g[r * OD + q->ooff + (int64_t)(u * q->ou) * q->n3 + q->m2[t] % q->n3];\n                        acc +="),
    "dbwd_term_dropped": ("if (ggY) { oracle_fwd(d, N, E, rowptr, src, x, ggY, W, rows, nrows, to); axpy(dg, to, nrows * OD); }",
                          "(void)0;"),
    # one-channel blocks (UVW products that reduce to the channel-wise one)
    "x_broadcast_ignored": ("double xv = x[s * XD + q->xoff + (int64_t)(u * q->xu) * q->n1 + q->m1[t]];\n                        double yv",
                            "double xv = x[s * XD + q->xoff + (int64_t)u * q->n1 + q->m1[t]];\n                        double yv"),
    "out_sum_first_channel_only": ("o[q->ooff + (int64_t)(u * q->ou) * q->n3 + q->m3[t]] += q->c[t] * xv * yv * w;",
                                   "if (q->ou || u == 0) o[q->ooff + (int64_t)(u * q->ou) * q->n3 + q->m3[t]] += q->c[t] * xv * yv * w;"),
    "gx_broadcast_not_summed": ("gx[q->xoff + (int64_t)(u * q->xu) * q->n1 + q->m1[t]] += q->c[t] * yv * w * gv;",
                                "if (q->xu || u == 0) gx[q->xoff + (int64_t)(u * q->xu) * q->n1 + q->m1[t]] += q->c[t] * yv * w * gv;"),
    "sender_csr_unstable": ("for (int64_t e = 0; e < E; ++e) sperm[fill[src[e]]++] = (int32_t)e;",
                            "for (int64_t e = E - 1; e >= 0; --e) sperm[fill[src[e]]++] = (int32_t)e;"),
}


def _build(tmp_path, name, text):
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"lib{name}.so"
    c.write_text(text)
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(c), "-lm"], check=True)
    return str(so)


def _pins_pass(so):
    env = dict(os.environ, ORACLE_SO=so, OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True)
    return r.returncode == 0, r.stdout[-400:]


def test_unmodified_copy_passes(tmp_path):
    ok, out = _pins_pass(_build(tmp_path, "orig", open(SRC).read()))
    assert ok, out


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) >= 1, f"mutation site for {name} not found"
    ok, out = _pins_pass(_build(tmp_path, name, text.replace(old, new, 1)))
    assert not ok, f"the pins did not catch {name}"
