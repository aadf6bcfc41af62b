"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source, builds it on
the CPU, and runs the pin suite against it: the suite has to fail.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

MUTATIONS = {
    "silu_on_w3_branch": ("hid[c] = orc_silu(a) * b;", "hid[c] = a * orc_silu(b);"),
    "no_residual": ("h[(size_t)r * d + i] = acc + x[i];", "h[(size_t)r * d + i] = acc;"),
    "ties_to_higher_index": ("(best < 0 || logit[i] > logit[best])",
                             "(best < 0 || logit[i] >= logit[best])"),
    "select_smallest": ("(best < 0 || logit[i] > logit[best])",
                        "(best < 0 || logit[i] < logit[best])"),
    "no_max_subtraction": ("s[i] = expf(logit[i] - mx);", "s[i] = expf(logit[i]);"),
    "renormalised_gates": ("topk_gate[(size_t)t * k + j] = s[sel[j]];",
                           "topk_gate[(size_t)t * k + j] = s[sel[j]] * (float)n / (float)k;"),
    "w2_transposed": ("orc_get(w2, o2 + (size_t)i * ldw2 + c, dtype)",
                      "orc_get(w2, o2 + (size_t)c * d + i, dtype)"),
    "shared_dropped": ("acc += sh[i];", "acc += 0.0f;"),
    "P_unnormalised": ("P[i] = acc / (float)T;", "P[i] = acc;"),
    "f_is_plain_fraction": ("f[i] = (float)((int64_t)counts[i] * n) / (float)((int64_t)k * T);",
                            "f[i] = (float)counts[i] / (float)T;"),
    "k_without_shared": ("*k = m * K - K_s;", "*k = m * K;"),
    "unstable_permute": ("int32_t pos = cursor[e]++;",
                         "int32_t pos = cursor[e + 1] - 1 - (cursor[e]++ - offsets[e]);"),
    "shared_slice_stride": ("(size_t)q * d_ff, ldws2, dtype, hid, tmp);",
                            "(size_t)q * d_ff * d, ldws2, dtype, hid, tmp);"),
    # backward pass
    "dsilu_first_term_only": ("const double dsilu = sg * (1.0 + a[c] * (1.0 - sg));",
                              "const double dsilu = sg;"),
    "gate_dropped_in_da": ("da[c] = g * dhid[c] * b[c] * dsilu;", "da[c] = dhid[c] * b[c] * dsilu;"),
    "softmax_bwd_uncentred": ("const double dl = s[i] * (ds[i] - sds);",
                              "const double dl = s[i] * ds[i];"),
    "balance_grad_without_1_over_T": ("ds[i] = alpha * (double)f[i] / (double)T;",
                                      "ds[i] = alpha * (double)f[i];"),
    "dw2_from_ungated_dy": ("dy[j] = g[r] * (double)dh[(size_t)tok[r] * d + j];",
                            "dy[j] = (double)dh[(size_t)tok[r] * d + j];"),
    "dx_w3_takes_da": ("(double)orc_get(w3, o13 + (size_t)c * ldw13 + j, dtype) * bc;",
                       "(double)orc_get(w3, o13 + (size_t)c * ldw13 + j, dtype) * ac;"),
    "residual_grad_dropped": ("dx[j] = (flags & ORC_BWD_NO_RESIDUAL) ? 0.0 : dy[j];",
                              "dx[j] = 0.0;"),
    "dcent_transposed_u": ("o[j] += dl * (double)orc_get(u, (size_t)t * d + j, dtype);",
                           "o[j] += dl * (double)orc_get(u, (size_t)j * d + t % d, dtype);"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-fopenmp", "-ffp-contract=off",
                    "-shared", "-o", str(lib), str(mut), "-lm"], check=True)
    env = dict(os.environ, MOE_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_bwd_pins.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True)
    assert r.returncode != 0, f"pins did not catch mutation {name}:\n{r.stdout[-2000:]}"
