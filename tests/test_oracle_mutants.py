"""Planted mistakes in the oracle (on the CPU only) must each fail some pin.

Each mutant is a copy of the oracle's C source with one plausible mistake
substituted (a flipped comparison, a swapped operand, a wrong row or uniform
index, a dropped term); it is compiled into a temporary library and every pin
in ``oracle_pins`` runs against it until one fails.  A mutant that passes every
pin means the pins are too weak to notice that mistake.
"""
import inspect
import os

import numpy as np
import pytest

import oracle
from tests import oracle_pins

MUTANTS = {
    "non-strict acceptance": ("accepted = (double)u[i] < P / Q;",
                              "accepted = (double)u[i] <= P / Q;"),
    "inverted ratio": ("accepted = (double)u[i] < P / Q;", "accepted = (double)u[i] < Q / P;"),
    "residual sign": ("double d = p[j] - q[j];", "double d = q[j] - p[j];"),
    "residual unclamped": ("w[j] = d > 0.0 ? d : 0.0;", "w[j] = d;"),
    "residual ignores draft": ("if (s < k) {", "if (0) {"),
    "bonus from row k-1": (
        "ROW_DIST(target_logits, ((size_t)b * (k + 1) + s) * (size_t)V, p);",
        "ROW_DIST(target_logits, ((size_t)b * (k + 1) + (s == k && s > 0 ? s - 1 : s)) * (size_t)V, p);"),
    "target row shifted": ("size_t t_row = ((size_t)b * (k + 1) + i) * (size_t)V;\n            size_t d_row = ((size_t)b * k + i) * (size_t)V;\n            ROW_DIST",
                           "size_t t_row = ((size_t)b * (k + 1) + i + 1) * (size_t)V;\n            size_t d_row = ((size_t)b * k + i) * (size_t)V;\n            ROW_DIST"),
    "final sample uses u[s]": ("inverse_cdf(w, V, (double)u[k], &final_margin);",
                               "inverse_cdf(w, V, (double)u[s], &final_margin);"),
    "cdf non-strict": ("if (above > target) {", "if (above >= target) {"),
    "temperature ignored": ("double z = logit_at(logits, dtype, row_offset + (size_t)j) / temperature;",
                            "double z = logit_at(logits, dtype, row_offset + (size_t)j);"),
    "argmax last tie": ("if (v > best_value) {", "if (v >= best_value) {"),
    "greedy emits draft at stop": ("out[s] = arg[s];", "out[s] = s < k ? x[s] : arg[s];"),
    "greedy off-by-one row": ("while (s < k && x[s] == arg[s])", "while (s < k && x[s] == arg[s + 1 <= k ? s + 1 : s])"),
    "tree highest tie": ("if (m > best_m) { /* strictly longer", "if (m >= best_m) { /* strictly longer"),
    "tree compares own row": ("if (tok[child] != a[row[m]])", "if (tok[child] != a[child])"),
    "tree emits last node token": ("out[best_m] = a[row[best_m]];", "out[best_m] = tok[row[best_m]];"),
    "ragged drops the final token": (
        "out_tokens[(size_t)b * (k + 1) + i] = i <= kb ? out1[i] : -1;\n            if (margins)",
        "out_tokens[(size_t)b * (k + 1) + i] = i < kb ? out1[i] : -1;\n            if (margins)"),
    "ragged ignores lengths": ("return kb < 0 ? 0 : (kb > k ? k : kb);", "return k;"),
    "ragged final uniform at k": ("uniforms + (size_t)b * (k + 1), temperature, 1, kb, V,",
                                  "uniforms + (size_t)b * (k + 1) + (k - kb), temperature, 1, kb, V,"),
    "greedy ragged reads full rows": ("rc = oracle_verify_greedy(t, dtype, draft_tokens + (size_t)b * k, 1, kb, V, out1, &acc,",
                                      "rc = oracle_verify_greedy(t, dtype, draft_tokens + (size_t)b * k, 1, kb < k ? kb + 1 : kb, V, out1, &acc,"),
    "top-k off by one": ("thr = scratch[f->top_k - 1];", "thr = scratch[f->top_k];"),
    "top-p not renormalised": ("double target = f->top_p * mass1;", "double target = f->top_p;"),
    "top-p one group late": ("            if (cum >= target) {\n                double lo", "            if (cum > target + 0.05) {\n                double lo"),
    "min_p sign": ("double tmin = xmax + temperature * log(f->min_p);", "double tmin = xmax - temperature * log(f->min_p);"),
    "filter target only": ("        if (filter) {                                                                   \\", "        if (filter && (logits) == target_logits) {                                      \\"),
    "tree residual not carried to siblings": ("                        p[j] = w[j] / Z;\n",
                                              "                        p[j] = p[j];\n"),
    "tree test uniform index": ("accepted = (double)u[c - 1] < P_ / Q_;",
                                "accepted = (double)u[c] < P_ / Q_;"),
    "tree accepts out-of-range ids": ("accepted = 0; /* an id outside the vocabulary is rejected */",
                                      "accepted = 1; /* an id outside the vocabulary is rejected */"),
    "tree siblings last first": ("for (int c = 1; c <= N && next < 0 && depth + 1 < L; ++c) {",
                                 "for (int c = N; c >= 1 && next < 0 && depth + 1 < L; --c) {"),
    "tree draft row of the child": (
        "softmax_row(draft_logits, dtype, ((size_t)b * (N + 1) + n) * (size_t)V, V,",
        "softmax_row(draft_logits, dtype, ((size_t)b * (N + 1) + (n < N ? n + 1 : n)) * (size_t)V, V,"),
    "philox wrong multiplier": ("M1 = 0xCA5A826395121157ull", "M1 = 0xCA5A826395121155ull"),
    "philox key not advanced": ("            k[0] += W0;\n", ""),
    "philox words swapped": ("    ctr[1] = lo1;\n", "    ctr[1] = lo0;\n"),
    "philox nine rounds": ("for (int round = 0; round < 10; ++round)", "for (int round = 0; round < 9; ++round)"),
    "philox uniform low bits": ("(block[i % 4] >> 40)", "(block[i % 4] & 0xFFFFFF)"),
    # guard band: the margins that classify requests as ambiguous
    "final margin not divided by Z": ("*margin = (lo < hi ? lo : hi) / Z;",
                                      "*margin = (lo < hi ? lo : hi);"),
    "accept margin without the min": ("double threshold = (P >= Q) ? 1.0 : P / Q;",
                                      "double threshold = P / Q;"),
    "accept margin at the final uniform": (
        "margin[i] = in_range ? fabs((double)u[i] - threshold) : INFINITY;",
        "margin[i] = in_range ? fabs((double)u[k] - threshold) : INFINITY;"),
    "top-p margin not relative to the survivors": ("double m = (lo < hi ? lo : hi) / mass1;",
                                                   "double m = (lo < hi ? lo : hi);"),
    "min-p margin from the maximum": (
        "double d = fabs(logit_at(logits, dtype, row_offset + (size_t)j) - tmin);",
        "double d = fabs(logit_at(logits, dtype, row_offset + (size_t)j) - xmax);"),
    "tree margin without the min": ("double threshold = (P_ >= Q_) ? 1.0 : P_ / Q_;",
                                    "double threshold = P_ / Q_;"),
    "tree final margin from p": ("out[depth] = inverse_cdf(rejected ? w : p, V, (double)u[N], &final_margin);",
                                 "out[depth] = inverse_cdf(rejected ? w : p, V, (double)u[N], &final_margin);\n                if (rejected) inverse_cdf(p, V, (double)u[N], &final_margin);"),
}

# Planted mistakes in the oracle's Python classifier of ambiguous requests.
PY_MUTANTS = {
    "ambiguous takes the largest margin": ("amb = np.min(margins, axis=1) < band",
                                           "amb = np.max(margins, axis=1) < band"),
    "ambiguous band inclusive": ("amb = np.min(margins, axis=1) < band",
                                 "amb = np.min(margins, axis=1) <= band"),
    "filter band ignored": ("amb |= np.asarray(filter_margins) < filter_band",
                            "amb |= np.asarray(filter_margins) < 0.0"),
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation anchor for {name!r} not found exactly once"
    src = tmp_path / "mutant.c"
    src.write_text(source.replace(old, new))
    lib_path = oracle.compile_source(str(src), str(tmp_path / f"libmutant_{os.getpid()}.so"))
    lib = oracle.open_library(lib_path)
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(lib)
        except AssertionError:
            return  # caught
    pytest.fail(f"planted mistake {name!r} passed every oracle pin")


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_classifier_mutant_is_caught(name):
    old, new = PY_MUTANTS[name]
    src = inspect.getsource(oracle.ambiguous_requests)
    assert src.count(old) == 1, f"mutation anchor for {name!r} not found exactly once"
    ns = {"np": np}
    exec(src.replace(old, new), ns)
    with pytest.raises(AssertionError):
        oracle_pins.check_ambiguous_requests(None, fn=ns["ambiguous_requests"])
