"""The pins must be able to fail: planted mistakes in the oracle are caught.

Each case below plants one plausible mistake in a copy of the oracle's C
source (a dropped term, a wrong sign or index, a transposed operand, a missed
CTC transition rule), compiles the copy with gcc and runs every pin of
tests/test_oracle_pins.py against it.  A mutant survives only if all pins
pass, which fails the test.  The unmodified source, compiled the same way,
must pass every pin (the harness itself is sound).

The transitions planted wrong here are the ones of the CTC recursion on the
blank-interleaved label sequence ("Pruned CTC for Memory-Efficient
Large-Vocabulary ASR Training", Sec. 3.1): stay, advance by one, and skip a
blank only between two different labels; alignments start on the first blank
or the first label and end on the last label or the final blank.
"""
import os

import numpy as np
import pytest

import oracle
from tests import test_oracle_pins as pins

# (name, original text, planted text); each original occurs exactly once.
MUTANTS = [
    ("log_add_drops_log1p", "return hi + log1p(exp(lo - hi));", "return hi + log(exp(lo - hi));"),
    ("normalizer_drops_max", "double lam = mx + log(s);", "double lam = log(s);"),
    ("normalizer_unshifted_exp", "s += exp(z[v] - mx);", "s += exp(z[v]);"),
    ("skip_between_repeats", "ext[s] != blank && ext[s] != ext[s - 2]", "ext[s] != blank"),
    ("skip_drops_a_label", "ext[s] != blank && ext[s] != ext[s - 2]",
     "(ext[s] == blank || ext[s] != ext[s - 2])"),
    ("beta_skip_between_repeats", "ext[s] != blank && ext[s] != ext[s + 2]", "ext[s] != blank"),
    ("no_start_on_label", "if (S > 1) alpha[1] = logp[ext[1]];", ";"),
    ("no_end_on_label", "if (S > 1) logP = log_add(logP, last[S - 2]);", ";"),
    ("beta_no_end_on_label", "if (S > 1)\n      beta[(size_t)(T - 1) * S + S - 2] =",
     "if (0)\n      beta[(size_t)(T - 1) * S + S - 2] ="),
    ("gamma_double_emission", "beta[(size_t)t * S + s] -\n                      lp[ext[s]] - logP;",
     "beta[(size_t)t * S + s] -\n                      logP;"),
    ("gradient_sign", "grad * (exp(lp[v]) - gam_row[v])", "grad * (gam_row[v] - exp(lp[v]))"),
    ("gradient_unscaled", "grad * (exp(lp[v]) - gam_row[v])", "(exp(lp[v]) - gam_row[v])"),
    ("alignability_ignores_repeats_ctc", "if (L + r > T) {", "if (L > T) {"),
    ("alignability_ignores_repeats_select", "flags[n] = (L + r <= frame_counts[n]) ? 1 : 0;",
     "flags[n] = (L <= frame_counts[n]) ? 1 : 0;"),
    ("relabel_off_by_one", "tgt_rel[i] = lo;", "tgt_rel[i] = lo - 1;"),
    ("selection_descending", "for (int v = 0; v < V; ++v)\n    if (present[v]",
     "for (int v = V - 1; v >= 0; --v)\n    if (present[v]"),
    ("bias_dropped", "acc + (b ? b[v] : 0.0)", "acc"),
    ("utterance_rows_unscaled", "const double* Xn = X + (size_t)row0 * D;",
     "const double* Xn = X + (size_t)row0;"),
    ("dW_transposed_operand", "const double* x = Xn + (size_t)t * D;\n            for",
     "const double* x = W + (size_t)v * D;\n            for"),
    ("dX_uses_X", "const double* w = W + (size_t)v * D;\n          for (int d = 0; d < D; ++d) dx[d]",
     "const double* w = Xn + (size_t)t * D;\n          for (int d = 0; d < D; ++d) dx[d]"),
    ("db_overwrites", "if (db) db[v] += g;", "if (db) db[v] = g;"),
    ("loss_counts_unalignable_as_inf", "if (L + r > T) {\n    status = 1;",
     "if (L + r > T) {\n    status = 1; loss = INFINITY;"),
    ("alpha_stay_dropped", "double a = prev[s];", "double a = -INFINITY;"),
    ("beta_drops_emission", "cur[s] = b + lp[ext[s]];", "cur[s] = b;"),
    ("alpha_emission_of_previous_frame", "cur[s] = a + lp[ext[s]];",
     "cur[s] = a + lp[ext[s] - V];"),
    ("normalizer_skips_last_class", "for (int v = 0; v < V; ++v) s += exp(z[v] - mx);",
     "for (int v = 0; v + 1 < V; ++v) s += exp(z[v] - mx);"),
    ("loss_from_first_state", "double logP = last[S - 1];", "double logP = last[0];"),
    ("gamma_overwrites_repeats", "gam_row[ext[s]] += exp(lg);", "gam_row[ext[s]] = exp(lg);"),
    ("relabel_search_includes_blank", "int lo = 1, hi = K - 1;", "int lo = 0, hi = K - 1;"),
    ("alignability_strict", "flags[n] = (L + r <= frame_counts[n]) ? 1 : 0;",
     "flags[n] = (L + r < frame_counts[n]) ? 1 : 0;"),
    ("gradient_log_probability", "grad * (exp(lp[v]) - gam_row[v])",
     "grad * (lp[v] - gam_row[v])"),
    ("gather_ignores_cols",
     "Zn[(size_t)t * V + cols[c]] - lam[t];\n        if (gamma_cols)\n"
     "          gamma_cols[(size_t)(row0 + t) * ncols + c] = gam[(size_t)t * V + cols[c]];",
     "Zn[(size_t)t * V + c] - lam[t];\n        if (gamma_cols)\n"
     "          gamma_cols[(size_t)(row0 + t) * ncols + c] = gam[(size_t)t * V + c];"),
    ("logp_gather_ignores_cols", "Zn[(size_t)t * V + cols[c]] - lam[t];",
     "Zn[(size_t)t * V + c] - lam[t];"),
    ("gamma_gather_ignores_cols", "= gam[(size_t)t * V + cols[c]];", "= gam[(size_t)t * V + c];"),
    ("gather_rows_of_first_utterance", "logp_cols[(size_t)(row0 + t) * ncols + c] =",
     "logp_cols[(size_t)t * ncols + c] ="),
    # finite-beam pruning (oracle_ctc_beam).  Dropping the check of the
    # initial or of the final arcs is no mistake under this reading: an arc
    # out of a first-frame node (into a last-frame node) never scores above
    # the initial (final) arc of that node, so those checks never decide.
    ("beam_threshold_sign", "const double thr = best - beam;", "const double thr = best + beam;"),
    ("beam_suffix_includes_emission",
     "vb[(size_t)(T - 1) * S + s] = s >= first_final ? 0.0 : -INFINITY;",
     "vb[(size_t)(T - 1) * S + s] = s >= first_final ? em[(size_t)(T - 1) * S + s] : -INFINITY;"),
    ("beam_backward_unmasked", "if (keep[((size_t)(t + 1) * S + s2) * 3 + k]) {", "if (1) {"),
    ("beam_forward_unmasked", "if (keep[((size_t)t * S + s) * 3 + k])\n          a = log_add",
     "if (1)\n          a = log_add"),
    ("beam_arc_score_drops_suffix",
     "em[(size_t)t * S + s]) +\n                          vb[(size_t)t * S + s];",
     "em[(size_t)t * S + s]);"),
    ("beam_skip_between_repeats", "if (s >= 2 && lab[s] != blank && y[s / 2 - 1] != lab[s]) pred",
     "if (s >= 2 && lab[s] != blank) pred"),
    ("beam_viterbi_sums", "        if (c > m) m = c;", "        m = log_add(m, c);"),
    ("beam_delta_sign", "-expm1(-(loss_n - full_n))", "-expm1(loss_n - full_n)"),
    ("beam_occupancy_double_emission", "occ[lab[s]] += exp(fa[o] + fb[o] - em[o] - logP);",
     "occ[lab[s]] += exp(fa[o] + fb[o] - logP);"),
    ("beam_best_over_all_states",
     "for (int s = first_final; s < S; ++s)\n    if (vf[(size_t)(T - 1) * S + s] > best)",
     "for (int s = 0; s < S; ++s)\n    if (vf[(size_t)(T - 1) * S + s] > best)"),
]


def _calls():
    """Every pin test with each of its parameter sets, as plain callables."""
    out = []
    for name in sorted(dir(pins)):
        fn = getattr(pins, name)
        if not name.startswith("test_") or not callable(fn):
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not marks:
            out.append((name, fn, {}))
            continue
        (mark,) = marks
        argnames = [a.strip() for a in mark.args[0].split(",")]
        for vals in mark.args[1]:
            vals = vals if len(argnames) > 1 else (vals,)
            out.append((name, fn, dict(zip(argnames, vals))))
    return out


def _failures(lib_path):
    saved = oracle._default
    oracle._default = oracle.Oracle(lib_path)
    failed = []
    try:
        # a planted mistake can zero a gradient or make a value infinite; the
        # pins then fail on the comparison, and numpy's warnings are noise
        with np.errstate(all="ignore"):
            for name, fn, kw in _calls():
                try:
                    fn(**kw)
                except Exception as e:  # an assertion, or the oracle rejecting its input
                    failed.append("%s%s: %s" % (name, kw or "", type(e).__name__))
    finally:
        oracle._default = saved
    return failed


@pytest.fixture(scope="module")
def variant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_variants")


def test_unmodified_copy_passes_every_pin(variant_dir):
    path = oracle.compile_variant(oracle.source_text(), os.path.join(variant_dir, "orig.so"))
    assert _failures(path) == []


@pytest.mark.parametrize("name,orig,planted", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(variant_dir, name, orig, planted):
    src = oracle.source_text()
    assert src.count(orig) == 1, "mutation anchor for %s not unique in the oracle" % name
    path = oracle.compile_variant(src.replace(orig, planted),
                                  os.path.join(variant_dir, name + ".so"))
    failed = _failures(path)
    assert failed, "no pin catches the planted mistake %s" % name
