"""Planted mistakes in a copy of the oracle, on the CPU: each mutant must fail
at least one pin, showing that the pins constrain every step of the oracle
(a dropped term, a wrong sign, a wrong index, a transposed operand)."""
import json
import os
import subprocess
import sys

import pytest

import _pins
import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "rkv_oracle.cpp")

# (name, original text, planted text): each original occurs exactly once
MUTANTS = [
    ("gqa_min_not_max", "std::max(imp[j], ibar[j])", "std::min(imp[j], ibar[j])"),
    ("sum_not_mean_over_window", "ibar[j] += (std::exp(logit[j] - mx) / den) / A;",
     "ibar[j] += (std::exp(logit[j] - mx) / den);"),
    ("not_causal", "const int pos = N - A + t;", "const int pos = N - 1;"),
    ("no_attention_scale", "logit[j] = s * inv_sqrt_d;", "logit[j] = s;"),
    ("transposed_query_index", "(int64_t)(g * A + t) * D + d", "(int64_t)(t * G + g) * D + d"),
    ("no_key_normalisation", "Kh[(size_t)j * D + d] = K[(size_t)j * D + d] / nrm;",
     "Kh[(size_t)j * D + d] = K[(size_t)j * D + d];"),
    ("count_on_newer_index", "if (s > p->tau) cnt[i] += 1;", "if (s > p->tau) cnt[j] += 1;"),
    ("non_strict_threshold", "if (s > p->tau) cnt[i] += 1;", "if (s >= p->tau) cnt[i] += 1;"),
    ("protection_off_by_one", "(cnt[i] < p->beta)", "(cnt[i] <= p->beta)"),
    ("rowmean_divides_by_n", "rowsum[i] / (double)(N - 1)", "rowsum[i] / (double)N"),
    ("rowsum_one_sided", "rowsum[j] += s;", ""),
    ("softmax_over_all_tokens", "for (int i = 0; i < nc; ++i) rden += std::exp(rbar[i] - rmax);",
     "for (int i = 0; i < N; ++i) rden += std::exp(rbar[i] - rmax);"),
    ("combination_sign", "p->lambda * imp[i] - (1.0 - p->lambda) * R[i]",
     "p->lambda * imp[i] + (1.0 - p->lambda) * R[i]"),
    ("combination_weights_swapped", "p->lambda * imp[i] - (1.0 - p->lambda) * R[i]",
     "(1.0 - p->lambda) * imp[i] - p->lambda * R[i]"),
    ("tie_to_older", "return a > b;", "return a < b;"),
    ("window_not_kept", "for (int j = nc; j < N; ++j) kept.push_back(j);",
     "for (int j = nc; j < N; ++j) kept.push_back(order[k]);"),
    ("budget_excludes_window", "const int k = B - A;", "const int k = B - A - 1;"),
    ("gather_shifted", "(const char*)src + (size_t)keep[j] * row_bytes",
     "(const char*)src + (size_t)(keep[j] > 0 ? keep[j] - 1 : 0) * row_bytes"),
    ("trigger_off_by_one", "if (*n_slots < B + p->buffer) return 0;", "if (*n_slots <= B + p->buffer) return 0;"),
    ("holefill_mover_to_last_free", "const int dst = free_rows[m++];",
     "const int dst = free_rows[free_rows.size() - 1 - m++];"),
    ("holefill_stayer_moves", "new_order[j] = order[keep[j]];", "new_order[j] = keep[j];"),
    ("holefill_v_not_moved", "std::memcpy((char*)v_rows + (size_t)dst * row_bytes",
     "if (0) std::memcpy((char*)v_rows + (size_t)dst * row_bytes"),
    ("sampled_gumbel_sign", "- std::log(-std::log((double)uniforms[i]));", "+ std::log(-std::log((double)uniforms[i]));"),
    ("sampled_no_temperature", "(double)scores[i] / temperature", "(double)scores[i]"),
    ("sampled_top_k_ignored", "  cand.resize(K);\n", "\n"),
    ("sampled_score_tie_to_older", "return sa != sb ? sa > sb : a > b;", "return sa != sb ? sa > sb : a < b;"),
    ("sentence_penalty_added", "if (token_penalty) Z[i] -= token_penalty[i];",
     "if (token_penalty) Z[i] += token_penalty[i];"),
    ("sentence_earlier_not_later", "for (int j = i + 1; j < n_sent; ++j) {", "for (int j = 0; j < i; ++j) {"),
    ("sentence_threshold_ignored", "if (c > tau_s && (!any || c > best)) {", "if ((!any || c > best)) {"),
    ("decode_no_attention_scale", "lg[j] = inv_sqrt_d * s;", "lg[j] = s;"),
    ("decode_drops_newest_key", "    for (int j = 0; j < n; ++j) den += std::exp(lg[j] - mx);",
     "    for (int j = 0; j < n - 1; ++j) den += std::exp(lg[j] - mx);"),
    ("decode_query_of_head_zero", "load(queries, dtype, (int64_t)g * D + d)", "load(queries, dtype, (int64_t)d)"),
    ("decode_value_of_key_zero", "load(values, dtype, (int64_t)j * D + d)", "load(values, dtype, (int64_t)d)"),
    ("holefill_padding_reuses_first_free", "for (int j = 0; j < lead; ++j) new_order[j] = free_rows[m + j];",
     "for (int j = 0; j < lead; ++j) new_order[j] = free_rows[j];"),
]


RUNNER = """
import json, sys
sys.path.insert(0, {tests!r}); sys.path.insert(0, {root!r})
import _pins, oracle
oracle._lib = oracle.load_library({so!r})
failed = []
for check in _pins.ALL_CHECKS:
    try:
        check()
    except Exception:
        failed.append(check.__name__)
print(json.dumps(failed))
"""


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("mutants")


def run_pins_on(so_path: str):
    """Runs every pin against a library in a child process; a crash counts as caught."""
    tests = os.path.dirname(os.path.abspath(__file__))
    code = RUNNER.format(tests=tests, root=os.path.dirname(tests), so=so_path)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        return ["<crashed>"]
    return json.loads(r.stdout.strip().splitlines()[-1])


def build_mutant(name, orig, planted, out_dir):
    src = open(SRC).read()
    assert src.count(orig) == 1, f"mutation anchor for {name} must occur once"
    path_cpp = os.path.join(out_dir, f"{name}.cpp")
    path_so = os.path.join(out_dir, f"{name}.so")
    with open(path_cpp, "w") as f:
        f.write(src.replace(orig, planted))
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", f"-I{os.path.dirname(SRC)}", path_cpp,
                           "-o", path_so])
    return path_so


def test_unmutated_oracle_passes_every_pin(mutant_dir):
    assert run_pins_on(oracle.build()) == []


@pytest.mark.parametrize("name,orig,planted", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, orig, planted, mutant_dir):
    failed = run_pins_on(build_mutant(name, orig, planted, str(mutant_dir)))
    assert failed, f"mutant {name} passed every pin"
