"""Plant plausible mistakes in copies of the oracle and check the pins catch them.

Each mutant is the oracle's C source with one textual edit (a dropped term, a
wrong sign, a wrong index, a transposed operand, a broken tie-break), built
into a temporary library on the CPU. The test passes only if at least one pin
of ``test_oracle_pins`` fails (or the oracle reports an error) for that
mutant. The real oracle is never modified.
"""
import os
import subprocess

import pytest

import oracle
from test_oracle_pins import PINS

MUTANTS = {
    "base_wrong_k_index": ("acc += (double)wn[k] * (double)xi[k];",
                           "acc += (double)wn[k] * (double)xi[d_in - 1 - k];"),
    "base_dropped": ("yq[n] = acc;\n", "yq[n] = 0.0 * acc;\n"),
    "scale_dropped": ("yq[n] = yq[n] + c * acc;", "yq[n] = yq[n] + acc;"),
    "lora_sign_flipped": ("yq[n] = yq[n] + c * acc;", "yq[n] = yq[n] - c * acc;"),
    "B_transposed": ("for (int j = 0; j < r; ++j) acc += (double)bn[j] * v[j];",
                     "for (int j = 0; j < r; ++j) acc += (double)Ba[(size_t)j * d_out + n] * v[j];"),
    "A_reads_W": ("const float* aj = Aa + (size_t)j * d_in;",
                  "const float* aj = W + (size_t)j * d_in;"),
    "segment_off_by_one": ("if (seg_start[ss] <= p && p < seg_start[ss + 1]) { s = ss; break; }",
                           "if (seg_start[ss] <= p && p <= seg_start[ss + 1]) { s = ss; break; }"),
    "token_index_not_inverted": ("if (token_index[pp] == i) { p = pp; break; }",
                                 "if (pp == i) { p = token_index[pp]; break; }"),
    "grouping_skips_base_only": ("for (int id = -1; id < capacity; ++id) {",
                                 "for (int id = 0; id < capacity; ++id) {"),
    "grouping_unstable": ("for (int t = 0; t < n_tokens; ++t) {\n      if (token_adapter[t] == id) {",
                          "for (int t = n_tokens - 1; t >= 0; --t) {\n      if (token_adapter[t] == id) {"),
    "rank_from_segment_plus_one": ("const int r = adapter_rank[a];",
                                   "const int r = adapter_rank[a] > 1 ? adapter_rank[a] - 1 : 1;"),
    "lora_on_ignored": ("if (!lora_on) continue;", "(void)0;"),
    "merge_scale_dropped": ("= (double)W[(size_t)n * d_in + k] + c * dw;",
                            "= (double)W[(size_t)n * d_in + k] + dw;"),
    "merge_sign_flipped": ("= (double)W[(size_t)n * d_in + k] + c * dw;",
                           "= (double)W[(size_t)n * d_in + k] - c * dw;"),
    "merge_A_transposed_index": ("dw += (double)bn[j] * (double)A[(size_t)j * d_in + k];",
                                 "dw += (double)bn[j] * (double)A[(size_t)k * rank + j];"),
    "merge_drops_last_rank_row": ("for (int j = 0; j < rank; ++j) dw +=",
                                  "for (int j = 0; j + 1 < rank; ++j) dw +="),
    "merge_drops_W": ("= (double)W[(size_t)n * d_in + k] + c * dw;", "= c * dw;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(oracle._SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new, 1)
    path = tmp_path / "mutant.c"
    path.write_text(mutated)
    so = str(tmp_path / f"libmutant_{name}.so")
    oracle.build(str(path), so)
    lib = oracle.load(so)
    failures = []
    for pin in PINS:
        try:
            pin(lib)
        except (AssertionError, oracle.OracleError, IndexError, ValueError) as e:
            failures.append((pin.__name__, type(e).__name__))
    assert failures, f"mutant {name} passed every pin"
