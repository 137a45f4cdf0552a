"""Altered copies of the oracle must fail at least one pin (CPU only).

Each mutant changes one plausible detail of s2r_oracle.cpp -- a dropped sign, a wrong
shift, a lost term, a wrong median index -- is compiled with g++ into a temporary
library, and the pin suite is run against it.  A mutant that passes every pin would mean
the pins cannot tell that mistake from the real thing.
"""
import json
import os
import subprocess
import sys

import pytest

import oracle

MUTANTS = {
    "drop_sign_in_insert": ("S[cell] += (double)orc_sign(p, j, i) * (double)g;",
                            "S[cell] += (double)g;"),
    "abs_mass_signed": ("A[cell] += std::fabs((double)g);", "A[cell] += (double)g;"),
    "shift_by_one": ("return low64 >> (64 - bits);", "return (low64 << 1) >> (64 - bits);"),
    "drop_add_term": ("(unsigned __int128)a * (unsigned __int128)x + c;",
                      "(unsigned __int128)a * (unsigned __int128)x;"),
    "add_after_shift": ("uint64_t low64 = (uint64_t)full;  // mod 2^64\n  return low64 >> (64 - bits);",
                        "uint64_t low64 = (uint64_t)full - c;\n  return (low64 >> (64 - bits)) + (c >> (64 - bits)) & ((1ull << bits) - 1);"),
    "partition_not_shifted": ("return (uint32_t)((part << K) | low);", "return (uint32_t)(part | low);"),
    "sign_uses_bucket_constant": ("mas_top(p->sA[j], p->sB[j], i, 1)", "mas_top(p->hA[j], p->sB[j], i, 1)"),
    "bitmap_bit_off_by_one": ("bitmap[b / 64] |= 1ull << (b % 64);\n    if (count < cap)",
                              "bitmap[b / 64] |= 1ull << ((b + 1) % 64);\n    if (count < cap)"),
    "block_bit_from_element_index": ("const uint64_t b = block_of(p, i);\n    bitmap[b / 64]",
                                     "const uint64_t b = i;\n    bitmap[b / 64]"),
    "block_rounds_up": ("return i >> p->log2_block; }", "return (i + 1) >> p->log2_block; }"),
    "topk_tie_prefers_higher_id": ("(norm2[a] == norm2[b] && a < b)", "(norm2[a] == norm2[b] && a > b)"),
    "topk_norm_of_abs": ("s += (double)g[i] * (double)g[i];", "s += std::fabs((double)g[i]);"),
    "topk_kept_residual_not_zeroed": ("residual[i] = kept ? 0.0f : g[i];", "residual[i] = g[i];"),
    "topk_ignores_residual_input": ("g[i] = residual ? grad[i] + residual[i] : grad[i];",
                                    "g[i] = grad[i];"),
    "topk_keeps_one_less": ("for (uint64_t r = 0; r < K && r < nb; ++r)",
                            "for (uint64_t r = 1; r < K && r < nb; ++r)"),
    "query_element_bits_only": ("const uint64_t b = block_of(p, i);\n    if (!((bitmap",
                                "const uint64_t b = i;\n    if (!((bitmap"),
    "negative_zero_counts": ("return (u & 0x7FFFFFFFu) != 0;", "return u != 0;"),
    "median_odd_takes_max": ("(d % 2) ? est[(d - 1) / 2]", "(d % 2) ? est[d - 1]"),
    "median_even_takes_lower": ("0.5 * (est[d / 2 - 1] + est[d / 2])", "est[d / 2 - 1]"),
    "tolerance_coefficient_loosened": ("out_tol[count] = 1e-5 * amax + 1e-12;",
                                       "out_tol[count] = 1e-2 * amax + 1e-12;"),
    "tolerance_mass_scaled": ("amax = std::max(amax, A[cell]);",
                              "amax = std::max(amax, 100 * A[cell]);"),
    "gather_drops_last_worker": ("for (uint32_t k = 0; k < W; ++k)\n    for (uint64_t t = 0; t < len[k]; ++t)",
                                 "for (uint32_t k = 0; k + 1 < W; ++k)\n    for (uint64_t t = 0; t < len[k]; ++t)"),
    "gather_skips_first_entry": ("for (uint64_t t = 0; t < len[k]; ++t) {\n      const uint64_t i = idx",
                                 "for (uint64_t t = 1; t < len[k]; ++t) {\n      const uint64_t i = idx"),
    "gather_mass_signed": ("mass[i] += std::fabs(v);", "mass[i] += v;"),
    "query_ignores_sign": ("est[j] = (double)orc_sign(p, j, (uint32_t)i) * S[cell];",
                           "est[j] = S[cell];"),
    "reduce_drops_last_worker": ("for (uint32_t k = 0; k < W; ++k) {\n      s += S",
                                 "for (uint32_t k = 0; k + 1 < W; ++k) {\n      s += S"),
    "merge_by_xor": ("m |= bitmaps[(uint64_t)k * words + q];", "m ^= bitmaps[(uint64_t)k * words + q];"),
    "draw_order_swapped": ("out->hA[j] = orc_splitmix64_next(&st);\n    out->hB[j] = orc_splitmix64_next(&st);",
                           "out->hB[j] = orc_splitmix64_next(&st);\n    out->hA[j] = orc_splitmix64_next(&st);"),
    "splitmix_wrong_gamma": ("*state += 0x9E3779B97F4A7C15ull;", "*state += 0x9E3779B97F4A7C17ull;"),
}


# Runs every pin against one compiled mutant and prints the names of the pins that failed.
# It runs in a child process: a mutant may index outside its arrays (a block bit computed
# from the element index, say), and its memory errors must not reach the test process.
_CHILD = """
import json, sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, pins
failed = []
with oracle.using({lib!r}):
    for pin in pins.ALL_PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
print(json.dumps(failed))
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.source_path()).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    mpath = tmp_path / f"{name}.cpp"
    mpath.write_text(src.replace(old, new))
    lib = oracle.compile_source(str(mpath), str(tmp_path / f"lib{name}.so"))
    tests = os.path.dirname(os.path.abspath(__file__))
    code = _CHILD.format(root=os.path.dirname(tests), tests=tests, lib=lib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        # the mutant crashed the pin run: it did not get through the pins unnoticed
        return
    failed = json.loads(r.stdout.strip().splitlines()[-1])
    assert failed, f"mutant {name} passes every pin"
