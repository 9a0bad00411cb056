"""The pins reject a broken oracle (CPU only).

Each case below plants one plausible mistake in a copy of oracle/moonep_oracle.c:
an off-by-one, a wrong order, a dropped term, a wrong operand, a wrong rounding or
tie-break. The copy is built with the oracle's own compiler flags, and the pin
tests named for the case are run against it in a child process (the oracle loads
the library that MOONEP_ORACLE_LIB names). Every mutant must fail at least one pin,
and the unmodified source, built and loaded the same way, must pass them all.

The slowest brute-force case (every routing of R=4, E=4, K=1, S=2) is left out of
the child runs to keep this test short; no mutant below needs it to be caught.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moonep_oracle.c")
PINS = "tests/test_oracle_pins.py"
BOUNDED = "tests/test_oracle_bounded_pins.py"
BACKWARD = "tests/test_oracle_backward_pins.py"

# (name, pin files to run, text to find, replacement, which occurrence of the text)
# Occurrence 0 of text shared by both plans is the water-fill's.
MUTANTS = [
    ("maxvio_without_minus_one", [PINS],
     "/ (double)NE - 1.0;", "/ (double)NE;", 0),
    ("maxvio_over_ranks", [PINS],
     "(double)(maxT * (int64_t)E) / (double)NE", "(double)(maxT * (int64_t)R) / (double)NE", 0),
    ("home_offset_inclusive", [PINS],
     "o->hoff[r * G + i] = (int32_t)acc;\n            acc += o->T[r * G + i];",
     "acc += o->T[r * G + i];\n            o->hoff[r * G + i] = (int32_t)acc;", 0),
    ("keep_one_short", [PINS],
     "o->keep[r] = o->L[r] < SK ? o->L[r] : (int32_t)SK;",
     "o->keep[r] = o->L[r] < SK ? o->L[r] : (int32_t)SK - 1;", 0),
    ("overflow_offset_from_deficit_prefix", [PINS],
     "int64_t j = o->Opre[r] + (h - SK);", "int64_t j = o->Dpre[r] + (h - SK);", 0),
    ("deficit_slot_without_kept_rows", [PINS],
     "slot = o->keep[d] + (j - o->Dpre[d]);", "slot = (j - o->Dpre[d]);", 0),
    ("deficit_search_closed_interval", [PINS],
     "if (Dpre[r] <= j && j < Dpre[r + 1]) return r;",
     "if (Dpre[r] <= j && j <= Dpre[r + 1]) return r;", 0),
    ("duplicate_walk_from_row_zero", [PINS],
     "int32_t nd = 0;\n        int64_t s = o->keep[r];", "int32_t nd = 0;\n        int64_t s = 0;", 0),
    ("over_b_at_b", [PINS],
     "if (nd > B) status |= ST_OVER_B;", "if (nd >= B) status |= ST_OVER_B;", 0),
    ("segment_start_unclamped", [PINS],
     "o->seg_ptr[r * sp + i] = (int32_t)(st < SK ? st : SK);",
     "o->seg_ptr[r * sp + i] = (int32_t)st;", 0),
    ("list_ranks_descending", [PINS],
     "for (int r = 0; r < R; ++r)\n            for (int b = 0; b < o->n_dup[r]; ++b)\n"
     "                if (o->dup_expert[(int64_t)r * dcap + b] == e) {\n"
     "                    if (p >= pcap)",
     "for (int r = R - 1; r >= 0; --r)\n            for (int b = 0; b < o->n_dup[r]; ++b)\n"
     "                if (o->dup_expert[(int64_t)r * dcap + b] == e) {\n"
     "                    if (p >= pcap)", 0),
    ("repeat_reported_as_bad_id", [PINS],
     "if (ids[g * K + k2] == e) status |= ST_REPEAT_ID;",
     "if (ids[g * K + k2] == e) status |= ST_BAD_ID;", 0),
    ("dispatch_drops_last_slot", [PINS],
     "if (d < slot_lo || d >= slot_hi) continue;\n        memcpy(recv_window",
     "if (d < slot_lo || d >= slot_hi - 1) continue;\n        memcpy(recv_window", 0),
    ("replicate_one_slot_short", [PINS, BOUNDED],
     "for (int b = 0; b < n_dup[r] && b < B; ++b)", "for (int b = 0; b < n_dup[r] && b < B - 1; ++b)", 0),
    ("combine_mul_then_add", [PINS],
     "acc = fmaf(w[g * K + k], x, acc);", "acc = w[g * K + k] * x + acc;", 0),
    ("combine_from_negative_zero", [PINS],
     "float acc = 0.0f;\n            for (int k = 0; k < K; ++k) {\n"
     "                int64_t d = dst[g * K + k];\n                if (d < 0) continue;\n"
     "                float x = in_dtype",
     "float acc = -0.0f;\n            for (int k = 0; k < K; ++k) {\n"
     "                int64_t d = dst[g * K + k];\n                if (d < 0) continue;\n"
     "                float x = in_dtype", 0),
    ("combine_k_descending", [PINS],
     "for (int k = 0; k < K; ++k) {\n                int64_t d = dst[g * K + k];\n"
     "                if (d < 0) continue;\n                float x = in_dtype",
     "for (int k = K - 1; k >= 0; --k) {\n                int64_t d = dst[g * K + k];\n"
     "                if (d < 0) continue;\n                float x = in_dtype", 0),
    ("bf16_ties_up", [PINS], "u += 0x7fffu + lsb;", "u += 0x7fffu;", 0),
    ("bf16_truncates", [PINS], "u += 0x7fffu + lsb;", "u += 0u * lsb;", 0),
    ("reduce_duplicates_descending", [PINS],
     "for (int32_t p = dup_ptr[e]; p < dup_ptr[e + 1]; ++p) {",
     "for (int32_t p = dup_ptr[e + 1] - 1; p >= dup_ptr[e]; --p) {", 0),
    ("reduce_skips_home_value", [PINS],
     "float v = home[(int64_t)e * n + i];", "float v = 0.0f;", 0),
    ("grad_y_unweighted", [BACKWARD], "float v = w[a] * x;", "float v = x;", 0),
    ("grad_w_token_row_of_y", [BACKWARD],
     "(double)load_elem(y_rows, y_dtype, a * H + i)", "(double)load_elem(y_rows, y_dtype, g * H + i)", 0),
    ("dispatch_backward_skips_k0", [BACKWARD],
     "for (int k = 0; k < K; ++k) {\n                int64_t d = dst[g * K + k];\n"
     "                if (d < 0) continue;\n                acc = acc +",
     "for (int k = 1; k < K; ++k) {\n                int64_t d = dst[g * K + k];\n"
     "                if (d < 0) continue;\n                acc = acc +", 0),
    ("duplicate_start_one_late", [PINS],
     "o->dup_start[(int64_t)r * dcap + nd] = (int32_t)s0;",
     "o->dup_start[(int64_t)r * dcap + nd] = (int32_t)(s0 + 1);", 0),
    ("duplicate_count_one_short", [PINS],
     "o->dup_count[(int64_t)r * dcap + nd] = (int32_t)(s - s0);",
     "o->dup_count[(int64_t)r * dcap + nd] = (int32_t)(s - s0 - 1);", 0),
    ("segment_end_at_kept_rows", [PINS],
     "o->seg_ptr[r * sp + G + o->n_dup[r]] = (int32_t)end;",
     "o->seg_ptr[r * sp + G + o->n_dup[r]] = (int32_t)o->keep[r];", 0),
    ("duplicate_csr_end_short", [PINS], "o->dup_ptr[E] = p;", "o->dup_ptr[E] = p > 0 ? p - 1 : 0;", 0),
    ("bad_id_not_reported", [PINS],
     "if (e < 0 || e >= E) { status |= ST_BAD_ID; continue; }",
     "if (e < 0 || e >= E) { continue; }", 0),
    ("grad_w_in_binary32", [BACKWARD], "double s = 0.0;", "float s = 0.0f;", 0),
    ("dispatch_backward_from_negative_zero", [BACKWARD],
     "float acc = 0.0f;\n            for (int k = 0; k < K; ++k) {\n"
     "                int64_t d = dst[g * K + k];\n                if (d < 0) continue;\n"
     "                acc = acc +",
     "float acc = -0.0f;\n            for (int k = 0; k < K; ++k) {\n"
     "                int64_t d = dst[g * K + k];\n                if (d < 0) continue;\n"
     "                acc = acc +", 0),
    ("grad_y_not_rounded_to_bf16", [BACKWARD],
     "if (dtype == DT_BF16) ((uint16_t *)base)[idx] = f32_to_bf16_rne(v);",
     "if (dtype == DT_BF16) { uint32_t u; memcpy(&u, &v, 4); ((uint16_t *)base)[idx] = (uint16_t)(u >> 16); }", 0),
    ("bounded_bad_id_not_reported", [BOUNDED],
     "if (e < 0 || e >= E) { status |= ST_BAD_ID; continue; }",
     "if (e < 0 || e >= E) { continue; }", 1),
    ("bounded_overflow_from_smallest", [BOUNDED],
     "(best < 0 || o->T[r * G + i] > o->T[r * G + best])",
     "(best < 0 || o->T[r * G + i] < o->T[r * G + best])", 0),
    ("bounded_overflow_ties_to_highest_id", [BOUNDED],
     "(best < 0 || o->T[r * G + i] > o->T[r * G + best])",
     "(best < 0 || o->T[r * G + i] >= o->T[r * G + best])", 0),
    ("bounded_smallest_deficit_first", [BOUNDED],
     "(r < 0 || o->D[q] > o->D[r])) r = q;", "(r < 0 || o->D[q] < o->D[r])) r = q;", 0),
    ("bounded_bth_rule_one_late", [BOUNDED], "if (used < B - 1) {", "if (used < B) {", 0),
    ("bounded_fit_strict", [BOUNDED],
     "if (left[x] > 0 && left[x] <= room && (e < 0 || left[x] > left[e])) e = x;",
     "if (left[x] > 0 && left[x] < room && (e < 0 || left[x] > left[e])) e = x;", 0),
    ("bounded_filler_largest", [BOUNDED],
     "if (left[x] >= room && (e < 0 || left[x] < left[e])) e = x;",
     "if (left[x] >= room && (e < 0 || left[x] > left[e])) e = x;", 0),
    ("bounded_piece_ignores_kept_rows", [BOUNDED],
     "pstart[np] = o->keep[r] + (o->D[r] - room);", "pstart[np] = (o->D[r] - room);", 0),
    ("bounded_maxvio_without_minus_one", [BOUNDED],
     "/ (double)NE - 1.0;", "/ (double)NE;", 1),
]


def _mutate(text, old, new, occurrence):
    at = -1
    for _ in range(occurrence + 1):
        at = text.find(old, at + 1)
        assert at >= 0, f"mutation text not found (occurrence {occurrence}): {old!r}"
    return text[:at] + new + text[at + len(old):]


def _build(src_text, out_dir, name):
    c = os.path.join(out_dir, name + ".c")
    so = os.path.join(out_dir, name + ".so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc"] + oracle.CFLAGS + ["-o", so, c, "-lm"])
    return so


def _run_pins(lib, files):
    # one thread per child: the children already run side by side
    env = dict(os.environ, MOONEP_ORACLE_LIB=lib, PYTHONDONTWRITEBYTECODE="1",
               OMP_NUM_THREADS="1")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
           "-m", "not gpu", "-k", "not 4-4-1-2"] + files
    p = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return p.returncode, (p.stdout + p.stderr)[-2000:]


@pytest.fixture(scope="module")
def results():
    with open(SRC) as f:
        text = f.read()
    with tempfile.TemporaryDirectory() as tmp:
        jobs = [("unmodified", [PINS, BOUNDED, BACKWARD], text)]
        for name, files, old, new, occ in MUTANTS:
            jobs.append((name, files, _mutate(text, old, new, occ)))
        libs = {name: _build(src, tmp, name) for name, _, src in jobs}
        workers = max(1, min(8, os.cpu_count() or 1))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            futs = {name: ex.submit(_run_pins, libs[name], files) for name, files, _ in jobs}
            return {name: f.result() for name, f in futs.items()}


def test_unmodified_oracle_passes_through_the_hook(results):
    rc, out = results["unmodified"]
    assert rc == 0, out


@pytest.mark.parametrize("name", [m[0] for m in MUTANTS])
def test_pins_reject_mutant(results, name):
    rc, out = results[name]
    # 1: some pin failed (a crash or an oracle error counts as failing too)
    assert rc != 0, f"mutant {name} passed every pin:\n{out}"
    assert rc != 5, f"no pin ran for mutant {name}:\n{out}"
