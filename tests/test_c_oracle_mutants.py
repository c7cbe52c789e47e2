"""Plausible mistakes planted in copies of the C oracle must fail a check
(CPU only).

Each mutant is one text substitution in a copy of oracle/verify_ref.c built
into a temporary library; the oracle's own source is never changed.  The
checks are the pins of the NumPy oracle and the agreement with it on small
seeded batches.
"""
import numpy as np
import pytest

import oracle.verify as vm
import oracle.verify_c as vc
import synth
from tests import oracle_pins as pins

MUTANTS = {
    "accept_le": ("return u * q_y < p_y;", "return u * q_y <= p_y;"),
    "accept_swapped": ("return u * q_y < p_y;", "return u * p_y < q_y;"),
    "accept_margin_absolute": ("return top == 0.0 ? 1.0 : fabs(a - b) / top;",
                               "return top == 0.0 ? 1.0 : fabs(a - b);"),
    "residual_transposed": ("const double d = p[v] - q[v];", "const double d = q[v] - p[v];"),
    "residual_unclamped": ("r[v] = d > 0.0 ? d : 0.0;", "r[v] = fabs(d);"),
    "cdf_left_side": ("if (c > thr) {", "if (c >= thr) {"),
    "draw_margin_absolute": (
        "*margin = tot > 0.0 ? fmin(fabs(lo - thr), fabs(hi - thr)) / tot : 0.0;",
        "*margin = tot > 0.0 ? fmin(fabs(lo - thr), fabs(hi - thr)) : 0.0;"),
    "softmax_ignores_T": ("p[v] = exp((z[v] - m) / T);", "p[v] = exp(z[v] - m);"),
    "temperature_not_widened": ("in.T = oracle_widen_temperature(temperature);",
                                "in.T = temperature;"),
    "argmax_highest_id": ("if (z[v] > z[best]) best = v;", "if (z[v] >= z[best]) best = v;"),
    "greedy_next_row": ("load_row(in->target, in->elem_bytes, t0 + i, in->target_ld, in->V, z);",
                        "load_row(in->target, in->elem_bytes, t0 + i + 1, in->target_ld, in->V, z);"),
    "q_from_target_rows": ("load_row(in->draft, in->elem_bytes, d0 + i, in->draft_ld, V, z);",
                           "load_row(in->target, in->elem_bytes, t0 + i, in->target_ld, V, z);"),
    "bonus_from_previous_row": (
        "load_row(in->target, in->elem_bytes, t0 + k, in->target_ld, V, z);",
        "load_row(in->target, in->elem_bytes, t0 + (k > 0 ? k - 1 : 0), in->target_ld, V, z);"),
    "no_cut_at_reject": ("if (cut) continue;", ";"),
    "final_uniform_flipped": ("(double)u_final[b]", "1.0 - (double)u_final[b]"),
    "last_kept_draft_dropped": ("for (int64_t i = 0; i < r.a; ++i) out_tokens[t0 + i]",
                                "for (int64_t i = 0; i + 1 < r.a; ++i) out_tokens[t0 + i]"),
}


def _agreement(co):
    for cfg, kw in ((3, dict(B=4, V=500)), (5, dict(B=16, V=3001)), (1, {})):
        d = synth.as_numpy(synth.make_batch(cfg, "cpu", **kw))
        ref = vm.verify_batch(**d)
        got = co.verify_batch(**d, threads=2)
        assert np.array_equal(got["accepted_len"], ref["accepted_len"])
        assert np.array_equal(got["out_tokens"], ref["out_tokens"])
        for key in ("p_draft", "q_draft"):
            assert np.all(np.abs(got[key] - ref[key]) <= 1e-12), key
        fin = np.isfinite(ref["margin"])
        assert np.array_equal(np.isfinite(got["margin"]), fin)
        assert np.all(np.abs(got["margin"][fin] - ref["margin"][fin]) <= 1e-9)


CHECKS = [pins.pin_abr_example, pins.pin_weather_example, pins.pin_t1_t4_round,
          pins.pin_greedy_ties, pins.pin_packed_batch, pins.pin_decision_margins,
          pins.pin_special_cases, pins.pin_greedy_invariants, pins.pin_temperature_reading,
          _agreement]


def test_unmutated_copy_passes(tmp_path):
    so = vc.build_library(source=vc.SOURCE, out=str(tmp_path / "liboracle_copy.so"))
    co = vc.COracle(so)
    for check in CHECKS:
        check(co)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    with open(vc.SOURCE) as f:
        src = f.read()
    assert src.count(old) == 1, f"{name}: the text to mutate must occur once"
    path = tmp_path / f"verify_{name}.c"
    path.write_text(src.replace(old, new))
    so = vc.build_library(source=str(path), out=str(tmp_path / f"lib_{name}.so"))
    co = vc.COracle(so)
    for check in CHECKS:
        try:
            check(co)
        except (AssertionError, ValueError, RuntimeError, IndexError):
            return
    pytest.fail(f"mutant {name} passed every check")
