"""Plant plausible mistakes in the oracle (on the CPU) and check that the
pins catch every one of them.

Each mutant is the oracle's C source with one textual change, compiled with
gcc into a temporary directory and loaded as a separate module; the pins of
tests/oracle_pins.py then run against it and at least one must fail.
"""
import importlib.util
import os
import shutil
import sys

import pytest

from tests import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_DIR = os.path.join(ROOT, "oracle")

# (name, original text, planted mistake)
MUTANTS = [
    ("drop_log_count", "(mean_fill == 1 ? log((double)ndrop) : 0.0)", "0.0"),
    ("unit_weight_logged", "(mean_fill == 1 ? log((double)ndrop)", "(mean_fill >= 1 ? log((double)ndrop)"),
    ("register_specials_see_all", "if (j % L >= gh * gw) col[nc++] = j;", "col[nc++] = j;"),
    ("register_specials_own_frame",
     "for (int64_t j = 0; j < T; ++j)\n          if (j % L >= gh * gw)",
     "for (int64_t j = (i / L) * L; j < (i / L) * L + L; ++j)\n          if (j % L >= gh * gw)"),
    ("register_first_special_as_patch", "(mode == ORC_MODE_REGISTER && i % L < gh * gw)",
     "(mode == ORC_MODE_REGISTER && i % L <= gh * gw)"),
    ("register_schedule_phase", "g % register_every == register_every - 1", "g % register_every == 0"),
    ("diag_double_count", "if (diagonal && !keep_mask[i])", "if (diagonal)"),
    ("diag_ignored", "if (diagonal && !keep_mask[i]) col[nc++] = i;", ";"),
    ("no_scale", "z[c] = scale * dot;\n", "z[c] = dot;\n"),
    ("max_sign", "double w = exp(z[c] - zmax);", "double w = exp(zmax - z[c]);"),
    ("value_index", "acc[e] += w * elem(v, dtype, (col[c] * H + h) * d + e);",
     "acc[e] += w * elem(v, dtype, (i * H + h) * d + e);"),
    ("key_head_transposed", "elem(k, dtype, (col[c] * H + h) * d + e)",
     "elem(k, dtype, ((int64_t)h * N * L + col[c]) % ((int64_t)N * L) * H * d + e)"),
    ("phase_swapped", "return (r % sh == oh) && (c % sw == ow);",
     "return (r % sh == ow) && (c % sw == oh);"),
    ("specials_dropped", "if (u >= gh * gw) return 1;", "if (u >= gh * gw) return 0;"),
    ("frame_start", "int64_t f0 = (i / L) * L;", "int64_t f0 = (i / L) * L + 1;"),
    ("mean_over_kept", "if (sga_keeps((int32_t)(t % L), gh, gw, sh, sw, oh, ow)) continue;",
     "if (!sga_keeps((int32_t)(t % L), gh, gw, sh, sw, oh, ow)) continue;"),
    ("mean_not_divided", "kmean[i] /= (double)nd;", ";"),
    ("schedule_off_by_one", "out[g] = g < num_early ?", "out[g] = g <= num_early ?"),
    ("mean_value_is_key", "acc[e] += w * vmean[h * d + e];", "acc[e] += w * kmean[h * d + e];"),
    ("linear_weight_transposed", "elem(w, dtype, (int64_t)n * K + k)",
     "elem(w, dtype, (int64_t)k * N + n)"),
    ("linear_bias_dropped", "y[m * N + n] = acc + (b ? elem(b, dtype, n) : 0.0);",
     "y[m * N + n] = acc;"),
    ("linear_bias_by_row", "elem(b, dtype, n)", "elem(b, dtype, m % N)"),
    ("qkv_k_v_swapped", "k[m * C + c] = y[m * 3 * C + C + c];",
     "k[m * C + c] = y[m * 3 * C + 2 * C + c];"),
    ("softmax_not_normalised", "out[(r * H + h) * d + e] = acc[e] / wsum;",
     "out[(r * H + h) * d + e] = acc[e];"),
    ("mean_column_outside_denominator", "wsum += w;\n        if (col[c] >= 0) {",
     "if (col[c] >= 0) {\n          wsum += w;"),
    ("frame_misses_last_key", "for (int64_t j = f0; j < f0 + L; ++j) col[nc++] = j;",
     "for (int64_t j = f0; j < f0 + L - 1; ++j) col[nc++] = j;"),
    ("keep_idx_without_frame_offset", "int64_t t = (int64_t)f * L + u;", "int64_t t = u;"),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(os.path.join(ORACLE_DIR, "vga_oracle.c")).read()
    assert src.count(old) >= 1, "mutation anchor not found: %s" % name
    pkg = tmp_path / ("oracle_mut_" + name)
    pkg.mkdir()
    for f in ("__init__.py", "brute.py"):
        shutil.copy(os.path.join(ORACLE_DIR, f), pkg / f)
    (pkg / "vga_oracle.c").write_text(src.replace(old, new, 1))
    modname = "oracle_mut_" + name
    spec = importlib.util.spec_from_file_location(modname, str(pkg / "__init__.py"))
    mod = importlib.util.module_from_spec(spec)
    sys.modules[modname] = mod
    spec.loader.exec_module(mod)
    mod.build(force=True)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    mod = _build_mutant(tmp_path, name, old, new)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, FloatingPointError) as exc:  # noqa: PERF203
            caught.append(pin.__name__)
    assert caught, "planted mistake %r passed every pin" % name
