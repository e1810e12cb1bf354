"""Plant plausible mistakes in a copy of the oracle and check a pin catches each.

The mutants are built on the CPU from a patched copy of oracle/afd_oracle.c in
a temporary directory; the committed oracle is never modified.
"""
import os

import pytest

import oracle_pins
from oracle import oracle as orc

SRC = os.path.join(os.path.dirname(orc.__file__), "afd_oracle.c")

MUTANTS = {
    "silu_sign": ("g[i] = (z / (1.0 + exp(-z))) * u[i];", "g[i] = (z / (1.0 + exp(z))) * u[i];"),
    "drop_up": ("g[i] = (z / (1.0 + exp(-z))) * u[i];", "g[i] = (z / (1.0 + exp(-z)));"),
    "silu_on_up": ("double z = g[i];", "double z = u[i]; u[i] = g[i];"),
    "drop_weight": ("y[h] += w * f[h];", "y[h] += f[h];"),
    "wrong_expert": ("ffn_view v = routed_view(p, e);", "ffn_view v = routed_view(p, e > 0 ? e - 1 : e);"),
    "skip_last_slot": ("for (int k = 0; k < K; ++k) {", "for (int k = 0; k + 1 < K; ++k) {"),
    "drop_shared": ("    if (p->shared_inter > 0) {\n        ffn_view v = shared_view(p);",
                    "    if (p->shared_inter < 0) {\n        ffn_view v = shared_view(p);"),
    "down_transposed": ("f[h] += a * elem(v->dtype, v->wd, v->od, H, v->sd, i, h);",
                        "f[h] += a * elem(v->dtype, v->wd, v->od, H, v->sd, h % Is, i % H);"),
    "scale_grid_transposed": ("scales[(size_t)(r / 128) * bc + (c / 128)]",
                              "scales[(size_t)(c / 128) * bc + (r / 128)]"),
    "act_scale_dropped": ("(double)p->hidden_scales[(size_t)t * (H / 128) + h / 128];", "1.0;"),
    "e4m3_bias": ("v = ldexp(1.0 + (double)m / 8.0, e - 7);", "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "bf16_shift": ("uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    "dispatch_unstable": ("for (int64_t f = 0; f < n; ++f) {\n        int e = ids[f];",
                          "for (int64_t f = n - 1; f >= 0; --f) {\n        int e = ids[f];"),
    "dispatch_inclusive": ("offsets[e + 1] = offsets[e] + counts[e];",
                           "offsets[e + 1] = offsets[e] + counts[e] + (e == 0);"),
    "row_of_skipped": ("row_of[f] = -1;", "row_of[f] = 0;"),
    "i8_unsigned": ("return (double)(raw < 128 ? (int)raw : (int)raw - 256);", "return (double)raw;"),
    "i8_scale_by_row": ("afd_oracle_i8_to_f64(((const uint8_t *)base)[i]) * (double)scales[c];",
                        "afd_oracle_i8_to_f64(((const uint8_t *)base)[i]) * (double)scales[r % cols];"),
    "i8_token_scale_dropped": ("(double)p->hidden_scales[t];", "1.0;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor for %s not unique" % name
    path = tmp_path / ("mut_%s.c" % name)
    path.write_text(src.replace(old, new))
    lib = orc.load(orc.build(force=True, src=str(path), out=str(tmp_path / ("libmut_%s.so" % name))))
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except Exception as exc:  # AssertionError or a rejected problem
            caught.append("%s: %s" % (pin.__name__, str(exc)[:60]))
    assert caught, "mutant %s passed every pin" % name
