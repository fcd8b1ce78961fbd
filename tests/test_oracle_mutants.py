"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a private copy of oracle/oracle_f64.c (on the
CPU, never on a GPU; built at session start by tests/native_builds.py) and requires that at least one pin from
tests/oracle_pins.py fails against the broken build while all pass against
the real one.
"""
import pytest

import oracle
from tests import native_builds
from tests import oracle_pins as pins

MUTANTS = {
    "window_off_by_one": ("lo = p - (int64_t)J->window + 1;", "lo = p - (int64_t)J->window;"),
    "causal_excludes_self": ("int64_t hi = is_causal ? p : T - 1;", "int64_t hi = is_causal ? p - 1 : T - 1;"),
    "noncausal_drops_last_key": ("int64_t hi = is_causal ? p : T - 1;", "int64_t hi = is_causal ? p : T - 2;"),
    "gqa_modulo_mapping": ("const int32_t g = h / G;", "const int32_t g = h % J->Hkv;"),
    "scale_dropped": ("z[j - lo] = J->scale * acc;", "z[j - lo] = acc;"),
    "exp_sign_flipped": ("z[j - lo] = exp(z[j - lo] - m);", "z[j - lo] = exp(m - z[j - lo]);"),
    "logits_use_values": ("const uint16_t *kr = J->k +", "const uint16_t *kr = J->v +"),
    "output_uses_keys": ("const uint16_t *vr = J->v +", "const uint16_t *vr = J->k +"),
    "missing_normalisation": ("o[d] = o[d] / s;", "o[d] = o[d];"),
    "wrong_request_base": ("const int64_t base = J->kv_start[r];", "const int64_t base = J->q_start[r];"),
    "window_ignored": ("if (J->window > 0) {", "if (J->window > 1000000) {"),
    "causal_ignored": ("int64_t hi = is_causal ? p : T - 1;", "int64_t hi = T - 1;"),
}


def _any_pin_fails(lib) -> bool:
    orc = lambda *a, **kw: oracle.block_attn_f64(*a, lib=lib, **kw)  # noqa: E731
    for check in pins.ALL_CHECKS:
        try:
            check(orc)
        except (AssertionError, RuntimeError, ValueError, FloatingPointError):
            return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    # the mutant libraries were compiled at session start (tests/native_builds.py)
    so = native_builds.get("mutants")[name]
    assert _any_pin_fails(oracle.bind(so)), f"no pin caught the planted mistake {name}"
