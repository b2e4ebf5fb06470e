"""Pin strength: oracle builds with one planted mistake each must fail at
least one pin. The mistakes are planted in a temporary copy of the oracle's
C source, compiled on the CPU; the real oracle is untouched. The verify composition
(Python) gets planted mistakes through a patched function."""

import os

import numpy as np
import pytest

from tests import oracle_pins

# (name, text in mtp_oracle.c, replacement)
MUTATIONS = [
    ("dropped_last_term", "for (int64_t j = 0; j < H; ++j) s += bf16_to_double(x[j]) * bf16_to_double(w[j]);", "for (int64_t j = 0; j + 1 < H; ++j) s += bf16_to_double(x[j]) * bf16_to_double(w[j]);"),
    ("wrong_bf16_shift", "(uint32_t)b << 16", "(uint32_t)b << 15"),
    ("reversed_operand_index", "bf16_to_double(x[j]) * bf16_to_double(w[j])", "bf16_to_double(x[j]) * bf16_to_double(w[H - 1 - j])"),
    ("highest_index_wins_ties", "if (best < 0 || f > best_f)", "if (best < 0 || f >= best_f)"),
    ("argmin_instead_of_argmax", "if (best < 0 || f > best_f)", "if (best < 0 || f < best_f)"),
    ("bonus_token_dropped", "p <= n ? target", "p < n ? target"),
    ("accept_wrong_target_stride", "draft[b * k + n] == target[b * (k + 1) + n]", "draft[b * k + n] == target[b * k + n]"),
    ("pack_ignores_ids", "head + (int64_t)ids[i] * H", "head + i * H"),
    ("runner_up_may_be_top", "if (n == best) continue;", ""),
    ("ids_may_repeat", "ids[i] <= ids[i - 1]", "ids[i] < ids[i - 1]"),
    ("id_map_dropped", "*top_id = ids ? ids[best] : (int32_t)best;", "*top_id = (int32_t)best;"),
    ("pair_rows_swapped", "x + rows[i] * H, w + cols[i] * H", "x + cols[i] * H, w + rows[i] * H"),
    ("logit_not_rounded_from_pick", "*top_logit = best_f;", "*top_logit = (float)z[0];"),
    ("e4m3_bias_8", "ldexp((double)(8 + m), e - 10)", "ldexp((double)(8 + m), e - 11)"),
    ("e4m3_ties_away_from_zero", "nearbyint(ldexp(a, 3 - ue))", "round(ldexp(a, 3 - ue))"),
    ("e4m3_subnormal_spacing", "nearbyint(ldexp(a, 9))", "nearbyint(ldexp(a, 8))"),
    ("e4m3_sign_lost", "const uint8_t s = signbit(x) ? 0x80 : 0x00;", "const uint8_t s = 0x00;"),
    ("fp8_scale_search_dropped", "while (ldexp(448.0, e) < amax) ++e;\n  while (ldexp(448.0, e - 1) >= amax) --e;", ""),
    ("fp8_scale_ignored", "return ldexp(s, e);", "return s;"),
    ("fp8_code_ignores_scale", "mtp_oracle_e4m3_round(ldexp(bf16_to_double(w[j]), -e))", "mtp_oracle_e4m3_round(bf16_to_double(w[j]))"),
    ("e2m1_bias_2", "ldexp((double)(2 + m), e - 2)", "ldexp((double)(2 + m), e - 3)"),
    ("e2m1_ties_away_from_zero", "nearbyint(ldexp(a, 1 - ue))", "round(ldexp(a, 1 - ue))"),
    ("e2m1_subnormal_ties_away", "nearbyint(2.0 * a)", "round(2.0 * a)"),
    ("e2m1_no_saturation", "if (!(a < 6.0)) return s | 7;", "if (!(a < 8.0)) return s | 7;"),
    ("e2m1_sign_lost", "const uint8_t s = x < 0.0 ? 8 : 0;", "const uint8_t s = 0;"),
    ("mx_scale_one_too_high", "ilogb(amax) - 2", "ilogb(amax) - 1"),
    ("mx_zero_block_scale", "amax == 0.0 ? -127", "amax == 0.0 ? 0"),
    ("mx_no_low_clamp", "ilogb(amax) - 2;\n  if (e < -127) e = -127;", "ilogb(amax) - 2;\n"),
    ("mx_fit_no_low_clamp", "++e;\n  }\n  if (e < -127) e = -127;", "++e;\n  }\n"),
    ("mx_nibbles_swapped", "(uint8_t)(lo | (hi << 4))", "(uint8_t)(hi | (lo << 4))"),
    ("mx_logit_scale_stride_16", "const int e = (int)scales[j / 32] - 127;", "const int e = (int)scales[j / 16] - 127;"),
    ("mx_logit_ignores_scale", "s += bf16_to_double(x[j]) * ldexp(mtp_oracle_e2m1_value(code), e);", "s += bf16_to_double(x[j]) * mtp_oracle_e2m1_value(code);"),
    ("mx_logit_nibble_order", "(j & 1) ? (q[j / 2] >> 4) : (q[j / 2] & 15)", "(j & 1) ? (q[j / 2] & 15) : (q[j / 2] >> 4)"),
    ("mx_fit_not_minimal_at_equality", "while (ldexp(6.0, e) < amax) ++e;", "while (ldexp(6.0, e) <= amax) ++e;"),
    ("mx_fit_search_starts_high", "e = ilogb(amax) - 3;", "e = ilogb(amax) - 1;"),
    ("mx_fit_bound_4", "while (ldexp(6.0, e) < amax) ++e;", "while (ldexp(4.0, e) < amax) ++e;"),
    ("mx_fit_rule_ignored", "const int r = rule == 0 ? mtp_oracle_mx_block_exponent(w + 32 * b, 32, &e)", "const int r = 1 ? mtp_oracle_mx_block_exponent(w + 32 * b, 32, &e)"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutant_fails_a_pin(oracle_mod, tmp_path, name, old, new):
    src = open(os.path.join(os.path.dirname(oracle_mod.__file__), "mtp_oracle.c")).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mut = tmp_path / f"{name}.c"
    mut.write_text(src.replace(old, new))
    lib = oracle_mod.build(force=True, src=str(mut), out=str(tmp_path / f"lib{name}.so"))
    failed = []
    with oracle_mod.use_library(lib):
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(oracle_mod)
            except (AssertionError, oracle_mod.OracleError, ValueError, IndexError):
                failed.append(pin.__name__)
                break
    assert failed, f"mutant {name} passed every pin"


def _verify_position_major(oracle_mod):
    """oracle.verify with the rows read position-major (a transposed reshape)."""
    def verify(hv, head, B, k, draft_ids=None):
        r = oracle_mod.argmax(hv, head, None)
        out = {key: v.reshape(k + 1, B).T.copy() for key, v in r.items()}
        if draft_ids is not None:
            out.update(oracle_mod.accept(draft_ids, out["id"]))
        return out
    return verify


def _verify_shifted_target(oracle_mod):
    """oracle.verify comparing draft p with the target of position p + 1."""
    def verify(hv, head, B, k, draft_ids=None):
        r = oracle_mod.argmax(hv, head, None)
        out = {key: v.reshape(B, k + 1) for key, v in r.items()}
        if draft_ids is not None:
            shifted = np.concatenate([out["id"][:, 1:], out["id"][:, -1:]], axis=1)
            out.update(oracle_mod.accept(draft_ids, shifted))
        return out
    return verify


@pytest.mark.parametrize("make", [_verify_position_major, _verify_shifted_target],
                         ids=["verify_position_major", "verify_shifted_target"])
def test_verify_mutant_fails_a_pin(oracle_mod, monkeypatch, make):
    """The verify composition (reshape to [B][k+1], acceptance on it) is
    Python; its planted mistakes must fail a pin too."""
    monkeypatch.setattr(oracle_mod, "verify", make(oracle_mod))
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(oracle_mod)
        except (AssertionError, oracle_mod.OracleError, ValueError, IndexError):
            failed.append(pin.__name__)
            break
    assert failed, "planted verify mistake passed every pin"
