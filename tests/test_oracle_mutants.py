"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins reject every one of them, so a passing pin suite means something."""
import os
import subprocess

import pytest

import oracle
from oracle import build as oracle_build
from oracle_pins import ALL_PINS

# (name, text in attn_ref.c, replacement)
MUTANTS = [
    ("dropped_scale", "s[j] = scale * dot;", "s[j] = dot;"),
    ("transposed_k", "dot += qrow[c] * K[j * d + c];", "dot += qrow[c] * K[c * N + j];"),
    ("transposed_v", "orow[c] += w * V[j * d + c];", "orow[c] += w * V[c * N + j];"),
    ("no_normalisation", "for (int64_t c = 0; c < d; ++c) orow[c] /= l;", ""),
    ("lse_without_max", "*lse_out = m + log(l);", "*lse_out = log(l);"),
    ("exp_sign_flipped", "s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    ("max_starts_at_zero", "double m = -INFINITY;", "double m = 0.0;"),
    ("min_instead_of_max", "if (s[j] > m) m = s[j];", "if (s[j] < m) m = s[j];"),
    ("bf16_shift", "(uint32_t)bits << 16;", "(uint32_t)bits << 15;"),
    ("fp16_bias", "expo - 25);", "expo - 24);"),
    ("fp16_subnormal", "ldexp((double)man, -24);", "ldexp((double)man, -25);"),
    ("q_row_ignores_head", "J->q + flat * d;", "J->q + (flat % Nq) * d;"),
    ("k_ignores_head", "J->k + kv_head * Nk * d;", "J->k;"),
    ("v_ignores_head", "J->v + kv_head * Nk * d;", "J->v;"),
    ("head_reload_skipped", "if (kv_head != loaded_head) {", "if (loaded_head < 0) {"),
    ("gqa_heads_interleaved", "(head % J->Hq) / group;", "(head % J->Hq) % J->Hkv;"),
    ("causal_off_by_one", "visible = i + 1 + Nk - Nq;", "visible = i + Nk - Nq;"),
    ("causal_top_left", "if (J->causal && i + 1 + Nk - Nq < visible) visible = i + 1 + Nk - Nq;",
     "if (J->causal && i + 1 < visible) visible = i + 1;"),
    ("empty_row_lse_zero", "*lse_out = -INFINITY;", "*lse_out = 0.0;"),
    ("sampled_row_position_from_sample", "int64_t head = flat / Nq, i = flat % Nq;",
     "int64_t head = flat / Nq, i = r % Nq;"),
    # INT8 key/value cache
    ("int8_truncates", "float code = rintf(u * inv);", "float code = truncf(u * inv);"),
    ("int8_ties_away", "float code = rintf(u * inv);", "float code = roundf(u * inv);"),
    ("int8_exact_rationals", "float code = rintf(u * inv);",
     "float code = (float)rint((double)u * 127.0 / (double)amax);"),
    ("int8_amax_signed", "if (fabsf(u) > amax) amax = fabsf(u);", "if (u > amax) amax = u;"),
    ("int8_sq_over_128", "return amax / 127.0f;", "return amax / 128.0f;"),
    ("int8_key_scale_not_folded", "const float u = (float)q[c] * ks[c];\n    if",
     "const float u = (float)q[c];\n    if"),
    ("int8_value_scale_dropped", "V[t] = (double)vs[t % d] * (double)vh[t];",
     "V[t] = (double)vh[t];"),
    ("int8_value_scale_by_key", "V[t] = (double)vs[t % d] * (double)vh[t];",
     "V[t] = (double)vs[(t / d) % d] * (double)vh[t];"),
    ("int8_row_scale_dropped", "row_scale = J->scale * (double)sq;", "row_scale = J->scale;"),
    ("int8_wrong_head_scales", "quantize_q_row(q, J->ks + kv_head * d, d, q);",
     "quantize_q_row(q, J->ks, d, q);"),
    # FP8 key/value cache
    ("fp8_bias_8", "mag = ldexp((double)(8 + m), e - 10);", "mag = ldexp((double)(8 + m), e - 11);"),
    ("fp8_subnormal_scale", "mag = ldexp((double)m, -9);", "mag = ldexp((double)m, -10);"),
    ("fp8_nan_code_finite", "if (e == 15 && m == 7)", "if (0)"),
    ("fp8_ties_up", "((lo & 1) == 0 ? lo : hi)", "hi"),
    ("fp8_ties_down", "((lo & 1) == 0 ? lo : hi)", "lo"),
    ("fp8_sign_dropped", "return signbit(x) ? (uint8_t)(code | 0x80) : code;", "return code;"),
    ("fp8_127_not_448", "const float to448 = 448.0f / top;", "const float to448 = 127.0f / top;"),
    ("fp8_sq_over_127", "return top / 448.0f;", "return top / 127.0f;"),
    ("fp8_key_scale_not_folded", "const float uk = (float)q[c] * ks[c];\n    const uint8_t",
     "const float uk = (float)q[c];\n    const uint8_t"),
    ("fp8_value_scale_dropped", "V[t] = (double)vs[t % d] * decode_e4m3(vh[t]);",
     "V[t] = decode_e4m3(vh[t]);"),
    ("fp8_row_scale_dropped", "row_scale = (double)sqf * J->scale;", "row_scale = J->scale;"),
    ("fp8_codes_as_int8", "K[t] = decode_e4m3(kh[t]);", "K[t] = (double)(int8_t)kh[t];"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(tmp_path, name, old, new):
    src = open(oracle_build.SRC).read()
    assert src.count(old) == 1, "mutation site not unique: %r" % old
    mutated = tmp_path / "attn_mut.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / ("liboracle_%s.so" % name)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                    "-w", "-o", str(lib), str(mutated), "-lm"], check=True)
    orc = oracle.Oracle(str(lib))
    caught = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "no pin rejects mutant %s" % name
