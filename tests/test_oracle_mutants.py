"""Plant plausible mistakes in copies of the oracle and check the pins catch them.

Each mutant is a one-line textual change to a copy of ``oracle/moe_oracle.c``
(a transposed operand, a dropped term, a wrong sign or index, a wrong
tie-break), built into a temporary library and run against
``test_oracle_pins.py`` in a subprocess through ``ORACLE_LIB``.  The pins must
fail for every mutant.  Everything here runs on the CPU; the real oracle is
never modified.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

MUTANTS = {
    "gate_transposed": ("g += oracle_bf16_to_f32(x[c]) * oracle_bf16_to_f32(Wg[i * H + c]);",
                        "g += oracle_bf16_to_f32(x[c]) * oracle_bf16_to_f32(Wg[c * I + i]);"),
    "down_transposed": ("acc += oracle_bf16_to_f32(h[i]) * oracle_bf16_to_f32(Wd[n * I + i]);",
                        "acc += oracle_bf16_to_f32(h[i]) * oracle_bf16_to_f32(Wd[i * H + n]);"),
    "silu_sign": ("float silu_g = g / (1.0f + expf(-g));\n        h[i] = oracle_f32_to_bf16(silu_g * u);\n    }\n#pragma omp parallel for schedule(static)\n    for (int64_t n = 0; n < H; ++n) {\n        float acc",
                  "float silu_g = g / (1.0f + expf(g));\n        h[i] = oracle_f32_to_bf16(silu_g * u);\n    }\n#pragma omp parallel for schedule(static)\n    for (int64_t n = 0; n < H; ++n) {\n        float acc"),
    "silu_on_up": ("float silu_g = g / (1.0f + expf(-g));\n        h[i] = oracle_f32_to_bf16(silu_g * u);\n    }\n#pragma omp parallel for schedule(static)\n    for (int64_t n = 0; n < H; ++n) {\n        float acc",
                   "float silu_g = u / (1.0f + expf(-u));\n        h[i] = oracle_f32_to_bf16(silu_g * g);\n    }\n#pragma omp parallel for schedule(static)\n    for (int64_t n = 0; n < H; ++n) {\n        float acc"),
    "dropped_route_weight": ("acc[n] += w[slot] * y[n];", "acc[n] += y[n];"),
    "slot_index": ("int64_t slot = t * k + j;", "int64_t slot = j * T + t;"),
    "dropped_last_term": ("for (int64_t c = 0; c < H; ++c)\n            g +=",
                          "for (int64_t c = 0; c < H - 1; ++c)\n            g +="),
    "router_tie_break": ("if (best < 0 || l[e] > l[best]) best = e;",
                         "if (best < 0 || l[e] >= l[best]) best = e;"),
    "router_no_renorm": ("topk_w[t * k + j] = (float)(p[topk_ids[t * k + j]] / kept);",
                         "topk_w[t * k + j] = (float)(p[topk_ids[t * k + j]]);"),
    "permute_reverse": ("for (int64_t s = 0; s < n_slots; ++s)\n            if (topk_ids[s] == e)",
                        "for (int64_t s = n_slots - 1; s >= 0; --s)\n            if (topk_ids[s] == e)"),
    "bf16_truncate": ("u += 0x7fffu + keep_lsb;", "u += 0u * keep_lsb;"),
    "int8_scale_dropped": ("acc += s[g0 / group] * part;", "acc += part;"),
    "int8_group_index": ("acc += s[g0 / group] * part;", "acc += s[0] * part;"),
    # decode attention (pins in test_oracle_attn_pins.py)
    "attn_head_mapping": ("const int32_t j = h / g;", "const int32_t j = h % h_kv;"),
    "attn_no_scale": ("s[t] = scale * dot;", "s[t] = dot;"),
    "attn_values_from_keys": ("acc[c] += s[t] * oracle_bf16_to_f32(vh[(size_t)t * d + c]);",
                              "acc[c] += s[t] * oracle_bf16_to_f32(kh[(size_t)t * d + c]);"),
    "attn_last_position_dropped": ("for (int32_t t = 0; t < n; ++t)\n                for (int32_t c = 0; c < d; ++c)\n                    acc[c]",
                                   "for (int32_t t = 0; t < n - 1; ++t)\n                for (int32_t c = 0; c < d; ++c)\n                    acc[c]"),
    "attn_not_normalised": ("oh[c] = oracle_f32_to_bf16(acc[c] / L);",
                            "oh[c] = oracle_f32_to_bf16(acc[c]);"),
    # residual-split weights (pins in test_oracle_resplit_pins.py)
    "resplit_gate_residual_dropped": (
        "g = g + grouped_dot(x, Rg + i * H, SRg + i * (H / group), H, group);", "g = g;"),
    "resplit_up_residual_dropped": (
        "u = u + grouped_dot(x, Ru + i * H, SRu + i * (H / group), H, group);", "u = u;"),
    "resplit_residual_with_first_scales": (
        "g = g + grouped_dot(x, Rg + i * H, SRg + i * (H / group), H, group);",
        "g = g + grouped_dot(x, Rg + i * H, Sg + i * (H / group), H, group);"),
    "resplit_down_copies_swapped": (
        "const int8_t* qd = crit ? Qd_hi[e] : Qd_lo[e];\n            const float* sd = crit ? Sd_hi[e] : Sd_lo[e];",
        "const int8_t* qd = crit ? Qd_lo[e] : Qd_hi[e];\n            const float* sd = crit ? Sd_lo[e] : Sd_hi[e];"),
    "resplit_flag_by_slot": ("int crit = critical[e] != 0;", "int crit = critical[slot % E] != 0;"),
    # grouped sigmoid router (pins in test_oracle_route_grouped_pins.py)
    "grouped_group_score_max_only": ("gs[g] = b2 < 0 ? c[b1] : c[b1] + c[b2];", "gs[g] = c[b1];"),
    "grouped_bias_in_weights": ("topk_w[t * k + j] = s[topk_ids[t * k + j]] / sum * scale;",
                                "topk_w[t * k + j] = c[topk_ids[t * k + j]] / sum * scale;"),
    "grouped_groups_not_masked": ("if (chosen[e] || !kept[e / G]) continue;",
                                  "if (chosen[e]) continue;"),
    "grouped_group_tie_break": ("if (!kept[g] && (best < 0 || gs[g] > gs[best])) best = g;",
                                "if (!kept[g] && (best < 0 || gs[g] >= gs[best])) best = g;"),
    "grouped_exp_not_sigmoid": ("s[e] = 1.0f / (1.0f + expf(-l[e]));", "s[e] = expf(l[e]);"),
}


def pin_file(name: str) -> str:
    if name.startswith("attn_"):
        return "test_oracle_attn_pins.py"
    if name.startswith("resplit_"):
        return "test_oracle_resplit_pins.py"
    if name.startswith("grouped_"):
        return "test_oracle_route_grouped_pins.py"
    return "test_oracle_pins.py"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not found exactly once"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-std=c11", str(src), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", pin_file(name))],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout or "Error" in r.stdout
