"""Plants one mistake at a time in a copy of the oracle's C source (on the CPU,
in a temporary directory) and checks that the pin tests catch every one."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = {
    "nibble_order": ("((c & 1) * 4)", "((1 - (c & 1)) * 4)"),
    "twos_complement": ("return (nib ^ 8) - 8;", "return nib - 8;"),
    "scale_index": ("srow[c / gs]", "srow[(c / gs + 1) % (cols / gs)]"),
    "swap_gate_up": ("silu(g[t]) * u[t]", "silu(u[t]) * g[t]"),
    "silu_sign": ("z / (1.0 + exp(-z))", "z / (1.0 + exp(z))"),
    "down_scale_array": ("oracle_dequant_row(v.down_q, v.down_s,", "oracle_dequant_row(v.down_q, v.up_s,"),
    "tie_to_highest_id": ("(sa == sb && ia < ib)", "(sa == sb && ia > ib)"),
    "bias_dropped": ("double l = b_router ? (double)b_router[e] : 0.0;", "double l = 0.0;"),
    "bias_sign": ("double l = b_router ? (double)b_router[e] : 0.0;",
                  "double l = b_router ? -(double)b_router[e] : 0.0;"),
    "shared_dropped": ("if (shared)\n        oracle_expert_mlp", "if (0)\n        oracle_expert_mlp"),
    "perm_order_reversed": ("perm[offsets[e] + cur[e]++] = a;", "perm[offsets[e + 1] - 1 - cur[e]++] = a;"),
    "combine_weight_slot": ("double w = (double)topk_w[(size_t)t * k + j];",
                            "double w = (double)topk_w[(size_t)t * k];"),
    "rms_mean": ("sqrt(ss / d + eps)", "sqrt(ss / (d - 1) + eps)"),
    "lru_evicts_most_recent": ("(victim < 0 || last_use[s] < last_use[victim])",
                               "(victim < 0 || last_use[s] > last_use[victim])"),
    "lru_ties_to_highest_slot": ("(victim < 0 || last_use[s] < last_use[victim])",
                                 "(victim < 0 || last_use[s] <= last_use[victim])"),
    "lru_hit_not_refreshed": ("                taken[s] = 1;\n                last_use[s] = *clock;\n                ++h;",
                              "                taken[s] = 1;\n                ++h;"),
    "hottest_ties_to_higher_id": ("counters[order[j - 1]] < counters[e]",
                                  "counters[order[j - 1]] <= counters[e]"),
}


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    old, new = MUTATIONS[name]
    assert old in src
    c = tmp_path / "oracle.c"
    c.write_text(src.replace(old, new, 1))
    so = tmp_path / "liboracle.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", str(c),
                           "-o", str(so), "-lm"])
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True)
    assert r.returncode != 0, f"planted mistake {name!r} passed every pin"
