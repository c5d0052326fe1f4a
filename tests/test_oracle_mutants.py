"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that the pins catch every one of them."""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "kvd_oracle.c")

MUTANTS = {
    "rope_sign": ("y[ia] = a * cs - c * sn;", "y[ia] = a * cs + c * sn;"),
    "rope_frequency": ("-2.0 * (double)i / (double)D", "-1.0 * (double)i / (double)D"),
    "rope_pairing": ("ia = 2 * i;", "ia = i;"),
    "q_position": ("rope_one(x, q_rot + o, D, pos, base, layout);",
                   "rope_one(x, q_rot + o, D, pos + 1, base, layout);"),
    "gqa_mapping": ("err |= attend_row(c, b, h / g, n_vis, q_rot + (size_t)row * D, scale,\n"
                    "                          out + (size_t)row * D,",
                    "err |= attend_row(c, b, h % c->n_kv_heads, n_vis, q_rot + (size_t)row * D, scale,\n"
                    "                          out + (size_t)row * D,"),
    "visible_range": ("int64_t n_vis = (int64_t)c->seq_lens[b] - T + t + 1;\n        err |= attend_row(c, b, h / g, n_vis, q_rot + (size_t)row * D, scale,\n                          out + (size_t)row * D,",
                      "int64_t n_vis = (int64_t)c->seq_lens[b] - T + t;\n        err |= attend_row(c, b, h / g, n_vis, q_rot + (size_t)row * D, scale,\n                          out + (size_t)row * D,"),
    "no_scale": ("s[j] = scale * dot;", "s[j] = dot;"),
    "no_running_max": ("s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
    "slot_offset": ("int64_t off = pos % c->block_size;", "int64_t off = 0;"),
    "v_from_k_pool": ("out[d] += w * load(c, c->v_pool, idx + d);",
                      "out[d] += w * load(c, c->k_pool, idx + d);"),
    "ties_away": ("double n = nearbyint(a / quantum);", "double n = floor(a / quantum + 0.5);"),
    "double_rounding": ("double a = fabs(x);", "double a = fabs((double)(float)x);"),
    "k_not_rotated": ("store(c, c->k_pool, s + d, y[d]);", "store(c, c->k_pool, s + d, x[d]);"),
    "window_off_by_one": ("? n_vis - c->window : 0;", "? n_vis - c->window + 1 : 0;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, f"mutation anchor for {name} not found exactly once"
    shutil.copy(os.path.join(os.path.dirname(SRC), "kvd_oracle.h"), tmp_path)
    mutant = tmp_path / "kvd_oracle.c"
    mutant.write_text(src.replace(before, after))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(lib),
                    str(mutant), "-lm"], check=True)
    r = subprocess.run([sys.executable, os.path.join(HERE, "run_pins.py"), str(lib)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout}\n{r.stderr}"
