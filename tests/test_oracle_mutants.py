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
    "gqa_mapping": ("err |= attend_row(c, b, h / g, q_pos0(c, b) + t, q_rot + (size_t)row * D,\n"
                    "                          scale, out + (size_t)row * D, lse ? lse + row : NULL,",
                    "err |= attend_row(c, b, h % c->n_kv_heads, q_pos0(c, b) + t, q_rot + (size_t)row * D,\n"
                    "                          scale, out + (size_t)row * D, lse ? lse + row : NULL,"),
    "visible_range": ("err |= attend_row(c, b, h / g, q_pos0(c, b) + t, q_rot + (size_t)row * D,\n"
                      "                          scale, out + (size_t)row * D, lse ? lse + row : NULL,",
                      "err |= attend_row(c, b, h / g, q_pos0(c, b) + t - 1, q_rot + (size_t)row * D,\n"
                      "                          scale, out + (size_t)row * D, lse ? lse + row : NULL,"),
    "no_scale": ("s[j - i0] = scale * dot;", "s[j - i0] = dot;"),
    "no_running_max": ("s[j - i0] = exp(s[j - i0] - m);", "s[j - i0] = exp(s[j - i0]);"),
    "slot_offset": ("int64_t off = pos % c->block_size;", "int64_t off = 0;"),
    "v_from_k_pool": ("out[d] += w * load(c, c->v_pool, idx + d);",
                      "out[d] += w * load(c, c->k_pool, idx + d);"),
    "ties_away": ("double n = nearbyint(a / quantum);", "double n = floor(a / quantum + 0.5);"),
    "double_rounding": ("double a = fabs(x);", "double a = fabs((double)(float)x);"),
    "k_not_rotated": ("store(c, c->k_pool, s + d, y[d]);", "store(c, c->k_pool, s + d, x[d]);"),
    "window_off_by_one": ("? p + 1 - c->window : 0;", "? p + 2 - c->window : 0;"),
    "shard_key_offset": ("int64_t i0 = g0 - k0, i1 = p + 1 - k0;", "int64_t i0 = g0, i1 = p + 1;"),
    "shard_append_slot": ("int64_t local = pos - key_pos0(c, b);", "int64_t local = pos;"),
    "shard_empty_lse": ("*lse = -INFINITY;", "*lse = 0.0;"),
    "ragged_positions": (": key_pos0(c, b) + (int64_t)c->seq_lens[b] - n_new(c, b);",
                         ": key_pos0(c, b) + (int64_t)c->seq_lens[b] - c->q_tokens;"),
    "ragged_padding_attended": ("if (t >= n_new(c, b)) {            /* padding row */\n            for (int32_t d = 0; d < D; ++d)\n                out[(size_t)row * D + d] = 0.0;",
                                "if (t >= n_new(c, b) && 0) {       /* padding row */\n            for (int32_t d = 0; d < D; ++d)\n                out[(size_t)row * D + d] = 0.0;"),
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
