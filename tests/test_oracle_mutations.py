"""Plant plausible mistakes in a copy of the oracle and check the pins catch them.

Each mutation is a textual edit of oracle/pkv_oracle.c compiled into a
temporary shared object (on the CPU, never near a GPU).  The pin suite
tests/test_oracle_pins.py is then run in a child process against that copy
and must fail.  This is what makes the pins evidence: a dropped term, a wrong
sign, a wrong index or a swapped operand cannot pass them.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "pkv_oracle.c")

MUTATIONS = {
    "causal-bound-exclusive": ("L - n + i + 1", "L - n + i"),
    "gqa-map-modulo": ("  int g = h / G;\n  int64_t page = p->k_table", "  int g = h % p->num_kv_heads;\n  int64_t page = p->k_table"),
    "drop-v-scale": ("out[d] = p->v_scale * out[d] / l;", "out[d] = out[d] / l;"),
    "drop-k-scale": ("return p->scale * p->k_scale * dot;", "return p->scale * dot;"),
    "softmax-sign": ("double w = exp(s[j - j0] - m);", "double w = exp(m - s[j - j0]);"),
    "token-offset-shift": ("int64_t off = key_offset(page, g, j % p->page_size, p->k_page_stride",
                           "int64_t off = key_offset(page, g, (j + 1) % p->page_size, p->k_page_stride"),
    "value-head-token-swap": ("p->v_page_stride, p->v_head_stride,\n                           p->v_tok_stride",
                              "p->v_page_stride, p->v_tok_stride,\n                           p->v_head_stride"),
    "lse-without-log": ("*lse = m + log(l);", "*lse = m + l;"),
    "e4m3-bias": ("mag = ldexp(1.0 + (double)m / 8.0, e - 7);", "mag = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "e4m3-subnormal-scale": ("mag = ldexp((double)m / 8.0, -6);", "mag = ldexp((double)m / 8.0, -7);"),
    "merge-weight-sign": ("double w = (ls == -INFINITY) ? 0.0 : exp(ls - mx);",
                          "double w = (ls == -INFINITY) ? 0.0 : exp(mx - ls);"),
    "bf16-shift": ("uint32_t u = (uint32_t)bits << 16;", "uint32_t u = (uint32_t)bits << 15;"),
    "split-drops-last-key": ("int64_t j1 = (int64_t)(sp + 1) * pps * p->page_size;",
                             "int64_t j1 = (int64_t)(sp + 1) * pps * p->page_size - 1;"),
    "value-table-is-key-table-row0": ("int64_t page = p->v_table[(int64_t)b * p->table_stride + j / p->page_size];",
                                      "int64_t page = p->v_table[j / p->page_size];"),
    "v-row-from-next-token": ("int64_t off = key_offset(page, g, j % p->page_size, p->v_page_stride",
                              "int64_t off = key_offset(page, g, (j + 1) % p->page_size, p->v_page_stride"),
    "max-not-subtracted-lse": ("*lse = m + log(l);", "*lse = log(l);"),
    "sink-weight-sign": ("double lse2 = hi + log(exp(a - hi) + exp(sigma - hi));",
                         "double lse2 = hi + log(exp(a - hi) + exp(hi - sigma));"),
    "sink-output-not-rescaled": ("for (int d = 0; d < dv; ++d) out[d] *= f;", "for (int d = 0; d < dv; ++d) out[d] *= 1.0;"),
}


def _run_pins_against(src_text: str, tmp_path) -> subprocess.CompletedProcess:
    mutated = tmp_path / "mut.c"
    mutated.write_text(src_text)
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", str(so), str(mutated), "-lm"])
    env = dict(os.environ, PKV_ORACLE_LIB=str(so))
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def test_control_unmutated_copy_passes(tmp_path):
    r = _run_pins_against(open(SRC).read(), tmp_path)
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/absent"
    r = _run_pins_against(src.replace(old, new), tmp_path)
    assert r.returncode == 1, f"pins did not catch mutation {name} (rc={r.returncode}):\n{r.stdout[-2000:]}"
