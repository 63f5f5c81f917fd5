"""Plant plausible mistakes in a copy of oracle/append.py and check that the
pins of tests/test_append_oracle.py catch every one (and pass on an unchanged
copy)."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "append.py")

MUTATIONS = {
    "rope-sign": ("return np.concatenate([lo * c - hi * s, hi * c + lo * s])",
                  "return np.concatenate([lo * c + hi * s, hi * c - lo * s])"),
    "rope-cos-sin-swapped": ("c, s = cs_row[:HALF], cs_row[HALF:]", "s, c = cs_row[:HALF], cs_row[HALF:]"),
    "rms-sum-not-mean": ("return x / np.sqrt(np.mean(x * x) + eps) * w", "return x / np.sqrt(np.sum(x * x) + eps) * w"),
    "rms-drops-eps": ("return x / np.sqrt(np.mean(x * x) + eps) * w", "return x / np.sqrt(np.mean(x * x)) * w"),
    "rms-drops-weight": ("return x / np.sqrt(np.mean(x * x) + eps) * w", "return x / np.sqrt(np.mean(x * x) + eps)"),
    "position-off-by-one": ("pos = r + L - hi", "pos = r + L - hi - 1"),
    "policies-swapped": ("if prob.norm_policy == 1:", "if prob.norm_policy == 2:"),
    "tail-starts-one-early": ("for slot in range((L - 1) % P + 1, P):", "for slot in range((L - 1) % P, P):"),
    "k-scale-multiplied": ("k_rows[(page, slot, g)] = k / prob.k_scale if e4m3 else k",
                           "k_rows[(page, slot, g)] = k * prob.k_scale if e4m3 else k"),
    "values-rotated": ("v = qkv[r, Hq + Hkv + g]", "v = rope(qkv[r, Hq + Hkv + g], cs[pos])"),
    "query-uses-key-weights": ("y = qk_transform(qkv[r, h], qw, cs[pos])",
                               "y = qk_transform(qkv[r, h], kw, cs[pos])"),
    "page-from-next-slot": ("page = int(prob.block_tables[b, pos // P])", "page = int(prob.block_tables[b, (pos + 1) // P])"),
    "bad-request-not-skipped": ("ok = 0 <= lo <= hi <= T and n <= L and", "ok = 0 <= lo <= hi <= T and"),
    "e4m3-bias": ("(1.0 + m / 8.0) * 2.0 ** (e - 7)", "(1.0 + m / 8.0) * 2.0 ** (e - 8)"),
    "q-scale-no-floor": ("max(float(np.max(np.abs(y))), Q_SCALE_FLOOR)", "float(np.max(np.abs(y)))"),
    "q-scale-mean-not-max": ("max(float(np.max(np.abs(y))), Q_SCALE_FLOOR)",
                             "max(float(np.mean(np.abs(y))), Q_SCALE_FLOOR)"),
    "q-payload-multiplied": ("y = y / sc", "y = y * sc"),
    "q-static-divides": ("y = y * prob.q_scale_inv", "y = y / prob.q_scale_inv"),
    "q-scale-index-global-row": ("* prob.q_scale_stride + (r - lo)", "* prob.q_scale_stride + r"),
    "q-scale-stride-not-checked": ("n > prob.q_scale_stride:", "n > prob.q_scale_stride + 8:"),
}


def _run_pins_against(src_text: str, tmp_path) -> subprocess.CompletedProcess:
    mutated = tmp_path / "append_mut.py"
    mutated.write_text(src_text)
    env = dict(os.environ, PKV_APPEND_ORACLE=str(mutated))
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_append_oracle.py")],
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
