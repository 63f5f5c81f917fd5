"""Shared helpers for the GPU parity tests: run a Problem through the C ABI
and compare it with the oracle element by element."""
from __future__ import annotations

import json
import os
import sys

import numpy as np
import torch

import oracle
from paged_kv_attention_15_amd import pkv
from tests import _refs as R

TOL = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tolerances.json")))


def tol_key(prob):
    return "e4m3" if prob.kv_dtype == "e4m3" else ("f32" if prob.kv_dtype == "f32" and prob.o_dtype == "f32"
                                                   and prob.q_dtype == "f32" else "bf16")


def tol_for(prob):
    key = tol_key(prob)
    return TOL[key]["atol"], TOL[key]["rtol"]


def norm_tol_for(prob):
    t = TOL["row_norm"][tol_key(prob)]
    return t["rtol"], t["floor"]


# Every comparison's errors, written out at the end of the session when
# PKV_PARITY_RECORD names a file (tests/conftest.py).
RECORD = []


def check_problem_output(prob, got, ref_o):
    """The comparison every GPU parity test applies (also run on the CPU
    against planted wrong outputs): elementwise bound and row-norm bound."""
    atol, rtol = tol_for(prob)
    nrt, nfl = norm_tol_for(prob)
    return R.check_output(got, ref_o, atol, rtol, nrt, nfl)


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def sample_pairs(prob, n: int, seed: int = 0) -> np.ndarray:
    """(row, head) pairs: first/last rows and heads of every request plus random ones."""
    rng = np.random.default_rng(seed)
    pairs = set()
    for b in range(prob.batch):
        lo, hi = int(prob.q_indptr[b]), int(prob.q_indptr[b + 1])
        if hi <= lo:
            continue
        for t in {lo, hi - 1}:
            for h in {0, prob.num_qo_heads - 1}:
                pairs.add((t, h))
    while len(pairs) < n + 4 * prob.batch:
        pairs.add((int(rng.integers(prob.total_q)), int(rng.integers(prob.num_qo_heads))))
        if len(pairs) >= prob.total_q * prob.num_qo_heads:
            break
    return np.array(sorted(pairs), dtype=np.int64)


def run_gpu(prob, num_splits=None, device_scales=False, stream=None):
    dp = pkv.upload(prob, "cuda", num_splits=num_splits, device_scales=device_scales)
    dp.run(stream=stream)
    torch.cuda.synchronize()
    return dp


def compare(prob, dp, pairs=None, check_lse=True, label="", expect_err=0, ref=None):
    """Check dp's output (and LSE, error word) against the oracle on `pairs`
    (default: every (row, head)); `ref` = the oracle's (out, lse) for those
    pairs when the caller already has them."""
    atol, rtol = tol_for(prob)
    nrt, nfl = norm_tol_for(prob)
    out = dp.out.float().cpu().numpy().reshape(prob.total_q * prob.num_qo_heads, prob.head_dim_v)
    lse = dp.lse.cpu().numpy().reshape(-1) if dp.lse is not None else None
    if pairs is None:
        pairs = oracle.all_pairs(prob)
    idx = pairs[:, 0] * prob.num_qo_heads + pairs[:, 1]
    ref_o, ref_l = oracle.attention(prob, pairs) if ref is None else ref
    got = out[idx]
    ok, rep = check_problem_output(prob, got, ref_o)
    lab = label or prob.name
    say(f"  [{lab}] rows={len(pairs)} max_abs={rep['max_abs']:.3e} max_rel={rep['max_rel']:.3e} "
        f"bad={rep['bad_elems']} row_norm_rel={rep['max_row_norm_rel']:.3e} bad_rows={rep['bad_rows']}")
    RECORD.append({"test": os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], "case": lab,
                   "kv_dtype": prob.kv_dtype, "rows": int(len(pairs)), "atol": atol, "rtol": rtol,
                   "norm_rtol": nrt, **{k: (round(v, 9) if isinstance(v, float) else v) for k, v in rep.items()}})
    assert rep["finite"], "non-finite output"
    assert ok, (f"{rep['bad_elems']} elements outside atol={atol} rtol={rtol} (max_abs {rep['max_abs']}) or "
                f"{rep['bad_rows']} rows above the row-norm bound {nrt} (worst {rep['max_row_norm_rel']})")
    if check_lse and lse is not None:
        fin = np.isfinite(ref_l)
        assert np.array_equal(np.isfinite(lse[idx]), fin)
        np.testing.assert_allclose(lse[idx][fin], ref_l[fin], atol=2e-3, rtol=1e-3)
    if dp.err is not None:
        err = int(dp.err.cpu().item())
        assert err == expect_err, f"device error word {err}, expected {expect_err}"
    return rep["max_abs"]
