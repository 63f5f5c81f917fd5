"""Peaked-logit problems shared by the GPU parity tests (tests/test_gpu_peaked.py)
and the CPU check that they move a row's running maximum where they claim
to (tests/test_peaked_inputs.py)."""
from __future__ import annotations

from paged_kv_attention_15_amd import workloads as W

# planted rises of the scaled logit, natural-log units (a standard-normal key
# against a shifted query has logits of about N(0, 2) here)
R1, R2, R3 = 16.0, 28.5, 46.0  # successive levels: jumps of ~+9..13, ~+18 and ~+25 log2 units
R_ABSORB = R1 + 4.0            # ~+5.8 log2 over R1: absorbed without moving the reference
R_MASKED = 80.0                # far above everything a row may see


def decode_case(T: int = 128):
    """Seven requests, each with its own pattern (T = the kernels' tile length)."""
    lens = [4 * T + 37, 5 * T, 3 * T + 50, 6 * T + 1, 1, 2 * T + 17, 7 * T + 3]
    levels = (
        (0, 2 * T + 5, 2 * T + 8, R1),                   # one jump inside a later tile
        (1, T, T + 1, R1), (1, 3 * T, 3 * T + 40, R2),   # jumps on tile boundaries, then a plateau
        (2, 10, 13, R1), (2, T + 64, T + 65, R2), (2, lens[2] - 1, lens[2], R3),  # last key
        (3, 0, 4, R1), (3, 2 * T + 1, 2 * T + 2, R_ABSORB),  # a rise below the threshold
        (5, lens[5] - 1, lens[5], R3),                   # one big jump in the last partial tile
        (6, T - 1, T, R2), (6, 5 * T, 5 * T + 2, R3),
    )
    return lens, levels


def decode_problem(kind: str, kv: str, q_len: int = 1, mla: bool = False):
    lens, levels = decode_case(64 if mla else 128)
    if kind == "peaked":
        prof = W.LogitProfile(levels=levels, tail_rise=R_MASKED)
    elif kind == "equal":
        prof = W.LogitProfile(equal_keys=True)
    else:
        prof = W.LogitProfile(negative=120.0)
    if mla:
        return W.make_problem(name=f"mla-{kind}-q{q_len}", seed=21, batch=len(lens), seq_lens=lens,
                              q_lens=[q_len] * len(lens), num_qo_heads=128, num_kv_heads=1, head_dim_qk=576,
                              head_dim_v=512, page_size=64, mla=True, scale=1 / 24.0, poison=True,
                              extra_page_frac=0.3, table_slack_pages=1, logits=prof)
    hq, P = (64, 64) if kv == W.E4M3 else (32, 32)
    return W.make_problem(name=f"gqa-{kv}-{kind}-q{q_len}", seed=22, batch=len(lens), seq_lens=lens,
                          q_lens=[q_len] * len(lens), num_qo_heads=hq, num_kv_heads=8, head_dim_qk=128,
                          head_dim_v=128, page_size=P, kv_dtype=kv, q_dtype=W.BF16, o_dtype=W.BF16,
                          poison=True, extra_page_frac=0.3, table_slack_pages=2, logits=prof)


def context_case():
    lens, qlens = [777, 300, 1100], [257, 100, 300]
    levels = (
        (0, 100, 103, R1), (0, 530, 531, R2),   # row i of request 0 sees keys 0 .. 520 + i
        (0, 650, 651, R_MASKED),                # masked for rows 0..129, visible to the rest
        (0, 700, 701, R3),
        (1, 0, 2, R1), (1, 250, 251, R3),       # request 1: rows i >= 50 see the second level
        (2, 31, 33, R1), (2, 64, 65, R2), (2, 896, 897, R3),
        (2, 1099, 1100, R_MASKED),              # only the last row of request 2 sees it
    )
    return lens, qlens, levels


def context_problem(kind: str):
    lens, qlens, levels = context_case()
    if kind == "peaked":
        prof = W.LogitProfile(levels=levels, tail_rise=R_MASKED)
    elif kind == "equal":
        prof = W.LogitProfile(equal_keys=True)
    else:
        prof = W.LogitProfile(negative=120.0)
    return W.make_problem(name=f"ctx-{kind}", seed=23, batch=3, seq_lens=lens, q_lens=qlens, num_qo_heads=16,
                          num_kv_heads=2, head_dim_qk=128, head_dim_v=128, page_size=16, is_decode=False,
                          poison=True, extra_page_frac=0.3, table_slack_pages=1, logits=prof)
