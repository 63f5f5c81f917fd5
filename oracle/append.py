"""CPU oracle for the paged-KV append producer -- TEST INFRASTRUCTURE ONLY.

Plain numpy in float64, one (token, head) at a time.  Only the tests, the
smoke check and the benchmark's CPU-baseline leg may use it; the HIP path
never does, and nothing here is shared with it (storage decoding included).

What it computes (PR #5952 page, "fused BF16 QK RMSNorm + NeoX RoPE + paged KV
append", summary paragraph; PR #5956 body quoted on it, section "Contract"):
  * the packed row qkv[r] holds Hq query heads, then Hkv key heads, then Hkv
    value heads, 128 channels each, in bf16;
  * query and key heads optionally get a per-head RMSNorm with fp32 arithmetic,
    y = x / sqrt(mean(x^2) + eps) * w, eps = 1e-6 (policy 0: none; 1: RoPE then
    norm; 2: norm then RoPE), w the bf16 weight vector of Q or of K;
  * NeoX rotary embedding from the caller's table cos_sin[pos] = (cos_0..63,
    sin_0..63): channel i < 64 pairs with i + 64,
      y_i = x_i cos_i - x_{i+64} sin_i,   y_{i+64} = x_{i+64} cos_i + x_i sin_i;
  * the position of row r of request b is r + seq_lens[b] - q_indptr[b+1]
    (seq_lens is the total length after the append, so the last new row is
    at seq_lens[b] - 1);
  * the query heads go to out_q[r]; key and value heads (values untouched) go
    to slot pos % P of page block_tables[b][pos / P] of the NHD caches, as bf16
    or as e4m3 codes of x / k_scale and x / v_scale;
  * with tail clearing, rows [last + 1, P) of every nonempty request's last
    page are zeroed in both caches, last = (seq_lens[b] - 1) % P;
  * optional e4m3 query output (the same Contract section): with the dynamic
    policy each (row, head) gets its own scale q_scale = max(max_i |y_i|,
    1e-6) / upper_max and the stored payload is y / q_scale; with the static
    policy the payload is y * q_scale_inv and no scale is written.  The
    dynamic scales sit at [T, Hq] (decode) or at [B, Hq, stride], entry
    (b, h, i) for the request's i-th new row (prefill; the pages size the
    last axis as max_seqlen rounded up to 128).
Reading where the pages are silent: a request whose rows do not fit its
length, the table or the rotary table (seq_lens[b] < rows, a position past
the table width or past max_pos) is skipped entirely (nothing written, its
tail not cleared) and reported; so is a request with more new rows than
the prefill scale layout's stride.  The static policy multiplies by
q_scale_inv (the argument's name: the inverse of a scale).

Returns expected *values* (float64), never storage bits: the tests compare the
HIP path's bf16 rows with the pages' tolerance and its e4m3 codes against the
unrounded payload, as the pages' own tests do.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple

import numpy as np

D = 128
HALF = 64


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (the bits are the top half of an fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP e4m3 ("fn") codes -> float64: sign, 4-bit exponent (bias 7), 3-bit
    mantissa; exponent 0 is subnormal (M/8 * 2^-6); S.1111.111 is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return s * val


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    return x / np.sqrt(np.mean(x * x) + eps) * w


def rope(x: np.ndarray, cs_row: np.ndarray) -> np.ndarray:
    c, s = cs_row[:HALF], cs_row[HALF:]
    lo, hi = x[:HALF], x[HALF:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s])


# query output policies
Q_BF16, Q_DYNAMIC, Q_STATIC = 0, 1, 2
Q_SCALE_FLOOR = 1e-6


def q_scale_index(prob, b: int, h: int, r: int, lo: int) -> int:
    """Flat position of the dynamic scale of row r (request b starting at row lo), head h."""
    if prob.q_scale_layout == 0:
        return r * prob.num_qo_heads + h
    return (b * prob.num_qo_heads + h) * prob.q_scale_stride + (r - lo)


@dataclasses.dataclass
class AppendResult:
    out_q: np.ndarray                      # [T, Hq, 128] float64 payload, NaN for rows not written
    q_scale: Dict[int, float]              # flat q_scale index -> dynamic scale (dynamic policy only)
    k_rows: Dict[Tuple[int, int, int], np.ndarray]  # (page, slot, kv head) -> value (x / k_scale for e4m3)
    v_rows: Dict[Tuple[int, int, int], np.ndarray]
    cleared: List[Tuple[int, int, int]]    # (page, slot, kv head) zeroed in both caches
    bad_requests: List[int]


def append(prob) -> AppendResult:
    """The plain definition above, written out for a workloads.AppendProblem."""
    Hq, Hkv, P = prob.num_qo_heads, prob.num_kv_heads, prob.page_size
    T = prob.total_tokens
    qkv = bf16_to_f64(prob.qkv).reshape(T, Hq + 2 * Hkv, D)
    cs = prob.cos_sin.astype(np.float64)
    qw, kw = bf16_to_f64(prob.q_weight), bf16_to_f64(prob.k_weight)
    e4m3 = prob.kv_dtype == "e4m3"
    out_q = np.full((T, Hq, D), np.nan)
    q_scale: Dict[int, float] = {}
    k_rows, v_rows, cleared, bad = {}, {}, [], []

    def qk_transform(x, w, cs_row):
        if prob.norm_policy == 1:
            return rms_norm(rope(x, cs_row), w, prob.eps)
        if prob.norm_policy == 2:
            return rope(rms_norm(x, w, prob.eps), cs_row)
        return rope(x, cs_row)

    for b in range(prob.batch):
        lo, hi = int(prob.q_indptr[b]), int(prob.q_indptr[b + 1])
        L = int(prob.seq_lens[b])
        n = hi - lo
        ok = 0 <= lo <= hi <= T and n <= L and L <= prob.max_pages * P and L <= prob.max_pos
        if prob.q_quant == Q_DYNAMIC and prob.q_scale_layout == 1 and n > prob.q_scale_stride:
            ok = False
        if not ok:
            bad.append(b)
            continue
        for r in range(lo, hi):
            pos = r + L - hi
            page = int(prob.block_tables[b, pos // P])
            slot = pos % P
            for h in range(Hq):
                y = qk_transform(qkv[r, h], qw, cs[pos])
                if prob.q_quant == Q_DYNAMIC:
                    sc = max(float(np.max(np.abs(y))), Q_SCALE_FLOOR) / prob.upper_max
                    q_scale[q_scale_index(prob, b, h, r, lo)] = sc
                    y = y / sc
                elif prob.q_quant == Q_STATIC:
                    y = y * prob.q_scale_inv
                out_q[r, h] = y
            for g in range(Hkv):
                k = qk_transform(qkv[r, Hq + g], kw, cs[pos])
                v = qkv[r, Hq + Hkv + g]
                k_rows[(page, slot, g)] = k / prob.k_scale if e4m3 else k
                v_rows[(page, slot, g)] = v / prob.v_scale if e4m3 else v
        if prob.clear_tail and L > 0:
            page = int(prob.block_tables[b, (L - 1) // P])
            for slot in range((L - 1) % P + 1, P):
                for g in range(Hkv):
                    cleared.append((page, slot, g))
    return AppendResult(out_q=out_q, q_scale=q_scale, k_rows=k_rows, v_rows=v_rows, cleared=cleared,
                        bad_requests=bad)
