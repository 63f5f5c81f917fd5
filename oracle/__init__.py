"""CPU oracle for paged-KV attention -- TEST INFRASTRUCTURE ONLY.

Thin ctypes wrapper around pkv_oracle.c (plain C, fp64, single-threaded).
Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package; the HIP product path never does.  It shares no code with
the HIP library: it reads the raw storage arrays of a workloads.Problem and
decodes every element itself.

The definition it computes, and the passages of the pages it follows, are in
the header comment of pkv_oracle.c.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkv_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD, "libpkv_oracle.so")
_lock = threading.Lock()
_lib = None

DTYPE_CODES = {"f32": 0, "bf16": 1, "e4m3": 2}


class _Problem(C.Structure):
    _fields_ = [
        ("batch", C.c_int32), ("num_qo_heads", C.c_int32), ("num_kv_heads", C.c_int32),
        ("head_dim_qk", C.c_int32), ("head_dim_v", C.c_int32), ("page_size", C.c_int32),
        ("causal", C.c_int32), ("q_dtype", C.c_int32), ("k_dtype", C.c_int32),
        ("v_dtype", C.c_int32),
        ("q_indptr", C.c_void_p), ("seq_lens", C.c_void_p), ("k_table", C.c_void_p),
        ("v_table", C.c_void_p), ("table_stride", C.c_int64),
        ("q", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p),
        ("k_page_stride", C.c_int64), ("k_head_stride", C.c_int64), ("k_tok_stride", C.c_int64),
        ("v_page_stride", C.c_int64), ("v_head_stride", C.c_int64), ("v_tok_stride", C.c_int64),
        ("scale", C.c_double), ("k_scale", C.c_double), ("v_scale", C.c_double),
        ("sinks", C.c_void_p),
    ]


def build(force: bool = False) -> str:
    """Compile pkv_oracle.c with gcc -O2 (no OpenMP, no SIMD intrinsics)."""
    os.makedirs(_BUILD, exist_ok=True)
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            # PKV_ORACLE_LIB lets the mutation tests load a deliberately broken
            # copy of the oracle in a child process; nothing else sets it.
            lib = C.CDLL(os.environ.get("PKV_ORACLE_LIB") or build())
            lib.orc_attention.argtypes = [C.POINTER(_Problem), C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p]
            lib.orc_attention.restype = C.c_int
            lib.orc_attention_split.argtypes = [C.POINTER(_Problem), C.c_int, C.c_void_p, C.c_int64,
                                                C.c_void_p, C.c_void_p]
            lib.orc_attention_split.restype = C.c_int
            lib.orc_merge.argtypes = [C.c_int, C.c_int64, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p,
                                      C.c_void_p, C.c_void_p]
            lib.orc_merge.restype = C.c_int
            lib.orc_e4m3_to_double.argtypes = [C.c_uint8]
            lib.orc_e4m3_to_double.restype = C.c_double
            lib.orc_bf16_to_double.argtypes = [C.c_uint16]
            lib.orc_bf16_to_double.restype = C.c_double
            _lib = lib
    return _lib


def _pool_strides(prob, pool: np.ndarray, dim_stride_source: np.ndarray):
    """Element strides (page, head, token) of a pool in HND or NHD layout."""
    if prob.layout == "HND":
        _, H, P, D = dim_stride_source.shape
        return H * P * D, P * D, D
    _, P, H, D = dim_stride_source.shape
    return P * H * D, D, H * D


def _make_struct(prob, keep: list):
    def ptr(a):
        a = np.ascontiguousarray(a)
        keep.append(a)
        return a.ctypes.data

    k_pool = np.ascontiguousarray(prob.k_pool)
    v_pool = k_pool if prob.mla else np.ascontiguousarray(prob.v_pool)
    keep.extend([k_pool, v_pool])
    ks = _pool_strides(prob, k_pool, k_pool)
    vs = _pool_strides(prob, v_pool, v_pool)
    s = _Problem()
    s.batch = prob.batch
    s.num_qo_heads = prob.num_qo_heads
    s.num_kv_heads = prob.num_kv_heads
    s.head_dim_qk = prob.head_dim_qk
    s.head_dim_v = prob.head_dim_v
    s.page_size = prob.page_size
    s.causal = 1 if prob.causal else 0
    s.q_dtype = DTYPE_CODES[prob.q_dtype]
    s.k_dtype = s.v_dtype = DTYPE_CODES[prob.kv_dtype]
    s.q_indptr = ptr(np.asarray(prob.q_indptr, dtype=np.int32))
    s.seq_lens = ptr(np.asarray(prob.seq_lens, dtype=np.int32))
    table = np.ascontiguousarray(prob.block_tables, dtype=np.int32)
    v_table = table if getattr(prob, "v_block_tables", None) is None else \
        np.ascontiguousarray(prob.v_block_tables, dtype=np.int32)
    assert v_table.shape == table.shape
    s.k_table = ptr(table)
    s.v_table = ptr(v_table)
    s.table_stride = table.shape[1]
    s.q = ptr(prob.q)
    s.k = k_pool.ctypes.data
    s.v = v_pool.ctypes.data
    s.k_page_stride, s.k_head_stride, s.k_tok_stride = ks
    s.v_page_stride, s.v_head_stride, s.v_tok_stride = vs
    s.scale = prob.scale
    s.k_scale = prob.k_scale
    s.v_scale = prob.v_scale
    sinks = getattr(prob, "sinks", None)
    s.sinks = ptr(np.asarray(sinks, dtype=np.float64)) if sinks is not None else None
    return s


def all_pairs(prob) -> np.ndarray:
    """Every (global query row, head) pair, row-major: shape [T_q*Hq, 2]."""
    t = np.repeat(np.arange(prob.total_q, dtype=np.int64), prob.num_qo_heads)
    h = np.tile(np.arange(prob.num_qo_heads, dtype=np.int64), prob.total_q)
    return np.stack([t, h], axis=1)


def attention(prob, pairs: np.ndarray | None = None):
    """fp64 attention output [n, D_v] and natural-log LSE [n] for (row, head) pairs."""
    lib = _load()
    if pairs is None:
        pairs = all_pairs(prob)
    pairs = np.ascontiguousarray(pairs, dtype=np.int64).reshape(-1, 2)
    n = pairs.shape[0]
    out = np.zeros((n, prob.head_dim_v), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    keep: list = []
    s = _make_struct(prob, keep)
    rc = lib.orc_attention(C.byref(s), pairs.ctypes.data, n, out.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle rejected the problem (rc={rc})")
    return out, lse


def attention_split(prob, num_splits: int, pairs: np.ndarray | None = None):
    """Per-partition outputs [S, n, D_v] and LSEs [S, n] (page-aligned partitions)."""
    lib = _load()
    if pairs is None:
        pairs = all_pairs(prob)
    pairs = np.ascontiguousarray(pairs, dtype=np.int64).reshape(-1, 2)
    n = pairs.shape[0]
    o_part = np.zeros((num_splits, n, prob.head_dim_v), dtype=np.float64)
    lse_part = np.zeros((num_splits, n), dtype=np.float64)
    keep: list = []
    s = _make_struct(prob, keep)
    rc = lib.orc_attention_split(C.byref(s), num_splits, pairs.ctypes.data, n, o_part.ctypes.data,
                                 lse_part.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle rejected the problem (rc={rc})")
    return o_part, lse_part


def merge(o_part: np.ndarray, lse_part: np.ndarray, row_sinks: np.ndarray | None = None):
    """Log-sum-exp merge of [S, n, D_v] partial outputs with [S, n] LSEs; row_sinks
    [n] (optional) folds one sink logit into each merged row."""
    lib = _load()
    o_part = np.ascontiguousarray(o_part, dtype=np.float64)
    lse_part = np.ascontiguousarray(lse_part, dtype=np.float64)
    S, n, dv = o_part.shape
    out = np.zeros((n, dv), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    rs = None if row_sinks is None else np.ascontiguousarray(row_sinks, dtype=np.float64)
    lib.orc_merge(S, n, dv, o_part.ctypes.data, lse_part.ctypes.data, out.ctypes.data, lse.ctypes.data,
                  None if rs is None else rs.ctypes.data)
    return out, lse


def e4m3_to_double(code: int) -> float:
    return float(_load().orc_e4m3_to_double(code))


def bf16_to_double(bits: int) -> float:
    return float(_load().orc_bf16_to_double(bits))


def e4m3_table() -> np.ndarray:
    """All 256 e4m3 codes decoded to fp64 (NaN for 0x7F / 0xFF)."""
    return np.array([e4m3_to_double(c) for c in range(256)], dtype=np.float64)
