"""ctypes binding of libpkv.so -- argument marshalling only.

Every function here has the name of the C entry point it calls (see
include/pkv.h) and does nothing but pack arguments; all attention work runs in
the library's HIP kernels.  Loading fails loudly when libpkv.so is missing:
there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build, unless PKV_LIBRARY_PATH names another build of the same sources
LIB_PATH = os.environ.get("PKV_LIBRARY_PATH") or os.path.join(HERE, "libpkv.so")

PKV_OK, PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED, PKV_ERR_WORKSPACE, PKV_ERR_HIP = range(5)
PKV_DTYPE_F32, PKV_DTYPE_BF16, PKV_DTYPE_FP8_E4M3 = range(3)
PKV_LAYOUT_HND, PKV_LAYOUT_NHD = range(2)
PKV_DEVERR_SEQ_LT_QLEN, PKV_DEVERR_SEQ_GT_TABLE, PKV_DEVERR_PAGE_RANGE, PKV_DEVERR_QINDPTR = 1, 2, 4, 8

# kernel ids of pkv_plan_info.kernel (stable; ids not listed are retired variants)
KERNEL_NAMES = {0: "none", 1: "generic", 2: "gqa_bf16", 3: "gqa_fp8", 4: "wide_bf16", 5: "wide_fp8",
                6: "mla_bf16", 7: "mla_fp8", 15: "dma_wide_bf16", 16: "dma_wide_fp8", 17: "dma_mla_bf16",
                18: "dma_mla_fp8", 31: "dma_gqa_fp8_n2", 36: "m32_ctx_w8t128", 37: "mla32_bf16"}
KERNEL_IDS = {v: k for k, v in KERNEL_NAMES.items()}

DTYPE_CODES = {"f32": PKV_DTYPE_F32, "bf16": PKV_DTYPE_BF16, "e4m3": PKV_DTYPE_FP8_E4M3}
EXPORTED = ["pkv_abi_version", "pkv_last_error", "pkv_plan", "pkv_workspace_bytes", "pkv_decode", "pkv_decode_noalloc",
            "pkv_context", "pkv_lse_merge", "pkv_append"]
PKV_DEVERR_POS_RANGE = 0x10
PKV_DEVERR_QSCALE_ROWS = 0x20
PKV_DEVERR_SEQ_GT_MAXLEN = 0x40


class PkvArgs(C.Structure):
    """Mirror of `pkv_args` in include/pkv.h (field order and types must match)."""
    _fields_ = [
        ("batch", C.c_int32), ("q_len", C.c_int32), ("num_qo_heads", C.c_int32),
        ("num_kv_heads", C.c_int32), ("head_dim_qk", C.c_int32), ("head_dim_v", C.c_int32),
        ("page_size", C.c_int32), ("max_pages_per_seq", C.c_int32), ("max_kv_len", C.c_int32),
        ("max_q_len", C.c_int32), ("total_q", C.c_int32), ("num_pages", C.c_int32),
        ("q_dtype", C.c_int32), ("kv_dtype", C.c_int32), ("o_dtype", C.c_int32),
        ("layout", C.c_int32), ("causal", C.c_int32), ("num_splits", C.c_int32),
        ("v_shares_k", C.c_int32), ("kernel_hint", C.c_int32),
        ("q", C.c_void_p), ("k_pages", C.c_void_p), ("v_pages", C.c_void_p),
        ("block_tables", C.c_void_p), ("seq_lens", C.c_void_p), ("q_indptr", C.c_void_p),
        ("out", C.c_void_p), ("lse_out", C.c_void_p), ("err_word", C.c_void_p),
        ("k_scale_dev", C.c_void_p), ("v_scale_dev", C.c_void_p), ("merge_counters", C.c_void_p),
        ("sinks", C.c_void_p), ("v_block_tables", C.c_void_p),
        ("q_stride_tok", C.c_int64), ("q_stride_head", C.c_int64),
        ("o_stride_tok", C.c_int64), ("o_stride_head", C.c_int64),
        ("k_stride_page", C.c_int64), ("k_stride_head", C.c_int64), ("k_stride_tok", C.c_int64),
        ("v_stride_page", C.c_int64), ("v_stride_head", C.c_int64), ("v_stride_tok", C.c_int64),
        ("table_stride", C.c_int64),
        ("scale", C.c_float), ("k_scale", C.c_float), ("v_scale", C.c_float), ("reserved1", C.c_float),
    ]


class PkvPlanInfo(C.Structure):
    _fields_ = [
        ("kernel", C.c_int32), ("num_splits", C.c_int32), ("pages_per_split", C.c_int32),
        ("grid_x", C.c_int32), ("grid_y", C.c_int32), ("grid_z", C.c_int32),
        ("block_threads", C.c_int32), ("schedule", C.c_int32), ("counter_words", C.c_int32),
        ("fused_merge", C.c_int32), ("workspace_bytes", C.c_size_t),
    ]


class PkvAppendArgs(C.Structure):
    """Mirror of `pkv_append_args` in include/pkv.h (field order and types must match)."""
    _fields_ = [
        ("num_tokens", C.c_int32), ("batch", C.c_int32), ("num_qo_heads", C.c_int32),
        ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("page_size", C.c_int32),
        ("max_pages_per_seq", C.c_int32), ("max_pos", C.c_int32), ("num_pages", C.c_int32),
        ("norm_policy", C.c_int32), ("clear_tail", C.c_int32), ("kv_dtype", C.c_int32),
        ("eps", C.c_float), ("k_scale", C.c_float), ("v_scale", C.c_float), ("reserved", C.c_float),
        ("qkv", C.c_void_p), ("qkv_stride_tok", C.c_int64), ("cos_sin", C.c_void_p),
        ("q_weight", C.c_void_p), ("k_weight", C.c_void_p), ("q_indptr", C.c_void_p),
        ("seq_lens", C.c_void_p), ("block_tables", C.c_void_p), ("table_stride", C.c_int64),
        ("out_q", C.c_void_p), ("k_cache", C.c_void_p), ("v_cache", C.c_void_p), ("err_word", C.c_void_p),
        ("q_quant", C.c_int32), ("upper_max", C.c_float), ("q_scale_inv", C.c_float),
        ("q_scale_layout", C.c_int32), ("q_scale_stride", C.c_int64), ("q_scale", C.c_void_p),
        ("layout", C.c_int32), ("reserved2", C.c_int32),
        ("k_stride_page", C.c_int64), ("k_stride_head", C.c_int64), ("k_stride_tok", C.c_int64),
        ("v_stride_page", C.c_int64), ("v_stride_head", C.c_int64), ("v_stride_tok", C.c_int64),
    ]


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"pkv status {status}: {message}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libpkv.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"libpkv.so not found at {path}; build it with "
                               f"`python -m paged_kv_attention_15_amd.build`")
        lib = C.CDLL(path)
        lib.pkv_abi_version.restype = C.c_int
        lib.pkv_last_error.restype = C.c_char_p
        lib.pkv_plan.argtypes = [C.POINTER(PkvArgs), C.c_int, C.c_int, C.POINTER(PkvPlanInfo)]
        lib.pkv_plan.restype = C.c_int
        lib.pkv_append.argtypes = [C.POINTER(PkvAppendArgs), C.c_void_p]
        lib.pkv_append.restype = C.c_int
        lib.pkv_workspace_bytes.argtypes = [C.POINTER(PkvArgs), C.c_int, C.POINTER(C.c_size_t)]
        lib.pkv_workspace_bytes.restype = C.c_int
        lib.pkv_decode_noalloc.argtypes = [C.POINTER(PkvArgs), C.c_void_p]
        lib.pkv_decode_noalloc.restype = C.c_int
        for fn in (lib.pkv_decode, lib.pkv_context):
            fn.argtypes = [C.POINTER(PkvArgs), C.c_void_p, C.c_size_t, C.c_void_p]
            fn.restype = C.c_int
        lib.pkv_lse_merge.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                      C.c_void_p, C.c_int32, C.c_int64, C.c_int64, C.c_void_p, C.c_void_p]
        lib.pkv_lse_merge.restype = C.c_int
        _lib = lib
    return _lib


def _check(status: int) -> int:
    if status != PKV_OK:
        raise PkvError(status, pkv_last_error())
    return status


def _require_gpu_tensors(args) -> None:
    """Arguments filled from tensors carry the tensors' device: refuse to
    launch on pointers that are not device memory (a kernel would fault)."""
    dev = getattr(args, "_tensor_device", None)
    if dev is not None and dev.type != "cuda":
        raise ValueError(f"the tensors behind these arguments are on {dev}, not on a GPU")


# ---------------------------------------------------------------- entry points

def pkv_abi_version() -> int:
    return int(load_library().pkv_abi_version())


def pkv_last_error() -> str:
    return load_library().pkv_last_error().decode()


def pkv_plan(args: PkvArgs, is_context: bool = False, num_cus: int = 0, check: bool = True) -> PkvPlanInfo:
    info = PkvPlanInfo()
    st = load_library().pkv_plan(C.byref(args), int(is_context), int(num_cus), C.byref(info))
    if check:
        _check(st)
    info.status = st
    return info


def pkv_workspace_bytes(args: PkvArgs, is_context: bool = False) -> int:
    n = C.c_size_t(0)
    _check(load_library().pkv_workspace_bytes(C.byref(args), int(is_context), C.byref(n)))
    return int(n.value)


PKV_NOALLOC_SCRATCH_BYTES = 32 << 20


def pkv_decode_noalloc(args: PkvArgs, stream: int, check: bool = True) -> int:
    _require_gpu_tensors(args)
    st = load_library().pkv_decode_noalloc(C.byref(args), C.c_void_p(stream))
    return _check(st) if check else st


def pkv_decode(args: PkvArgs, workspace: int, workspace_bytes: int, stream: int, check: bool = True) -> int:
    _require_gpu_tensors(args)
    st = load_library().pkv_decode(C.byref(args), C.c_void_p(workspace or None), workspace_bytes,
                                   C.c_void_p(stream or None))
    return _check(st) if check else st


def pkv_context(args: PkvArgs, workspace: int, workspace_bytes: int, stream: int, check: bool = True) -> int:
    _require_gpu_tensors(args)
    st = load_library().pkv_context(C.byref(args), C.c_void_p(workspace or None), workspace_bytes,
                                    C.c_void_p(stream or None))
    return _check(st) if check else st


def pkv_lse_merge(num_splits: int, num_rows: int, num_qo_heads: int, head_dim_v: int, o_part: int,
                  lse_part: int, out: int, o_dtype: int, o_stride_tok: int, o_stride_head: int,
                  lse_out: int, stream: int, check: bool = True) -> int:
    st = load_library().pkv_lse_merge(num_splits, num_rows, num_qo_heads, head_dim_v, C.c_void_p(o_part or None),
                                      C.c_void_p(lse_part or None), C.c_void_p(out or None), o_dtype,
                                      o_stride_tok, o_stride_head, C.c_void_p(lse_out or None),
                                      C.c_void_p(stream or None))
    return _check(st) if check else st


# ---------------------------------------------------------------- torch marshalling

def pkv_append(args: PkvAppendArgs, stream: int, check: bool = True) -> int:
    _require_gpu_tensors(args)
    st = load_library().pkv_append(C.byref(args), C.c_void_p(stream or None))
    if check:
        _check(st)
    return st


def _torch():
    import torch
    return torch


@dataclass
class DeviceProblem:
    """A workloads.Problem copied to device tensors plus the matching pkv_args."""
    args: PkvArgs
    is_context: bool
    tensors: dict
    workspace: Optional[object]
    workspace_bytes: int

    @property
    def out(self):
        return self.tensors["out"]

    @property
    def lse(self):
        return self.tensors.get("lse")

    @property
    def err(self):
        return self.tensors.get("err")

    def stream_ptr(self, stream=None) -> int:
        torch = _torch()
        s = stream if stream is not None else torch.cuda.current_stream()
        return int(s.cuda_stream)

    def run(self, stream=None, check: bool = True) -> int:
        ws = int(self.workspace.data_ptr()) if self.workspace is not None else 0
        fn = pkv_context if self.is_context else pkv_decode
        return fn(self.args, ws, self.workspace_bytes, self.stream_ptr(stream), check=check)


def _to_device(arr, device):
    import numpy as np
    torch = _torch()
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to(device).view(torch.bfloat16)
    if arr.dtype == np.uint8:
        return torch.from_numpy(arr).to(device)
    return torch.from_numpy(arr).to(device)


def upload(prob, device="cuda", with_lse: bool = True, with_err: bool = True, num_splits: Optional[int] = None,
           device_scales: bool = False, kernel: Optional[str] = None,
           merge_counters: bool = False) -> DeviceProblem:
    """Copy a workloads.Problem to `device` and fill pkv_args for it.

    merge_counters: give the balanced decode schedule a zeroed counter buffer
    (the in-kernel reducer); other plans ignore it."""
    import numpy as np
    torch = _torch()
    t = {}
    t["q"] = _to_device(prob.q, device)
    t["k"] = _to_device(prob.k_pool, device)
    if not prob.mla:
        t["v"] = _to_device(prob.v_pool, device)
    t["table"] = torch.from_numpy(prob.block_tables).to(device)
    t["seq_lens"] = torch.from_numpy(prob.seq_lens).to(device)
    t["q_indptr"] = torch.from_numpy(prob.q_indptr).to(device)
    odt = torch.bfloat16 if prob.o_dtype == "bf16" else torch.float32
    t["out"] = torch.full((prob.total_q, prob.num_qo_heads, prob.head_dim_v), float("nan"), dtype=odt, device=device)
    if with_lse:
        t["lse"] = torch.full((prob.total_q, prob.num_qo_heads), float("nan"), dtype=torch.float32, device=device)
    if with_err:
        t["err"] = torch.zeros(1, dtype=torch.int32, device=device)
    if getattr(prob, "sinks", None) is not None:
        t["sinks"] = torch.from_numpy(np.ascontiguousarray(prob.sinks, dtype=np.float32)).to(device)
    if getattr(prob, "v_block_tables", None) is not None:
        t["v_table"] = torch.from_numpy(np.ascontiguousarray(prob.v_block_tables, dtype=np.int32)).to(device)
    if device_scales:
        t["k_scale"] = torch.tensor([prob.k_scale], dtype=torch.float32, device=device)
        t["v_scale"] = torch.tensor([prob.v_scale], dtype=torch.float32, device=device)
    a = fill_args(prob, t, num_splits=num_splits)
    if kernel is not None:
        a.kernel_hint = KERNEL_IDS[kernel]
    is_ctx = not prob.is_decode
    if merge_counters:
        words = pkv_plan(a, is_ctx).counter_words
        if words > 0:
            t["counters"] = torch.zeros(words, dtype=torch.int32, device=device)
            a.merge_counters = t["counters"].data_ptr()
    ws_bytes = pkv_workspace_bytes(a, is_ctx)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=device) if ws_bytes > 0 else None
    return DeviceProblem(args=a, is_context=is_ctx, tensors=t, workspace=ws, workspace_bytes=ws_bytes)


def fill_args(prob, t: dict, num_splits: Optional[int] = None) -> PkvArgs:
    """pkv_args for a workloads.Problem whose arrays live in the tensors of `t`."""
    a = PkvArgs()
    H, P = prob.num_kv_heads, prob.page_size
    a.batch = prob.batch
    a.q_len = prob.q_len if prob.is_decode else 0
    a.num_qo_heads = prob.num_qo_heads
    a.num_kv_heads = H
    a.head_dim_qk = prob.head_dim_qk
    a.head_dim_v = prob.head_dim_v
    a.page_size = P
    a.max_pages_per_seq = prob.max_pages
    a.max_kv_len = prob.max_kv_len
    a.max_q_len = prob.q_len
    a.total_q = prob.total_q
    a.num_pages = prob.num_pages
    a.q_dtype = DTYPE_CODES[prob.q_dtype]
    a.kv_dtype = DTYPE_CODES[prob.kv_dtype]
    a.o_dtype = DTYPE_CODES[prob.o_dtype]
    a.layout = PKV_LAYOUT_HND if prob.layout == "HND" else PKV_LAYOUT_NHD
    a.causal = 1 if prob.causal else 0
    a.num_splits = prob.num_splits if num_splits is None else num_splits
    a.v_shares_k = 1 if prob.mla else 0
    a.q = t["q"].data_ptr()
    a.k_pages = t["k"].data_ptr()
    a.v_pages = t["v"].data_ptr() if "v" in t else 0
    a.block_tables = t["table"].data_ptr()
    a.seq_lens = t["seq_lens"].data_ptr()
    a.q_indptr = t["q_indptr"].data_ptr()
    a.out = t["out"].data_ptr()
    a.lse_out = t["lse"].data_ptr() if t.get("lse") is not None else 0
    a.err_word = t["err"].data_ptr() if t.get("err") is not None else 0
    a.k_scale_dev = t["k_scale"].data_ptr() if "k_scale" in t else 0
    a.v_scale_dev = t["v_scale"].data_ptr() if "v_scale" in t else 0
    a.sinks = t["sinks"].data_ptr() if "sinks" in t else 0
    a.v_block_tables = t["v_table"].data_ptr() if "v_table" in t else 0
    D, Dv = prob.head_dim_qk, prob.head_dim_v
    a.q_stride_tok = prob.num_qo_heads * D
    a.q_stride_head = D
    a.o_stride_tok = prob.num_qo_heads * Dv
    a.o_stride_head = Dv
    if prob.layout == "HND":
        k_sp, k_sh, k_st = H * P * D, P * D, D
    else:
        k_sp, k_sh, k_st = P * H * D, D, H * D
    a.k_stride_page, a.k_stride_head, a.k_stride_tok = k_sp, k_sh, k_st
    if prob.mla:
        a.v_stride_page, a.v_stride_head, a.v_stride_tok = k_sp, k_sh, k_st
    elif prob.layout == "HND":
        a.v_stride_page, a.v_stride_head, a.v_stride_tok = H * P * Dv, P * Dv, Dv
    else:
        a.v_stride_page, a.v_stride_head, a.v_stride_tok = P * H * Dv, Dv, H * Dv
    a.table_stride = prob.block_tables.shape[1]
    a.scale = prob.scale
    a.k_scale = prob.k_scale
    a.v_scale = prob.v_scale
    return a


# ---------------------------------------------------------------- torch tensors in, pkv_args out

def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return PKV_DTYPE_BF16
    if t.dtype == torch.float32:
        return PKV_DTYPE_F32
    if t.dtype in (getattr(torch, "float8_e4m3fn", None), torch.uint8):  # e4m3 codes, or their raw bytes
        return PKV_DTYPE_FP8_E4M3
    raise ValueError(f"unsupported dtype {t.dtype}")


def _check_tensors(device, named: dict) -> None:
    """Every tensor on `device`; (tensor, dtypes) pairs also checked for dtype."""
    for name, spec in named.items():
        t, dtypes = spec if isinstance(spec, tuple) else (spec, None)
        if t is None:
            continue
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, the query on {device}")
        if dtypes is not None and t.dtype not in dtypes:
            raise ValueError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, not {t.dtype}")


def _stride(t, dim: int, natural: int) -> int:
    """Element stride of `dim`; a dimension of extent 1 is never stepped, so
    the contiguous value stands in for whatever its stride says."""
    return natural if int(t.shape[dim]) == 1 else int(t.stride(dim))


def args_from_tensors(q, k_pages, v_pages, block_tables, seq_lens, out, *, scale: float, max_kv_len: int,
                      layout: str = "HND", q_indptr=None, max_q_len: Optional[int] = None, causal: bool = True,
                      k_scale: float = 1.0, v_scale: float = 1.0, head_dim_v: Optional[int] = None, lse=None,
                      err=None, sinks=None, v_block_tables=None, num_splits: int = 0,
                      kernel: Optional[str] = None) -> PkvArgs:
    """pkv_args for caller-owned device tensors: shapes, dtypes and element
    strides are read off the tensors, nothing is copied.

    q [total_q, Hq, D]; k_pages / v_pages HND [num_pages, Hkv, P, D] or NHD
    [num_pages, P, Hkv, D] (v_pages None: MLA, V is the first head_dim_v
    channels of the K rows); block_tables int32 [B, >= max pages];
    seq_lens int32 [B]; out [total_q, Hq, Dv].  Decode when q_indptr is
    None (every request has total_q / B rows), context otherwise (int32
    [B + 1] row offsets; max_q_len is then the host-side bound on a request's
    rows).  max_kv_len is the host-side bound on seq_lens that sizes the
    plan."""
    if layout not in ("HND", "NHD"):
        raise ValueError("layout must be 'HND' or 'NHD'")
    torch = _torch()
    i32, f32 = (torch.int32,), (torch.float32,)
    _check_tensors(q.device, {"k_pages": k_pages, "v_pages": v_pages, "out": out,
                              "block_tables": (block_tables, i32), "seq_lens": (seq_lens, i32),
                              "q_indptr": (q_indptr, i32), "v_block_tables": (v_block_tables, i32),
                              "lse": (lse, f32), "err": (err, i32), "sinks": (sinks, f32)})
    for name, t in (("q", q), ("k_pages", k_pages), ("out", out)) + ((("v_pages", v_pages),) if v_pages is not None else ()):
        if t.stride(-1) != 1:
            raise ValueError(f"{name}: the last (channel) dimension must be contiguous")
    B = int(block_tables.shape[0])
    total_q, Hq, D = (int(x) for x in q.shape)
    def pool_strides(t):  # (page, head, token) element strides of a K or V pool
        W_ = int(t.shape[3])
        if layout == "HND":
            return (_stride(t, 0, Hkv * P * W_), _stride(t, 1, P * W_), _stride(t, 2, W_))
        return (_stride(t, 0, P * Hkv * W_), _stride(t, 2, W_), _stride(t, 1, Hkv * W_))

    if layout == "HND":
        num_pages, Hkv, P, Dk = (int(x) for x in k_pages.shape)
    else:
        num_pages, P, Hkv, Dk = (int(x) for x in k_pages.shape)
    k_sp, k_sh, k_st = pool_strides(k_pages)
    if Dk != D:
        raise ValueError(f"q has {D} channels, the K rows {Dk}")
    a = PkvArgs()
    a.batch = B
    a.num_qo_heads, a.num_kv_heads = Hq, Hkv
    a.head_dim_qk = D
    a.page_size = P
    a.max_pages_per_seq = int(block_tables.shape[1])
    a.table_stride = _stride(block_tables, 0, int(block_tables.shape[1]))
    a.max_kv_len = int(max_kv_len)
    a.total_q = total_q
    a.num_pages = num_pages
    if q_indptr is None:
        if B == 0 or total_q % B:
            raise ValueError("decode needs the same number of rows for every request (total_q % B == 0)")
        a.q_len = total_q // B
        a.max_q_len = a.q_len
    else:
        if max_q_len is None:
            raise ValueError("context calls need max_q_len")
        a.q_len = 0
        a.max_q_len = int(max_q_len)
        a.q_indptr = q_indptr.data_ptr()
    a.q_dtype, a.kv_dtype, a.o_dtype = _dtype_code(q), _dtype_code(k_pages), _dtype_code(out)
    a.layout = PKV_LAYOUT_HND if layout == "HND" else PKV_LAYOUT_NHD
    a.causal = 1 if causal else 0
    a.num_splits = int(num_splits)
    a.q, a.k_pages = q.data_ptr(), k_pages.data_ptr()
    a.q_stride_tok, a.q_stride_head = _stride(q, 0, Hq * D), _stride(q, 1, D)
    a.k_stride_page, a.k_stride_head, a.k_stride_tok = k_sp, k_sh, k_st
    if v_pages is None:
        a.v_shares_k = 1
        a.head_dim_v = int(head_dim_v if head_dim_v is not None else out.shape[2])
        a.v_stride_page, a.v_stride_head, a.v_stride_tok = k_sp, k_sh, k_st
    else:
        a.head_dim_v = int(v_pages.shape[3])
        a.v_pages = v_pages.data_ptr()
        a.v_stride_page, a.v_stride_head, a.v_stride_tok = pool_strides(v_pages)
    a.block_tables, a.seq_lens = block_tables.data_ptr(), seq_lens.data_ptr()
    a.out = out.data_ptr()
    a.o_stride_tok, a.o_stride_head = _stride(out, 0, Hq * int(out.shape[2])), _stride(out, 1, int(out.shape[2]))
    a.lse_out = lse.data_ptr() if lse is not None else 0
    a.err_word = err.data_ptr() if err is not None else 0
    a.sinks = sinks.data_ptr() if sinks is not None else 0
    a.v_block_tables = v_block_tables.data_ptr() if v_block_tables is not None else 0
    a.scale, a.k_scale, a.v_scale = float(scale), float(k_scale), float(v_scale)
    if kernel is not None:
        a.kernel_hint = KERNEL_IDS[kernel]
    a._tensor_device = q.device
    return a


def run_tensors(args: PkvArgs, stream=None, workspace=None):
    """pkv_decode or pkv_context (by args.q_len) on `stream` (default: torch's
    current stream), with `workspace` (a uint8 device tensor) or one
    allocated here at the size pkv_workspace_bytes asks for.  Returns the
    workspace so that a caller can keep it for the next call."""
    _require_gpu_tensors(args)
    torch = _torch()
    is_ctx = args.q_len == 0
    need = pkv_workspace_bytes(args, is_ctx)
    if need > 0 and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=torch.device("cuda", torch.cuda.current_device()))
    ws_ptr = int(workspace.data_ptr()) if (workspace is not None and need > 0) else 0
    s = stream if stream is not None else torch.cuda.current_stream()
    (pkv_context if is_ctx else pkv_decode)(args, ws_ptr, need, int(s.cuda_stream))
    return workspace


def append_args_from_tensors(qkv, cos_sin, q_weight, k_weight, q_indptr, seq_lens, block_tables, out_q, k_cache,
                             v_cache, *, max_pos: int, norm_policy: int, eps: float, layout: str = "NHD",
                             clear_tail: bool = True, k_scale: float = 1.0, v_scale: float = 1.0,
                             q_quant: int = 0, upper_max: float = 448.0, q_scale_inv: float = 1.0, q_scale=None,
                             q_scale_layout: int = 0, q_scale_stride: int = 0, err=None) -> PkvAppendArgs:
    """pkv_append_args for caller-owned device tensors (the append producer of
    include/pkv.h): qkv bf16 [T, (Hq + 2 Hkv) 128] with any token stride;
    k_cache / v_cache NHD [num_pages, P, Hkv, >= 128] or HND [num_pages, Hkv,
    P, >= 128] (bf16, or e4m3 codes as uint8 / float8_e4m3fn; channels past 128
    are padding the producer leaves alone); block_tables int32 [B, pages];
    q_indptr int32 [B + 1]; seq_lens int32 [B] (lengths after the append);
    out_q [T, Hq, 128].  Every other field is passed through."""
    if layout not in ("HND", "NHD"):
        raise ValueError("layout must be 'HND' or 'NHD'")
    torch = _torch()
    i32, f32, b16 = (torch.int32,), (torch.float32,), (torch.bfloat16, torch.int16)
    _check_tensors(qkv.device, {"qkv": (qkv, b16), "cos_sin": (cos_sin, f32), "q_weight": (q_weight, b16),
                                "k_weight": (k_weight, b16), "q_indptr": (q_indptr, i32),
                                "seq_lens": (seq_lens, i32), "block_tables": (block_tables, i32),
                                "out_q": out_q, "k_cache": k_cache, "v_cache": v_cache,
                                "q_scale": (q_scale, f32), "err": (err, i32)})
    if qkv.stride(-1) != 1 or k_cache.stride(-1) != 1 or v_cache.stride(-1) != 1:
        raise ValueError("the channel dimension of qkv and the caches must be contiguous")
    if tuple(k_cache.shape) != tuple(v_cache.shape):
        raise ValueError("K and V caches must have the same shape")
    a = PkvAppendArgs()
    a.num_tokens = int(qkv.shape[0])
    a.batch = int(block_tables.shape[0])
    a.num_qo_heads = int(out_q.shape[1])
    a.head_dim = 128
    if layout == "NHD":
        num_pages, P, Hkv, W_ = (int(x) for x in k_cache.shape)
    else:
        num_pages, Hkv, P, W_ = (int(x) for x in k_cache.shape)
    if W_ < 128:
        raise ValueError("cache rows need at least 128 channels")
    a.num_kv_heads, a.page_size, a.num_pages = Hkv, P, num_pages
    a.max_pages_per_seq = int(block_tables.shape[1])
    a.table_stride = _stride(block_tables, 0, int(block_tables.shape[1]))
    a.max_pos = int(max_pos)
    a.norm_policy = int(norm_policy)
    a.clear_tail = 1 if clear_tail else 0
    a.kv_dtype = _dtype_code(k_cache)
    a.eps, a.k_scale, a.v_scale = float(eps), float(k_scale), float(v_scale)
    a.qkv = qkv.data_ptr()
    a.qkv_stride_tok = _stride(qkv, 0, int(qkv.shape[1]))
    a.cos_sin = cos_sin.data_ptr()
    a.q_weight, a.k_weight = q_weight.data_ptr(), k_weight.data_ptr()
    a.q_indptr, a.seq_lens, a.block_tables = q_indptr.data_ptr(), seq_lens.data_ptr(), block_tables.data_ptr()
    a.out_q, a.k_cache, a.v_cache = out_q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr()
    a.err_word = err.data_ptr() if err is not None else 0
    a.q_quant = int(q_quant)
    a.upper_max, a.q_scale_inv = float(upper_max), float(q_scale_inv)
    a.q_scale_layout, a.q_scale_stride = int(q_scale_layout), int(q_scale_stride)
    a.q_scale = q_scale.data_ptr() if q_scale is not None else 0
    a.layout = PKV_LAYOUT_HND if layout == "HND" else PKV_LAYOUT_NHD
    a._tensor_device = qkv.device
    for prefix, t in (("k", k_cache), ("v", v_cache)):
        if layout == "NHD":
            sp, sh, st = _stride(t, 0, P * Hkv * W_), _stride(t, 2, W_), _stride(t, 1, Hkv * W_)
        else:
            sp, sh, st = _stride(t, 0, Hkv * P * W_), _stride(t, 1, P * W_), _stride(t, 2, W_)
        setattr(a, f"{prefix}_stride_page", sp)
        setattr(a, f"{prefix}_stride_head", sh)
        setattr(a, f"{prefix}_stride_tok", st)
    return a


@dataclass
class DeviceAppend:
    args: PkvAppendArgs
    tensors: dict

    def run(self, stream=None, check: bool = True) -> int:
        torch = _torch()
        s = stream if stream is not None else torch.cuda.current_stream()
        return pkv_append(self.args, int(s.cuda_stream), check=check)


def upload_append(prob, device="cuda", with_err: bool = True) -> DeviceAppend:
    """Copy a workloads.AppendProblem to `device` (caches from their initial
    contents, out_q NaN-filled) and fill pkv_append_args for it."""
    import numpy as np
    torch = _torch()
    t = {}
    t["qkv"] = torch.from_numpy(prob.qkv.view(np.int16)).to(device)
    t["cos_sin"] = torch.from_numpy(prob.cos_sin).to(device)
    t["q_w"] = torch.from_numpy(prob.q_weight.view(np.int16)).to(device)
    t["k_w"] = torch.from_numpy(prob.k_weight.view(np.int16)).to(device)
    t["q_indptr"] = torch.from_numpy(prob.q_indptr).to(device)
    t["seq_lens"] = torch.from_numpy(prob.seq_lens).to(device)
    t["table"] = torch.from_numpy(prob.block_tables).to(device)
    if prob.kv_dtype == "bf16":
        t["k_cache"] = torch.from_numpy(prob.k_cache0.view(np.int16)).to(device)
        t["v_cache"] = torch.from_numpy(prob.v_cache0.view(np.int16)).to(device)
    else:
        t["k_cache"] = torch.from_numpy(prob.k_cache0).to(device)
        t["v_cache"] = torch.from_numpy(prob.v_cache0).to(device)
    T = prob.total_tokens
    if prob.q_quant == 0:
        t["out_q"] = torch.full((max(T, 1), prob.num_qo_heads, 128), -1, dtype=torch.int16, device=device)
    else:  # e4m3 codes; 0xFF (a NaN code) marks bytes never written
        t["out_q"] = torch.full((max(T, 1), prob.num_qo_heads, 128), 0xFF, dtype=torch.uint8, device=device)
    if prob.q_quant == 1:  # NaN-filled: entries no row writes stay NaN
        t["q_scale"] = torch.full((max(prob.q_scale_entries, 1),), float("nan"), dtype=torch.float32, device=device)
    if with_err:
        t["err"] = torch.zeros(1, dtype=torch.int32, device=device)
    a = PkvAppendArgs()
    a.num_tokens = T
    a.batch = prob.batch
    a.num_qo_heads = prob.num_qo_heads
    a.num_kv_heads = prob.num_kv_heads
    a.head_dim = 128
    a.page_size = prob.page_size
    a.max_pages_per_seq = prob.max_pages
    a.max_pos = prob.max_pos
    a.num_pages = prob.num_pages
    a.norm_policy = prob.norm_policy
    a.clear_tail = 1 if prob.clear_tail else 0
    a.kv_dtype = DTYPE_CODES[prob.kv_dtype]
    a.eps = prob.eps
    a.k_scale = prob.k_scale
    a.v_scale = prob.v_scale
    a.qkv = t["qkv"].data_ptr()
    a.qkv_stride_tok = prob.qkv.shape[1]
    a.cos_sin = t["cos_sin"].data_ptr()
    a.q_weight = t["q_w"].data_ptr()
    a.k_weight = t["k_w"].data_ptr()
    a.q_indptr = t["q_indptr"].data_ptr()
    a.seq_lens = t["seq_lens"].data_ptr()
    a.block_tables = t["table"].data_ptr()
    a.table_stride = prob.block_tables.shape[1]
    a.out_q = t["out_q"].data_ptr()
    a.k_cache = t["k_cache"].data_ptr()
    a.v_cache = t["v_cache"].data_ptr()
    a.err_word = t["err"].data_ptr() if with_err else 0
    a.q_quant = prob.q_quant
    a.upper_max = prob.upper_max
    a.q_scale_inv = prob.q_scale_inv
    a.q_scale_layout = prob.q_scale_layout
    a.q_scale_stride = prob.q_scale_stride
    a.q_scale = t["q_scale"].data_ptr() if prob.q_quant == 1 else 0
    a.layout = PKV_LAYOUT_HND if prob.layout == "HND" else PKV_LAYOUT_NHD
    sp, sh, st = prob.cache_strides()
    a.k_stride_page = a.v_stride_page = sp
    a.k_stride_head = a.v_stride_head = sh
    a.k_stride_tok = a.v_stride_tok = st
    return DeviceAppend(args=a, tensors=t)
