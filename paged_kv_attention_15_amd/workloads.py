"""Seeded synthetic inputs for paged-KV attention.

This module only draws random numbers and lays them out in memory: it rounds
fp32 draws to the storage dtypes (bf16, OCP e4m3) and scatters per-request KV
rows into a shuffled page pool with a block table.  It holds none of the
attention arithmetic, so both the CPU oracle and the HIP path can consume its
arrays without sharing any code with each other.

Layout facts it follows (cited from the pages):
  * flashinfer.cake_fmha API page, paragraph on the BF16 context profiles and
    the FP8 qualification: HND pages, a shared K/V page table, page sizes 32 /
    64, a batch-four q511/KV2047 context profile.
  * PR #5952 page (fused QK RMSNorm + RoPE + paged KV append), summary: a dense
    [B, max_pages] page table; FP8 append contract (PR #5956 section
    "Contract"): NHD caches [num_pages, page_size, Hkv, D], K/V stored as
    x / scale with round-to-nearest saturating e4m3 (max 448), seq_lens is the
    total length including the rows being appended.
  * PR #4557 page, MLA decode description: one latent KV head, 512 latent +
    64 rope channels, V is the latent part of the same row.

Draw order for every workload: seq_lens (ragged workloads only), then the
page permutation, then Q, K and V, each standard normal in fp32, from one
numpy.random.default_rng(seed).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

# dtype tags shared by the binding, the oracle wrapper and the tests
F32, BF16, E4M3 = "f32", "bf16", "e4m3"
HND, NHD = "HND", "NHD"

E4M3_MAX = 448.0
_NAN_BITS = {BF16: np.uint16(0x7FC0), E4M3: np.uint8(0x7F)}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def e4m3_bytes(x: np.ndarray) -> np.ndarray:
    """fp32 -> OCP e4m3 ("fn", max 448) bytes, round to nearest even, saturated.

    Uses torch's float8_e4m3fn cast as the rounding primitive after clamping to
    the finite range (the pages' "RN satfinite" storage rule)."""
    import torch

    t = torch.from_numpy(np.clip(np.ascontiguousarray(x, dtype=np.float32), -E4M3_MAX, E4M3_MAX))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == BF16:
        return bf16_bits(x)
    raise ValueError(dtype)


def _nan_fill(arr: np.ndarray, dtype: str) -> None:
    if dtype == F32:
        arr[...] = np.float32(np.nan)
    else:
        arr[...] = _NAN_BITS[dtype]


def _np_storage(dtype: str):
    return {F32: np.float32, BF16: np.uint16, E4M3: np.uint8}[dtype]


@dataclasses.dataclass
class LogitProfile:
    """Shapes the scaled logits of a drawn problem (inputs that move a row's
    running maximum where a test wants it, or hold every logit equal or far
    below zero).

    Every KV head g gets a random unit direction u_g (its own generator, so the
    main draws are unchanged).  Every query row of a head of group g is shifted
    by q_shift * u_g.  A key listed in `levels` as (request b, first key j0,
    end key j1, rise) has its K row replaced by c * u_g in every KV head g,
    with c = rise / (scale * q_shift): its logit against a query row of the
    group is then rise * (1 + <z, u_g> / q_shift) in natural-log units, z the
    row's own standard-normal part (about 5 % of spread per sigma for the
    default shift), while the other keys' logits stay near N(0, 2).  `tail_rise`
    does the same to the keys past each request's length in its last page
    (they must stay invisible; V keeps its poison there).  `equal_keys` makes
    every key row of a (request, KV head) one shared random vector, so all of
    a row's logits are equal; `negative` (> 0) shifts Q by +a u_g and every K
    row by -a u_g with a = sqrt(negative / scale), putting every logit near
    -negative."""

    q_shift: float = 20.0
    levels: tuple = ()
    tail_rise: Optional[float] = None
    equal_keys: bool = False
    negative: float = 0.0
    seed: int = 7919


@dataclasses.dataclass
class Problem:
    """One paged attention call, held in host memory.

    Arrays hold raw storage: float32 values, uint16 bf16 bit patterns or uint8
    e4m3 codes.  Shapes:
      q            [T_q, Hq, D_qk]       rows of request b are q_indptr[b]..q_indptr[b+1]
      k_pool       HND [num_pages, Hkv, P, D_qk]  or  NHD [num_pages, P, Hkv, D_qk]
      v_pool       same with D_v, or None when V is the first D_v channels of K (MLA)
      block_tables int32 [B, max_pages]  (shared by K and V)
      seq_lens     int32 [B]  total KV length, including the request's own q rows
      q_indptr     int32 [B+1]
    """

    name: str
    batch: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim_qk: int
    head_dim_v: int
    page_size: int
    layout: str
    q_dtype: str
    kv_dtype: str
    o_dtype: str
    q: np.ndarray
    k_pool: np.ndarray
    v_pool: Optional[np.ndarray]
    block_tables: np.ndarray
    seq_lens: np.ndarray
    q_indptr: np.ndarray
    scale: float
    k_scale: float = 1.0
    v_scale: float = 1.0
    causal: bool = True
    is_decode: bool = True      # uniform q rows per request (decode / speculative rows)
    mla: bool = False           # V shares the K rows
    num_splits: int = 0         # 0 = let the planner choose
    sinks: Optional[np.ndarray] = None           # float32 [Hq] sink logits, or None
    v_block_tables: Optional[np.ndarray] = None  # int32 [B, max_pages] for V, None = shared

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def q_len(self) -> int:
        """Uniform q rows per request (decode); for context, the maximum."""
        d = np.diff(self.q_indptr)
        return int(d.max()) if d.size else 0

    @property
    def total_q(self) -> int:
        return int(self.q_indptr[-1])

    @property
    def max_kv_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.size else 0

    def kv_bytes(self) -> int:
        """Algorithmic KV bytes: every visible token of every request once per
        KV head (MLA rows counted once since V shares them)."""
        eb = {F32: 4, BF16: 2, E4M3: 1}[self.kv_dtype]
        per_tok = self.head_dim_qk * eb if self.mla else (self.head_dim_qk + self.head_dim_v) * eb
        return int(self.seq_lens.astype(np.int64).sum()) * self.num_kv_heads * per_tok

    def flops(self) -> int:
        """2*(D_qk + D_v) per visible (query row, head, key) triple."""
        total = 0
        for b in range(self.batch):
            n = int(self.q_indptr[b + 1] - self.q_indptr[b])
            L = int(self.seq_lens[b])
            for i in range(n):
                c = (L - n + i + 1) if self.causal else L
                total += max(0, min(c, L))
        return 2 * (self.head_dim_qk + self.head_dim_v) * self.num_qo_heads * total


def make_problem(
    *,
    name: str,
    seed: int,
    batch: int,
    seq_lens,
    q_lens,
    num_qo_heads: int,
    num_kv_heads: int,
    head_dim_qk: int,
    head_dim_v: int,
    page_size: int,
    layout: str = HND,
    q_dtype: str = BF16,
    kv_dtype: str = BF16,
    o_dtype: Optional[str] = None,
    scale: Optional[float] = None,
    causal: bool = True,
    is_decode: bool = True,
    mla: bool = False,
    poison: bool = False,
    extra_page_frac: float = 0.0,
    table_slack_pages: int = 0,
    rng: Optional[np.random.Generator] = None,
    num_splits: int = 0,
    sinks: bool = False,
    separate_v_table: bool = False,
    logits: Optional[LogitProfile] = None,
) -> Problem:
    """Draw one problem.  `seq_lens` / `q_lens` are int sequences of length B.

    poison=True fills page tails (tokens >= L in a request's last page), the
    extra pages and the unused block-table slots' target pages with NaN, so a
    kernel that reads anything it should not turns the output non-finite.

    sinks=True draws one sink logit per query head (N(1, 1)) after everything
    else; separate_v_table=True then moves every V page to a second random
    placement with its own table (the key pages stay where they are)."""
    if rng is None:
        rng = np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32).reshape(batch)
    q_lens = np.asarray(q_lens, dtype=np.int32).reshape(batch)
    q_indptr = np.zeros(batch + 1, dtype=np.int32)
    q_indptr[1:] = np.cumsum(q_lens)
    P = page_size
    Hkv = num_kv_heads
    pages_per_req = [(int(L) + P - 1) // P for L in seq_lens]
    needed = int(sum(pages_per_req))
    extra = int(math.ceil(needed * extra_page_frac))
    if poison and extra == 0:
        extra = 1
    num_pages = needed + extra
    max_pages = max(pages_per_req + [1]) + table_slack_pages

    perm = rng.permutation(num_pages).astype(np.int32)

    if o_dtype is None:
        o_dtype = q_dtype
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim_qk)

    T_q = int(q_indptr[-1])
    q32 = rng.standard_normal((T_q, num_qo_heads, head_dim_qk), dtype=np.float32)
    G = num_qo_heads // Hkv
    page_start = np.concatenate([[0], np.cumsum(pages_per_req)]).astype(np.int64)
    if logits is not None:
        prng = np.random.default_rng(logits.seed)
        u = prng.standard_normal((Hkv, head_dim_qk))
        u = (u / np.linalg.norm(u, axis=1, keepdims=True)).astype(np.float32)  # [Hkv, D]
        a_q = math.sqrt(logits.negative / scale) if logits.negative > 0 else logits.q_shift
        q32 += a_q * np.repeat(u, G, axis=0)[None, :, :]
        k_equal = prng.standard_normal((Hkv, head_dim_qk)).astype(np.float32)
        # (logical page, token, rise) of every planted key
        plants = []
        for (b, j0, j1, rise) in logits.levels:
            for j in range(int(j0), int(j1)):
                if 0 <= j < int(seq_lens[b]):
                    plants.append((int(page_start[b]) + j // P, j % P, float(rise)))
        if logits.tail_rise is not None:
            for b in range(batch):
                L = int(seq_lens[b])
                if L % P:
                    lp = int(page_start[b]) + L // P
                    plants += [(lp, t, float(logits.tail_rise)) for t in range(L % P, P)]
    q = _store(q32, q_dtype)
    del q32

    # logical page i of the concatenated requests lives at physical page perm[i]
    def draw_pool(dim: int, dtype_tag: str):
        store_dtype = F32 if dtype_tag == E4M3 else dtype_tag
        pool = np.zeros((num_pages, Hkv, P, dim), dtype=_np_storage(store_dtype))
        chunk = max(1, (1 << 24) // max(1, Hkv * P * dim))
        for start in range(0, needed, chunk):
            stop = min(needed, start + chunk)
            vals = rng.standard_normal((stop - start, Hkv, P, dim), dtype=np.float32)
            if is_k and logits is not None:
                if logits.equal_keys:
                    vals[...] = k_equal[None, :, None, :]
                if logits.negative > 0:
                    vals -= math.sqrt(logits.negative / scale) * u[None, :, None, :]
                for (lp, t, rise) in plants:
                    if start <= lp < stop:
                        vals[lp - start, :, t, :] = (rise / (scale * logits.q_shift)) * u
            pool[perm[start:stop]] = _store(vals, store_dtype)
        return pool

    is_k = True
    k_pool = draw_pool(head_dim_qk, kv_dtype)
    is_k = False
    v_pool = None if mla else draw_pool(head_dim_v, kv_dtype)

    k_scale = v_scale = 1.0
    if kv_dtype == E4M3:
        # per-tensor scalar scale s = max|x| / 448 over the needed pages; stored = x / s
        used = perm[:needed]
        k_scale = float(np.abs(k_pool[used]).max()) / E4M3_MAX
        k_pool = e4m3_bytes(k_pool / np.float32(k_scale))
        if v_pool is not None:
            v_scale = float(np.abs(v_pool[used]).max()) / E4M3_MAX
            v_pool = e4m3_bytes(v_pool / np.float32(v_scale))

    block_tables = np.zeros((batch, max_pages), dtype=np.int32)
    poison_page = int(perm[needed]) if extra > 0 else 0
    cursor = 0
    for b, npg in enumerate(pages_per_req):
        block_tables[b, :npg] = perm[cursor:cursor + npg]
        block_tables[b, npg:] = poison_page
        cursor += npg

    if poison:
        for pool in (k_pool, v_pool):
            if pool is None:
                continue
            for phys in perm[needed:]:
                _nan_fill(pool[phys], kv_dtype)
            if pool is k_pool and logits is not None and logits.tail_rise is not None:
                continue  # the K tails hold the planted keys instead
            cursor = 0
            for b, npg in enumerate(pages_per_req):
                L = int(seq_lens[b])
                if npg > 0 and L % P != 0:
                    _nan_fill(pool[perm[cursor + npg - 1], :, L % P:, :], kv_dtype)
                cursor += npg

    sink_vals = None
    if sinks:
        sink_vals = (1.0 + rng.standard_normal(num_qo_heads)).astype(np.float32)
    v_tables = None
    if separate_v_table:
        if v_pool is None:
            raise ValueError("separate V tables need a separate V pool")
        perm_v = rng.permutation(num_pages).astype(np.int32)
        moved = np.empty_like(v_pool)
        moved[perm_v] = v_pool[perm]  # logical page i: from perm[i] to perm_v[i]
        v_pool = moved
        v_tables = np.zeros_like(block_tables)
        v_poison = int(perm_v[needed]) if extra > 0 else 0
        cursor = 0
        for b, npg in enumerate(pages_per_req):
            v_tables[b, :npg] = perm_v[cursor:cursor + npg]
            v_tables[b, npg:] = v_poison
            cursor += npg

    if layout == NHD:
        k_pool = np.ascontiguousarray(k_pool.transpose(0, 2, 1, 3))
        if v_pool is not None:
            v_pool = np.ascontiguousarray(v_pool.transpose(0, 2, 1, 3))
    elif layout != HND:
        raise ValueError(layout)

    return Problem(
        name=name, batch=batch, num_qo_heads=num_qo_heads, num_kv_heads=Hkv,
        head_dim_qk=head_dim_qk, head_dim_v=head_dim_v, page_size=P, layout=layout,
        q_dtype=q_dtype, kv_dtype=kv_dtype, o_dtype=o_dtype, q=q, k_pool=k_pool,
        v_pool=v_pool, block_tables=block_tables, seq_lens=seq_lens, q_indptr=q_indptr,
        scale=float(scale), k_scale=k_scale, v_scale=v_scale, causal=causal,
        is_decode=is_decode, mla=mla, num_splits=num_splits, sinks=sink_vals, v_block_tables=v_tables,
    )


def ragged_log_uniform_lens(rng: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    """L = floor(exp(U(ln lo, ln hi))), drawn before anything else."""
    return np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size=n))).astype(np.int32)


# ---------------------------------------------------------------------------
# The five workloads.  Sizes are the method's decode / context profiles; the
# names say what each one is.
# ---------------------------------------------------------------------------

def tiny_gqa_fp32(seed: int = 0, poison: bool = True) -> Problem:
    """B=2, one q row, Hq=8 on one KV head, D=128, pages of 16, L={37,100},
    fp32 end to end, a 16-page pool (10 used + 6 NaN pages), two KV splits."""
    return make_problem(
        name="tiny-gqa-fp32-b2", seed=seed, batch=2, seq_lens=[37, 100], q_lens=[1, 1],
        num_qo_heads=8, num_kv_heads=1, head_dim_qk=128, head_dim_v=128, page_size=16,
        q_dtype=F32, kv_dtype=F32, poison=poison, extra_page_frac=0.6, num_splits=2,
    )


def gqa_bf16_b32_kv4096(seed: int = 0, poison: bool = False) -> Problem:
    """B=32, one q row, Hq=32 / Hkv=8, D=128, HND pages of 32, L=4096, bf16."""
    return make_problem(
        name="bf16-gqa-b32-h32x8-kv4096-p32", seed=seed, batch=32, seq_lens=[4096] * 32,
        q_lens=[1] * 32, num_qo_heads=32, num_kv_heads=8, head_dim_qk=128, head_dim_v=128,
        page_size=32, q_dtype=BF16, kv_dtype=BF16, poison=poison,
        extra_page_frac=0.25 if poison else 0.0,
    )


def gqa_fp8_b16_ragged(seed: int = 0, poison: bool = False) -> Problem:
    """B=16, one q row, Hq=64 / Hkv=8, D=128, HND pages of 64, e4m3 K/V with
    per-tensor scales, bf16 Q and output, L log-uniform in [512, 32768]."""
    rng = np.random.default_rng(seed)
    lens = ragged_log_uniform_lens(rng, 16, 512, 32768)
    return make_problem(
        name="fp8-gqa-b16-h64x8-ragged-p64", seed=seed, batch=16, seq_lens=lens, q_lens=[1] * 16,
        num_qo_heads=64, num_kv_heads=8, head_dim_qk=128, head_dim_v=128, page_size=64,
        q_dtype=BF16, kv_dtype=E4M3, o_dtype=BF16, poison=poison,
        extra_page_frac=0.25 if poison else 0.0, rng=rng,
    )


def mla_b512_kv4096(seed: int = 0, q_len: int = 1, batch: int = 512, seq_len: int = 4096,
                    poison: bool = False) -> Problem:
    """MLA decode: Hq=128 on one shared latent head, D_qk=576 (512+64),
    D_v=512 (V = first 512 channels of the K row), pages of 64, bf16,
    q_len in {1, 2} (speculative rows are causal within the draft)."""
    return make_problem(
        name=f"mla-b{batch}-q{q_len}-h128-kv{seq_len}-p64", seed=seed, batch=batch,
        seq_lens=[seq_len] * batch, q_lens=[q_len] * batch, num_qo_heads=128, num_kv_heads=1,
        head_dim_qk=576, head_dim_v=512, page_size=64, q_dtype=BF16, kv_dtype=BF16,
        scale=1.0 / math.sqrt(576.0), mla=True, poison=poison,
        extra_page_frac=0.25 if poison else 0.0,
    )


def context_b4_q511_kv2047(seed: int = 0, poison: bool = False) -> Problem:
    """Causal paged context: B=4, 511 new rows per request whose total KV
    length (including those rows) is 2047, Hq=64 / Hkv=8, D=128, HND pages
    of 32, bf16, explicit q_indptr {0,511,1022,1533,2044}."""
    return make_problem(
        name="ctx-b4-q511-kv2047-h64x8-p32", seed=seed, batch=4, seq_lens=[2047] * 4,
        q_lens=[511] * 4, num_qo_heads=64, num_kv_heads=8, head_dim_qk=128, head_dim_v=128,
        page_size=32, q_dtype=BF16, kv_dtype=BF16, is_decode=False, poison=poison,
        extra_page_frac=0.25 if poison else 0.0,
    )


def context_b4_q257_kv1024_p1024(seed: int = 0, separate: bool = True, poison: bool = False) -> Problem:
    """The API page's second BF16 context profile: B=4, 257 new rows per
    request over 1024 keys, Hq=64 / Hkv=8, D=128, 1024-token pages, with
    separate K/V page tables (or the shared table)."""
    return make_problem(
        name=f"ctx-b4-q257-kv1024-p1024-sep{int(separate)}", seed=seed, batch=4, seq_lens=[1024] * 4,
        q_lens=[257] * 4, num_qo_heads=64, num_kv_heads=8, head_dim_qk=128, head_dim_v=128,
        page_size=1024, q_dtype=BF16, kv_dtype=BF16, is_decode=False, poison=poison,
        extra_page_frac=0.25 if poison else 0.0, separate_v_table=separate,
    )


WORKLOADS: Dict[str, callable] = {
    "tiny-gqa-fp32": tiny_gqa_fp32,
    "bf16-gqa-b32-kv4096": gqa_bf16_b32_kv4096,
    "fp8-gqa-b16-ragged": gqa_fp8_b16_ragged,
    "mla-b512-kv4096": mla_b512_kv4096,
    "ctx-b4-q511-kv2047": context_b4_q511_kv2047,
}


# ---------------------------------------------------------------- paged KV append producer inputs
#
# PR #5952 page (fused BF16 QK RMSNorm + NeoX RoPE + paged KV append), summary:
# a packed BF16 qkv [T, (Hq + 2 Hkv) * 128] (Q heads, then K heads, then V
# heads), an FP32 cos_sin [max_pos, 128] table, optional per-head RMSNorm
# weights, NHD caches [num_pages, page_size, Hkv, 128] reached through a dense
# [B, max_pages] table; PR #5956 "Contract": seq_lens is the total length after
# the append and K/V may be stored as e4m3 codes of x / scale.

ROPE_DIM = 128


@dataclasses.dataclass
class AppendProblem:
    """One append call, held in host memory (raw storage arrays).

      qkv          uint16 bf16 bits [T, (Hq + 2 Hkv) * 128]
      cos_sin      float32 [max_pos, 128]: cos of the 64 frequencies, then their sin
      q_weight     uint16 bf16 bits [128] (RMSNorm weights of the Q heads)
      k_weight     uint16 bf16 bits [128]
      q_indptr     int32 [B + 1]   rows of request b are q_indptr[b] .. q_indptr[b+1]
      seq_lens     int32 [B]       total length after the append
      block_tables int32 [B, max_pages]
      k_cache0     initial K cache (uint16 bf16 bits or uint8 e4m3), NHD [num_pages, P, Hkv, 128 + pad]
                   or HND [num_pages, Hkv, P, 128 + pad]; the last `cache_pad` elements of each
                   row are padding no call may write
      v_cache0     same for V
    """

    name: str
    batch: int
    num_qo_heads: int
    num_kv_heads: int
    page_size: int
    qkv: np.ndarray
    cos_sin: np.ndarray
    q_weight: np.ndarray
    k_weight: np.ndarray
    q_indptr: np.ndarray
    seq_lens: np.ndarray
    block_tables: np.ndarray
    k_cache0: np.ndarray
    v_cache0: np.ndarray
    norm_policy: int = 0
    eps: float = 1e-6
    kv_dtype: str = BF16
    k_scale: float = 1.0
    v_scale: float = 1.0
    clear_tail: bool = True
    head_dim: int = ROPE_DIM
    # query output: 0 bf16; 1 e4m3 with a dynamic scale per (row, head)
    # (q_scale = max(|q|, 1e-6) / upper_max); 2 e4m3 of q * q_scale_inv
    q_quant: int = 0
    upper_max: float = 448.0
    q_scale_inv: float = 1.0
    # dynamic scales: 0 -> [T, Hq]; 1 -> [B, Hq, q_scale_stride] indexed by the row inside its request
    q_scale_layout: int = 0
    q_scale_stride: int = 0
    layout: str = "NHD"
    cache_pad: int = 0

    def cache_rows(self, cache: np.ndarray) -> np.ndarray:
        """View [num_pages, P, Hkv, 128] of a cache array of this problem's
        layout (writes through the view reach the array)."""
        rows = cache[..., :self.head_dim]
        return rows if self.layout == "NHD" else rows.transpose(0, 2, 1, 3)

    def cache_strides(self):
        """(page, head, token) strides of the caches in elements."""
        H, P, W = self.num_kv_heads, self.page_size, self.head_dim + self.cache_pad
        return (P * H * W, W, H * W) if self.layout == "NHD" else (H * P * W, P * W, W)

    @property
    def q_scale_entries(self) -> int:
        """Length of the dynamic scale buffer (0 without the dynamic policy)."""
        if self.q_quant != 1:
            return 0
        if self.q_scale_layout == 0:
            return self.total_tokens * self.num_qo_heads
        return self.batch * self.num_qo_heads * self.q_scale_stride

    @property
    def total_tokens(self) -> int:
        return int(self.q_indptr[-1])

    @property
    def num_pages(self) -> int:
        return int(self.k_cache0.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_pos(self) -> int:
        return int(self.cos_sin.shape[0])

    def bytes_moved(self) -> int:
        """Algorithmic HBM bytes of one call: qkv read, Q written, K and V rows
        written, and the cleared tail rows of every nonempty request."""
        T, Hq, Hkv, D, P = self.total_tokens, self.num_qo_heads, self.num_kv_heads, self.head_dim, self.page_size
        eb = 1 if self.kv_dtype == E4M3 else 2
        tail = 0
        if self.clear_tail:
            for L in self.seq_lens.tolist():
                if L > 0:
                    tail += P - 1 - (L - 1) % P
        qb = 2 if self.q_quant == 0 else 1
        qs = 4 * T * Hq if self.q_quant == 1 else 0
        return (T * (Hq + 2 * Hkv) * D * 2 + T * Hq * D * qb + qs + 2 * T * Hkv * D * eb
                + 2 * tail * Hkv * D * eb)


def rope_table(max_pos: int, base: float = 10000.0) -> np.ndarray:
    """A standard NeoX rotary table [max_pos, 128]: frequency i = base^(-2i/128),
    row p = cos(p * f_0..63) then sin(p * f_0..63), in fp32."""
    half = ROPE_DIM // 2
    inv = base ** (-np.arange(half, dtype=np.float64) * 2.0 / ROPE_DIM)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def make_append_problem(*, name: str, seed: int, new_lens, seq_lens, num_qo_heads: int, num_kv_heads: int,
                        page_size: int, norm_policy: int = 0, kv_dtype: str = BF16, clear_tail: bool = True,
                        k_scale: float = 1.0, v_scale: float = 1.0, extra_pages: int = 2,
                        table_slack_pages: int = 1, max_pos: Optional[int] = None, q_quant: int = 0,
                        upper_max: float = 448.0, q_scale_inv: float = 1.0, q_scale_layout: int = 0,
                        q_scale_stride: int = 0, layout: str = "NHD", cache_pad: int = 0) -> AppendProblem:
    """Draw order: page permutation, qkv, the two weight vectors, the initial
    cache contents (random non-zero storage so that untouched and cleared rows
    are told apart, padding included).  Unused table slots point at a spare
    page that no request owns, so any stray write through them shows up."""
    rng = np.random.default_rng(seed)
    new_lens = [int(x) for x in new_lens]
    seq_lens = [int(x) for x in seq_lens]
    B = len(seq_lens)
    D, P, Hq, Hkv = ROPE_DIM, int(page_size), int(num_qo_heads), int(num_kv_heads)
    pages_per = [(L + P - 1) // P for L in seq_lens]
    used = sum(pages_per)
    num_pages = used + max(1, extra_pages)
    perm = rng.permutation(num_pages).astype(np.int32)
    spare = int(perm[-1])
    width = max(1, max(pages_per) if pages_per else 1) + table_slack_pages
    table = np.full((B, width), spare, dtype=np.int32)
    off = 0
    for b, n in enumerate(pages_per):
        table[b, :n] = perm[off:off + n]
        off += n
    q_indptr = np.zeros(B + 1, dtype=np.int32)
    q_indptr[1:] = np.cumsum(new_lens)
    T = int(q_indptr[-1])
    qkv = bf16_bits(rng.standard_normal((T, (Hq + 2 * Hkv) * D)).astype(np.float32))
    q_w = bf16_bits((1.0 + 0.25 * rng.standard_normal(D)).astype(np.float32))
    k_w = bf16_bits((1.0 + 0.25 * rng.standard_normal(D)).astype(np.float32))
    if layout not in ("NHD", "HND"):
        raise ValueError(layout)
    shape = (num_pages, P, Hkv, D + cache_pad) if layout == "NHD" else (num_pages, Hkv, P, D + cache_pad)
    if kv_dtype == BF16:
        k0 = bf16_bits((rng.standard_normal(shape) + 3.0).astype(np.float32))
        v0 = bf16_bits((rng.standard_normal(shape) + 3.0).astype(np.float32))
    elif kv_dtype == E4M3:
        k0 = rng.integers(1, 0x7E, size=shape, dtype=np.uint8)  # finite, non-zero codes
        v0 = rng.integers(1, 0x7E, size=shape, dtype=np.uint8)
    else:
        raise ValueError(kv_dtype)
    mp = max_pos if max_pos is not None else max(1, max(seq_lens) if seq_lens else 1) + 7
    return AppendProblem(name=name, batch=B, num_qo_heads=Hq, num_kv_heads=Hkv, page_size=P, qkv=qkv,
                         cos_sin=rope_table(mp), q_weight=q_w, k_weight=k_w, q_indptr=q_indptr,
                         seq_lens=np.array(seq_lens, dtype=np.int32), block_tables=table, k_cache0=k0,
                         v_cache0=v0, norm_policy=norm_policy, kv_dtype=kv_dtype, k_scale=float(k_scale),
                         v_scale=float(v_scale), clear_tail=clear_tail, q_quant=int(q_quant),
                         upper_max=float(upper_max), q_scale_inv=float(q_scale_inv),
                         q_scale_layout=int(q_scale_layout), q_scale_stride=int(q_scale_stride),
                         layout=layout, cache_pad=int(cache_pad))


def append_h64x8_b32_decode(seed: int = 0, norm_policy: int = 2, kv_dtype: str = BF16,
                            q_quant: int = 0, layout: str = "NHD") -> AppendProblem:
    """The pages' H1 row: Hq=64 / Hkv=8, 32 requests appending one row each,
    here at total lengths 2048 with 64-token pages (q_quant 1: e4m3 queries
    with a dynamic scale per (row, head) in the [T, Hq] layout, upper_max 448).
    The pages' caches are NHD; layout "HND" writes the attention pools' layout."""
    tag = "" if layout == "NHD" else f"-{layout.lower()}"
    return make_append_problem(name=f"append-h64x8-b32-decode-p{norm_policy}-{kv_dtype}-q{q_quant}{tag}", seed=seed,
                               layout=layout,
                               new_lens=[1] * 32, seq_lens=[2048] * 32, num_qo_heads=64, num_kv_heads=8,
                               page_size=64, norm_policy=norm_policy, kv_dtype=kv_dtype,
                               k_scale=0.05 if kv_dtype == E4M3 else 1.0, v_scale=0.05 if kv_dtype == E4M3 else 1.0,
                               q_quant=q_quant, upper_max=448.0)
