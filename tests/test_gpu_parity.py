"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small problems are compared on every output element; the full-size workloads
are compared on sampled (row, head) pairs that the oracle computes one by one,
in the launch configuration the benchmark times.  Tolerances are the pages'
(tests/golden/tolerances.json).  Inputs poison page tails, spare pages and
unused table slots with NaN where noted, so any stray read shows up as a
non-finite output.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from paged_kv_attention_15_amd import pkv, workloads as W
from tests._gpu import compare, run_gpu, sample_pairs, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pkv.load_library()
    torch.cuda.init()


def _gqa(seq_lens, hq=32, hkv=8, P=32, kv=W.BF16, poison=True, layout=W.HND, seed=1, q_lens=None, **kw):
    B = len(seq_lens)
    return W.make_problem(name=f"gqa-{kv}-P{P}-h{hq}x{hkv}", seed=seed, batch=B, seq_lens=seq_lens,
                          q_lens=q_lens or [1] * B, num_qo_heads=hq, num_kv_heads=hkv, head_dim_qk=128,
                          head_dim_v=128, page_size=P, kv_dtype=kv, q_dtype=W.BF16, o_dtype=W.BF16,
                          poison=poison, extra_page_frac=0.25, table_slack_pages=2, layout=layout, **kw)


# ----------------------------------------------------------------- the five workloads

def test_tiny_gqa_fp32_workload():
    prob = W.tiny_gqa_fp32(poison=True)
    say(f"case {prob.name}")
    dp = run_gpu(prob)
    assert dp.workspace_bytes > 0  # two KV partitions + the reducer
    compare(prob, dp)


@pytest.mark.parametrize("splits", [None, 1, 3, -1])
def test_gqa_bf16_ragged_small(splits):
    prob = _gqa([1, 31, 32, 33, 700, 129])
    say(f"case {prob.name} splits={splits}")
    compare(prob, run_gpu(prob, num_splits=splits))


@pytest.mark.parametrize("splits", [None, 1, 4, -1])
def test_gqa_fp8_ragged_small(splits):
    prob = _gqa([5, 64, 65, 1500], hq=64, hkv=8, P=64, kv=W.E4M3)
    say(f"case {prob.name} splits={splits}")
    compare(prob, run_gpu(prob, num_splits=splits))


def test_gqa_bf16_full_size():
    prob = W.gqa_bf16_b32_kv4096()
    say(f"case {prob.name} (sampled)")
    dp = run_gpu(prob)
    compare(prob, dp, sample_pairs(prob, 96))


@pytest.mark.parametrize("splits", [None, 12])
def test_gqa_fp8_full_size(splits):
    prob = W.gqa_fp8_b16_ragged()
    say(f"case {prob.name} splits={splits} (sampled)")
    dp = run_gpu(prob, num_splits=splits)
    compare(prob, dp, sample_pairs(prob, 96))


def test_balanced_schedule_one_long_request():
    # 8 units of 250 pages spread over every workgroup: each unit has ~32 partial slots
    prob = _gqa([8000], hq=32, hkv=8, P=32)
    dp = run_gpu(prob)
    assert pkv.pkv_plan(dp.args).schedule == 1
    compare(prob, dp)


@pytest.mark.parametrize("kv", [W.BF16, W.E4M3])
def test_decode_one_128k_token_request(kv):
    # the longest context here: one request of 131,072 keys (537 MB of bf16 K/V in 8 KV heads),
    # spread by the balanced schedule over every workgroup: ~128 partial slots per row
    prob = _gqa([131072], hq=32 if kv == W.BF16 else 64, hkv=8, P=32 if kv == W.BF16 else 64, kv=kv, poison=False)
    say(f"case decode one 128k-token request kv={kv}")
    dp = run_gpu(prob)
    info = pkv.pkv_plan(dp.args)
    assert info.schedule == 1
    compare(prob, dp, sample_pairs(prob, 16), label=f"128k {kv} kernel={pkv.KERNEL_NAMES[info.kernel]}")


def test_balanced_schedule_fewer_pages_than_workgroups():
    prob = _gqa([1, 2, 40], hq=16, hkv=2, P=16, q_lens=[1, 1, 1])
    dp = run_gpu(prob, num_splits=-1)
    compare(prob, dp)


def test_balanced_schedule_speculative_rows_and_empty_request():
    prob = _gqa([3, 0, 300, 77], q_lens=[3, 3, 3, 3], hq=16, hkv=4)
    compare(prob, run_gpu(prob, num_splits=-1), expect_err=pkv.PKV_DEVERR_SEQ_LT_QLEN)


# ----------------------------------------------------------------- balanced schedule with the in-kernel reducer

def _fused_runs(prob, kernel=None, runs=3, expect_err=0, pairs=None):
    """Run the balanced schedule with merge counters `runs` times on one counter
    buffer: every run must match the oracle and leave the counters at zero."""
    dp = pkv.upload(prob, "cuda", num_splits=-1, kernel=kernel, merge_counters=True)
    plan = pkv.pkv_plan(dp.args)
    assert plan.schedule == 1 and plan.fused_merge == 1, (plan.schedule, plan.fused_merge)
    assert dp.tensors["counters"].numel() == prob.batch * prob.num_kv_heads
    for r in range(runs):
        dp.tensors["out"].fill_(float("nan"))
        dp.tensors["lse"].fill_(float("nan"))
        dp.run()
        torch.cuda.synchronize()
        compare(prob, dp, pairs=pairs, label=f"{kernel}/fused run {r}", expect_err=expect_err)
        assert int(dp.tensors["counters"].abs().sum().item()) == 0, "counters not reset"
    return dp


@pytest.mark.parametrize("kernel,kv", [("dma_gqa_fp8_n2", W.E4M3)])
def test_fused_merge_kernel_families(kernel, kv):
    P = 64 if kv == W.E4M3 else 32
    prob = _gqa([1, 31, 64, 65, 700, 1300], hq=64 if kv == W.E4M3 else 32, hkv=8, P=P, kv=kv)
    say(f"case {kernel} fused merge")
    _fused_runs(prob, kernel)


def test_fused_merge_one_long_request():
    prob = _gqa([8000], hq=32, hkv=8, P=32, kv=W.E4M3)
    say("case fused one long request")
    _fused_runs(prob, "dma_gqa_fp8_n2")


def test_fused_merge_fewer_pages_than_workgroups():
    prob = _gqa([1, 2, 40], hq=16, hkv=2, P=16, kv=W.E4M3)
    say("case fused fewer pages than workgroups")
    _fused_runs(prob, "dma_gqa_fp8_n2")


def test_fused_merge_speculative_rows_and_empty_request():
    prob = _gqa([3, 0, 300, 77], q_lens=[3, 3, 3, 3], hq=16, hkv=4, kv=W.E4M3, P=64)
    say("case fused speculative rows + empty request")
    _fused_runs(prob, "dma_gqa_fp8_n2", expect_err=pkv.PKV_DEVERR_SEQ_LT_QLEN)


def test_fused_merge_separate_value_tables():
    prob = _gqa([1, 31, 64, 65, 700, 1300], hq=64, hkv=8, P=64, kv=W.E4M3, separate_v_table=True, seed=5)
    say("case fused merge with separate V tables")
    _fused_runs(prob, "dma_gqa_fp8_n2")


def test_fp8_ragged_full_size_separate_value_tables():
    # the e4m3 benchmark workload's shape with its V pages behind a table of their own
    lens = W.ragged_log_uniform_lens(np.random.default_rng(0), 16, 512, 32768)
    prob = W.make_problem(name="fp8-gqa-b16-ragged-vtab", seed=0, batch=16, seq_lens=lens, q_lens=[1] * 16,
                          num_qo_heads=64,
                          num_kv_heads=8, head_dim_qk=128, head_dim_v=128, page_size=64, kv_dtype=W.E4M3,
                          q_dtype=W.BF16, o_dtype=W.BF16, separate_v_table=True)
    dp = run_gpu(prob)
    plan = pkv.pkv_plan(dp.args)
    say(f"case {prob.name}: kernel={pkv.KERNEL_NAMES[plan.kernel]} schedule={plan.schedule}")
    assert pkv.KERNEL_NAMES[plan.kernel] == "dma_gqa_fp8_n2" and plan.schedule == 1
    compare(prob, dp, sample_pairs(prob, 96))


def test_fused_merge_full_size_fp8():
    prob = W.gqa_fp8_b16_ragged()
    say(f"case {prob.name} fused merge (sampled)")
    _fused_runs(prob, None, runs=2, pairs=sample_pairs(prob, 96))


@pytest.mark.parametrize("q_len,kernel", [(1, None), (2, None), (1, "dma_mla_bf16"), (2, "dma_mla_bf16"),
                                          (1, "mla_bf16"), (1, "mla32_bf16"), (2, "mla32_bf16"),
                                          (3, "mla32_bf16")])
def test_mla_small(q_len, kernel):
    prob = W.make_problem(name=f"mla-small-q{q_len}", seed=3, batch=3, seq_lens=[2, 70, 300],
                          q_lens=[q_len] * 3, num_qo_heads=128, num_kv_heads=1, head_dim_qk=576,
                          head_dim_v=512, page_size=64, mla=True, scale=1 / 24.0, poison=True,
                          extra_page_frac=0.3, table_slack_pages=1)
    say(f"case {prob.name} kernel={kernel}")
    dp = pkv.upload(prob, "cuda", kernel=kernel)
    dp.run()
    torch.cuda.synchronize()
    # with three draft rows the 2-key request has a row that sees no key (flagged)
    compare(prob, dp, expect_err=pkv.PKV_DEVERR_SEQ_LT_QLEN if q_len > 2 else 0)


def test_mla_fp8_latent_small():
    prob = W.make_problem(name="mla-fp8-small", seed=11, batch=2, seq_lens=[65, 200], q_lens=[2, 2],
                          num_qo_heads=128, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, page_size=64,
                          mla=True, kv_dtype=W.E4M3, scale=1 / 24.0, poison=True, extra_page_frac=0.3)
    for kernel in ["dma_mla_fp8", "mla_fp8"]:
        dp = pkv.upload(prob, "cuda", kernel=kernel)
        dp.run()
        torch.cuda.synchronize()
        compare(prob, dp, label=kernel)


@pytest.mark.parametrize("q_len,kernel", [(1, "mla32_bf16"), (2, "mla32_bf16")])
def test_mla_full_size_mla32(q_len, kernel):
    prob = W.mla_b512_kv4096(q_len=q_len)
    say(f"case {prob.name} kernel={kernel}")
    dp = pkv.upload(prob, "cuda", kernel=kernel)
    dp.run()
    torch.cuda.synchronize()
    compare(prob, dp, pairs=sample_pairs(prob, 256), label=kernel)


@pytest.mark.parametrize("P,hq,q_len", [(32, 128, 1), (128, 128, 2), (256, 64, 1), (64, 16, 2), (32, 48, 1)])
def test_mla32_page_sizes_and_head_counts(P, hq, q_len):
    # pages of 32 .. 256 tokens (a 32-key block never crosses a page), head
    # counts that leave whole waves of a workgroup without a valid row, and
    # lengths around the block and page boundaries
    prob = W.make_problem(name=f"mla32-p{P}-h{hq}-q{q_len}", seed=16, batch=6,
                          seq_lens=[2, 31, 32, 33, 257, 700], q_lens=[q_len] * 6, num_qo_heads=hq,
                          num_kv_heads=1, head_dim_qk=576, head_dim_v=512, page_size=P, mla=True,
                          scale=1 / 24.0, poison=True, extra_page_frac=0.3, table_slack_pages=1)
    say(f"case {prob.name}")
    dp = pkv.upload(prob, "cuda", kernel="mla32_bf16")
    dp.run()
    torch.cuda.synchronize()
    compare(prob, dp, label=prob.name)


@pytest.mark.parametrize("kernel,splits", [("mla32_bf16", 3), ("mla32_bf16", 7), ("mla32_bf16", 2)])
def test_mla32_split_partitions(kernel, splits):
    prob = W.make_problem(name="mla32-split", seed=15, batch=3, seq_lens=[1000, 64, 2050], q_lens=[2] * 3,
                          num_qo_heads=128, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, page_size=64,
                          mla=True, scale=1 / 24.0, poison=True, extra_page_frac=0.3, table_slack_pages=1,
                          sinks=True)
    say(f"case mla32 split {kernel} {splits}")
    dp = pkv.upload(prob, "cuda", kernel=kernel, num_splits=splits)
    dp.run()
    torch.cuda.synchronize()
    compare(prob, dp, label=f"{kernel}/{splits}")


# every context option at once: ragged rows (one request whose rows exceed its
# keys, one with a single row), sinks, a separate V table, poisoned pages, NHD
@pytest.mark.parametrize("kernel,kv,splits,layout", [
    (None, W.BF16, None, W.HND), ("m32_ctx_w8t128", W.BF16, 3, W.NHD), ("dma_wide_fp8", W.E4M3, 2, W.HND),
    ("wide_bf16", W.BF16, None, W.NHD),
])
def test_context_with_every_option(kernel, kv, splits, layout):
    prob = W.make_problem(name="ctx-every", seed=21, batch=4, seq_lens=[70, 5, 333, 1], q_lens=[64, 7, 130, 1],
                          num_qo_heads=16, num_kv_heads=2, head_dim_qk=128, head_dim_v=128, page_size=16,
                          kv_dtype=kv, q_dtype=W.BF16, o_dtype=W.BF16, layout=layout, is_decode=False, poison=True,
                          extra_page_frac=0.3, table_slack_pages=1, sinks=True, separate_v_table=True)
    say(f"case every context option {kernel} {kv} splits={splits} {layout}")
    dp = pkv.upload(prob, "cuda", kernel=kernel, num_splits=splits)
    dp.run()
    torch.cuda.synchronize()
    compare(prob, dp, label=f"ctx every option {kernel}/{kv}/{splits}/{layout}", expect_err=pkv.PKV_DEVERR_SEQ_LT_QLEN)


@pytest.mark.parametrize("q_len", [1, 2])
def test_mla_full_size(q_len):
    prob = W.mla_b512_kv4096(q_len=q_len)
    say(f"case {prob.name} (sampled)")
    dp = run_gpu(prob)
    compare(prob, dp, sample_pairs(prob, 48))


def test_context_small_ragged():
    prob = W.make_problem(name="ctx-small", seed=4, batch=3, seq_lens=[50, 1, 300], q_lens=[20, 1, 70],
                          num_qo_heads=64, num_kv_heads=8, head_dim_qk=128, head_dim_v=128, page_size=32,
                          is_decode=False, poison=True, extra_page_frac=0.3, table_slack_pages=1)
    say(f"case {prob.name}")
    compare(prob, run_gpu(prob))


def test_context_full_size():
    prob = W.context_b4_q511_kv2047()
    say(f"case {prob.name} (sampled)")
    dp = run_gpu(prob)
    compare(prob, dp, sample_pairs(prob, 96))


# ----------------------------------------------------------------- reducer, codec, invariants

def test_lse_merge_entry_point_matches_oracle_merge():
    prob = W.make_problem(name="merge", seed=5, batch=3, seq_lens=[37, 100, 5], q_lens=[1, 1, 1],
                          num_qo_heads=4, num_kv_heads=1, head_dim_qk=64, head_dim_v=64, page_size=16,
                          q_dtype=W.F32, kv_dtype=W.F32, o_dtype=W.F32)
    S = 5  # includes empty partitions for the short requests
    o_part, l_part = oracle.attention_split(prob, S)
    ref_o, ref_l = oracle.merge(o_part, l_part)
    n = o_part.shape[1]
    o_dev = torch.from_numpy(o_part.astype(np.float32)).cuda()
    l_dev = torch.from_numpy(l_part.astype(np.float32)).cuda()
    out = torch.full((prob.total_q, prob.num_qo_heads, 64), float("nan"), device="cuda")
    lse = torch.full((n,), float("nan"), device="cuda")
    pkv.pkv_lse_merge(S, n, prob.num_qo_heads, 64, o_dev.data_ptr(), l_dev.data_ptr(), out.data_ptr(),
                      pkv.PKV_DTYPE_F32, prob.num_qo_heads * 64, 64, lse.data_ptr(),
                      torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    np.testing.assert_allclose(out.cpu().numpy().reshape(n, 64), ref_o, atol=1e-5, rtol=1e-5)
    np.testing.assert_allclose(lse.cpu().numpy(), ref_l, atol=1e-5, rtol=1e-5)


def test_fp8_dequant_all_256_codes_exact():
    # one key per request, v_scale = 1: the output row is the decoded value row itself
    prob = _gqa([1, 1], hq=8, hkv=1, P=64, kv=W.E4M3, poison=False)
    codes = np.arange(256, dtype=np.uint8).reshape(2, 128)
    for b in range(2):
        page = prob.block_tables[b, 0]
        prob.v_pool[page, 0, 0, :] = codes[b]
    prob = dataclasses.replace(prob, v_scale=1.0)
    dp = run_gpu(prob)
    got = dp.out.float().cpu().numpy()  # [2, 8, 128]
    table = oracle.e4m3_table()
    for b in range(2):
        exp = table[codes[b].astype(int)]
        for h in range(8):
            nan = np.isnan(exp)
            assert np.array_equal(np.isnan(got[b, h]), nan)
            assert np.array_equal(got[b, h][~nan], exp[~nan])


def test_page_permutation_invariance_bitwise():
    prob = _gqa([300, 77], poison=False)
    dp1 = run_gpu(prob)
    rng = np.random.default_rng(7)
    relabel = rng.permutation(prob.num_pages)
    k2 = np.empty_like(prob.k_pool)
    v2 = np.empty_like(prob.v_pool)
    k2[relabel] = prob.k_pool
    v2[relabel] = prob.v_pool
    p2 = dataclasses.replace(prob, k_pool=k2, v_pool=v2, block_tables=relabel[prob.block_tables].astype(np.int32))
    dp2 = run_gpu(p2)
    assert torch.equal(dp1.out, dp2.out)


def test_repeated_calls_are_bitwise_deterministic():
    prob = _gqa([513, 1000], poison=True)
    dp = pkv.upload(prob, "cuda")
    dp.run()
    first = dp.out.clone()
    for _ in range(3):
        dp.run()
    torch.cuda.synchronize()
    assert torch.equal(first, dp.out)


@pytest.mark.parametrize("case", ["gqa_bf16", "fp8_balanced_merge", "fp8_fused_merge", "context"])
def test_graph_replay_matches_eager(case):
    # the calls enqueue kernels only (no allocation, no memset, no host sync), so
    # they can be captured; every replay, with eager work and synchronizations in
    # between, must reproduce the eager result bitwise
    if case == "gqa_bf16":
        prob, kw = _gqa([513, 1000], poison=True), {}
    elif case == "context":
        prob = W.make_problem(name="ctx-graph", seed=4, batch=3, seq_lens=[50, 1, 300], q_lens=[20, 1, 70],
                              num_qo_heads=64, num_kv_heads=8, head_dim_qk=128, head_dim_v=128, page_size=32,
                              is_decode=False, poison=True, extra_page_frac=0.3, table_slack_pages=1)
        kw = {}
    else:
        prob = _gqa([5, 64, 65, 1500], hq=64, hkv=8, P=64, kv=W.E4M3)
        kw = {"num_splits": -1, "merge_counters": case == "fp8_fused_merge"}
    say(f"case graph {case}")
    dp = pkv.upload(prob, "cuda", **kw)
    dp.run()
    torch.cuda.synchronize()
    eager_out, eager_lse = dp.out.clone(), dp.lse.clone()
    compare(prob, dp, label=f"graph {case} eager")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dp.run()  # warm the side stream once outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        dp.run()
    for r in range(3):
        dp.tensors["out"].fill_(float("nan"))
        dp.tensors["lse"].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dp.out, eager_out), f"replay {r} differs from the eager output"
        assert torch.equal(dp.lse, eager_lse), f"replay {r} lse differs from the eager lse"
        if "counters" in dp.tensors:
            assert int(dp.tensors["counters"].abs().sum().item()) == 0
        dp.run()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(dp.out, eager_out)


# ----------------------------------------------------------------- attention sinks, separate V tables

@pytest.mark.parametrize("kernel,kv,splits,counters", [
    (None, W.BF16, None, False), ("gqa_bf16", W.BF16, 3, False), ("gqa_fp8", W.E4M3, 1, False),
    ("dma_gqa_fp8_n2", W.E4M3, -1, False), ("dma_gqa_fp8_n2", W.E4M3, -1, True), ("generic", W.BF16, None, False),
])
def test_sinks_decode(kernel, kv, splits, counters):
    P = 64 if kv == W.E4M3 else 32
    prob = _gqa([1, 31, 64, 65, 700, 1300], hq=64 if kv == W.E4M3 else 32, hkv=8, P=P, kv=kv, sinks=True)
    say(f"case sinks decode {kernel} splits={splits} counters={counters}")
    dp = pkv.upload(prob, "cuda", num_splits=splits, kernel=kernel, merge_counters=counters)
    dp.run()
    torch.cuda.synchronize()
    compare(prob, dp, label=f"sinks {kernel}/{splits}/{counters}")


# every contract option of a decode call at once: speculative rows (one
# request with fewer keys than rows), sinks, a separate V table, NaN-poisoned
# page tails and spare pages, on the balanced schedule with either reducer
@pytest.mark.parametrize("kernel,kv,counters", [
    ("dma_gqa_fp8_n2", W.E4M3, False), ("dma_gqa_fp8_n2", W.E4M3, True), ("gqa_bf16", W.BF16, False),
    ("gqa_fp8", W.E4M3, False),
])
def test_decode_with_every_option_on_the_balanced_schedule(kernel, kv, counters):
    prob = _gqa([1, 300, 77, 1300, 64], q_lens=[2] * 5, hq=16, hkv=2, P=64 if kv == W.E4M3 else 32, kv=kv,
                sinks=True, separate_v_table=True, seed=9)
    say(f"case every option {kernel} counters={counters}")
    dp = pkv.upload(prob, "cuda", num_splits=-1, kernel=kernel, merge_counters=counters)
    assert pkv.pkv_plan(dp.args).schedule == 1
    for r in range(2 if counters else 1):
        dp.tensors["out"].fill_(float("nan"))
        dp.run()
        torch.cuda.synchronize()
        compare(prob, dp, label=f"every option {kernel}/{counters} run {r}", expect_err=pkv.PKV_DEVERR_SEQ_LT_QLEN)
        if counters:
            assert int(dp.tensors["counters"].abs().sum().item()) == 0


def test_sinks_speculative_rows_with_an_empty_row():
    # request 0 has 3 rows over 2 keys: its first row sees no key and reports lse = sink
    prob = _gqa([2, 300, 77], q_lens=[3, 3, 3], hq=16, hkv=4, sinks=True)
    compare(prob, run_gpu(prob, num_splits=-1), expect_err=pkv.PKV_DEVERR_SEQ_LT_QLEN)


@pytest.mark.parametrize("kernel,splits", [(None, None), ("m32_ctx_w8t128", 3), ("dma_wide_bf16", None)])
def test_sinks_context(kernel, splits):
    prob = W.make_problem(name="ctx-sinks", seed=9, batch=3, seq_lens=[70, 5, 333], q_lens=[64, 5, 130],
                          num_qo_heads=16, num_kv_heads=2, head_dim_qk=128, head_dim_v=128, page_size=16,
                          is_decode=False, poison=True, extra_page_frac=0.3, table_slack_pages=1, sinks=True)
    dp = pkv.upload(prob, "cuda", kernel=kernel, num_splits=splits)
    dp.run()
    torch.cuda.synchronize()
    compare(prob, dp, label=f"ctx sinks {kernel}/{splits}")


@pytest.mark.parametrize("q_len", [1, 2])
def test_sinks_mla(q_len):
    prob = W.make_problem(name=f"mla-sinks-q{q_len}", seed=3, batch=3, seq_lens=[2, 70, 300],
                          q_lens=[q_len] * 3, num_qo_heads=128, num_kv_heads=1, head_dim_qk=576,
                          head_dim_v=512, page_size=64, mla=True, scale=1 / 24.0, poison=True,
                          extra_page_frac=0.3, table_slack_pages=1, sinks=True)
    compare(prob, run_gpu(prob))


# every MLA option at once: two speculative rows with a request shorter than
# them, sinks, poisoned pages, Split-KV partitions, on each MLA family
@pytest.mark.parametrize("kernel,kv,splits", [
    ("mla32_bf16", W.BF16, 3), ("mla32_bf16", W.BF16, None), ("dma_mla_bf16", W.BF16, 2), ("dma_mla_fp8", W.E4M3, 3),
])
def test_mla_with_every_option(kernel, kv, splits):
    prob = W.make_problem(name="mla-every", seed=23, batch=4, seq_lens=[1, 70, 300, 129], q_lens=[2] * 4,
                          num_qo_heads=128, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, page_size=64,
                          kv_dtype=kv, mla=True, scale=1 / 24.0, poison=True, extra_page_frac=0.3,
                          table_slack_pages=1, sinks=True)
    say(f"case every MLA option {kernel} {kv} splits={splits}")
    dp = pkv.upload(prob, "cuda", kernel=kernel, num_splits=splits)
    dp.run()
    torch.cuda.synchronize()
    compare(prob, dp, label=f"mla every option {kernel}/{kv}/{splits}", expect_err=pkv.PKV_DEVERR_SEQ_LT_QLEN)


# separate V page tables: the planner's choice per shape (the same as with a
# shared table: register-staged tiles for bf16 decode, the direct-to-LDS ring
# on the balanced schedule for e4m3 decode, the 32x32 kernel for bf16
# context, the ring's wide tiles for e4m3 context), forced split partitions
# and the balanced schedule on request, and the other families
@pytest.mark.parametrize("decode,kv,kernel,splits,expect", [
    (True, W.BF16, None, None, "gqa_bf16"),
    (True, W.E4M3, None, None, "dma_gqa_fp8_n2"),
    (True, W.BF16, None, 3, "gqa_bf16"),
    (True, W.BF16, None, -1, "gqa_bf16"),
    (True, W.BF16, "generic", None, "generic"),
    (True, W.E4M3, "gqa_fp8", 2, "gqa_fp8"),
    (True, W.E4M3, "gqa_fp8", -1, "gqa_fp8"),
    (True, W.E4M3, "dma_gqa_fp8_n2", 3, "dma_gqa_fp8_n2"),
    (False, W.BF16, None, None, "m32_ctx_w8t128"),
    (False, W.BF16, "m32_ctx_w8t128", 3, "m32_ctx_w8t128"),
    (False, W.E4M3, None, None, "dma_wide_fp8"),
    (False, W.E4M3, "wide_fp8", None, "wide_fp8"),
    (False, W.BF16, "wide_bf16", None, "wide_bf16"),
    (False, W.BF16, "dma_wide_bf16", 2, "dma_wide_bf16"),
    (False, W.BF16, "generic", None, "generic"),
])
def test_separate_value_tables(decode, kv, kernel, splits, expect):
    if decode:
        prob = _gqa([1, 31, 64, 65, 700], kv=kv, separate_v_table=True, sinks=True)
    else:
        prob = W.make_problem(name="ctx-vtab", seed=12, batch=2, seq_lens=[300, 40], q_lens=[30, 40],
                              num_qo_heads=16, num_kv_heads=2, head_dim_qk=128, head_dim_v=128, page_size=16,
                              kv_dtype=kv, q_dtype=W.BF16, o_dtype=W.BF16, is_decode=False, poison=True,
                              extra_page_frac=0.3, table_slack_pages=1, separate_v_table=True)
    dp = pkv.upload(prob, "cuda", kernel=kernel, num_splits=splits)
    info = pkv.pkv_plan(dp.args, dp.is_context)
    assert pkv.KERNEL_NAMES[info.kernel] == expect
    say(f"case separate V tables decode={decode} kv={kv} kernel={expect} splits={info.num_splits}")
    dp.run()
    torch.cuda.synchronize()
    compare(prob, dp, label=f"separate V tables decode={decode} {kv} {expect}")


@pytest.mark.parametrize("separate", [False, True])
def test_context_q257_kv1024_page1024_profile(separate):
    # the API page's second BF16 context profile: four requests of 257 rows over
    # 1024 keys, 1024-token pages, separate K/V page tables (and the shared form)
    prob = W.make_problem(name=f"ctx-q257-kv1024-p1024-sep{int(separate)}", seed=13, batch=4,
                          seq_lens=[1024] * 4, q_lens=[257] * 4, num_qo_heads=64, num_kv_heads=8,
                          head_dim_qk=128, head_dim_v=128, page_size=1024, is_decode=False, poison=True,
                          extra_page_frac=0.25, table_slack_pages=1, separate_v_table=separate)
    say(f"case {prob.name}")
    dp = run_gpu(prob)
    assert pkv.KERNEL_NAMES[pkv.pkv_plan(dp.args, dp.is_context).kernel] == "m32_ctx_w8t128"
    compare(prob, dp, sample_pairs(prob, 192))
    # the benchmark's configuration of this profile (no poison, the planner's plan)
    bprob = W.context_b4_q257_kv1024_p1024(separate=separate)
    bdp = run_gpu(bprob)
    compare(bprob, bdp, sample_pairs(bprob, 192), label=f"{bprob.name} (bench configuration)")


@pytest.mark.parametrize("P", [1, 2, 1024])
def test_extreme_page_sizes_decode(P):
    prob = _gqa([1, 3, 1000, 2049], P=P)
    say(f"case decode P={P}")
    dp = run_gpu(prob)
    say(f"  kernel {pkv.KERNEL_NAMES[pkv.pkv_plan(dp.args).kernel]}")
    compare(prob, dp)


def test_nhd_layout_matches_oracle():
    prob = _gqa([40, 129], layout=W.NHD)
    say(f"case {prob.name} NHD")
    compare(prob, run_gpu(prob))


def test_device_scalar_fp8_scales():
    prob = _gqa([100, 260], hq=64, hkv=8, P=64, kv=W.E4M3)
    compare(prob, run_gpu(prob, device_scales=True))


@pytest.mark.parametrize("kv,P,D,qd", [(W.F32, 24, 64, W.F32), (W.BF16, 16, 96, W.BF16), (W.E4M3, 8, 64, W.BF16)])
def test_generic_kernel_other_shapes(kv, P, D, qd):
    prob = W.make_problem(name=f"generic-{kv}-P{P}-D{D}", seed=6, batch=3, seq_lens=[1, 47, 130],
                          q_lens=[2, 2, 2], num_qo_heads=6, num_kv_heads=2, head_dim_qk=D, head_dim_v=D,
                          page_size=P, q_dtype=qd, kv_dtype=kv, o_dtype=W.F32 if qd == W.F32 else W.BF16,
                          poison=True, extra_page_frac=0.3)
    say(f"case {prob.name}")
    # the first request holds one key for two query rows: its first row sees nothing (flagged, zeros)
    compare(prob, run_gpu(prob), expect_err=pkv.PKV_DEVERR_SEQ_LT_QLEN)


def test_speculative_rows_on_gqa_kernel():
    prob = _gqa([3, 90, 400], q_lens=[3, 3, 3], hq=32, hkv=8)  # 3 rows x 4 heads = 12 packed rows
    compare(prob, run_gpu(prob))
    short = _gqa([2, 90, 400], q_lens=[3, 3, 3], hq=32, hkv=8)  # 2 keys for 3 rows: flagged
    compare(short, run_gpu(short), expect_err=pkv.PKV_DEVERR_SEQ_LT_QLEN)


# ----------------------------------------------------------------- device-side validation

def test_error_word_flags_and_clamping():
    prob = _gqa([60, 100], poison=False)
    dp = pkv.upload(prob, "cuda")
    # seq_lens beyond the table capacity: flagged, clamped to capacity
    cap = prob.max_pages * prob.page_size
    dp.tensors["seq_lens"][1] = cap + 50
    dp.run()
    torch.cuda.synchronize()
    assert int(dp.err.item()) & pkv.PKV_DEVERR_SEQ_GT_TABLE
    assert torch.isfinite(dp.out.float()).all()
    # a page index outside the pool: flagged, clamped
    dp.tensors["err"].zero_()
    dp.tensors["seq_lens"][1] = 100
    dp.tensors["table"][0, 0] = prob.num_pages + 1000
    dp.run()
    torch.cuda.synchronize()
    assert int(dp.err.item()) & pkv.PKV_DEVERR_PAGE_RANGE
    # fewer keys than query rows
    dp.tensors["err"].zero_()
    dp.tensors["table"][0, 0] = int(prob.block_tables[0, 0])
    dp.tensors["seq_lens"][0] = 0
    dp.run()
    torch.cuda.synchronize()
    assert int(dp.err.item()) & pkv.PKV_DEVERR_SEQ_LT_QLEN
    assert torch.all(dp.out[0].float() == 0)
    assert torch.isneginf(dp.lse[0]).all()


def test_malformed_q_indptr_flagged_without_writes():
    prob = W.make_problem(name="ctx-bad", seed=8, batch=2, seq_lens=[40, 50], q_lens=[10, 12],
                          num_qo_heads=16, num_kv_heads=2, head_dim_qk=128, head_dim_v=128, page_size=32,
                          is_decode=False)
    dp = pkv.upload(prob, "cuda")
    dp.tensors["q_indptr"][1] = 50  # > total_q (22) and rows > max_q_len
    dp.run()
    torch.cuda.synchronize()
    assert int(dp.err.item()) & pkv.PKV_DEVERR_QINDPTR


# ----------------------------------------------------------------- every kernel family on the same inputs

@pytest.mark.parametrize("kernel,kv,splits", [
    ("gqa_bf16", W.BF16, None), ("gqa_bf16", W.BF16, 1), ("gqa_bf16", W.BF16, 3), ("gqa_bf16", W.BF16, -1),
    ("gqa_fp8", W.E4M3, None), ("gqa_fp8", W.E4M3, 1), ("gqa_fp8", W.E4M3, 5), ("gqa_fp8", W.E4M3, -1),
    ("dma_gqa_fp8_n2", W.E4M3, None), ("dma_gqa_fp8_n2", W.E4M3, 1), ("dma_gqa_fp8_n2", W.E4M3, 5),
    ("dma_gqa_fp8_n2", W.E4M3, -1),
])
def test_gqa_kernel_families_match_oracle(kernel, kv, splits):
    P = 64 if kv == W.E4M3 else 32
    prob = _gqa([1, 31, 64, 65, 700, 1300], hq=64 if kv == W.E4M3 else 32, hkv=8, P=P, kv=kv)
    say(f"case {kernel} splits={splits}")
    dp = pkv.upload(prob, "cuda", num_splits=splits, kernel=kernel)
    dp.run()
    torch.cuda.synchronize()
    compare(prob, dp, label=f"{kernel}/{splits}")


@pytest.mark.parametrize("kernel,splits", [("dma_wide_bf16", None), ("wide_bf16", None), ("wide_bf16", 2),
                                           ("m32_ctx_w8t128", None), ("m32_ctx_w8t128", 2),
                                           ("m32_ctx_w8t128", 3)])
def test_context_kernel_families_match_oracle(kernel, splits):
    prob = W.make_problem(name="ctx-fam", seed=9, batch=3, seq_lens=[70, 5, 333], q_lens=[64, 5, 130],
                          num_qo_heads=16, num_kv_heads=2, head_dim_qk=128, head_dim_v=128, page_size=16,
                          is_decode=False, poison=True, extra_page_frac=0.3, table_slack_pages=1)
    say(f"case {kernel} splits={splits}")
    dp = pkv.upload(prob, "cuda", kernel=kernel, num_splits=splits)
    dp.run()
    torch.cuda.synchronize()
    compare(prob, dp, label=f"{kernel}/{splits}")


@pytest.mark.parametrize("kernel", ["m32_ctx_w8t128", "dma_wide_bf16"])
def test_context_full_size_m32(kernel):
    prob = W.context_b4_q511_kv2047()
    say(f"case {prob.name} kernel={kernel}")
    dp = pkv.upload(prob, "cuda", kernel=kernel)
    dp.run()
    torch.cuda.synchronize()
    compare(prob, dp, pairs=sample_pairs(prob, 512), label=kernel)


def test_context_fp8_kv_families_match_oracle():
    prob = W.make_problem(name="ctx-fp8", seed=10, batch=2, seq_lens=[90, 300], q_lens=[40, 100],
                          num_qo_heads=16, num_kv_heads=2, head_dim_qk=128, head_dim_v=128, page_size=32,
                          kv_dtype=W.E4M3, is_decode=False, poison=True, extra_page_frac=0.3)
    for kernel in ["dma_wide_fp8", "wide_fp8"]:
        dp = pkv.upload(prob, "cuda", kernel=kernel)
        dp.run()
        torch.cuda.synchronize()
        compare(prob, dp, label=kernel)


# ----------------------------------------------------------------- lengths above the host bound

@pytest.mark.parametrize("kernel,splits,kv,ctx", [
    ("gqa_bf16", 1, W.BF16, False), ("gqa_bf16", 3, W.BF16, False), ("dma_gqa_fp8_n2", 4, W.E4M3, False),
    ("generic", 2, W.BF16, False), ("gqa_bf16", -1, W.BF16, False), ("dma_mla_bf16", None, W.BF16, False),
    ("mla32_bf16", None, W.BF16, False),
    ("m32_ctx_w8t128", None, W.BF16, True), ("m32_ctx_w8t128", 2, W.BF16, True),
])
def test_seq_len_above_max_kv_len_is_flagged_and_cut_to_the_plan(kernel, splits, kv, ctx):
    # the plan is sized from max_kv_len = 700 while the device says 1000: the
    # request is cut to the keys the plan's partitions cover (the balanced
    # schedule covers the whole table) and PKV_DEVERR_SEQ_GT_MAXLEN is set
    mla = kernel in ("dma_mla_bf16", "mla32_bf16")
    if ctx:
        prob = W.make_problem(name="ctx-gt-maxlen", seed=14, batch=2, seq_lens=[300, 1000], q_lens=[40, 90],
                              num_qo_heads=16, num_kv_heads=2, head_dim_qk=128, head_dim_v=128, page_size=32,
                              is_decode=False, poison=True, extra_page_frac=0.3, table_slack_pages=12)
    elif mla:
        prob = W.make_problem(name="mla-gt-maxlen", seed=14, batch=2, seq_lens=[300, 1000], q_lens=[1, 1],
                              num_qo_heads=128, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, page_size=64,
                              mla=True, scale=1 / 24.0, poison=True, extra_page_frac=0.3, table_slack_pages=6)
    else:
        P = 64 if kv == W.E4M3 else 32
        prob = _gqa([300, 1000], hq=64 if kv == W.E4M3 else 32, hkv=8, P=P, kv=kv)
        prob = dataclasses.replace(prob, block_tables=np.pad(prob.block_tables, ((0, 0), (0, 12)), mode="edge"))
    short = dataclasses.replace(prob, seq_lens=np.array([300, 700], dtype=np.int32))
    dp = pkv.upload(short, "cuda", num_splits=splits, kernel=kernel)
    info = pkv.pkv_plan(dp.args, dp.is_context)
    cap = prob.max_pages * prob.page_size
    span = cap if info.schedule == 1 else min(cap, info.num_splits * info.pages_per_split * prob.page_size)
    assert 700 <= span < 1000 or info.schedule == 1
    dp.tensors["seq_lens"][1] = 1000
    say(f"case seq_len 1000 > max_kv_len 700: {kernel} splits={info.num_splits} schedule={info.schedule} "
        f"span={span}")
    dp.run()
    torch.cuda.synchronize()
    cut = dataclasses.replace(prob, seq_lens=np.array([300, min(1000, span)], dtype=np.int32))
    compare(cut, dp, label=f"gt-maxlen {kernel}/{splits}", expect_err=pkv.PKV_DEVERR_SEQ_GT_MAXLEN)
