"""GPU parity of pkv_decode_noalloc (the decode entry point for callers that
cannot allocate): through the C ABI, two calls in a row on the library's
static scratch, the second with a smaller input, each checked bitwise against
pkv_decode with a caller workspace and against the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from paged_kv_attention_15_amd import pkv, workloads as W
from tests._gpu import compare, sample_pairs, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pkv.load_library()
    torch.cuda.init()


def _noalloc_against_decode(prob, pairs=None, **kw):
    dp = pkv.upload(prob, "cuda", **kw)
    info = pkv.pkv_plan(dp.args)
    assert 0 < info.workspace_bytes <= pkv.PKV_NOALLOC_SCRATCH_BYTES  # the call uses scratch
    stream = torch.cuda.current_stream().cuda_stream
    dp.run()
    torch.cuda.synchronize()
    ref_out, ref_lse, ref_err = dp.out.clone(), dp.lse.clone(), dp.err.clone()
    dp.tensors["out"].fill_(float("nan"))
    dp.tensors["lse"].fill_(float("nan"))
    dp.tensors["err"].zero_()
    torch.cuda.synchronize()
    pkv.pkv_decode_noalloc(dp.args, stream)
    torch.cuda.synchronize()
    say(f"case noalloc {prob.name}: kernel={pkv.KERNEL_NAMES[info.kernel]} schedule={info.schedule} "
        f"splits={info.num_splits} scratch={info.workspace_bytes}")
    assert torch.equal(dp.out, ref_out), "noalloc output differs from pkv_decode"
    assert torch.equal(dp.lse, ref_lse), "noalloc lse differs from pkv_decode"
    assert torch.equal(dp.err, ref_err)
    compare(prob, dp, pairs=pairs, label=f"noalloc {prob.name}")


def test_noalloc_two_calls_second_smaller():
    # 1: the ragged e4m3 workload on the balanced schedule (about 4.8 MB of partials)
    big = W.gqa_fp8_b16_ragged()
    _noalloc_against_decode(big, pairs=sample_pairs(big, 64))
    # 2: a smaller bf16 problem on three Split-KV partitions, reusing the same scratch
    small = W.make_problem(name="noalloc-small", seed=31, batch=3, seq_lens=[1, 700, 129], q_lens=[1, 1, 1],
                           num_qo_heads=32, num_kv_heads=8, head_dim_qk=128, head_dim_v=128, page_size=32,
                           poison=True, extra_page_frac=0.25, table_slack_pages=2)
    _noalloc_against_decode(small, num_splits=3)
