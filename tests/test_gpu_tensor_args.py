"""The binding's tensor-level entry (args_from_tensors + run_tensors) on the
GPU: for the same device tensors it must produce bit for bit the output of
the field-by-field path the parity tests check against the oracle."""
import pytest

from paged_kv_attention_15_amd import pkv

from .test_tensor_args_cpu import PROBLEMS

torch = pytest.importorskip("torch")


@pytest.mark.gpu
@pytest.mark.parametrize("label,make", PROBLEMS, ids=[p[0] for p in PROBLEMS])
def test_tensor_entry_matches_the_harness_path(label, make):
    prob = make()
    print(f"case tensor-args {label}", flush=True)
    dp = pkv.upload(prob, "cuda", with_lse=True, with_err=True)
    dp.run()
    torch.cuda.synchronize()
    ref_o, ref_l = dp.out.clone(), dp.lse.clone()
    assert int(dp.err.item()) == 0
    t = dp.tensors
    out = torch.full_like(ref_o, float("nan"))
    lse = torch.full_like(ref_l, float("nan"))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    args = pkv.args_from_tensors(
        t["q"], t["k"], t.get("v"), t["table"], t["seq_lens"], out, scale=prob.scale, max_kv_len=prob.max_kv_len,
        layout=prob.layout, q_indptr=None if prob.is_decode else t["q_indptr"],
        max_q_len=None if prob.is_decode else prob.q_len, causal=prob.causal, k_scale=prob.k_scale,
        v_scale=prob.v_scale, lse=lse, err=err, num_splits=prob.num_splits)
    ws = pkv.run_tensors(args)
    ws = pkv.run_tensors(args, workspace=ws)  # a kept workspace serves the next call
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                       ref_o.view(torch.int16) if ref_o.dtype == torch.bfloat16 else ref_o)
    assert torch.equal(lse, ref_l)


@pytest.mark.gpu
def test_tensor_entry_refuses_host_tensors_beside_device_ones():
    # a host seq_lens beside device tensors would be read by a kernel through a
    # host address: refused on the host, before any launch
    prob = PROBLEMS[0][1]()
    dp = pkv.upload(prob, "cuda", with_lse=False, with_err=False)
    t = dp.tensors
    out = torch.empty_like(dp.out)
    with pytest.raises(ValueError, match="seq_lens"):
        pkv.args_from_tensors(t["q"], t["k"], t.get("v"), t["table"], t["seq_lens"].cpu(), out, scale=prob.scale,
                              max_kv_len=prob.max_kv_len, layout=prob.layout)
    with pytest.raises(ValueError, match="block_tables"):
        pkv.args_from_tensors(t["q"], t["k"], t.get("v"), t["table"].long(), t["seq_lens"], out, scale=prob.scale,
                              max_kv_len=prob.max_kv_len, layout=prob.layout)
