"""The binding's tensor-level append entry on the GPU: from fresh copies of
the same initial caches it must write bit for bit what the field-by-field
path writes (which the append parity tests check against the oracle)."""
import pytest

from paged_kv_attention_15_amd import pkv

from .test_append_tensor_args_cpu import APPEND_PROBLEMS, tensor_args

torch = pytest.importorskip("torch")


@pytest.mark.gpu
@pytest.mark.parametrize("label,make", APPEND_PROBLEMS, ids=[p[0] for p in APPEND_PROBLEMS])
def test_append_tensor_entry_matches_the_harness_path(label, make):
    prob = make()
    print(f"case append tensor-args {label}", flush=True)
    ref = pkv.upload_append(prob, "cuda")
    got = pkv.upload_append(prob, "cuda")  # its own copies of the initial caches and outputs
    stream = int(torch.cuda.current_stream().cuda_stream)
    pkv.pkv_append(ref.args, stream)
    pkv.pkv_append(tensor_args(prob, got.tensors), stream)
    torch.cuda.synchronize()
    assert int(ref.tensors["err"].item()) == 0 and int(got.tensors["err"].item()) == 0
    for name in ("k_cache", "v_cache", "out_q", "q_scale"):
        if name in ref.tensors:
            a, b = ref.tensors[name], got.tensors[name]
            if a.is_floating_point():
                a, b = a.view(torch.int32), b.view(torch.int32)  # NaN markers compare by bits
            assert torch.equal(a, b), (label, name)
