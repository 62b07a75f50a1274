"""The allocation-free attention entry point (static per-device split
records) against mk_t_attention, which allocates its records per call: the
same kernels on the same inputs, so the outputs are bitwise equal.  Two calls
in a row, the second smaller (fewer splits and heads), so the second reads a
scratch array that still holds the first call's records."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def abi():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_persistent_megakernel_02_amd import abi as a
    return a


def case(seed, nq, nkv, hd, S, f32):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(nq, hd, generator=g)
    k = torch.randn(nkv, S, hd, generator=g)
    v = torch.randn(nkv, S, hd, generator=g)
    if not f32:
        k, v = k.to(torch.bfloat16), v.to(torch.bfloat16)
    return q.cuda(), k.cuda(), v.cuda()


@pytest.mark.parametrize("f32", [True, False], ids=["kv_f32", "kv_bf16"])
def test_noalloc_matches_allocating_entry_point_on_two_calls(abi, f32):
    calls = [(32, 8, 128, 600, 551, 16), (8, 2, 64, 40, 37, 8)]  # nq, nkv, hd, S, T, split
    for i, (nq, nkv, hd, S, T, split) in enumerate(calls):
        print(f"no-alloc attention call {i}: nq {nq} nkv {nkv} hd {hd} T {T} split {split} f32 {f32}", flush=True)
        q, k, v = case(100 + i, nq, nkv, hd, S, f32)
        ref = torch.empty(nq, hd, dtype=torch.float32, device="cuda")
        out = torch.full((nq, hd), float("nan"), dtype=torch.float32, device="cuda")
        abi.mk_t_attention(q, k, v, T, split, ref)
        abi.mk_t_attention_noalloc(q, k, v, T, split, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"call {i}: max diff {(out - ref).abs().max().item()}"


def test_noalloc_rejects_records_beyond_the_static_array(abi):
    # 8 groups x 4 heads x 130 floats per split: 1100 splits need 4.6M floats > 2^20
    q, k, v = case(7, 32, 8, 128, 1100, True)
    out = torch.empty(32, 128, dtype=torch.float32, device="cuda")
    with pytest.raises(abi.MkError) as e:
        abi.mk_t_attention_noalloc(q, k, v, 1100, 1, out)
    assert e.value.status == abi.MK_ERR_CAPACITY
