"""Single task bodies on the GPU against the oracle's operators.

The GEMV pin: with weights k * 2^-4 (|k| <= 8, exact in bf16) and small
integer activations every fp32 partial sum is exact, so any summation order
gives the exact result; the GPU must match the fp64 product bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import decoder as D
from synth import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def abi():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_persistent_megakernel_02_amd import abi as a
    return a


def bits_of(f32):
    return gen.f32_to_bf16_bits(np.asarray(f32, dtype=np.float32))


def dev_bits(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


@pytest.mark.parametrize("N,K", [(4096, 4096), (6, 8), (13, 520), (1025, 14336), (7, 688), (3, 32768)])
def test_gemv_exact_on_representable_data(abi, N, K):
    rng = np.random.default_rng(N * 7 + K)
    W = rng.integers(-8, 9, size=(N, K)).astype(np.float32) / 16.0
    x = rng.integers(-4, 5, size=K).astype(np.float32)
    y = torch.empty(N, dtype=torch.float32, device="cuda")
    abi.mk_t_gemv(dev_bits(bits_of(W)).view(N, K), torch.from_numpy(x).cuda(), y)
    torch.cuda.synchronize()
    ref = W.astype(np.float64) @ x.astype(np.float64)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("N,K", [(6144, 4096), (4096, 14336), (255, 2048)])
def test_gemv_random_within_fp32_accumulation_error(abi, N, K):
    Wb = gen.bf16_normal(0, 99, 0, N * K).reshape(N, K)
    x = np.random.default_rng(K).normal(size=K).astype(np.float32)
    y = torch.empty(N, dtype=torch.float32, device="cuda")
    abi.mk_t_gemv(dev_bits(Wb).view(N, K), torch.from_numpy(x).cuda(), y)
    torch.cuda.synchronize()
    Wd = D.widen_bf16(Wb)
    ref = Wd @ x.astype(np.float64)
    # each lane sums K/64 fused products in order, then 6 tree levels and the
    # 4-row combine: |err| <= (K/64 + 8) * 2^-24 * sum|w x| (a strict bound)
    bound = (K / 64 + 8) * 2.0 ** -24 * (np.abs(Wd) @ np.abs(x.astype(np.float64))) * 1.01
    assert np.all(np.abs(y.cpu().numpy() - ref) <= bound)


@pytest.mark.parametrize("n", [8, 256, 4096, 8200])
def test_rmsnorm(abi, n):
    rng = np.random.default_rng(n)
    x = (rng.normal(size=n) * 3).astype(np.float32)
    g = gen.bf16_normal(1, 2, 0, n, 0.1, 1.0)
    y = torch.empty(n, dtype=torch.float32, device="cuda")
    abi.mk_t_rmsnorm(torch.from_numpy(x).cuda(), dev_bits(g), 1e-5, y)
    torch.cuda.synchronize()
    ref = D.rmsnorm(x.astype(np.float64), D.widen_bf16(g), 1e-5)
    np.testing.assert_allclose(y.cpu().numpy(), ref, rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("kv", ["bf16", "fp32"])
@pytest.mark.parametrize("nq,nkv,hd", [(4, 2, 64), (32, 8, 128), (8, 1, 128), (2, 2, 64)])
@pytest.mark.parametrize("T,split", [(1, 64), (7, 64), (64, 64), (65, 64), (200, 16), (37, 1), (130, 13),
                                     (600, 256), (300, 1000)])
def test_attention_split_kv(abi, nq, nkv, hd, T, split, kv):
    rng = np.random.default_rng(T * 131 + split + nq)
    S = T + 3
    q = rng.normal(size=(nq, hd)).astype(np.float32)
    kb = gen.bf16_normal(2, 7, 0, nkv * S * hd, 1.0).reshape(nkv, S, hd)
    vb = gen.bf16_normal(2, 8, 0, nkv * S * hd, 1.0).reshape(nkv, S, hd)
    if kv == "bf16":
        kd, vd = dev_bits(kb).view(nkv, S, hd), dev_bits(vb).view(nkv, S, hd)
        K, V = D.widen_bf16(kb), D.widen_bf16(vb)
    else:  # fp32 values that are not bf16-representable
        K = rng.normal(size=(nkv, S, hd)).astype(np.float32)
        V = rng.normal(size=(nkv, S, hd)).astype(np.float32)
        kd, vd = torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda()
        K, V = K.astype(np.float64), V.astype(np.float64)
    o = torch.empty(nq, hd, dtype=torch.float32, device="cuda")
    abi.mk_t_attention(torch.from_numpy(q).cuda(), kd, vd, T, split, o)
    ref = D.gqa_attention(q.astype(np.float64), K[:, :T], V[:, :T])
    np.testing.assert_allclose(o.cpu().numpy(), ref, rtol=1e-5, atol=2e-6)


def test_attention_single_position_returns_v(abi):
    nq, nkv, hd = 8, 2, 128
    q = np.random.default_rng(0).normal(size=(nq, hd)).astype(np.float32)
    kb = gen.bf16_normal(3, 7, 0, nkv * 4 * hd, 1.0).reshape(nkv, 4, hd)
    vb = gen.bf16_normal(3, 8, 0, nkv * 4 * hd, 1.0).reshape(nkv, 4, hd)
    o = torch.empty(nq, hd, dtype=torch.float32, device="cuda")
    abi.mk_t_attention(torch.from_numpy(q).cuda(), dev_bits(kb).view(nkv, 4, hd), dev_bits(vb).view(nkv, 4, hd),
                       1, 64, o)
    v0 = D.widen_bf16(vb)[:, 0]
    assert np.array_equal(o.cpu().numpy().astype(np.float64), np.repeat(v0, nq // nkv, 0))


@pytest.mark.parametrize("n", [1, 5, 1000, 128256])
def test_argmax_lowest_index_on_ties(abi, n):
    rng = np.random.default_rng(n)
    x = rng.normal(size=n).astype(np.float32)
    if n > 4:
        m = x.max() + 1
        x[[n // 3, n // 2, n - 1]] = m  # ties: lowest index wins
    out = torch.empty(1, dtype=torch.int32, device="cuda")
    abi.mk_t_argmax(torch.from_numpy(x).cuda(), out)
    assert int(out.item()) == int(np.argmax(x))
    x2 = -np.abs(x) - 1  # all negative
    abi.mk_t_argmax(torch.from_numpy(x2).cuda(), out)
    assert int(out.item()) == int(np.argmax(x2))
