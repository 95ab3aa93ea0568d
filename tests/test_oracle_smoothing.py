"""Pins of the oracle's sequence-mean smoothing (TeleFuser blog "FP8 Sol-Attn", MiniMax-H3
section: K' = K - mean_T(K), V' = V - mean_T(V) per head with FP32 statistics, mean_T(V) added
back to the output, optional compensation of the residual mean bias that rounding V' to E4M3
leaves)."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads


def _bits(t):
    return workloads.bits(t)


def _cos(a, b):
    a, b = a.ravel(), b.ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def _exact(q, k, v):
    tr = lambda a: np.ascontiguousarray(oracle.bf16_decode(a).transpose(0, 2, 1, 3))
    ex, _, _ = oracle.attention_ref(oracle.MODE_EXACT, tr(q), tr(k), tr(v))
    return ex


def test_constant_v_restored_exactly():
    # V = c per (head, channel): V' = 0, every code 0, and the output must be c exactly.
    B, N, H, D = 1, 1000, 2, 128
    q, k, _ = workloads.make_qkv(B, N, H, seed=71)
    g = torch.Generator("cpu").manual_seed(72)
    c = torch.randn((1, 1, H, D), generator=g).to(torch.bfloat16)
    v = c.expand(B, N, H, D).contiguous()
    qz = oracle.quantize(_bits(q), _bits(k), _bits(v), smoothing=2)
    cbits = _bits(c)[0, 0]
    assert np.array_equal(qz["v_shift"][0], oracle.bf16_decode(cbits).astype(np.float32))
    assert not qz["v8t"].any() and not qz["v_scale"].any()
    _, ob, _, _ = oracle.attention_fp8(qz, kv_reverse=True)
    assert np.array_equal(ob[0], np.broadcast_to(cbits[:, None, :], ob[0].shape))


@pytest.mark.parametrize("sta", [False, True])
def test_mean_over_valid_tokens(sta):
    # v_shift equals the mean of V over the valid tokens (not the padding) to within the
    # rounding of an FP32 tree sum.
    q, k, v = workloads.make_qkv(1, 21 * 10 * 16, 2, seed=73)
    v = (v.float() + 3.0).to(torch.bfloat16)  # a nonzero mean
    perm = None
    if sta:
        lay = oracle.sta_layout(21, 10, 16, 6, 8, 8, 1, 1, 1)
        perm = lay["perm"]
    qz = oracle.quantize(_bits(q), _bits(k), _bits(v), perm_q=perm, perm_kv=perm, smoothing=2)
    x = oracle.bf16_decode(_bits(v)).astype(np.float64)[0]  # [N, H, D]
    want = x.mean(axis=0)  # [H, D]
    n = x.shape[0]
    bound = (64 + math.log2(n) + 2) * 2.0 ** -24 * np.abs(x).mean(axis=0) + 2.0 ** -22 * np.abs(want)
    assert np.all(np.abs(qz["v_shift"][0] - want) <= bound)


@pytest.mark.parametrize("sta", [False, True])
def test_mean_exact_when_every_partial_sum_is_exact(sta):
    # Values k/8 with |k| <= 64 over 3000 tokens: every partial sum of them, in any order, is a
    # multiple of 1/8 below 2^15 and so exact in FP32. The mean is then the plain definition's
    # value bit for bit: the exact sum over the valid tokens divided by their count, rounded once
    # (a dropped or doubled token, a padding row counted, or a wrong count fails this).
    N, H = 3000, 2
    g = torch.Generator("cpu").manual_seed(78)
    kk = torch.randint(-64, 65, (1, N, H, 128), generator=g).float() / 8.0
    v = kk.to(torch.bfloat16)
    assert torch.equal(v.float(), kk)
    q, k, _ = workloads.make_qkv(1, N, H, seed=79)
    perm = None
    if sta:
        lay = oracle.sta_layout(15, 10, 20, 6, 8, 8, 1, 1, 1)  # 3000 tokens, padded tiles
        perm = lay["perm"]
        assert (perm >= 0).sum() == N and perm.shape[0] > N
    qz = oracle.quantize(_bits(q), _bits(k), _bits(v), perm_q=perm, perm_kv=perm, smoothing=2)
    exact_sum = kk[0].double().sum(dim=0).numpy()  # [H, 128], exact
    want = (exact_sum.astype(np.float32) / np.float32(N)).astype(np.float32)
    assert np.array_equal(qz["v_shift"][0].view(np.uint32), want.view(np.uint32))


def _offset_error(which, smoothing):
    B, N, H = 1, 2048, 2
    q, k, v = workloads.make_qkv(B, N, H, seed=74)
    g = torch.Generator("cpu").manual_seed(75)
    off = 12.0 * torch.randn((1, 1, H, 128), generator=g)
    if which == "k":
        k = (k.float() + off).to(torch.bfloat16)
    else:
        v = (v.float() + off).to(torch.bfloat16)
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    qz = oracle.quantize(qb, kb, vb, smoothing=smoothing)
    out, _, _, _ = oracle.attention_fp8(qz, kv_reverse=True)
    ex = _exact(qb, kb, vb)
    return float(np.sqrt(np.mean((out - ex) ** 2)))


def test_k_offset_removed_by_k_smoothing():
    # A per-channel offset on K moves every logit of a row by one constant (softmax-invariant)
    # but spends the block scales' range; removing it must cut the FP8 error.
    e0, e1 = _offset_error("k", 0), _offset_error("k", 1)
    assert e1 < 0.5 * e0, (e0, e1)


def test_v_offset_removed_by_v_smoothing():
    e1, e2 = _offset_error("v", 1), _offset_error("v", 2)
    assert e2 < 0.5 * e1, (e1, e2)


def test_bias_correction_restores_the_mean_of_v():
    # With the correction, the token mean of the dequantised V' plus the output shift equals the
    # token mean of V (the rounding bias of V' is compensated); without it the two differ by
    # exactly that bias.
    q, k, v = workloads.make_qkv(1, 3000, 2, seed=76, kind="token_outliers", n_outlier_channels=8)
    v = (v.float() * 0.37 + 0.11).to(torch.bfloat16)
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    x = oracle.bf16_decode(vb).astype(np.float64)[0].mean(axis=0)  # [H, D]
    res = {}
    for corr in (False, True):
        qz = oracle.quantize(qb, kb, vb, smoothing=2, v_bias_correction=corr)
        deq = oracle.e4m3_decode(qz["v8t"][0, :, :, :3000]) * qz["v_scale"][0][:, :, None]
        res[corr] = deq.mean(axis=2) + qz["v_shift"][0] - x
    scale = np.abs(x).max()
    assert np.abs(res[True]).max() <= 1e-6 * scale + 1e-6
    assert np.abs(res[False]).max() > 10 * np.abs(res[True]).max()


def test_smoothing_argument_errors():
    q, k, v = workloads.make_qkv(1, 128, 1, seed=77)
    with pytest.raises(ValueError):
        oracle.quantize(_bits(q), _bits(k), _bits(v), vsmooth=True, smoothing=2)
    with pytest.raises(ValueError):
        oracle.quantize(_bits(q), _bits(k), _bits(v), smoothing=1, v_bias_correction=True)
