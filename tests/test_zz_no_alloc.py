"""fp8attn_forward_noalloc (no workspace: the library's static per-device scratch) against
fp8attn_forward (caller's workspace) through the C ABI. The same kernels run, so the outputs
must agree bit for bit; two calls in a row, the second on a smaller input, reuse the scratch
(its work-queue counters are cleared by a kernel at the start of every call). A shape that needs
more scratch than the array holds is rejected before anything is enqueued."""
import sys

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print("[no-alloc]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_attention_video_qkv_amd as m
    m.lib()
    return m


def _quantized(m, N, H, seed, vsmooth=False):
    q, k, v = workloads.make_qkv(1, N, H, seed, kind="token_outliers" if vsmooth else "normal")
    perm = None
    if vsmooth:
        perm = torch.argsort(v.float()[0, :, :, 0].t().contiguous(), dim=1, stable=True).to(torch.int32)[None]
        perm = perm.contiguous().to(DEV)
    return m.quantize_qkv(q.to(DEV), k.to(DEV), v.to(DEV), perm_kv=perm, vsmooth=vsmooth)


@pytest.mark.parametrize("vsmooth,pcast", [(False, 0), (True, 1)])
def test_noalloc_matches_forward(m, vsmooth, pcast):
    for N, H, seed in ((5000, 8, 1), (777, 3, 2)):      # the second call smaller than the first
        say("shape", N, H, "vsmooth", vsmooth, "pcast", pcast)
        qz = _quantized(m, N, H, seed, vsmooth)
        want = m.forward(qz, kv_order=1, pcast=pcast)
        out = torch.full_like(want, float("nan"))
        got = m.forward_noalloc(qz, kv_order=1, pcast=pcast, out=out)
        torch.cuda.synchronize()
        assert torch.isfinite(got.float()).all()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))


def test_noalloc_rejects_oversized_scratch(m):
    qz = _quantized(m, 20000, 4, 3)
    before = torch.zeros((1, 20000, 4, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(m.Fp8AttnError) as e:
        m.forward_noalloc(qz, kv_splits=8, out=before)   # 8 pieces of FP32 partials: far above
    assert e.value.status == m.FP8ATTN_ESCRATCH
    torch.cuda.synchronize()
    assert not before.any()                               # nothing was enqueued
