"""Pins of the oracle's Sol routing (TeleFuser blog "FP8 Sol-Attn", sections "Sol Routing" and
"SM90 CuTe Mainloop"): block summaries, the threshold estimators, the exact-block mask, and the
two routes of the attention.

* every block exact (tau -> -inf) is the dense FP8 path bit for bit;
* summaries are the block means of the dequantised K and V; quantised K summaries decode back
  within half an E4M3 step;
* the "exact" estimator's mu and sigma are the mean and standard deviation of all route scores
  of the Q block (computed here by brute force over the pairs); "diag" equals it when only one
  channel is non-zero;
* the mask is the brute-force rule "some query of the block reaches theta, or a sink block";
* on inputs whose K and V rows are constant inside each KV block (and exactly representable),
  the summary route is exact: all-summary Sol equals FP64 softmax attention.
"""
import math

import numpy as np
import pytest

import workloads

SS = 1.0 / math.sqrt(128.0)


def _qz(orc, N, H, seed, kind="normal"):
    q, k, v = workloads.make_qkv(1, N, H, seed, kind=kind)
    b = workloads.bits
    return orc.quantize(b(q), b(k), b(v))


@pytest.mark.parametrize("N,rev,expcast", [(1000, True, False), (777, False, True), (64, True, False)])
def test_all_exact_is_dense(orc, N, rev, expcast):
    qz = _qz(orc, N, 2, 5 + N)
    sol = orc.sol_prepare(qz, tau=-1e9, estimator=1, sink_blocks=0)
    assert orc.mask_bits(sol["mask"], -(-N // 64)).all()
    a = orc.attention_fp8(qz, kv_reverse=rev, expcast=expcast, sol=sol)
    b = orc.attention_fp8(qz, kv_reverse=rev, expcast=expcast)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_summaries_are_block_means(orc):
    N, H = 1000, 2
    qz = _qz(orc, N, H, 21, kind="channel_outliers")
    sol = orc.sol_prepare(qz)
    NB = -(-N // 64)
    kd = orc.e4m3_decode(qz["k8"][:, :, :N]) * np.repeat(qz["k_scale"], 64, axis=2)[:, :, :N, None]
    vd = orc.e4m3_decode(qz["v8t"][:, :, :, :N]).transpose(0, 1, 3, 2) * qz["v_scale"][:, :, None, :]
    for j in range(NB):
        lo, hi = 64 * j, min(N, 64 * j + 64)
        km = kd[:, :, lo:hi].mean(axis=2)
        vm = vd[:, :, lo:hi].mean(axis=2)
        ks = sol["ksum"][:, :, j].astype(np.float64)
        assert np.all(np.abs(ks - km) <= 2 * 2.0 ** -23 * np.abs(km) + 1e-30)
        vs = orc.bf16_decode(sol["vsum"][:, :, j])
        assert np.all(np.abs(vs - vm) <= (2.0 ** -8 + 2.0 ** -22) * np.abs(vm) + 1e-30)
    # quantised summaries: decode(kq8) * scale within half an E4M3 step (2^-4 relative, plus the
    # subnormal spacing 2^-9 * scale) of the FP32 summary
    NBg = -(-NB // 64)
    for g in range(NBg):
        s = qz_s = sol["kq_scale"][:, :, g][:, :, None, None].astype(np.float64)
        rec = orc.e4m3_decode(sol["kq8"][:, :, 64 * g:64 * g + 64]) * s
        ref = np.zeros_like(rec)
        n = min(NB, 64 * g + 64) - 64 * g
        ref[:, :, :n] = sol["ksum"][:, :, 64 * g:64 * g + n]
        assert np.all(np.abs(rec - ref) <= 2.0 ** -4 * np.abs(ref) + 2.0 ** -10 * qz_s)
        amax = np.abs(sol["ksum"][:, :, 64 * g:64 * g + n]).max(axis=(2, 3))
        assert np.allclose(sol["kq_scale"][:, :, g], amax / 448.0, rtol=2e-7)


def _pair_stats(orc, qz, sol, u):
    """Brute force: mean and std of r_ij = ss * q_i . kbar_j over the valid queries i of Q block
    u and every KV block j, per head (FP32 summaries, dequantised queries)."""
    N = qz["N"]
    lo, hi = 64 * u, min(N, 64 * u + 64)
    qd = orc.e4m3_decode(qz["q8"][:, :, lo:hi]) * qz["q_scale"][:, :, u][:, :, None, None]
    r = np.einsum("bhid,bhjd->bhij", qd, sol["ksum"].astype(np.float64)) * SS
    return r.mean(axis=(2, 3)), r.std(axis=(2, 3))


@pytest.mark.parametrize("tau", [0.0, 2.5, -1.0])
def test_exact_estimator_is_the_pair_statistics(orc, tau):
    N = 700
    qz = _qz(orc, N, 2, 33, kind="channel_outliers")
    sol = orc.sol_prepare(qz, tau=tau, estimator=1)
    for u in range(-(-N // 64)):
        mu, sd = _pair_stats(orc, qz, sol, u)
        want = mu + tau * sd
        assert np.allclose(sol["theta"][:, :, u], want, rtol=1e-9, atol=1e-12)


def test_diag_estimator_equals_exact_with_one_channel(orc):
    N, H = 500, 1
    q, k, v = workloads.make_qkv(1, N, H, 44)
    k = k * 0
    k[..., 3] = 2.0
    k[0, ::7, :, 3] = -1.0
    b = workloads.bits
    qz = orc.quantize(b(q), b(k), b(v))
    t0 = orc.sol_prepare(qz, tau=2.0, estimator=0)["theta"]
    t1 = orc.sol_prepare(qz, tau=2.0, estimator=1)["theta"]
    assert np.allclose(t0, t1, rtol=1e-12, atol=1e-15)
    # with many channels the two differ
    qz2 = _qz(orc, N, H, 45, kind="channel_outliers")
    assert not np.allclose(orc.sol_prepare(qz2, tau=2.0, estimator=0)["theta"],
                           orc.sol_prepare(qz2, tau=2.0, estimator=1)["theta"])


@pytest.mark.parametrize("tau,sinks", [(2.0, 1), (3.0, 0), (2.5, 3)])
def test_mask_is_the_bruteforce_rule(orc, tau, sinks):
    N, H = 900, 2
    qz = _qz(orc, N, H, 55)
    sol = orc.sol_prepare(qz, tau=tau, estimator=0, sink_blocks=sinks)
    NB = -(-N // 64)
    bits = orc.mask_bits(sol["mask"], NB)
    amb = orc.mask_bits(sol["amb_mask"], NB)
    kq = orc.e4m3_decode(sol["kq8"][:, :, :NB]) * np.repeat(sol["kq_scale"], 64, axis=2)[:, :, :NB, None]
    exact_frac = bits.mean()
    assert 0.0 < exact_frac < 1.0
    for u in range(NB):
        lo, hi = 64 * u, min(N, 64 * u + 64)
        qd = orc.e4m3_decode(qz["q8"][:, :, lo:hi]) * qz["q_scale"][:, :, u][:, :, None, None]
        r = np.einsum("bhid,bhjd->bhij", qd, kq) * SS
        want = (r >= sol["theta"][:, :, u][:, :, None, None]).any(axis=2)
        want[:, :, :sinks] = True
        ok = (want == bits[:, :, u]) | amb[:, :, u]
        assert ok.all()


def _block_constant_grid(orc, rng, N, H, D=128):
    """K and V rows constant inside each 64-token block, all values on the E4M3 grid, every
    scale exactly 1: summaries equal the rows and the summary route is exact."""
    NB = -(-N // 64)

    def grid(shape):
        codes = rng.integers(0x08, 0x40, size=shape).astype(np.uint8)
        codes = np.where(rng.random(shape) < 0.5, codes | 0x80, codes).astype(np.uint8)
        return orc.e4m3_decode(codes)

    q = grid((1, N, H, D))
    kb = grid((1, NB, H, D))
    vb = grid((1, NB, H, D))
    for b in range(NB):
        q[0, 64 * b, :, 0] = 448.0
    kb[0, :, :, 1] = 448.0                      # every K block (and summary group) has amax 448
    vb[0, 0, :, :] = 448.0                      # every V channel has amax 448
    k = np.repeat(kb, 64, axis=1)[:, :N]
    v = np.repeat(vb, 64, axis=1)[:, :N]
    return q, k, v


@pytest.mark.parametrize("N,rev", [(1000, True), (320, False)])
def test_summary_route_exact_on_block_constant_inputs(orc, N, rev):
    import torch
    rng = np.random.default_rng(N)
    H = 2
    q, k, v = _block_constant_grid(orc, rng, N, H)
    to_bits = lambda a: workloads.bits(torch.from_numpy(a).to(torch.bfloat16))
    qz = orc.quantize(to_bits(q), to_bits(k), to_bits(v))
    assert np.all(qz["q_scale"] == 1.0) and np.all(qz["k_scale"] == 1.0) and np.all(qz["v_scale"] == 1.0)
    ss = 1e-3
    sol = orc.sol_prepare(qz, tau=1e9, estimator=0, sink_blocks=0, softmax_scale=ss)
    assert not orc.mask_bits(sol["mask"], -(-N // 64)).any()
    out, _, _, _ = orc.attention_fp8(qz, softmax_scale=ss, kv_reverse=rev, sol=sol)
    tr = lambda a: np.ascontiguousarray(a.transpose(0, 2, 1, 3))
    ex, _, _ = orc.attention_ref(orc.MODE_EXACT, tr(q), tr(k), tr(v), softmax_scale=ss)
    assert np.max(np.abs(out - ex)) < 1e-9 * np.max(np.abs(ex))
