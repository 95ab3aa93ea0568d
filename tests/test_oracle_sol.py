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
  the summary route is exact: all-summary Sol equals FP64 softmax attention;
* both routes update one online-softmax state, route group by route group of 64 KV blocks in KV
  order, a group's summary blocks before its exact blocks: where summary blocks score above the
  exact blocks, the oracle equals an independent numpy model of that shared loop (exact blocks'
  P codes taken against the summary-set running max) and differs from the reading with two
  states merged by log-sum-exp; with several groups, a group's exact blocks see the summaries of
  that group and of the groups before it in KV order, and not those of later groups.
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


# ------------------------------------------------------------------------------------------
# One shared online-softmax state (TeleFuser blog, "Sol Routing": the summary route keeps its
# compressed contribution in the same online-softmax state; "SM90 CuTe Mainloop": both routes
# update one row max, row sum and output accumulator)
# ------------------------------------------------------------------------------------------
def _decoded(orc, qz):
    N = qz["N"]
    qd = orc.e4m3_decode(qz["q8"][:, :, :N]).astype(np.float64)
    kd = orc.e4m3_decode(qz["k8"][:, :, :N]).astype(np.float64)
    vd = orc.e4m3_decode(qz["v8t"][:, :, :, :N]).transpose(0, 1, 3, 2).astype(np.float64)
    return qd, kd, vd


def _logits(qz, qd, kd, b, h, i, ss):
    """Logits of query i against every key, exact in FP64 (E4M3 products, 128-term sums)."""
    u = i // 64
    ks = np.repeat(qz["k_scale"][b, h].astype(np.float64), 64)[: kd.shape[2]]
    return (kd[b, h] @ qd[b, h, i]) * float(qz["q_scale"][b, h, u]) * ks * ss


def _route_scores(orc, qz, sol, qd, b, h, i, ss):
    NB = -(-qz["N"] // 64)
    kq = orc.e4m3_decode(sol["kq8"][b, h, :NB]).astype(np.float64)
    sc = np.repeat(sol["kq_scale"][b, h].astype(np.float64), 64)[:NB]
    return (kq @ qd[b, h, i]) * float(qz["q_scale"][b, h, i // 64]) * sc * ss


def _sol_model(orc, qz, sol, exact, rev, S, ss, shared=True, rows=None):
    """numpy: per row, the KV blocks in route groups of 64 (groups in KV order; a group's summary
    blocks, then its exact blocks, each in KV order). shared=True: one (m, l, acc) for both routes;
    an exact block takes m' = max(m, max x), P8 = E4M3(fl32(S exp(x - m'))), l += sum p,
    acc += P8 . V8; a summary block takes m' = max(m, r_j), w = n_j exp(r_j - m'), l += w,
    acc += w vbar_j. shared=False: the exact blocks run their own state, the summary blocks
    theirs, and the two are merged by log-sum-exp (the reading this pin rules out)."""
    B, H = qz["q8"].shape[:2]
    N = qz["N"]
    NB = -(-N // 64)
    qd, kd, vd = _decoded(orc, qz)
    rows = range(N) if rows is None else rows
    out = np.zeros((B, H, len(rows), 128))
    kv = list(range(NB))[::-1] if rev else list(range(NB))
    groups = sorted({j // 64 for j in kv}, reverse=rev)
    for b in range(B):
        for h in range(H):
            vs = vd[b, h] * qz["v_scale"][b, h].astype(np.float64)[None, :]
            vbar = orc.bf16_decode(sol["vsum"][b, h]).astype(np.float64)
            for ri, i in enumerate(rows):
                x_all = _logits(qz, qd, kd, b, h, i, ss)
                r_all = _route_scores(orc, qz, sol, qd, b, h, i, ss)
                states = {True: [-np.inf, 0.0, np.zeros(128)], False: [-np.inf, 0.0, np.zeros(128)]}
                u = i // 64
                # route groups in KV order; a group's summary blocks, then its exact blocks
                order = [j for g in groups for ex in (False, True) for j in kv
                         if j // 64 == g and bool(exact[b, h, u, j]) == ex]
                for j in order:
                    ex = bool(exact[b, h, i // 64, j])
                    st = states[True] if shared else states[ex]
                    m, l, acc = st
                    if ex:
                        xs = x_all[64 * j:min(N, 64 * j + 64)]
                        m_new = max(m, xs.max())
                        alpha = 0.0 if m == -np.inf else math.exp(m - m_new)
                        p = np.exp(xs - m_new)
                        codes = orc.e4m3_encode((S * p).astype(np.float32).astype(np.float64))
                        pd = orc.e4m3_decode(codes).astype(np.float64) / S
                        st[:] = [m_new, alpha * l + p.sum(), alpha * acc + pd @ vs[64 * j:64 * j + len(xs)]]
                    else:
                        n_j = min(64, N - 64 * j)
                        m_new = max(m, r_all[j])
                        alpha = 0.0 if m == -np.inf else math.exp(m - m_new)
                        w = n_j * math.exp(r_all[j] - m_new)
                        st[:] = [m_new, alpha * l + w, alpha * acc + w * vbar[j]]
                if shared:
                    m, l, acc = states[True]
                    out[b, h, ri] = acc / l
                else:
                    ms = [s_[0] for s_ in states.values() if s_[1] > 0]
                    mx = max(ms)
                    num, den = np.zeros(128), 0.0
                    for m, l, acc in states.values():
                        if l > 0:
                            num += math.exp(m - mx) * acc
                            den += math.exp(m - mx) * l
                    out[b, h, ri] = num / den
    return out


def _sink_block_inputs(N, H, seed, summary_blocks, delta):
    """N(0,1) Q, K, V; channel 127 carries a bias (Q = 4, K = delta * sqrt(128) / 4 on every key
    of the listed blocks, 0 elsewhere), so those blocks' logits, and hence their summaries'
    route scores, sit about delta above the others."""
    import torch
    q, k, v = workloads.make_qkv(1, N, H, seed)
    q = q.float()
    k = k.float()
    q[..., 127] = 4.0
    k[..., 127] = 0.0
    for j in summary_blocks:
        k[:, 64 * j:64 * j + 64, :, 127] = delta * math.sqrt(128.0) / 4.0
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v


@pytest.mark.parametrize("rev,S", [(False, 256.0), (True, 256.0), (False, 1.0)])
def test_shared_state_matches_model(orc, rev, S):
    """Summary blocks scoring about 4 above the exact blocks' logits sit before them in KV order,
    so the exact blocks' P codes are taken against a running max that a summary set. The
    oracle equals the shared-state model, and the two-state reading gives a different result."""
    N, H, ss = 640, 1, 1.0 / math.sqrt(128.0)
    NB = N // 64
    summary = [0, 3, 4, 7, 8] if not rev else [9, 6, 5, 2, 1]
    q, k, v = _sink_block_inputs(N, H, 61, summary, 4.0)
    b = workloads.bits
    qz = orc.quantize(b(q), b(k), b(v))
    sol = dict(orc.sol_prepare(qz, tau=0.0, estimator=0, sink_blocks=0))
    exact = np.ones((1, H, NB, NB), bool)
    exact[..., summary] = False
    words = np.zeros((1, H, NB, 1), np.uint64)
    for j in range(NB):
        words[..., 0] |= (exact[..., j].astype(np.uint64) << np.uint64(j))
    sol["mask"] = words
    out, _, uf, _ = orc.attention_fp8(qz, p_scale=S, kv_reverse=rev, sol=sol)
    want = _sol_model(orc, qz, sol, exact, rev, S, ss, shared=True)
    other = _sol_model(orc, qz, sol, exact, rev, S, ss, shared=False)
    # the situation the pin is about: the first block visited is a summary scoring above the
    # largest logit of the first exact block after it, for most rows
    qd, kd, _ = _decoded(orc, qz)
    first_ex = next(j for j in (range(NB)[::-1] if rev else range(NB)) if exact[0, 0, 0, j])
    hits = 0
    for i in range(0, N, 7):
        r = _route_scores(orc, qz, sol, qd, 0, 0, i, ss)
        x = _logits(qz, qd, kd, 0, 0, i, ss)[64 * first_ex:64 * first_ex + 64]
        hits += r[summary[0]] > x.max()
    assert hits >= 0.9 * len(range(0, N, 7))
    scale = np.abs(want).max()
    assert np.max(np.abs(out - want)) <= 1e-10 * scale
    assert np.max(np.abs(out - other)) > 1e-3 * scale
    if S == 1.0:
        # with S = 1 the exact blocks' codes against the summary-set max underflow more than
        # against their own max
        assert uf.sum() > 0


@pytest.mark.parametrize("rev", [False, True])
def test_shared_state_route_groups(orc, rev):
    """70 KV blocks, two route groups. Summary block 66 (group 1) scores about 6 above every
    other block. Forward: group 0's exact blocks run before it and are unaffected; group 1's see
    it. Reverse: group 1 comes first, so every exact block sees it. Sampled rows of the oracle
    equal the numpy model of the grouped shared loop, not the two-state reading."""
    NBk = 70
    N, H, S, ss = 64 * NBk, 1, 256.0, 1.0 / math.sqrt(128.0)
    summary = [3, 10, 66, 68]
    q, k, v = _sink_block_inputs(N, H, 62, [66], 6.0)
    b = workloads.bits
    qz = orc.quantize(b(q), b(k), b(v))
    sol = dict(orc.sol_prepare(qz, tau=0.0, estimator=0, sink_blocks=0))
    exact = np.ones((1, H, NBk, NBk), bool)
    exact[..., summary] = False
    words = np.zeros((1, H, NBk, 2), np.uint64)
    for j in range(NBk):
        words[..., j // 64] |= (exact[..., j].astype(np.uint64) << np.uint64(j % 64))
    sol["mask"] = words
    rows = np.array([0, 1, 777, 2048, 3000, N - 1], np.int32)
    out, _, _, _ = orc.attention_fp8(qz, rows=rows, p_scale=S, kv_reverse=rev, sol=sol)
    want = _sol_model(orc, qz, sol, exact, rev, S, ss, shared=True, rows=rows)
    other = _sol_model(orc, qz, sol, exact, rev, S, ss, shared=False, rows=rows)
    scale = np.abs(want).max()
    assert np.max(np.abs(out - want)) <= 1e-10 * scale
    assert np.max(np.abs(out - other)) > 1e-3 * scale
