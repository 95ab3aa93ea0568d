"""Pins of the oracle's split-KV (TeleFuser blog "FP8 Sol-Attn", long-sequence split-KV: pieces
of the KV sequence run their own online softmax and are merged by log-sum-exp).

* With every cast off, the merge is exact mathematics: split or not, the streaming result
  equals brute-force FP64 softmax attention.
* With the P cast on (the P-cast paper's kernel-faithful mode), each piece's codes depend on its
  own running max; a numpy re-implementation of the pieces (cut at absolute multiples of
  L = 2*ceil(NB/(2*splits)) blocks, each visited in KV order) and of the merge must agree.
* One piece, or kv_splits 0/1, is the unsplit loop bit for bit.
"""
import math

import numpy as np
import pytest

import workloads


def _layout(orc, N, H, seed):
    q, k, v = workloads.make_qkv(1, N, H, seed)
    tr = lambda a: np.ascontiguousarray(orc.bf16_decode(workloads.bits(a)).transpose(0, 2, 1, 3))
    return tr(q), tr(k), tr(v)


def _bruteforce(q, k, v, scale):
    x = (q @ k.T) * scale
    p = np.exp(x - x.max(axis=1, keepdims=True))
    return (p @ v) / p.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("N,splits,rev", [(1000, 2, False), (1000, 3, True), (300, 2, True),
                                          (4096, 16, False), (64, 4, True)])
def test_noquant_split_equals_bruteforce(orc, N, splits, rev):
    q, k, v = _layout(orc, N, 2, seed=N + splits)
    scale = 1.0 / math.sqrt(128.0)
    out, _, _ = orc.attention_ref(orc.MODE_NOQUANT, q, k, v, kv_reverse=rev, kv_splits=splits)
    for h in range(2):
        ref = _bruteforce(q[0, h], k[0, h], v[0, h], scale)
        assert np.max(np.abs(out[0, h] - ref)) < 1e-12


def _pcast_pieces(orc, q, k, v, splits, rev, S, scale):
    """numpy: per row, the pieces' streaming loops with P8 = E4M3(fl32(S p)), then the merge."""
    N = q.shape[0]
    NB = -(-N // 64)
    L = 2 * -(-NB // (2 * splits)) if splits > 1 else NB
    pieces = [list(range(lo, min(NB, lo + L))) for lo in range(0, NB, L)]
    x_all = (q @ k.T) * scale
    out = np.zeros_like(q)
    for i in range(N):
        parts = []
        for blocks in pieces:
            seq = blocks[::-1] if rev else blocks
            m, l, acc = -np.inf, 0.0, np.zeros(q.shape[1])
            for kb in seq:
                xs = x_all[i, kb * 64:min(N, kb * 64 + 64)]
                m_new = max(m, xs.max())
                alpha = 0.0 if m == -np.inf else math.exp(m - m_new)
                p = np.exp(xs - m_new)
                codes = orc.e4m3_encode((S * p).astype(np.float32).astype(np.float64))
                pv = orc.e4m3_decode(codes) / S
                l = alpha * l + p.sum()
                acc = alpha * acc + pv @ v[kb * 64:min(N, kb * 64 + 64)]
                m = m_new
            parts.append((acc / l, m, l))
        mm = max(pm for _, pm, _ in parts)
        w = np.array([pl * math.exp(pm - mm) for _, pm, pl in parts])
        out[i] = sum(wi * po for wi, (po, _, _) in zip(w, parts)) / w.sum()
    return out


@pytest.mark.parametrize("N,splits,rev", [(300, 2, True), (300, 2, False), (700, 3, True),
                                          (1000, 4, False)])
def test_pcast_split_matches_numpy_pieces(orc, N, splits, rev):
    q, k, v = _layout(orc, N, 1, seed=7 * N + splits)
    scale = 1.0 / math.sqrt(128.0)
    S = 256.0
    out, _, _ = orc.attention_ref(orc.MODE_PCAST, q, k, v, kv_reverse=rev, kv_splits=splits,
                                  p_scale=S)
    ref = _pcast_pieces(orc, q[0, 0], k[0, 0], v[0, 0], splits, rev, S, scale)
    assert np.max(np.abs(out[0, 0] - ref)) < 1e-12
    # the pieces' own maxima change P codes: the split result is not the unsplit one
    one, _, _ = orc.attention_ref(orc.MODE_PCAST, q, k, v, kv_reverse=rev, p_scale=S)
    assert np.max(np.abs(out - one)) > 1e-6


def test_one_piece_is_the_unsplit_loop(orc):
    q8 = workloads.make_qkv(1, 500, 2, 3)
    b = workloads.bits
    qz = orc.quantize(b(q8[0]), b(q8[1]), b(q8[2]))
    base = orc.attention_fp8(qz, kv_reverse=True)
    for sp in (0, 1):
        alt = orc.attention_fp8(qz, kv_reverse=True, kv_splits=sp)
        for a, c in zip(base, alt):
            assert np.array_equal(a, c)
    # 128 tokens = 2 blocks: L = 2 for 2 requested pieces, so one piece
    qz2 = orc.quantize(*(b(t[:, :128]) for t in q8))
    a = orc.attention_fp8(qz2, kv_reverse=True)
    c = orc.attention_fp8(qz2, kv_reverse=True, kv_splits=2)
    assert np.array_equal(a[0], c[0])


def test_split_underflow_counts_add_up(orc):
    """Sink inputs: the piece without the sink keys has its own max, so its keys underflow
    less; the counts of the pieces add up to the row's count."""
    q, k, v = workloads.workload("sink4096", delta=9, heads=1)
    b = workloads.bits
    qz = orc.quantize(b(q), b(k), b(v))
    rows = np.arange(0, 4096, 97, dtype=np.int32)
    _, _, uf1, _ = orc.attention_fp8(qz, rows=rows, p_scale=1.0, kv_reverse=False)
    _, _, uf2, _ = orc.attention_fp8(qz, rows=rows, p_scale=1.0, kv_reverse=False, kv_splits=2)
    assert uf2.sum() < uf1.sum()
    assert uf2.sum() > 0
