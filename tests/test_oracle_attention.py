"""Pins of the oracle's quantisation and attention paths.

Each check ties the oracle to something other than itself: brute-force FP64 softmax in numpy,
a token-level sparse mask built from raster coordinates, exactly representable inputs on
which quantisation is the identity, closed-form counts of the sliding-tile layout, and the
algebraic identities the pages rely on (V-Smooth's mean split, permutation invariance of
non-causal attention, constant-value preservation).

Sources: TeleFuser blog ("面向注意力的 FP8 Preparation", "SM90 CuTe Mainloop", "输出验证":
non-aligned tails and constant-value preservation); FPSAttention write-up 2.2/3.1 (STA);
VC-Attention article 二/三 (V-Smooth, ExpCast); P-cast paper 三 (order, S).
"""
import math

import numpy as np
import pytest
import torch


def _softmax_attn(q, k, v, scale, mask=None):
    """numpy FP64 brute force: q [N,D], k [M,D], v [M,D], optional bool mask [N,M]."""
    x = (q @ k.T) * scale
    if mask is not None:
        x = np.where(mask, x, -np.inf)
    x = x - x.max(axis=1, keepdims=True)
    p = np.exp(x)
    return (p @ v) / p.sum(axis=1, keepdims=True)


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def _grid_values(orc, rng, shape):
    """Random E4M3 grid values with exponent fields 1..7 (2^-6 <= |x| < 2), as float64."""
    codes = rng.integers(0x08, 0x40, size=shape).astype(np.uint8)
    codes = np.where(rng.random(shape) < 0.5, codes | 0x80, codes).astype(np.uint8)
    return orc.e4m3_decode(codes)


@pytest.mark.parametrize("N,D,rev", [(37, 16, False), (64, 128, True), (200, 128, False),
                                     (300, 32, True)])
def test_noquant_and_exact_match_bruteforce(orc, N, D, rev):
    rng = np.random.default_rng(N + D)
    q, k, v = (rng.standard_normal((1, 2, N, D)) for _ in range(3))
    scale = 1 / math.sqrt(D)
    for mode in (orc.MODE_EXACT, orc.MODE_NOQUANT):
        out, _, rv = orc.attention_ref(mode, q, k, v, softmax_scale=scale, kv_reverse=rev)
        assert rv.all()
        for h in range(2):
            ref = _softmax_attn(q[0, h], k[0, h], v[0, h], scale)
            assert np.max(np.abs(out[0, h] - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def _raster_mask(T, Hg, W, tt, th, tw, rt, rh, rw, perm):
    """Token-level STA mask in the layout order, from raster coordinates only."""
    n = perm.shape[0]
    valid = perm >= 0
    src = np.where(valid, perm, 0)
    t, y, x = src // (Hg * W), (src // W) % Hg, src % W
    ct, cy, cx = t // tt, y // th, x // tw
    m = ((np.abs(ct[:, None] - ct[None, :]) <= rt) & (np.abs(cy[:, None] - cy[None, :]) <= rh)
         & (np.abs(cx[:, None] - cx[None, :]) <= rw))
    return m & valid[:, None] & valid[None, :], valid


@pytest.mark.parametrize("rev", [False, True])
def test_sparse_noquant_matches_token_mask(orc, rev):
    T, Hg, W, tt, th, tw = 5, 7, 9, 2, 4, 8          # tiles of 64 tokens, ragged in T and H
    lay = orc.sta_layout(T, Hg, W, tt, th, tw, 1, 1, 0)
    perm = lay["perm"]
    n = perm.shape[0]
    D = 32
    rng = np.random.default_rng(5)
    src = rng.standard_normal((3, T * Hg * W, D))
    q, k, v = (np.where(perm[:, None] >= 0, s[np.maximum(perm, 0)], 0.0)[None, None] for s in src)
    mask, valid = _raster_mask(T, Hg, W, tt, th, tw, 1, 1, 0, perm)
    scale = 1 / math.sqrt(D)
    out, _, rv = orc.attention_ref(orc.MODE_NOQUANT, q, k, v, softmax_scale=scale,
                                   kv_reverse=rev, sparse=lay)
    assert np.array_equal(rv[0, 0].astype(bool), valid)
    ref = _softmax_attn(q[0, 0][valid], k[0, 0], v[0, 0], scale, mask=mask[valid])
    assert np.max(np.abs(out[0, 0][valid] - ref)) <= 1e-12
    ex, _, _ = orc.attention_ref(orc.MODE_EXACT, q, k, v, softmax_scale=scale, sparse=lay)
    assert np.max(np.abs(ex[0, 0][valid] - ref)) <= 1e-12


def test_sta_layout_wan14b_counts(orc):
    lay = orc.sta_layout(21, 45, 80, 6, 8, 8, 1, 1, 1)
    assert lay["n_tiles"] == 240 and lay["tile_tokens"] == 384
    assert lay["perm"].shape[0] == 92160
    nnz_per_row = np.diff(lay["row_ptr"])
    assert nnz_per_row.sum() == 4480 == 10 * 16 * 28      # per-axis neighbour-count product
    assert nnz_per_row.min() == 8 and nnz_per_row.max() == 27
    perm = lay["perm"]
    assert np.array_equal(np.sort(perm[perm >= 0]), np.arange(75600))
    assert (perm < 0).sum() == 92160 - 75600
    # independent count from raster coordinates: valid tokens per tile and neighbour tiles
    t, y, x = np.meshgrid(np.arange(21), np.arange(45), np.arange(80), indexing="ij")
    tile_of = ((t // 6) * 6 + (y // 8)) * 10 + (x // 8)
    per_tile = np.bincount(tile_of.ravel(), minlength=240)
    assert np.array_equal(per_tile, lay["tile_len"])
    ct, cy, cx = np.meshgrid(np.arange(4), np.arange(6), np.arange(10), indexing="ij")
    ct, cy, cx = ct.ravel(), cy.ravel(), cx.ravel()
    nb = ((np.abs(ct[:, None] - ct[None]) <= 1) & (np.abs(cy[:, None] - cy[None]) <= 1)
          & (np.abs(cx[:, None] - cx[None]) <= 1))
    pairs = int((per_tile[:, None] * per_tile[None, :] * nb).sum())
    assert pairs == 498_693_888
    cols = [set(lay["col_idx"][lay["row_ptr"][u]:lay["row_ptr"][u + 1]]) for u in range(240)]
    assert all(cols[u] == set(np.flatnonzero(nb[u])) for u in range(240))
    assert all(np.all(np.diff(lay["col_idx"][lay["row_ptr"][u]:lay["row_ptr"][u + 1]]) > 0)
               for u in range(240))


def _exact_grid_inputs(orc, rng, N, H, D=128):
    """Q, K, V whose bf16 values lie on the E4M3 grid and whose every Q/K 64-block and every V
    channel contains 448: all scales are exactly 1 and quantisation is the identity."""
    NB = (N + 63) // 64
    q = _grid_values(orc, rng, (1, N, H, D))
    k = _grid_values(orc, rng, (1, N, H, D))
    v = _grid_values(orc, rng, (1, N, H, D))
    for b in range(NB):
        q[0, b * 64, :, 0] = 448.0
        k[0, b * 64 + 1 if b * 64 + 1 < N else b * 64, :, 1] = 448.0
    v[0, 0, :, :] = 448.0
    return q, k, v


@pytest.mark.parametrize("N,rev,S", [(130, False, 256.0), (200, True, 448.0), (64, True, 1.0)])
def test_fp8_on_exact_grid_equals_pcast(orc, N, rev, S):
    rng = np.random.default_rng(N)
    H = 2
    q, k, v = _exact_grid_inputs(orc, rng, N, H)
    qz = orc.quantize(_bf16(q), _bf16(k), _bf16(v))
    assert np.all(qz["q_scale"] == 1.0) and np.all(qz["k_scale"] == 1.0)
    assert np.all(qz["v_scale"] == 1.0)
    # codes decode back to the inputs, V stored token-contiguous
    N64 = qz["q8"].shape[2]
    assert np.array_equal(orc.e4m3_decode(qz["q8"][0, :, :N]), q[0].transpose(1, 0, 2))
    assert np.array_equal(orc.e4m3_decode(qz["v8t"][0, :, :, :N]), v[0].transpose(1, 2, 0))
    assert np.all(qz["q8"][0, :, N:] == 0) and np.all(qz["v8t"][0, :, :, N:] == 0)
    out, ob, _, _ = orc.attention_fp8(qz, p_scale=S, kv_reverse=rev)
    tr = lambda a: np.ascontiguousarray(a.transpose(0, 2, 1, 3))
    ref, _, _ = orc.attention_ref(orc.MODE_PCAST, tr(q), tr(k), tr(v), p_scale=S, kv_reverse=rev)
    assert np.max(np.abs(out - ref)) <= 1e-9 * np.max(np.abs(ref))
    assert np.array_equal(ob, orc.bf16_encode(out.astype(np.float32)))
    # per-channel V scale plumbing: scaling channel d by 2^j scales output channel d by 2^j
    j = rng.integers(-3, 4, size=128)
    qz2 = orc.quantize(_bf16(q), _bf16(k), _bf16(v * 2.0 ** j))
    assert np.array_equal(qz2["v8t"], qz["v8t"])
    out2, _, _, _ = orc.attention_fp8(qz2, p_scale=S, kv_reverse=rev)
    assert np.allclose(out2, out * 2.0 ** j, rtol=1e-12, atol=0)


def test_quantize_block_rules(orc):
    rng = np.random.default_rng(7)
    N, H, D = 150, 3, 128
    x = rng.standard_normal((1, N, H, D)).astype(np.float32) * 3
    x[0, 64:128, 1, :] = 0.0                              # an all-zero block
    xb = _bf16(x)
    qz = orc.quantize(xb, xb, xb)
    xf = orc.bf16_decode(xb)[0].transpose(1, 0, 2)       # [H, N, D]
    NB = 3
    for h in range(H):
        for b in range(NB):
            blk = xf[h, b * 64:min(N, b * 64 + 64)]
            amax = np.float32(np.abs(blk).max())
            assert qz["q_scale"][0, h, b] == np.float32(amax / np.float32(448.0))
            codes = qz["q8"][0, h, b * 64:b * 64 + blk.shape[0]]
            if amax == 0:
                assert np.all(codes == 0)
                continue
            deq = orc.e4m3_decode(codes) * qz["q_scale"][0, h, b]
            # RNE on E4M3: relative error <= 2^-4 in the normal range, abs 2^-10 below it
            err = np.abs(deq - blk)
            assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(blk), 2.0 ** -10 * amax / 448 * 1.01))
            # the block maximum maps to +-448
            i = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
            assert codes[i] & 0x7F == 0x7E
    assert np.all(qz["q8"][0, :, N:] == 0)               # tail rows of the last block
    # V: per channel over all tokens
    amax_v = np.abs(xf).max(axis=1).astype(np.float32)
    assert np.array_equal(qz["v_scale"][0], (amax_v / np.float32(448.0)).astype(np.float32))


def test_quantize_gather_equals_pregathered(orc):
    rng = np.random.default_rng(8)
    Nsrc, H, D = 120, 2, 128
    x = [rng.standard_normal((1, Nsrc, H, D)).astype(np.float32) for _ in range(3)]
    xb = [_bf16(a) for a in x]
    perm_q = rng.permutation(Nsrc + 20).astype(np.int32)
    perm_q = np.where(perm_q >= Nsrc, -1, perm_q).astype(np.int32)
    perm_kv = np.stack([rng.permutation(Nsrc + 20) for _ in range(H)])[None].astype(np.int32)
    perm_kv = np.where(perm_kv >= Nsrc, -1, perm_kv).astype(np.int32)
    qz = orc.quantize(*xb, perm_q=perm_q, perm_kv=perm_kv)

    def gather(a, p):                                     # p: [N] -> rows, -1 -> zero row
        keep = (p >= 0).reshape((-1,) + (1,) * (a.ndim - 1))
        return np.where(keep, a[np.maximum(p, 0)], 0).astype(np.uint16)

    qg = gather(xb[0][0], perm_q)[None]
    kg = np.stack([gather(xb[1][0][:, h], perm_kv[0, h]) for h in range(H)], axis=1)[None]
    vg = np.stack([gather(xb[2][0][:, h], perm_kv[0, h]) for h in range(H)], axis=1)[None]
    ref = orc.quantize(qg, kg, vg)
    for key in ("q8", "k8", "v8t", "q_scale", "k_scale", "v_scale"):
        assert np.array_equal(qz[key], ref[key]), key


def test_exact_attention_invariant_to_joint_key_permutation(orc):
    rng = np.random.default_rng(9)
    N, D = 256, 128
    q, k, v = (rng.standard_normal((1, 1, N, D)) for _ in range(3))
    p = rng.permutation(N)
    a, _, _ = orc.attention_ref(orc.MODE_EXACT, q, k, v)
    b, _, _ = orc.attention_ref(orc.MODE_EXACT, q, k[:, :, p], v[:, :, p])
    assert np.max(np.abs(a - b)) <= 1e-12


def test_vsmooth_constant_value_preserved_exactly(orc):
    # TeleFuser "输出验证": constant-value preservation; with V-Smooth R = 0, s_r = 0 and the
    # output is the stored mean, exactly.
    rng = np.random.default_rng(10)
    N, H, D = 300, 2, 128
    q, k = (rng.standard_normal((1, N, H, D)).astype(np.float32) for _ in range(2))
    c = rng.standard_normal(D).astype(np.float32) * 5
    v = np.broadcast_to(c, (1, N, H, D)).astype(np.float32)
    qz = orc.quantize(_bf16(q), _bf16(k), _bf16(v), vsmooth=True)
    assert np.all(qz["v_scale"] == 0) and np.all(qz["v8t"] == 0)
    for rev, ec in ((False, False), (True, True)):
        _, ob, _, _ = orc.attention_fp8(qz, kv_reverse=rev, expcast=ec)
        assert np.array_equal(ob, np.broadcast_to(_bf16(c), ob.shape))
    # without V-Smooth the plain FP8 path is only close
    qz0 = orc.quantize(_bf16(q), _bf16(k), _bf16(v))
    out0, _, _, _ = orc.attention_fp8(qz0)
    cb = orc.bf16_decode(_bf16(c))
    assert np.max(np.abs(out0 - cb)) <= 2e-2 * np.max(np.abs(cb))
    assert not np.array_equal(orc.bf16_encode(out0.astype(np.float32)), np.broadcast_to(_bf16(c), out0.shape))


def test_vsmooth_block_means_restore_exactly(orc):
    # V' = per-128-block constant means (zero residual): the rank-one restore alone must
    # reproduce the exact softmax average of the block means when Q, K quantise exactly.
    rng = np.random.default_rng(11)
    N, H, D = 320, 2, 128
    q, k, _ = _exact_grid_inputs(orc, rng, N, H)
    means = rng.standard_normal((3, H, D)).astype(np.float32)
    v = np.concatenate([np.broadcast_to(means[j], (min(128, N - 128 * j), H, D))
                        for j in range(3)])[None]
    vb = _bf16(v)
    qz = orc.quantize(_bf16(q), _bf16(k), vb, vsmooth=True)
    assert np.all(qz["v8t"] == 0)
    assert np.array_equal(qz["v_mean"][0].transpose(1, 0, 2), _bf16(means))
    tr = lambda a: np.ascontiguousarray(a.transpose(0, 2, 1, 3))
    vf = orc.bf16_decode(vb)
    for rev in (False, True):
        out, _, _, _ = orc.attention_fp8(qz, kv_reverse=rev)
        ex, _, _ = orc.attention_ref(orc.MODE_EXACT, tr(q), tr(k), tr(vf))
        assert np.max(np.abs(out - ex)) <= 1e-12 * np.max(np.abs(ex))


def test_vsmooth_means_and_residual_rules(orc):
    rng = np.random.default_rng(12)
    N, H, D = 200, 1, 128
    v = (rng.standard_normal((1, N, H, D)) * 2 + 3).astype(np.float32)
    vb = _bf16(v)
    perm = np.stack([rng.permutation(N)])[None].astype(np.int32)
    qz = orc.quantize(vb, vb, vb, perm_kv=perm, vsmooth=True)
    vp = orc.bf16_decode(vb)[0, perm[0, 0], 0]            # permuted V' [N, D]
    for j in range(2):
        blk = vp[j * 128:min(N, j * 128 + 128)]
        mean = (blk.sum(axis=0) / blk.shape[0]).astype(np.float32)
        assert np.array_equal(qz["v_mean"][0, 0, j], _bf16(mean))
    mhat = orc.bf16_decode(qz["v_mean"][0, 0])
    resid = (vp.astype(np.float32) - np.repeat(mhat, 128, axis=0)[:N].astype(np.float32))
    amax = np.abs(resid).max(axis=0).astype(np.float32)
    assert np.array_equal(qz["v_scale"][0, 0], amax / np.float32(448))
    # energy removed by the block means is positive on a shifted V
    assert (np.sum(np.repeat(mhat, 128, axis=0)[:N] ** 2) / np.sum(vp ** 2)) > 0.5


def test_expcast_codes(orc):
    # c = round(8 z + 56 + beta), z = log2(S p); with S = 256 and p = 1 the code is 120 (256.0)
    z = math.log2(256.0)
    assert int(np.rint(np.float32(8 * z + 56 - 0.35))) == 0x78
    # beta = -0.35 balances the linear approximation within a doubling (midrange of
    # 8(f + 1 - 2^f) over f in [0, 1) is max/2 = 0.344)
    f = np.linspace(0, 1, 100001)
    assert -0.5 * np.max(8 * (f + 1 - 2.0 ** f)) == pytest.approx(-0.35, abs=0.01)
    # in the normal range the ExpCast code is within one step of the RNE code of S p
    rng = np.random.default_rng(13)
    zz = rng.uniform(-6.0, 8.0, 2_000_000)
    c_exp = np.clip(np.rint((8 * zz + 56 - 0.35).astype(np.float32)), 0, 126)
    c_rne = orc.e4m3_encode(2.0 ** zz).astype(np.float64)
    assert np.max(np.abs(c_exp - c_rne)) <= 1
    assert 0.05 < np.mean(c_exp != c_rne) < 0.5


def test_expcast_total_variation_soft(orc):
    # VC-Attention 三: mean total variation between ExpCast and standard-cast probability rows
    # is 1.6 % on Wan2.2 rows; synthetic N(0,1) logit rows stay in the same range.
    rng = np.random.default_rng(14)
    x = rng.standard_normal((256, 4096))
    z = (x - x.max(axis=1, keepdims=True)) / math.log(2) + 8.0
    dec = orc.e4m3_decode
    c_exp = np.clip(np.rint((8 * z + 56 - 0.35).astype(np.float32)), 0, 126).astype(np.uint8)
    p_exp = dec(c_exp)
    p_std = dec(orc.e4m3_encode(2.0 ** z))
    p_exp /= p_exp.sum(axis=1, keepdims=True)
    p_std /= p_std.sum(axis=1, keepdims=True)
    tv = 0.5 * np.abs(p_exp - p_std).sum(axis=1).mean()
    assert 0.002 < tv < 0.025


def test_fp8_expcast_close_to_exact(orc):
    rng = np.random.default_rng(15)
    N, H, D = 256, 2, 128
    q, k, v = (rng.standard_normal((1, N, H, D)).astype(np.float32) for _ in range(3))
    qz = orc.quantize(_bf16(q), _bf16(k), _bf16(v))
    tr = lambda a: np.ascontiguousarray(orc.bf16_decode(_bf16(a)).transpose(0, 2, 1, 3))
    ex, _, _ = orc.attention_ref(orc.MODE_EXACT, tr(q), tr(k), tr(v))
    for ec in (False, True):
        out, _, _, _ = orc.attention_fp8(qz, expcast=ec)
        cos = np.sum(out * ex) / np.sqrt(np.sum(out ** 2) * np.sum(ex ** 2))
        assert cos > 0.995


def test_sparse_all_neighbours_close_to_exact(orc):
    T, Hg, W, tt, th, tw = 3, 5, 8, 2, 4, 8
    lay = orc.sta_layout(T, Hg, W, tt, th, tw, 1, 1, 0)
    full = orc.sta_layout(T, Hg, W, tt, th, tw, 9, 9, 9)
    assert np.array_equal(full["perm"], lay["perm"])
    rng = np.random.default_rng(16)
    n_src = T * Hg * W
    q, k, v = (rng.standard_normal((1, n_src, 2, 128)).astype(np.float32) for _ in range(3))
    perm = full["perm"]
    qz = orc.quantize(_bf16(q), _bf16(k), _bf16(v), perm_q=perm, perm_kv=perm)
    # with every tile a neighbour, the sparse FP8 path attends to all valid tokens
    for rev in (False, True):
        o_sp, ob_sp, _, rv = orc.attention_fp8(qz, kv_reverse=rev, sparse=full)
        tr = lambda a: np.ascontiguousarray(orc.bf16_decode(_bf16(a))[:, perm[perm >= 0]].transpose(0, 2, 1, 3))
        ex, _, _ = orc.attention_ref(orc.MODE_EXACT, tr(q), tr(k), tr(v))
        valid = rv[0, 0].astype(bool)
        assert valid.sum() == n_src
        cos = np.sum(o_sp[0][:, valid] * ex[0]) / np.sqrt(np.sum(o_sp[0][:, valid] ** 2) * np.sum(ex[0] ** 2))
        assert cos > 0.995


def test_vsmooth_perm_properties(orc):
    rng = np.random.default_rng(17)
    N, H, D = 600, 2, 128
    v = rng.standard_normal((1, N, H, D)).astype(np.float32)
    grp = rng.random(N) < 0.3                             # two groups far apart on 8 channels
    v[0, grp, :, 8:16] += 25.0
    vb = _bf16(v)
    perm, labels = orc.vsmooth_perm(vb, iters=60, return_labels=True)
    vf = orc.bf16_decode(vb)[0]
    for h in range(H):
        p, lab = perm[0, h], labels[0, h]
        assert np.array_equal(p, np.argsort(lab, kind="stable"))   # stable sort by cluster id
        for c in np.unique(lab):
            assert len(set(grp[lab == c])) == 1                    # clusters never mix groups
        # features: the 8 largest-variance channels (independent numpy computation)
        x = vf[:, h, :]
        feat = np.sort(np.argsort(-x.var(axis=0), kind="stable")[:8])
        assert set(feat) == set(range(8, 16))
        # Lloyd fixed point: every token is nearest to the mean of its own cluster
        f = x[:, feat]
        cent = np.stack([f[lab == c].mean(axis=0) for c in range(16) if np.any(lab == c)])
        ids = [c for c in range(16) if np.any(lab == c)]
        d2 = ((f[:, None, :] - cent[None]) ** 2).sum(axis=2)
        assert np.array_equal(np.array(ids)[d2.argmin(axis=1)], lab)


def test_ambiguity_bound_flags_a_midpoint(orc):
    # Two keys on exactly representable operands (all scales 1); the softmax scale puts S p of
    # the second key exactly on the midpoint 248 between the E4M3 values 240 and 256 (S = 256),
    # so either code is a correct FP32 outcome and the bound must cover one grid step.
    D = 128
    qb = np.zeros((1, 2, 1, D), np.float32)
    kb = np.zeros((1, 2, 1, D), np.float32)
    vb = np.zeros((1, 2, 1, D), np.float32)
    qb[0, :, 0, 0] = 448.0
    kb[0, 0, 0, 0] = 448.0
    kb[0, 1, 0, 0] = 416.0
    vb[0, 1, 0, :] = 448.0
    to = lambda a: torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    qz = orc.quantize(to(qb), to(kb), to(vb))
    x_gap = 448.0 * 32.0                                  # logit gap of the two keys, code units
    sc = -math.log(248.0 / 256.0) / x_gap                 # exp(-gap * sc) = 248 / 256
    rows = np.array([0], np.int32)
    _, _, _, _, amb = orc.attention_fp8(qz, rows=rows, softmax_scale=sc, return_amb=True)
    l = 1.0 + 248.0 / 256.0
    flip = 16.0 * 448.0 / (256.0 * l)                     # one grid step of key 2, |V_2| = 448
    # plus the matrix-core truncation allowance (2^-11 of the largest P8 V of the key group)
    assert flip <= amb[0, 0, 0].min() and amb[0, 0, 0].max() <= flip * 1.03
    _, _, _, _, amb2 = orc.attention_fp8(qz, rows=rows, softmax_scale=sc * 1.3, return_amb=True)
    assert amb2[0, 0, 0].max() < 0.03 * flip              # no ambiguous code: truncation only


def _expcast_model(orc, q, k, v, rev, S, scale, precast_l=False):
    """numpy, per row: 64-key blocks in KV order; m' = max(m, block max); the ExpCast byte
    c = clamp(rint(fl32(8 z + 56 - 0.35)), 0, 126) with z = (x - m') log2(e) + log2(S) (VC-Attention
    article section 三, S folded into z); l = exp(m - m') l + sum decode(c) / S; acc = exp(m - m')
    acc + decode(c) . V; O = acc / (S l). precast_l: l sums exp(x - m') instead (the standard
    cast's rule, which ExpCast has no FP32 value for)."""
    N = q.shape[0]
    NB = -(-N // 64)
    order = list(range(NB))[::-1] if rev else list(range(NB))
    x_all = (q @ k.T) * scale
    out = np.zeros_like(q)
    for i in range(N):
        m, l, acc = -np.inf, 0.0, np.zeros(q.shape[1])
        for kb in order:
            xs = x_all[i, kb * 64:min(N, kb * 64 + 64)]
            m_new = max(m, xs.max())
            alpha = 0.0 if m == -np.inf else math.exp(m - m_new)
            z = (xs - m_new) / math.log(2.0) + math.log2(S)
            c = np.clip(np.rint((8.0 * z + 56.0 - 0.35).astype(np.float32).astype(np.float64)), 0, 126)
            pd = orc.e4m3_decode(c.astype(np.uint8)).astype(np.float64)
            inc = np.exp(xs - m_new).sum() if precast_l else pd.sum() / S
            l = alpha * l + inc
            acc = alpha * acc + pd @ v[kb * 64:kb * 64 + len(xs)]
            m = m_new
        out[i] = acc / (S * l)
    return out


@pytest.mark.parametrize("N,rev,S", [(200, True, 256.0), (130, False, 448.0), (64, False, 256.0)])
def test_expcast_loop_matches_numpy_model(orc, N, rev, S):
    """The oracle's ExpCast path element by element against an independent model of the loop, on
    inputs where quantisation is the identity (all scales 1, so logits are exact). The row sum
    must be the sum of the decoded codes over S: summing the pre-cast exp(x - m) instead (as the
    standard cast does) gives a visibly different output."""
    rng = np.random.default_rng(300 + N)
    H = 2
    q, k, v = _exact_grid_inputs(orc, rng, N, H)
    qz = orc.quantize(_bf16(q), _bf16(k), _bf16(v))
    assert np.all(qz["q_scale"] == 1.0) and np.all(qz["k_scale"] == 1.0) and np.all(qz["v_scale"] == 1.0)
    scale = 1.0 / 256.0      # keeps the exact-grid logits in a range where many codes are non-zero
    out, _, _, _ = orc.attention_fp8(qz, softmax_scale=scale, p_scale=S, kv_reverse=rev, expcast=True)
    for h in range(H):
        want = _expcast_model(orc, q[0, :, h], k[0, :, h], v[0, :, h], rev, S, scale)
        assert np.max(np.abs(out[0, h] - want)) <= 1e-10 * np.max(np.abs(want))
        other = _expcast_model(orc, q[0, :, h], k[0, :, h], v[0, :, h], rev, S, scale, precast_l=True)
        assert np.max(np.abs(out[0, h] - other)) > 1e-3 * np.max(np.abs(want))
