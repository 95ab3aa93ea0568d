"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Bar: quantisation codes, scales and V-Smooth means bit-exact; attention outputs within
max-abs 1e-2 and rel-L2 5e-3 of the oracle's FP8-path output on the compared rows (cosine
against FP64 unquantised attention is checked >= 0.995 where the inputs are unstructured).
Small cases run every row across several tiles and ragged tails; the full-size workloads run
the same launch configuration as the benchmark and compare sampled rows of sampled heads.
"""
import math
import sys

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

ATOL, RTOL_L2, COS_MIN = 1e-2, 5e-3, 0.995


def say(*a):
    print("[gpu-parity]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_attention_video_qkv_amd as m
    m.lib()
    return m


DEV = "cuda:0"


def _bits(t):
    return workloads.bits(t)


def _np(t):
    return t.detach().cpu().numpy()


def _gpu_quantize(m, q, k, v, perm_q=None, perm_kv=None, vsmooth=False, n_layout=None,
                  smoothing=0, bias=False):
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    pq = None if perm_q is None else torch.from_numpy(np.ascontiguousarray(perm_q)).to(DEV)
    pkv = None if perm_kv is None else torch.from_numpy(np.ascontiguousarray(perm_kv)).to(DEV)
    qz = m.quantize_qkv(qd, kd, vd, perm_q=pq, perm_kv=pkv, vsmooth=vsmooth, n_layout=n_layout,
                        smoothing=smoothing, v_bias_correction=bias)
    torch.cuda.synchronize()
    return qz


def _compare_quant(qz, ref):
    assert np.array_equal(_np(qz.q8), ref["q8"]), "q8"
    assert np.array_equal(_np(qz.k8), ref["k8"]), "k8"
    assert np.array_equal(_np(qz.v8t), ref["v8t"]), "v8t"
    for key in ("q_scale", "k_scale", "v_scale"):
        assert np.array_equal(_np(getattr(qz, key)).view(np.uint32), ref[key].view(np.uint32)), key
    if ref.get("v_mean") is not None:
        assert np.array_equal(_np(qz.v_mean).view(np.uint16), ref["v_mean"]), "v_mean"
    if ref.get("v_shift") is not None:
        assert np.array_equal(_np(qz.v_shift).view(np.uint32), ref["v_shift"].view(np.uint32)), "v_shift"
    else:
        assert qz.v_shift is None


def _compare_out(gpu_rows, ref_rows, what, amb=None, peaked=False, wide=False):
    """gpu_rows (BF16 values), ref_rows: [B, H, R, D] float64 over the compared rows (the
    oracle's FP8-path output before its BF16 rounding).

    Default: every element within max-abs 1e-2 of the oracle and rel-L2 <= 5e-3, no allowance.
    Two documented exceptions, each printing how many elements needed it:
      wide    inputs whose outputs reach |O| >= 2 (channel offsets, token outliers): there the
              BF16 output grid is coarser than the bar (one step is 2^-6 for |O| in [2, 4)), so
              an element may exceed 1e-2 by half a BF16 step of its value, 2^-8 |O|;
      peaked  rows dominated by a few keys (attention sinks, outlier channels): one P code sits
              next to a rounding boundary within the device's evaluation error and decides a
              visible part of the output, so an element may exceed 1e-2 by what flipping the
              codes the oracle flags as ambiguous (each to its one neighbouring code) changes.
    rel-L2 is never given an allowance."""
    diff = np.abs(gpu_rows - ref_rows)
    allow = np.zeros(diff.shape)
    if wide:
        allow = allow + 2.0 ** -8 * np.abs(ref_rows)
    if peaked:
        assert amb is not None
        allow = allow + amb
    max_all = float(diff.max()) if diff.size else 0.0
    over = diff > ATOL
    rel = float(np.linalg.norm(gpu_rows - ref_rows) / max(np.linalg.norm(ref_rows), 1e-30))
    excess = diff - (ATOL + allow)
    note = ""
    if wide:
        # elements above the bar whose GPU value is exactly the oracle's value rounded to BF16
        ref_bf16 = torch.from_numpy(ref_rows.astype(np.float32)).to(torch.bfloat16).double().numpy()
        note += (f" (|O| max {float(np.abs(ref_rows).max()):.2f}; half BF16 step allowed; "
                 f"{int((over & (gpu_rows == ref_bf16)).sum())} of them equal the oracle rounded to BF16)")
    if peaked:
        note += f" (ambiguous-code allowance: median {float(np.median(amb)):.2e})"
    say(f"{what}: max_abs {max_all:.3e}, rel_l2 {rel:.3e}, {int(over.sum())} of {diff.size} elements "
        f"above 1e-2" + note)
    if not (wide or peaked):
        assert max_all <= ATOL, (what, max_all)
    assert np.all(excess <= 0), (what, float(excess.max()))
    assert rel <= RTOL_L2, (what, rel)
    return max_all, rel


def _cos(a, b):
    return float(np.sum(a * b) / math.sqrt(np.sum(a * a) * np.sum(b * b)))


def _gpu_rows(out, rows):
    """GPU out [B, N, H, D] bf16 -> [B, H, R, D] float64 at the given source rows."""
    o = out.float().cpu().numpy()[:, rows]
    return np.ascontiguousarray(o.transpose(0, 2, 1, 3)).astype(np.float64)


# ------------------------------------------------------------------------------------------
# Quantisation: bit-exact
# ------------------------------------------------------------------------------------------
QUANT_CASES = [
    ("dense512", dict(B=1, N=512, H=2, seed=1)),
    ("ragged1000", dict(B=1, N=1000, H=3, seed=2)),
    ("tiny37", dict(B=2, N=37, H=1, seed=3)),
]


@pytest.mark.parametrize("name,c", QUANT_CASES)
@pytest.mark.parametrize("vsmooth", [False, True])
def test_quantize_bit_exact(m, orc, name, c, vsmooth):
    say("quantize", name, "vsmooth", vsmooth)
    q, k, v = workloads.make_qkv(c["B"], c["N"], c["H"], c["seed"], kind="channel_outliers")
    ref = orc.quantize(_bits(q), _bits(k), _bits(v), vsmooth=vsmooth)
    qz = _gpu_quantize(m, q, k, v, vsmooth=vsmooth)
    _compare_quant(qz, ref)


@pytest.mark.parametrize("per_head", [False, True])
@pytest.mark.parametrize("N", [384, 350])
def test_quantize_gather_bit_exact(m, orc, per_head, N):
    """Permutations with entries past the source (padding rows); N = 350 also leaves layout
    positions past N inside the last 64- and 128-row blocks."""
    say("quantize gather, per_head", per_head, "N", N)
    rng = np.random.default_rng(5)
    Nsrc, H = 300, 2
    q, k, v = workloads.make_qkv(1, Nsrc, H, 7, kind="token_outliers")
    perm_q = rng.permutation(N).astype(np.int32)
    perm_q = np.where(perm_q >= Nsrc, -1, perm_q).astype(np.int32)
    if per_head:
        pkv = np.stack([rng.permutation(N) for _ in range(H)])[None].astype(np.int32)
    else:
        pkv = rng.permutation(N).astype(np.int32)
    pkv = np.where(pkv >= Nsrc, -1, pkv).astype(np.int32)
    for vs in (False, True):
        ref = orc.quantize(_bits(q), _bits(k), _bits(v), perm_q=perm_q, perm_kv=pkv, vsmooth=vs)
        qz = _gpu_quantize(m, q, k, v, perm_q=perm_q, perm_kv=pkv, vsmooth=vs, n_layout=N)
        _compare_quant(qz, ref)


def test_quantize_encoder_boundaries(m, orc):
    """Every Q/K block holds 448 so its scale is 1 and codes are E4M3(x) itself: the values sit
    on and around every rounding boundary of the E4M3 grid (the device conversion against
    the oracle's round-to-nearest-even)."""
    say("quantize boundaries")
    grid = orc.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = (grid[:-1] + grid[1:]) / 2
    vals = np.concatenate([grid, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9)])
    vals = torch.tensor(np.concatenate([vals, -vals]), dtype=torch.float32)
    # keep only values exactly representable in bf16 (the inputs are bf16)
    vals = vals[vals.to(torch.bfloat16).float() == vals]
    n_per_row = 127
    rows = -(-vals.numel() // n_per_row)
    N = ((rows + 63) // 64) * 64
    x = torch.zeros((1, N, 1, 128), dtype=torch.float32)
    flat = torch.zeros(N * n_per_row)
    flat[: vals.numel()] = vals
    x[0, :, 0, 1:] = flat.view(N, n_per_row)
    x[0, :, 0, 0] = 448.0
    xb = x.to(torch.bfloat16)
    ref = orc.quantize(_bits(xb), _bits(xb), _bits(xb))
    assert np.all(ref["q_scale"] == 1.0)
    qz = _gpu_quantize(m, xb, xb, xb)
    _compare_quant(qz, ref)


# ------------------------------------------------------------------------------------------
# Attention: small cases, every row
# ------------------------------------------------------------------------------------------
def _run_attn(m, qz, **kw):
    out = m.forward(qz, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("N,H,reverse,S", [
    (512, 2, True, 256.0), (512, 2, False, 256.0), (512, 2, False, 1.0), (512, 2, True, 448.0),
    (1000, 3, True, 256.0), (1000, 3, False, 448.0), (37, 2, False, 256.0), (64, 1, True, 1.0),
    (2500, 2, False, 256.0), (1, 2, True, 256.0), (65, 2, False, 256.0), (65, 1, True, 448.0)])
def test_attention_dense_small(m, orc, N, H, reverse, S):
    say("dense", N, H, "reverse" if reverse else "forward", S)
    q, k, v = workloads.make_qkv(1, N, H, seed=N + H)
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    ref_q = orc.quantize(qb, kb, vb)
    ref, _, _, _, amb = orc.attention_fp8(ref_q, p_scale=S, kv_reverse=reverse, return_amb=True)
    qz = _gpu_quantize(m, q, k, v)
    out = _run_attn(m, qz, p_scale=S, kv_order=int(reverse))
    got = _gpu_rows(out, np.arange(N))
    _compare_out(got, ref, f"dense N={N}", amb)
    tr = lambda a: np.ascontiguousarray(orc.bf16_decode(a).transpose(0, 2, 1, 3))
    ex, _, _ = orc.attention_ref(orc.MODE_EXACT, tr(qb), tr(kb), tr(vb))
    c = _cos(got, ex)
    say(f"cosine vs FP64 exact {c:.6f}")
    assert c >= COS_MIN


@pytest.mark.parametrize("N,reverse", [(512, True), (1000, False), (1, True), (65, False)])
def test_attention_expcast_small(m, orc, N, reverse):
    say("expcast", N, reverse)
    q, k, v = workloads.make_qkv(1, N, 2, seed=11 + N)
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    ref, _, _, _, amb = orc.attention_fp8(orc.quantize(qb, kb, vb), kv_reverse=reverse,
                                          expcast=True, return_amb=True)
    qz = _gpu_quantize(m, q, k, v)
    out = _run_attn(m, qz, kv_order=int(reverse), pcast=m.FP8ATTN_PCAST_EXPCAST)
    _compare_out(_gpu_rows(out, np.arange(N)), ref, "expcast", amb)


@pytest.mark.parametrize("S", [256.0, 448.0])
def test_attention_expcast_extreme_logits(m, orc, S):
    """ExpCast with Q and K scaled by 48 (logits of order 1e4 in log2 units). This is outside the
    range where element-wise parity is claimed: the E4M3 matrix core's accumulation error on a
    logit (below 2^-11 of the summed group maxima of the products) is then worth several code
    steps, so the codes of the device and of the exact oracle differ by more than one step. What
    is claimed there: the output is finite (no byte 0x7F, E4M3 NaN, ever reaches the PV) and it
    stays within rel-L2 5e-3 of the oracle (the rows are nearly one-hot, and the dominant keys
    agree)."""
    say("expcast extreme logits", S)
    N, H = 640, 2
    q, k, v = workloads.make_qkv(1, N, H, seed=77)
    q = (q.float() * 48.0).to(torch.bfloat16)
    k = (k.float() * 48.0).to(torch.bfloat16)
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    ref, _, _, _ = orc.attention_fp8(orc.quantize(qb, kb, vb), p_scale=S, kv_reverse=True, expcast=True)
    qz = _gpu_quantize(m, q, k, v)
    out = _run_attn(m, qz, p_scale=S, kv_order=1, pcast=m.FP8ATTN_PCAST_EXPCAST)
    assert torch.isfinite(out.float()).all()
    got = _gpu_rows(out, np.arange(N))
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    say(f"expcast extreme S={S}: max_abs {float(np.abs(got - ref).max()):.3e} (no element-wise claim), "
        f"rel_l2 {rel:.3e}")
    assert rel <= RTOL_L2


@pytest.mark.parametrize("S", [256.0, 448.0])
def test_attention_expcast_clamped_top_code(m, orc, S):
    """Logits of order 1e6 in log2 units (Q and K scaled by 1024): the FP32 rounding of the
    per-block bias can then carry the byte of a row's maximum past 126.5, which would round to
    0x7F (E4M3 NaN); such blocks clamp every byte at 126. The output must be finite and every
    row must be a convex combination of the dequantised V rows, whatever the codes: each output
    channel lies within the range of that channel's V values widened by the E4M3 rounding of V
    (2^-4 of the channel maximum) and the BF16 output rounding."""
    say("expcast clamped top code", S)
    N, H = 640, 2
    q, k, v = workloads.make_qkv(1, N, H, seed=78)
    q = (q.float() * 1024.0).to(torch.bfloat16)
    k = (k.float() * 1024.0).to(torch.bfloat16)
    qz = _gpu_quantize(m, q, k, v)
    for rev in (0, 1):
        out = _run_attn(m, qz, p_scale=S, kv_order=rev, pcast=m.FP8ATTN_PCAST_EXPCAST).float()
        assert torch.isfinite(out).all()
        vf = v.float().to(DEV)
        vmax, vmin = vf.amax(dim=1, keepdim=True), vf.amin(dim=1, keepdim=True)
        slack = 2.0 ** -4 * vf.abs().amax(dim=1, keepdim=True) + 2.0 ** -8 * vf.abs().amax()
        assert torch.all(out <= vmax + slack) and torch.all(out >= vmin - slack)


@pytest.mark.parametrize("N,reverse,expcast", [(1000, True, False), (768, False, True),
                                               (300, False, False), (300, True, True),
                                               (1100, True, True), (1100, False, False)])
def test_attention_vsmooth_small(m, orc, N, reverse, expcast):
    """V-Smooth against the oracle. The restore runs per group of four 128-row V blocks (eight
    key blocks): the sizes cover an odd block count (300: 5 blocks, one partial group) and a
    group cut by the sequence end in both orders (1100: 18 blocks, groups of 8, 8 and 2)."""
    say("vsmooth", N, reverse, expcast)
    H = 2
    q, k, v = workloads.make_qkv(1, N, H, seed=21 + N, kind="token_outliers")
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    perm = orc.vsmooth_perm(vb)                         # [1, H, N], an input to both sides
    ref_q = orc.quantize(qb, kb, vb, perm_kv=perm, vsmooth=True)
    ref, _, _, _, amb = orc.attention_fp8(ref_q, kv_reverse=reverse, expcast=expcast,
                                          return_amb=True)
    qz = _gpu_quantize(m, q, k, v, perm_kv=perm, vsmooth=True)
    _compare_quant(qz, ref_q)
    out = _run_attn(m, qz, kv_order=int(reverse),
                    pcast=m.FP8ATTN_PCAST_EXPCAST if expcast else m.FP8ATTN_PCAST_RNE)
    _compare_out(_gpu_rows(out, np.arange(N)), ref, "vsmooth", amb, peaked=True, wide=True)


def test_vsmooth_constant_value_exact(m, orc):
    say("vsmooth constant")
    N, H = 700, 2
    q, k, _ = workloads.make_qkv(1, N, H, seed=31)
    c = torch.randn(128, generator=torch.Generator().manual_seed(3)) * 4
    v = c.view(1, 1, 1, 128).expand(1, N, H, 128).contiguous().to(torch.bfloat16)
    qz = _gpu_quantize(m, q, k, v, vsmooth=True)
    for rev, pc in ((True, 0), (False, 1)):
        out = _run_attn(m, qz, kv_order=int(rev), pcast=pc)
        want = v.to(DEV)
        assert torch.equal(out.view(torch.int16), want.view(torch.int16))


def _sparse_case(m, orc, grid, H, seed, reverse, expcast=False, smoothing=0, bias=False):
    T, Hg, W, tt, th, tw, rt, rh, rw = grid
    lay = orc.sta_layout(*grid)
    perm = lay["perm"]
    n_src = T * Hg * W
    q, k, v = workloads.make_qkv(1, n_src, H, seed=seed,
                                 kind="channel_offset" if smoothing else "normal")
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    ref_q = orc.quantize(qb, kb, vb, perm_q=perm, perm_kv=perm, smoothing=smoothing,
                         v_bias_correction=bias)
    ref, _, _, rv, amb = orc.attention_fp8(ref_q, kv_reverse=reverse, expcast=expcast, sparse=lay,
                                           return_amb=True)
    qz = _gpu_quantize(m, q, k, v, perm_q=perm, perm_kv=perm, smoothing=smoothing, bias=bias)
    _compare_quant(qz, ref_q)
    sp = m.sparse_to_device(m.sta_build(*grid), DEV)
    out_rows = torch.from_numpy(perm).to(DEV)
    out = _run_attn(m, qz, kv_order=int(reverse), sparse=sp, out_rows=out_rows, n_out=n_src,
                    pcast=m.FP8ATTN_PCAST_EXPCAST if expcast else m.FP8ATTN_PCAST_RNE)
    valid = perm >= 0
    got = _gpu_rows(out, perm[valid])                    # GPU wrote O in source order
    assert np.all(rv[0, 0][valid] == 1)
    _compare_out(got, ref[:, :, valid], f"sparse {grid[:3]}", amb[:, :, valid], wide=smoothing > 0)


@pytest.mark.parametrize("reverse", [False, True])
def test_attention_sparse_small(m, orc, reverse):
    say("sparse (10,20,20) tiles (6,8,8)", reverse)
    _sparse_case(m, orc, (10, 20, 20, 6, 8, 8, 1, 1, 1), H=2, seed=41, reverse=reverse)


def test_attention_sparse_expcast_and_odd_tiles(m, orc):
    say("sparse expcast; 64-token tiles")
    _sparse_case(m, orc, (10, 20, 20, 6, 8, 8, 1, 1, 1), H=1, seed=42, reverse=True, expcast=True)
    _sparse_case(m, orc, (5, 7, 9, 2, 4, 8, 1, 1, 0), H=2, seed=43, reverse=False)
    _sparse_case(m, orc, (9, 10, 11, 3, 8, 8, 1, 0, 1), H=1, seed=44, reverse=True)


# ------------------------------------------------------------------------------------------
# Sequence-mean smoothing (K, K+V, K+V with the V bias correction)
# ------------------------------------------------------------------------------------------
SMOOTH_MODES = [(1, False), (2, False), (2, True)]


@pytest.mark.parametrize("smoothing,bias", SMOOTH_MODES)
@pytest.mark.parametrize("B,N,H,seed", [(1, 1000, 3, 51), (2, 37, 1, 52), (1, 8256, 2, 53),
                                         (1, 16448, 1, 57)])
def test_quantize_smoothing_bit_exact(m, orc, smoothing, bias, B, N, H, seed):
    """Codes, scales and v_shift bit-exact: the means use one fixed FP32 summation order on
    both sides (N = 8256 gives 129 64-row blocks, an odd tree level; N = 16448 gives 257
    blocks, more than one 256-node group of the device's tree passes)."""
    say("quantize smoothing", smoothing, bias, B, N, H)
    q, k, v = workloads.make_qkv(B, N, H, seed, kind="channel_offset")
    ref = orc.quantize(_bits(q), _bits(k), _bits(v), smoothing=smoothing, v_bias_correction=bias)
    qz = _gpu_quantize(m, q, k, v, smoothing=smoothing, bias=bias)
    _compare_quant(qz, ref)


@pytest.mark.parametrize("per_head", [False, True])
def test_quantize_smoothing_gather_bit_exact(m, orc, per_head):
    """Padding positions (-1) are left out of every mean and stay code 0."""
    say("quantize smoothing gather, per_head", per_head)
    rng = np.random.default_rng(54)
    Nsrc, N, H = 700, 900, 2
    q, k, v = workloads.make_qkv(1, Nsrc, H, 55, kind="channel_offset")
    perm_q = np.where(np.arange(N) < Nsrc, np.arange(N), -1).astype(np.int32)
    if per_head:
        pkv = np.stack([rng.permutation(N) for _ in range(H)])[None]
    else:
        pkv = rng.permutation(N)
    pkv = np.where(pkv >= Nsrc, -1, pkv).astype(np.int32)
    for smoothing, bias in SMOOTH_MODES:
        ref = orc.quantize(_bits(q), _bits(k), _bits(v), perm_q=perm_q, perm_kv=pkv,
                           smoothing=smoothing, v_bias_correction=bias)
        qz = _gpu_quantize(m, q, k, v, perm_q=perm_q, perm_kv=pkv, n_layout=N,
                           smoothing=smoothing, bias=bias)
        _compare_quant(qz, ref)


def test_quantize_smoothing_all_padding_head(m, orc):
    """A layout whose K/V positions are all padding: means 0, scales 0, codes 0, v_shift 0."""
    say("quantize smoothing, all padding")
    q, k, v = workloads.make_qkv(1, 64, 1, 56, kind="channel_offset")
    pkv = np.full(128, -1, np.int32)
    pq = np.arange(128, dtype=np.int32) % 64
    ref = orc.quantize(_bits(q), _bits(k), _bits(v), perm_q=pq, perm_kv=pkv, smoothing=2,
                       v_bias_correction=True)
    assert np.all(ref["v_shift"] == 0)
    qz = _gpu_quantize(m, q, k, v, perm_q=pq, perm_kv=pkv, n_layout=128, smoothing=2, bias=True)
    _compare_quant(qz, ref)


@pytest.mark.parametrize("N,smoothing,bias,reverse,expcast", [
    (1000, 2, True, True, False), (777, 1, False, False, False), (512, 2, False, True, True),
    (2500, 2, True, False, False)])
def test_attention_smoothing_small(m, orc, N, smoothing, bias, reverse, expcast):
    say("attention smoothing", N, smoothing, bias, reverse, expcast)
    H = 2
    q, k, v = workloads.make_qkv(1, N, H, seed=60 + N, kind="channel_offset")
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    ref_q = orc.quantize(qb, kb, vb, smoothing=smoothing, v_bias_correction=bias)
    ref, _, _, _, amb = orc.attention_fp8(ref_q, kv_reverse=reverse, expcast=expcast,
                                          return_amb=True)
    qz = _gpu_quantize(m, q, k, v, smoothing=smoothing, bias=bias)
    _compare_quant(qz, ref_q)
    out = _run_attn(m, qz, kv_order=int(reverse),
                    pcast=m.FP8ATTN_PCAST_EXPCAST if expcast else m.FP8ATTN_PCAST_RNE)
    got = _gpu_rows(out, np.arange(N))
    _compare_out(got, ref, f"smoothing {smoothing} bias {bias}", amb, wide=True)
    tr = lambda a: np.ascontiguousarray(orc.bf16_decode(a).transpose(0, 2, 1, 3))
    ex, _, _ = orc.attention_ref(orc.MODE_EXACT, tr(qb), tr(kb), tr(vb))
    c = _cos(got, ex)
    say(f"cosine vs FP64 exact {c:.6f}")
    assert c >= COS_MIN


def test_attention_smoothing_sparse(m, orc):
    say("sparse + smoothing")
    _sparse_case(m, orc, (10, 20, 20, 6, 8, 8, 1, 1, 1), H=2, seed=61, reverse=True, smoothing=2,
                 bias=True)
    _sparse_case(m, orc, (5, 7, 9, 2, 4, 8, 1, 1, 0), H=1, seed=62, reverse=False, smoothing=1)


# ------------------------------------------------------------------------------------------
# Split-KV (pieces of the key sequence merged by log-sum-exp)
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("N,H,splits,reverse,expcast", [
    (1000, 2, 2, True, False), (2500, 2, 3, False, False), (300, 1, 2, True, False),
    (4096, 8, 4, True, False), (777, 2, 16, False, True), (64, 1, 2, True, False)])
def test_attention_split_kv_small(m, orc, N, H, splits, reverse, expcast):
    say("split-KV", N, H, splits, reverse, expcast)
    q, k, v = workloads.make_qkv(1, N, H, seed=70 + N + splits)
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    ref_q = orc.quantize(qb, kb, vb)
    ref, _, _, _, amb = orc.attention_fp8(ref_q, kv_reverse=reverse, expcast=expcast,
                                          return_amb=True, kv_splits=splits)
    qz = _gpu_quantize(m, q, k, v)
    out = _run_attn(m, qz, kv_order=int(reverse), kv_splits=splits,
                    pcast=m.FP8ATTN_PCAST_EXPCAST if expcast else m.FP8ATTN_PCAST_RNE)
    _compare_out(_gpu_rows(out, np.arange(N)), ref, f"split-KV {splits}", amb)


def test_attention_split_kv_vsmooth_and_smoothing(m, orc):
    """V-Smooth: every piece holds whole 128-row V blocks (odd block counts included); sequence
    mean smoothing: v_shift is added after the merge."""
    say("split-KV + V-Smooth, + smoothing")
    N, H = 1000, 2
    q, k, v = workloads.make_qkv(1, N, H, seed=81, kind="token_outliers")
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    perm = orc.vsmooth_perm(vb)
    ref_q = orc.quantize(qb, kb, vb, perm_kv=perm, vsmooth=True)
    for splits, rev in ((3, True), (2, False)):
        ref, _, _, _, amb = orc.attention_fp8(ref_q, kv_reverse=rev, expcast=True, return_amb=True,
                                              kv_splits=splits)
        qz = _gpu_quantize(m, q, k, v, perm_kv=perm, vsmooth=True)
        out = _run_attn(m, qz, kv_order=int(rev), kv_splits=splits, pcast=m.FP8ATTN_PCAST_EXPCAST)
        _compare_out(_gpu_rows(out, np.arange(N)), ref, f"split-KV {splits} vsmooth", amb, peaked=True,
                     wide=True)
    q, k, v = workloads.make_qkv(1, N, H, seed=82, kind="channel_offset")
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    ref_q = orc.quantize(qb, kb, vb, smoothing=2, v_bias_correction=True)
    ref, _, _, _, amb = orc.attention_fp8(ref_q, kv_reverse=True, return_amb=True, kv_splits=2)
    qz = _gpu_quantize(m, q, k, v, smoothing=2, bias=True)
    out = _run_attn(m, qz, kv_order=1, kv_splits=2)
    _compare_out(_gpu_rows(out, np.arange(N)), ref, "split-KV 2 smoothing", amb, wide=True)


def _auto_splits(m, B, N, H):
    """The documented AUTO policy, evaluated here from the device's compute-unit count."""
    slots = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    base = B * H * -(-N // 128)
    last = base % slots
    if -(-N // 64) >= 256:
        if base < slots:
            return min(8, -(-slots // base))
        if base < 4 * slots and 0 < last and 20 * last <= 7 * slots:
            return 3
    return 1


def test_attention_split_kv_auto(m, orc):
    """A long sequence with few heads (H=2, N=20000) fills under one round of the machine, so
    AUTO splits it; sampled rows against the oracle with the same piece count. The sink-stress
    shape (N=4096) stays whole."""
    assert _auto_splits(m, 1, 4096, 8) == 1
    N, H = 20000, 2
    splits = _auto_splits(m, 1, N, H)
    say("split-KV auto on H=2 N=20000:", splits, "pieces")
    assert splits > 1
    q, k, v = workloads.make_qkv(1, N, H, seed=83, kind="channel_outliers")
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    ref_q = orc.quantize(qb, kb, vb)
    rows = workloads.sample_rows(N, 200, seed=9)
    ref, _, _, _, amb = orc.attention_fp8(ref_q, rows=rows, kv_reverse=True, return_amb=True,
                                          kv_splits=splits)
    qz = _gpu_quantize(m, q, k, v)
    out = _run_attn(m, qz, kv_order=1, kv_splits=m.FP8ATTN_KV_SPLITS_AUTO)
    _compare_out(_gpu_rows(out, rows), ref, "auto split", amb, peaked=True, wide=True)


@pytest.mark.parametrize("delta,S,reverse", [(9, 256.0, False), (7, 1.0, True)])
def test_attention_split_kv_sink_underflow(m, orc, delta, S, reverse):
    """Sink stress (H=8, N=4096) in 4 pieces: outputs and underflow counts against the oracle."""
    q, k, v = workloads.workload("sink4096", delta=delta)
    B, N, H, _ = q.shape
    splits = 4
    say("split-KV on sink4096:", splits, "pieces")
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    ref_q = orc.quantize(qb, kb, vb)
    ref, _, uf, _, amb = orc.attention_fp8(ref_q, p_scale=S, kv_reverse=reverse, return_amb=True,
                                           kv_splits=splits)
    qz = _gpu_quantize(m, q, k, v)
    cnt = torch.zeros(H, dtype=torch.int64, device=DEV)
    out = _run_attn(m, qz, p_scale=S, kv_order=int(reverse), underflow=cnt, kv_splits=splits)
    _compare_out(_gpu_rows(out, np.arange(N)), ref, "sink split", amb, peaked=True)
    g = _np(cnt).astype(np.float64)
    o = uf.sum(axis=2)[0].astype(np.float64)
    say("underflow gpu", g, "oracle", o)
    assert np.all(np.abs(g - o) <= 1e-4 * N * N + 1e-3 * o)


# ------------------------------------------------------------------------------------------
# Sol routing (exact / summary routes chosen per 64-token Q block)
# ------------------------------------------------------------------------------------------
def _check_route_mask(orc, gpu_words, ref, NB):
    """Every bit the oracle decides beyond the device's evaluation error must match; flagged
    (ambiguous) bits may go either way. Returns the device mask as the oracle's uint64 words."""
    words = np.ascontiguousarray(gpu_words).view(np.uint64)
    g = orc.mask_bits(words, NB)
    r = orc.mask_bits(ref["mask"], NB)
    a = orc.mask_bits(ref["amb_mask"], NB)
    bad = (g != r) & ~a
    say(f"route: {g.mean():.3f} of blocks exact, {int(a.sum())} ambiguous, "
        f"{int(((g != r) & a).sum())} decided the other way, {int(bad.sum())} wrong")
    assert not bad.any()
    return words


@pytest.mark.parametrize("N,H,tau,est,sinks,reverse,expcast", [
    (1000, 2, 2.0, 0, 1, True, False), (2500, 2, 3.0, 1, 2, False, False),
    (300, 1, 1.0, 1, 0, True, False), (777, 2, 2.5, 0, 1, True, True),
    (4160, 2, 3.0, 0, 1, True, False), (1000, 2, -50.0, 0, 0, True, False),
    (1000, 2, 50.0, 0, 0, False, False)])
def test_sol_small(m, orc, N, H, tau, est, sinks, reverse, expcast):
    say("sol", N, H, tau, est, sinks, reverse, expcast)
    q, k, v = workloads.make_qkv(1, N, H, seed=90 + N, kind="channel_outliers")
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    ref_q = orc.quantize(qb, kb, vb)
    ref_sol = orc.sol_prepare(ref_q, tau=tau, estimator=est, sink_blocks=sinks)
    qz = _gpu_quantize(m, q, k, v)
    out, mask = m.sol_forward(qz, tau=tau, estimator=est, sink_blocks=sinks, kv_order=int(reverse),
                              pcast=m.FP8ATTN_PCAST_EXPCAST if expcast else m.FP8ATTN_PCAST_RNE,
                              return_mask=True)
    torch.cuda.synchronize()
    NB = -(-N // 64)
    sol = dict(ref_sol)
    sol["mask"] = _check_route_mask(orc, _np(mask), ref_sol, NB)
    ref, _, _, _, amb = orc.attention_fp8(ref_q, kv_reverse=reverse, expcast=expcast,
                                          return_amb=True, sol=sol)
    _compare_out(_gpu_rows(out, np.arange(N)), ref, f"sol tau={tau}", amb, peaked=True, wide=True)


@pytest.mark.parametrize("N,tau,est,reverse,expcast", [
    (1000, 1.0, 0, True, False), (2500, 2.0, 1, False, False), (4500, 1.5, 0, True, False),
    (777, 1.0, 1, False, True), (4160, 2.5, 0, True, True)])
def test_sol_unstructured(m, orc, N, tau, est, reverse, expcast):
    """Sol on N(0,1) inputs, at the plain bar (max-abs 1e-2, no allowance): route masks with a
    large share of summary blocks, one and two route groups."""
    H = 2
    say("sol unstructured", N, tau, est, reverse, expcast)
    q, k, v = workloads.make_qkv(1, N, H, seed=150 + N)
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    ref_q = orc.quantize(qb, kb, vb)
    ref_sol = orc.sol_prepare(ref_q, tau=tau, estimator=est, sink_blocks=1)
    qz = _gpu_quantize(m, q, k, v)
    out, mask = m.sol_forward(qz, tau=tau, estimator=est, sink_blocks=1, kv_order=int(reverse),
                              pcast=m.FP8ATTN_PCAST_EXPCAST if expcast else m.FP8ATTN_PCAST_RNE,
                              return_mask=True)
    torch.cuda.synchronize()
    sol = dict(ref_sol)
    sol["mask"] = _check_route_mask(orc, _np(mask), ref_sol, -(-N // 64))
    ref, _, _, _, amb = orc.attention_fp8(ref_q, kv_reverse=reverse, expcast=expcast, return_amb=True,
                                          sol=sol)
    _compare_out(_gpu_rows(out, np.arange(N)), ref, f"sol unstructured tau={tau}", amb)


@pytest.mark.parametrize("reverse,expcast", [(False, False), (True, False), (False, True)])
def test_sol_shared_state(m, orc, reverse, expcast):
    """Both routes in one online-softmax state. The one-key tail block (a summary block) scores
    about 7 above every other key and shares the route group with the exact sink blocks 0 and 1
    (V = 4 there, S = 1), so the sinks' P codes are taken against the running max that summary
    sets, and many underflow. Device against the oracle; the reading with two states merged by
    log-sum-exp fails the same comparison on sampled rows by a wide margin."""
    from test_oracle_sol import _sol_model
    N, H, S, delta = 641, 2, 1.0, 7.0
    say("sol shared state", reverse, expcast)
    q, k, v = workloads.make_qkv(1, N, H, 64)
    q, k, v = q.float(), k.float(), v.float()
    q[..., 127] = 4.0
    k[..., 127] = 0.0
    k[:, N - 1, :, 127] = delta * math.sqrt(128.0) / 4.0
    v[:, :128] = 4.0
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    ref_q = orc.quantize(qb, kb, vb)
    ref_sol = orc.sol_prepare(ref_q, tau=50.0, estimator=0, sink_blocks=2)
    qz = _gpu_quantize(m, q, k, v)
    _compare_quant(qz, ref_q)
    out, mask = m.sol_forward(qz, tau=50.0, sink_blocks=2, kv_order=int(reverse), p_scale=S,
                              pcast=m.FP8ATTN_PCAST_EXPCAST if expcast else m.FP8ATTN_PCAST_RNE,
                              return_mask=True)
    torch.cuda.synchronize()
    NB = -(-N // 64)
    sol = dict(ref_sol)
    sol["mask"] = _check_route_mask(orc, _np(mask), ref_sol, NB)
    exact = orc.mask_bits(sol["mask"], NB)
    assert exact[..., :2].all() and not exact[..., 2:].any()
    ref, _, _, _, amb = orc.attention_fp8(ref_q, p_scale=S, kv_reverse=reverse, expcast=expcast,
                                          return_amb=True, sol=sol)
    got = _gpu_rows(out, np.arange(N))
    _compare_out(got, ref, "sol shared state", amb, peaked=True, wide=True)
    if not expcast:
        rows = np.arange(0, N, 37)
        two = _sol_model(orc, ref_q, sol, exact, reverse, S, 1.0 / math.sqrt(128.0), shared=False,
                         rows=rows)
        allow = ATOL + 2.0 ** -8 * np.abs(ref[:, :, rows]) + amb[:, :, rows]
        miss = float((np.abs(two - ref[:, :, rows]) - allow).max())
        say(f"two-state reading: misses the same bar by up to {miss:.3e}")
        assert miss > 0.03


@pytest.mark.parametrize("grid,tau,reverse", [((5, 12, 16), 3.0, True), ((4, 9, 20), 2.0, False)])
def test_sol_video_local(m, orc, grid, tau, reverse):
    """Video-like inputs (logits falling off with 3D distance): exact blocks cluster around the
    query; same checks as above."""
    N, H = grid[0] * grid[1] * grid[2], 2
    say("sol video-local", grid, tau)
    q, k, v = workloads.make_qkv(1, N, H, seed=98, kind="video_local", grid=grid)
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    ref_q = orc.quantize(qb, kb, vb)
    ref_sol = orc.sol_prepare(ref_q, tau=tau, estimator=0, sink_blocks=1)
    qz = _gpu_quantize(m, q, k, v)
    out, mask = m.sol_forward(qz, tau=tau, kv_order=int(reverse), return_mask=True)
    torch.cuda.synchronize()
    sol = dict(ref_sol)
    sol["mask"] = _check_route_mask(orc, _np(mask), ref_sol, -(-N // 64))
    ref, _, _, _, amb = orc.attention_fp8(ref_q, kv_reverse=reverse, return_amb=True, sol=sol)
    _compare_out(_gpu_rows(out, np.arange(N)), ref, f"sol video-local tau={tau}", amb, peaked=True)


def test_sol_with_smoothing(m, orc):
    """Sequence-mean smoothing under Sol: K shifted before the summaries, V shift restored."""
    say("sol + smoothing")
    N, H = 1500, 2
    q, k, v = workloads.make_qkv(1, N, H, seed=97, kind="channel_offset")
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    ref_q = orc.quantize(qb, kb, vb, smoothing=2, v_bias_correction=True)
    ref_sol = orc.sol_prepare(ref_q, tau=2.5, estimator=1, sink_blocks=1)
    qz = _gpu_quantize(m, q, k, v, smoothing=2, bias=True)
    out, mask = m.sol_forward(qz, tau=2.5, estimator=1, sink_blocks=1, return_mask=True)
    torch.cuda.synchronize()
    sol = dict(ref_sol)
    sol["mask"] = _check_route_mask(orc, _np(mask), ref_sol, -(-N // 64))
    ref, _, _, _, amb = orc.attention_fp8(ref_q, kv_reverse=True, return_amb=True, sol=sol)
    _compare_out(_gpu_rows(out, np.arange(N)), ref, "sol smoothing", amb, peaked=True, wide=True)


@pytest.mark.parametrize("delta,S,reverse", [(7, 1.0, False), (7, 256.0, True), (9, 256.0, False)])
def test_underflow_counter(m, orc, delta, S, reverse):
    say("underflow", delta, S, reverse)
    q, k, v = workloads.workload("sink4096", delta=delta, heads=2)
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    ref_q = orc.quantize(qb, kb, vb)
    ref, _, uf, _, amb = orc.attention_fp8(ref_q, p_scale=S, kv_reverse=reverse, return_amb=True)
    qz = _gpu_quantize(m, q, k, v)
    cnt = torch.zeros(2, dtype=torch.int64, device=DEV)
    out = _run_attn(m, qz, p_scale=S, kv_order=int(reverse), underflow=cnt)
    _compare_out(_gpu_rows(out, np.arange(4096)), ref, "sink", amb, peaked=True)
    g = _np(cnt).astype(np.float64)
    o = uf.sum(axis=2)[0].astype(np.float64)
    say("underflow gpu", g, "oracle", o)
    total = 4096 * 4096
    assert np.all(np.abs(g - o) <= 1e-4 * total + 1e-3 * o)


# ------------------------------------------------------------------------------------------
# V-Smooth clustering (fp8attn_vsmooth_cluster) against the oracle's clustering
# ------------------------------------------------------------------------------------------
def _check_perm_valid(perm, labels):
    """Every (b, h) row of perm is a permutation of its tokens, grouped by ascending cluster id,
    in ascending token order inside a cluster (a stable sort)."""
    B, H, N = perm.shape
    for b in range(B):
        for h in range(H):
            p, lab = perm[b, h], labels[b, h]
            assert np.array_equal(np.sort(p), np.arange(N))
            key = lab[p].astype(np.int64) * N + p
            assert np.all(np.diff(key) > 0)


@pytest.mark.parametrize("N,H,K,F,iters", [(49152, 2, 16, 8, 10), (1000, 3, 16, 8, 10), (37, 1, 16, 8, 3),
                                           (5, 1, 16, 4, 2), (3000, 1, 32, 16, 0)])
def test_vsmooth_cluster_matches_oracle(m, orc, N, H, K, F, iters):
    say("cluster", N, H, K, F, iters)
    if N == 49152:
        _, _, v = workloads.workload("vsmooth", heads=H)
    else:
        _, _, v = workloads.make_qkv(1, N, H, seed=N + K, kind="token_outliers", n_outlier_channels=8)
    perm_g, lab_g = m.vsmooth_cluster(v.to(DEV), n_clusters=K, n_feat=F, iters=iters, labels=True)
    torch.cuda.synchronize()
    perm_g, lab_g = _np(perm_g), _np(lab_g)
    perm_o, lab_o = orc.vsmooth_perm(_bits(v), n_clusters=K, n_feat=F, iters=iters, return_labels=True)
    _check_perm_valid(perm_g, lab_g)
    # the same deterministic algorithm: only the order of FP64 sums differs, which could move a
    # token only if it were equidistant to two centroids to within rounding
    agree = float(np.mean(lab_g == lab_o))
    say(f"cluster labels agree with the oracle on {agree * 100:.4f}% of tokens")
    assert np.array_equal(lab_g, lab_o)
    assert np.array_equal(perm_g, perm_o)


@pytest.mark.parametrize("B,N,H,K,F,iters,smoothing,rev_q", [
    (1, 49152, 2, 16, 8, 10, 0, False), (2, 1000, 3, 16, 8, 10, 0, False), (1, 37, 1, 16, 8, 3, 0, False),
    (1, 5, 1, 16, 4, 2, 0, False), (1, 3000, 1, 32, 16, 0, 0, False), (1, 4099, 2, 1, 8, 2, 0, False),
    (1, 2000, 2, 16, 8, 4, 1, True)])
def test_vsmooth_prepare_fused_scatter(m, orc, B, N, H, K, F, iters, smoothing, rev_q):
    """The fused preparation (stable scatter inside the V block statistics) against the two-call
    path (clustering, then quantisation through its permutation): every output bit-exact, the
    permutation and labels equal; both against the oracle's clustering and quantisation. Covers
    a full V-Smooth head pair, B = 2, fewer tokens than one 256-token sub-chunk, fewer tokens
    than clusters, 32 clusters, one cluster (identity permutation), K smoothing with a query
    permutation."""
    say("vsmooth prepare", B, N, H, K, F, iters, smoothing, rev_q)
    if N == 49152:
        q, k, v = workloads.workload("vsmooth", heads=H)
    else:
        q, k, v = workloads.make_qkv(B, N, H, seed=N + 7 * K, kind="token_outliers", n_outlier_channels=8)
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    perm_q = np.arange(N - 1, -1, -1, dtype=np.int32) if rev_q else None
    pq = None if perm_q is None else torch.from_numpy(perm_q).to(DEV)
    qz, perm, lab = m.vsmooth_prepare(qd, kd, vd, n_clusters=K, n_feat=F, iters=iters, perm_q=pq,
                                      smoothing=smoothing, labels=True)
    perm2, lab2 = m.vsmooth_cluster(vd, n_clusters=K, n_feat=F, iters=iters, labels=True)
    qz2 = m.quantize_qkv(qd, kd, vd, perm_q=pq, perm_kv=perm2, vsmooth=True, smoothing=smoothing)
    torch.cuda.synchronize()
    assert np.array_equal(_np(perm), _np(perm2)), "perm"
    assert np.array_equal(_np(lab), _np(lab2)), "labels"
    for key in ("q8", "k8", "v8t", "q_scale", "k_scale", "v_scale", "v_mean"):
        a, b = _np(getattr(qz, key)), _np(getattr(qz2, key))
        assert a.dtype == b.dtype and np.array_equal(a.view(np.uint8), b.view(np.uint8)), key
    perm_np, lab_np = _np(perm), _np(lab)
    _check_perm_valid(perm_np, lab_np)
    if N <= 4099:
        perm_o = orc.vsmooth_perm(_bits(v), n_clusters=K, n_feat=F, iters=iters)
        assert np.array_equal(perm_np, perm_o)
        ref = orc.quantize(_bits(q), _bits(k), _bits(v), perm_q=perm_q, perm_kv=perm_o, vsmooth=True,
                           smoothing=smoothing)
        _compare_quant(qz, ref)
    if K == 1:
        assert np.array_equal(perm_np, np.broadcast_to(np.arange(N, dtype=np.int32), perm_np.shape))


# ------------------------------------------------------------------------------------------
# Full-size workloads (benchmark launch configuration), sampled heads and rows
# ------------------------------------------------------------------------------------------
def test_maximum_batch_heads(m, orc):
    """B * H = 65535 (the largest count the library takes) with a ragged two-block sequence:
    codes, scales and outputs of sampled (b, h) against the oracle. Inputs are drawn on the
    device from a seeded generator; the oracle receives the same bf16 bytes of those heads."""
    B, H, N = 3, 21845, 101
    say("maximum batch*heads", B, H, N)
    g = torch.Generator(device=DEV).manual_seed(123)
    q, k, v = (torch.randn((B, N, H, 128), generator=g, device=DEV).to(torch.bfloat16) for _ in range(3))
    qz = m.quantize_qkv(q, k, v)
    out = m.forward(qz, kv_order=1)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (1, 12345), (2, H - 1)):
        sl = lambda t: _bits(t[b:b + 1, :, h:h + 1].contiguous().cpu())
        ref_q = orc.quantize(sl(q), sl(k), sl(v))
        for key in ("q8", "k8", "v8t", "q_scale", "k_scale", "v_scale"):
            assert np.array_equal(_np(getattr(qz, key)[b:b + 1, h:h + 1]), ref_q[key]), (key, b, h)
        ref, _, _, _, amb = orc.attention_fp8(ref_q, kv_reverse=True, return_amb=True)
        got = out[b:b + 1, :, h:h + 1].float().cpu().numpy().transpose(0, 2, 1, 3).astype(np.float64)
        _compare_out(got, ref, f"max heads ({b}, {h})", amb)
    del q, k, v, qz, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("sparse", [False, True])
def test_work_queues_streams_and_reuse(m, orc, sparse):
    """The persistent workgroups take their work items from counters in the workspace. Several
    items per workgroup, with items taken across XCD ranges, must still write every output row
    exactly once. The outputs start as NaN, so a skipped item shows. Calls must agree bit for bit:
    - with a workspace full of 0xFF bytes (the counters are reset by the launch);
    - with one workspace reused;
    - on two streams at once with one workspace each.
    One dense head of the first call is checked against the oracle."""
    if sparse:
        # 10x15x24 grid in (6,8,8) tiles: 12 tiles of 384 tokens, ragged in t and h
        lay = m.sta_build(10, 15, 24, 6, 8, 8, 1, 1, 1)
        Nsrc, H = 10 * 15 * 24, 40
        N = lay["perm"].shape[0]
        sp = m.sparse_to_device(lay, DEV)
        perm = torch.from_numpy(lay["perm"]).to(DEV)
    else:
        Nsrc, H = 20000, 8
        N, sp, perm = Nsrc, None, None
    say("work queues", "sparse" if sparse else "dense", Nsrc, N, H)
    g = torch.Generator(device=DEV).manual_seed(77)
    ins = [[torch.randn((1, Nsrc, H, 128), generator=g, device=DEV).to(torch.bfloat16) for _ in range(3)]
           for _ in range(2)]
    qz = [m.quantize_qkv(*x, perm_q=perm, perm_kv=perm, n_layout=N) for x in ins]

    def run(i, ws, stream=None):
        out = torch.full((1, Nsrc, H, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
        kw = dict(kv_order=1, sparse=sp, out_rows=perm, n_out=Nsrc, out=out, workspace=ws)
        if stream is None:
            m.forward(qz[i], **kw)
        else:
            with torch.cuda.stream(stream):
                m.forward(qz[i], **kw)
        return out

    def new_ws():
        ws = m.forward_workspace(1, N, H, False, DEV, 1)
        ws.fill_(255)
        return ws

    ref = [run(i, new_ws()) for i in range(2)]
    torch.cuda.synchronize()
    for r in ref:
        assert not torch.isnan(r.float()).any(), "a work item was skipped"
    ws = new_ws()
    for _ in range(3):
        assert torch.equal(run(0, ws).view(torch.int16), ref[0].view(torch.int16))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    w1, w2 = new_ws(), new_ws()
    torch.cuda.synchronize()
    o1, o2 = run(0, w1, s1), run(1, w2, s2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), ref[0].view(torch.int16))
    assert torch.equal(o2.view(torch.int16), ref[1].view(torch.int16))
    if not sparse:
        h = 5
        sl = lambda t: _bits(t[:, :, h:h + 1].contiguous().cpu())
        ref_q = orc.quantize(*(sl(t) for t in ins[0]))
        want, _, _, _, amb = orc.attention_fp8(ref_q, kv_reverse=True, return_amb=True)
        got = ref[0][:, :, h:h + 1].float().cpu().numpy().transpose(0, 2, 1, 3).astype(np.float64)
        _compare_out(got, want, "work queues, head 5", amb)


def _slice_heads(t, heads):
    return t[:, :, heads, :].contiguous()


@pytest.mark.parametrize("name", ["wan13b", "wan14b", "vsmooth", "wan14b+smoothing", "wan13b+split3"])
def test_full_size_sampled(m, orc, name):
    say("full size", name)
    smooth = name.endswith("+smoothing")      # K and V smoothing with the bias correction
    splits = int(name.split("+split")[1]) if "+split" in name else 1
    name = name.split("+")[0]
    q, k, v = workloads.workload(name)
    B, N, H, _ = q.shape
    heads = [0, H - 1]
    vs = name == "vsmooth"
    perm = None
    if vs:
        perm_s = orc.vsmooth_perm(_bits(_slice_heads(v, heads)))     # [1, 2, N]
        perm = np.zeros((1, H, N), np.int32)
        perm[:] = np.arange(N, dtype=np.int32)
        perm[0, heads] = perm_s[0]
    sm = 2 if smooth else 0
    qz = _gpu_quantize(m, q, k, v, perm_kv=perm, vsmooth=vs, smoothing=sm, bias=smooth)
    out = _run_attn(m, qz, kv_order=1, pcast=m.FP8ATTN_PCAST_EXPCAST if vs else m.FP8ATTN_PCAST_RNE,
                    kv_splits=splits)
    qs, ks, vsl = (_bits(_slice_heads(t, heads)) for t in (q, k, v))
    ref_q = orc.quantize(qs, ks, vsl, perm_kv=None if perm is None else perm[:, heads], vsmooth=vs,
                         smoothing=sm, v_bias_correction=smooth)
    for key in ("q8", "k8", "v8t"):
        assert np.array_equal(_np(getattr(qz, key)[:, heads]), ref_q[key]), key
    keys = ("q_scale", "k_scale", "v_scale") + (("v_shift",) if smooth else ())
    for key in keys:
        assert np.array_equal(_np(getattr(qz, key)[:, heads]), ref_q[key]), key
    rows = workloads.sample_rows(N, 48, seed=7)
    ref, _, _, _, amb = orc.attention_fp8(ref_q, rows=rows, kv_reverse=True, expcast=vs,
                                          return_amb=True, kv_splits=splits)
    got = _gpu_rows(out[:, :, heads], rows)
    # outlier channels (Wan-1.3B) and outlier tokens (V-Smooth) decide outputs through single P
    # codes and reach |O| >= 2; the channel offsets of the smoothing inputs reach |O| >= 2
    _compare_out(got, ref, name, amb, peaked=name in ("wan13b", "vsmooth"),
                 wide=smooth or name in ("wan13b", "vsmooth"))


def test_full_size_sparse_sampled(m, orc):
    say("full size wan14b sparse")
    q, k, v = workloads.workload("wan14b")
    B, N, H, _ = q.shape
    grid = (21, 45, 80, 6, 8, 8, 1, 1, 1)
    lay = m.sta_build(*grid)
    perm = lay["perm"]
    qz = _gpu_quantize(m, q, k, v, perm_q=perm, perm_kv=perm)
    sp = m.sparse_to_device(lay, DEV)
    out = _run_attn(m, qz, kv_order=1, sparse=sp, out_rows=torch.from_numpy(perm).to(DEV), n_out=N)
    heads = [0, H - 1]
    qs, ks, vsl = (_bits(_slice_heads(t, heads)) for t in (q, k, v))
    ref_q = orc.quantize(qs, ks, vsl, perm_q=perm, perm_kv=perm)
    assert np.array_equal(_np(qz.k8[:, heads]), ref_q["k8"])
    valid_pos = np.flatnonzero(perm >= 0)
    rng = np.random.default_rng(9)
    pos = np.unique(np.concatenate([valid_pos[:2], valid_pos[-2:], rng.choice(valid_pos, 96)]))
    ref, _, _, _, amb = orc.attention_fp8(ref_q, rows=pos.astype(np.int32), kv_reverse=True,
                                          sparse=orc.sta_layout(*grid), return_amb=True)
    got = _gpu_rows(out[:, :, heads], perm[pos])
    _compare_out(got, ref, "wan14b sparse", amb)
