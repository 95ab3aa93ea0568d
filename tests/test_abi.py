"""Host-side checks of the C ABI (no GPU needed): the library loads and exports every entry
point declared in include/fp8attn.h, argument validation rejects bad calls before any HIP
call, and the host STA layout helper agrees with the oracle's independent implementation."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "fp8attn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8attn_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def m():
    import bit_attention_video_qkv_amd as m
    m.lib()
    return m


def test_exports_every_declared_symbol(m):
    names = _declared()
    assert len(names) >= 6
    for n in names:
        assert hasattr(m.lib(), n), n
    assert set(names) == set(m.EXPORTED)


def test_status_strings(m):
    L = m.lib()
    for s in range(4):
        assert L.fp8attn_status_string(s)
    assert L.fp8attn_status_string(99) == b"unknown status"


def _fake(n=0x10000):
    return ctypes.c_void_p(n)   # never dereferenced: validation fails first


def test_quantize_rejects_bad_arguments(m):
    L = m.lib()
    A = m._QuantArgs
    ptrs = [_fake()] * 10
    ws = ctypes.c_size_t(1 << 20)
    call = lambda a, p=ptrs: L.fp8attn_quantize_qkv(ctypes.byref(a), *p, _fake(), ws, None)
    assert call(A(1, 64, 64, 2, 64, None, None, 0, 0)) == 2            # D != 128
    assert call(A(0, 64, 64, 2, 128, None, None, 0, 0)) == 1           # B < 1
    assert call(A(2, 64, 64, 32768, 128, None, None, 0, 0)) == 2       # B * H > 65535
    assert call(A(1, 64, 65, 2, 128, None, None, 0, 0)) == 1           # N != N_src, no perm
    bad = list(ptrs)
    bad[0] = None
    assert call(A(1, 64, 64, 2, 128, None, None, 0, 0), bad) == 1      # null q
    bad = list(ptrs)
    bad[3] = _fake(0x10001)
    assert call(A(1, 64, 64, 2, 128, None, None, 0, 0), bad) == 1      # misaligned q8
    assert L.fp8attn_quantize_qkv(ctypes.byref(A(1, 64, 64, 2, 128, None, None, 0, 0)), *ptrs,
                                  _fake(), ctypes.c_size_t(16), None) == 1   # workspace too small
    assert call(A(1, 64, 64, 2, 128, None, None, 0, 1), ptrs[:9] + [None]) == 1  # vsmooth, no mean
    assert L.fp8attn_quantize_qkv(None, *ptrs, _fake(), ws, None) == 1
    # sequence-mean smoothing options
    assert call(A(1, 64, 64, 2, 128, None, None, 0, 0, 3, 0, _fake())) == 1   # smoothing 3
    assert call(A(1, 64, 64, 2, 128, None, None, 0, 0, -1, 0, _fake())) == 1  # smoothing -1
    assert call(A(1, 64, 64, 2, 128, None, None, 0, 1, 2, 0, _fake())) == 1   # + V-Smooth
    assert call(A(1, 64, 64, 2, 128, None, None, 0, 0, 1, 1, _fake())) == 1   # bias, smoothing 1
    assert call(A(1, 64, 64, 2, 128, None, None, 0, 0, 2, 2, _fake())) == 1   # bias flag 2
    assert call(A(1, 64, 64, 2, 128, None, None, 0, 0, 2, 0, None)) == 1      # no v_shift
    assert call(A(1, 64, 64, 2, 128, None, None, 0, 0, 2, 1, _fake(0x10004))) == 1  # misaligned


def _opts(m, **kw):
    o = dict(softmax_scale=0.088, p_scale=256.0, kv_order=1, pcast=0, sparse=None, out_rows=None,
             n_out=256, underflow=None, v_shift=None, kv_splits=1)
    o.update(kw)
    return m._FwdOpts(o["softmax_scale"], o["p_scale"], o["kv_order"], o["pcast"], o["sparse"],
                      o["out_rows"], o["n_out"], o["underflow"], o["v_shift"], o["kv_splits"])


def test_forward_rejects_bad_arguments(m):
    L = m.lib()
    P = [_fake()] * 7

    def call(opts, D=128, N=256, v_mean=None, ws=0):
        args = P[:6] + [v_mean]
        return L.fp8attn_forward(1, N, 2, D, *args, ctypes.byref(opts), _fake(), None,
                                 ctypes.c_size_t(ws), None)

    assert call(_opts(m), D=64) == 2
    assert L.fp8attn_forward(2, 256, 32768, 128, *P, ctypes.byref(_opts(m)), _fake(), None,
                             ctypes.c_size_t(0), None) == 2            # B * H > 65535
    assert call(_opts(m, p_scale=500.0)) == 1
    assert call(_opts(m, p_scale=0.0)) == 1
    assert call(_opts(m, p_scale=float("nan"))) == 1
    assert call(_opts(m, softmax_scale=-1.0)) == 1
    assert call(_opts(m, kv_order=3)) == 1
    assert call(_opts(m, pcast=2)) == 1
    assert call(_opts(m, n_out=100)) == 1                               # n_out != N without out_rows
    assert call(_opts(m, pcast=1, underflow=_fake())) == 1              # ExpCast + counting
    sp = m._Sparse(64, 3, _fake(), _fake(), _fake())                    # 3 * 64 != 256
    assert call(_opts(m, sparse=ctypes.pointer(sp))) == 1
    sp = m._Sparse(96, 2, _fake(), _fake(), _fake())                    # not a multiple of 64
    assert call(_opts(m, sparse=ctypes.pointer(sp)), N=192) == 1
    sp = m._Sparse(128, 2, _fake(), _fake(), _fake())
    assert call(_opts(m, sparse=ctypes.pointer(sp)), v_mean=_fake()) == 1   # sparse + V-Smooth
    assert call(_opts(m), v_mean=_fake(), ws=0) == 1                    # V-Smooth needs workspace
    assert call(_opts(m, v_shift=_fake()), v_mean=_fake(), ws=1 << 24) == 1  # V shift + V-Smooth
    assert call(_opts(m, v_shift=_fake(0x10008))) == 1                  # misaligned v_shift
    assert call(_opts(m, kv_splits=17)) == 1                             # > FP8ATTN_KV_SPLITS_MAX
    assert call(_opts(m, kv_splits=-2)) == 1
    sp = m._Sparse(128, 2, _fake(), _fake(), _fake())
    assert call(_opts(m, sparse=ctypes.pointer(sp), kv_splits=2)) == 1   # split-KV is dense only
    assert call(_opts(m, kv_splits=2), ws=0) == 1                         # pieces need workspace
    assert call(_opts(m), ws=0) == 1                                      # work queues need workspace
    assert call(_opts(m), ws=255) == 1
    big = (1 << 25) + 1                                                   # N64 > 2^25 tokens per head
    assert call(_opts(m, n_out=big), N=big, ws=1 << 40) == 2
    assert call(_opts(m, n_out=(1 << 25) - 63), N=(1 << 25) - 63, ws=0) == 1   # N64 = 2^25 is accepted


@pytest.mark.parametrize("grid", [(21, 45, 80, 6, 8, 8, 1, 1, 1), (5, 7, 9, 2, 4, 8, 1, 1, 0),
                                  (3, 5, 8, 2, 4, 8, 9, 9, 9), (4, 4, 4, 4, 4, 4, 0, 0, 0)])
def test_sta_build_matches_oracle(m, orc, grid):
    a = m.sta_build(*grid)
    b = orc.sta_layout(*grid)
    for key in ("perm", "tile_len", "row_ptr", "col_idx"):
        assert np.array_equal(a[key], b[key]), key
    assert a["tile_tokens"] == b["tile_tokens"] and a["n_tiles"] == b["n_tiles"]


def test_sta_build_capacity_error(m):
    L = m.lib()
    perm = np.zeros(92160, np.int32)
    tl = np.zeros(240, np.int32)
    rp = np.zeros(241, np.int32)
    ci = np.zeros(10, np.int32)
    nnz = ctypes.c_int32(0)
    st = L.fp8attn_sta_build(21, 45, 80, 6, 8, 8, 1, 1, 1, perm.ctypes.data, tl.ctypes.data,
                             rp.ctypes.data, ci.ctypes.data, 10, ctypes.byref(nnz))
    assert st == 1 and nnz.value == 4480


def test_workspace_sizes(m):
    L = m.lib()
    assert L.fp8attn_quantize_workspace_bytes(1, 75600, 40, 128, 0) >= 40 * 591 * 128 * 4 + \
        2 * 40 * 1182 * 128 * 4   # + the smoothing block sums of K and V
    q = 256  # the eight work-queue counters, padded to 256 bytes
    assert L.fp8attn_forward_workspace_bytes(1, 75600, 40, 128, 0, 1) == q
    # V-Smooth: one 32-byte mean operand record per (b, h, group of four 128-row blocks, channel)
    assert L.fp8attn_forward_workspace_bytes(1, 49152, 24, 128, 1, 0) == q + 24 * 96 * 128 * 32
    assert L.fp8attn_forward_workspace_bytes(1, 129, 1, 128, 1, 0) == q + 128 * 32   # 2 blocks, one group
    # split-KV: 4096 tokens = 64 key blocks, 2 pieces of 32 blocks; 3 requested -> L = 22, 3 pieces
    assert L.fp8attn_forward_workspace_bytes(1, 4096, 8, 128, 0, 2) == q + 2 * 8 * 4096 * 129 * 4
    assert L.fp8attn_forward_workspace_bytes(1, 4096, 8, 128, 0, 3) == q + 3 * 8 * 4096 * 129 * 4
    # 5 blocks, 16 requested: L = 2, 3 pieces
    assert L.fp8attn_forward_workspace_bytes(1, 300, 1, 128, 0, 16) == \
        q + -(-3 * 300 * 128 * 4 // 256) * 256 + -(-3 * 300 * 4 // 256) * 256
    assert L.fp8attn_forward_workspace_bytes(1, 4096, 8, 128, 0, 17) == 0
    # auto (no device here: 256 compute units assumed): one piece for the large shapes and for
    # short sequences; H=1, N=75600 (591 query tiles, 1.15 rounds) -> ceil(3 * 512 / 591) = 3
    auto = m.FP8ATTN_KV_SPLITS_AUTO
    assert L.fp8attn_forward_workspace_bytes(1, 75600, 40, 128, 0, auto) == q
    assert L.fp8attn_forward_workspace_bytes(1, 4096, 8, 128, 0, auto) == q
    assert L.fp8attn_forward_workspace_bytes(1, 75600, 1, 128, 0, auto) == \
        L.fp8attn_forward_workspace_bytes(1, 75600, 1, 128, 0, 3) > q
    assert L.fp8attn_quantize_workspace_bytes(1, 100, 2, 64, 0) == 0


def test_cluster_rejects_bad_arguments(m):
    L = m.lib()
    need = L.fp8attn_vsmooth_cluster_workspace_bytes(1, 100, 2, 128, 8)
    assert need >= 100 * 2 * (8 * 4 + 4)
    assert L.fp8attn_vsmooth_cluster_workspace_bytes(1, 100, 2, 64, 8) == 0
    assert L.fp8attn_vsmooth_cluster_workspace_bytes(1, 100, 2, 128, 17) == 0
    good = dict(B=1, N=100, H=2, D=128, v=_fake(), K=16, F=8, it=10, perm=_fake(), lab=None,
                ws=_fake(), wsb=need)

    def call(**kw):
        a = dict(good, **kw)
        return L.fp8attn_vsmooth_cluster(a["B"], a["N"], a["H"], a["D"], a["v"], a["K"], a["F"], a["it"],
                                         a["perm"], a["lab"], a["ws"], a["wsb"], None)
    EINVAL, EUNSUPPORTED = 1, 2
    assert call(B=0) == EINVAL
    assert call(N=0) == EINVAL
    assert call(D=64) == EUNSUPPORTED
    assert call(B=300, H=300) == EINVAL
    assert call(K=0) == EINVAL and call(K=33) == EINVAL
    assert call(F=0) == EINVAL and call(F=17) == EINVAL
    assert call(it=-1) == EINVAL and call(it=1001) == EINVAL
    assert call(v=None) == EINVAL and call(v=_fake(0x10008)) == EINVAL
    assert call(perm=None) == EINVAL and call(lab=_fake(0x10002)) == EINVAL
    assert call(ws=None) == EINVAL and call(wsb=need - 1) == EINVAL


def test_vsmooth_prepare_rejects_bad_arguments(m):
    L = m.lib()
    A = m._QuantArgs
    need = L.fp8attn_vsmooth_prepare_workspace_bytes(1, 1000, 2, 128, 8)
    assert need >= L.fp8attn_quantize_workspace_bytes(1, 1000, 2, 128, 1) + \
        L.fp8attn_vsmooth_cluster_workspace_bytes(1, 1000, 2, 128, 8)
    assert L.fp8attn_vsmooth_prepare_workspace_bytes(1, 1000, 2, 64, 8) == 0
    assert L.fp8attn_vsmooth_prepare_workspace_bytes(1, 1000, 2, 128, 17) == 0

    def call(a, K=16, F=8, it=10, perm=_fake(), lab=None, ws=_fake(), wsb=need, qkv=(_fake(),) * 3):
        return L.fp8attn_vsmooth_prepare(ctypes.byref(a), *qkv, K, F, it, perm, lab, *([_fake()] * 7), ws,
                                         ctypes.c_size_t(wsb), None)
    EINVAL, EUNSUPPORTED = 1, 2
    good = lambda **kw: A(**dict(dict(B=1, N_src=1000, N=1000, H=2, D=128, perm_q=None, perm_kv=None,
                                      perm_kv_per_head=0, vsmooth=1, smoothing=0, v_bias_correction=0,
                                      v_shift=None), **kw))
    assert L.fp8attn_vsmooth_prepare(None, *([_fake()] * 3), 16, 8, 10, _fake(), None, *([_fake()] * 7),
                                     _fake(), ctypes.c_size_t(need), None) == EINVAL
    assert call(good(D=64)) == EUNSUPPORTED
    assert call(good(B=0)) == EINVAL
    assert call(good(perm_kv=_fake().value)) == EINVAL                 # the clustering supplies perm_kv
    assert call(good(vsmooth=0)) == EINVAL
    assert call(good(N=999)) == EINVAL                                 # N != N_src
    assert call(good(smoothing=2)) == EINVAL                           # smoothing 2 excludes V-Smooth
    assert call(good(), K=0) == EINVAL and call(good(), K=33) == EINVAL
    assert call(good(), F=0) == EINVAL and call(good(), it=1001) == EINVAL
    assert call(good(), perm=None) == EINVAL and call(good(), lab=_fake(0x10002)) == EINVAL
    assert call(good(), ws=None) == EINVAL and call(good(), wsb=need - 1) == EINVAL
    assert call(good(), qkv=(None, _fake(), _fake())) == EINVAL


def test_sol_rejects_bad_arguments(m):
    L = m.lib()
    need = L.fp8attn_sol_workspace_bytes(1, 1000, 2, 128)
    assert need > 2 * 1000 * 128 * 4  # at least the summary route's FP32 output
    assert L.fp8attn_sol_workspace_bytes(1, 1000, 2, 64) == 0
    P = [_fake()] * 6

    def call(D=128, ws=need, mask=None, **kw):
        o = dict(softmax_scale=0.088, p_scale=256.0, kv_order=1, pcast=0, tau=3.0, estimator=0,
                 sink_blocks=1, v_shift=None)
        o.update(kw)
        opts = m._SolOpts(o["softmax_scale"], o["p_scale"], o["kv_order"], o["pcast"], o["tau"],
                          o["estimator"], o["sink_blocks"], o["v_shift"])
        return L.fp8attn_sol_forward(1, 1000, 2, D, *P, ctypes.byref(opts), _fake(), mask,
                                     _fake(), ctypes.c_size_t(ws), None)

    assert call(D=64) == 2
    assert call(ws=need - 1) == 1
    opts = m._SolOpts(0.088, 256.0, 1, 0, 3.0, 0, 1, None)
    assert L.fp8attn_sol_forward(1, (1 << 25) + 1, 2, 128, *P, ctypes.byref(opts), _fake(), None,
                                 _fake(), ctypes.c_size_t(1 << 40), None) == 2   # N64 > 2^25
    assert call(estimator=2) == 1
    assert call(sink_blocks=-1) == 1
    assert call(tau=float("nan")) == 1
    assert call(tau=float("inf")) == 1
    assert call(p_scale=449.0) == 1
    assert call(softmax_scale=0.0) == 1
    assert call(kv_order=2) == 1
    assert call(mask=_fake(0x10004)) == 1
    assert call(v_shift=_fake(0x10004)) == 1
    assert L.fp8attn_sol_forward(1, 1000, 2, 128, *P, None, _fake(), None, _fake(),
                                 ctypes.c_size_t(need), None) == 1


def test_diagnostics_argument_errors(m):
    L = m.lib()
    fake = ctypes.c_void_p(0x10000)
    assert L.fp8attn_diag_e4m3_encode(0, 6, fake, None) == 1              # not a multiple of 4
    assert L.fp8attn_diag_e4m3_encode(0, -4, fake, None) == 1
    assert L.fp8attn_diag_e4m3_encode(0, 8, None, None) == 1
    assert L.fp8attn_diag_e4m3_encode(0, 8, ctypes.c_void_p(0x10001), None) == 1
    assert L.fp8attn_diag_e4m3_encode(0xFFFFFFFC, 8, fake, None) == 1     # past pattern 2^32 - 1
    assert L.fp8attn_diag_e4m3_encode(0, 0, None, None) == 0              # nothing to do
    assert L.fp8attn_diag_e4m3_decode(fake, 6, fake, None) == 1              # not a multiple of 4
    assert L.fp8attn_diag_e4m3_decode(fake, -4, fake, None) == 1
    assert L.fp8attn_diag_e4m3_decode(None, 8, fake, None) == 1
    assert L.fp8attn_diag_e4m3_decode(fake, 8, ctypes.c_void_p(0x10004), None) == 1  # out misaligned
    assert L.fp8attn_diag_e4m3_decode(None, 0, None, None) == 0              # nothing to do
    assert L.fp8attn_diag_mfma_e4m3(fake, fake, fake, -1, None) == 1
    assert L.fp8attn_diag_mfma_e4m3(None, fake, fake, 2, None) == 1
    assert L.fp8attn_diag_mfma_e4m3(ctypes.c_void_p(0x10008), fake, fake, 2, None) == 1
    assert L.fp8attn_diag_mfma_e4m3(None, None, None, 0, None) == 0
