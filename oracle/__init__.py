"""CPU oracle for block-scaled FP8 (OCP E4M3) attention forward.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package. It shares no code with the HIP library
(``bit_attention_video_qkv_amd``) and never imports it.

The arithmetic lives in ``fp8attn_oracle.cpp`` (plain C++17 + OpenMP, loaded with ctypes);
this module marshals numpy arrays and holds the closed forms of the P-underflow analysis.
Every function cites the passage of the pages it follows:

* TeleFuser blog "FP8 Sol-Attn: H100 视频 DiT 的量化稀疏注意力", section
  "面向注意力的 FP8 Preparation" (block / channel scales) and "SM90 CuTe Mainloop".
* FPSAttention write-up, sections 2.1-2.2 and 3.1 (fake-quant form, STA window, tiling).
* VC-Attention article, sections 二 (V-Smooth) and 三 (ExpCast).
* "FP8 P-Cast Precision in Attention: Sink-Induced Collapse and the Optimality of S=2^8",
  sections 三 (F(Delta, S), dp(S), Theorem 4) and 五 (Table I, MSE table).

Parity pins: every function here is pinned by a ``-m "not gpu"`` test against page values,
closed forms or brute force, except the absolute attention outputs on the large synthetic
configurations, which nothing on the pages fixes (parity unpinned beyond the pins listed in
the tests).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8attn_oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "libfp8attn_oracle.so")
_lib = None

MODE_EXACT, MODE_NOQUANT, MODE_PCAST, MODE_FP8 = 0, 1, 2, 3


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (OpenMP); returns the library path."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["g++", "-O2", "-std=c++17", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
               _SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        _lib = ctypes.CDLL(_LIB_PATH)
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().orc_num_threads())


# ----------------------------------------------------------------------------------------
# E4M3 / BF16 codecs (OCP E4M3FN; the pages fix max 448, 8 values per binade, underflow below
# 2^-10 for round-to-nearest, and 56 as the code of 1.0 used by ExpCast).
# ----------------------------------------------------------------------------------------
def e4m3_encode(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    _load().orc_e4m3_encode(_p(x), _p(out), ctypes.c_int64(x.size))
    return out


def e4m3_encode_f32(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    _load().orc_e4m3_encode_f32(_p(x), _p(out), ctypes.c_int64(x.size))
    return out


def e4m3_decode(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    _load().orc_e4m3_decode(_p(c), _p(out), ctypes.c_int64(c.size))
    return out


def bf16_encode(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().orc_bf16_encode(_p(x), _p(out), ctypes.c_int64(x.size))
    return out


def bf16_decode(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------------
# Quantisation: TeleFuser "面向注意力的 FP8 Preparation" eq. s_q, s_k (per 64-token block),
# s_v (per channel), V stored token-contiguous; VC-Attention 二 (V-Smooth residual).
# ----------------------------------------------------------------------------------------
def quantize(q, k, v, perm_q=None, perm_kv=None, vsmooth=False, n_layout=None, smoothing=0,
             v_bias_correction=False):
    """q, k, v: uint16 bf16 bits [B, Nsrc, H, D]. perm_q: int32 [N] or None; perm_kv: int32
    [N] (shared) or [B, H, N] (per head) or None. smoothing: 0 none, 1 K, 2 K and V
    (sequence-mean smoothing, TeleFuser MiniMax-H3 section); v_bias_correction only with 2.
    Returns a dict of numpy arrays: q8, k8 [B,H,N64,D] uint8; v8t [B,H,D,N64] uint8;
    q_scale, k_scale [B,H,NB] f32; v_scale [B,H,D] f32; v_mean [B,H,ceil(N/128),D] uint16
    (V-Smooth only); v_shift [B,H,D] f32 (smoothing 2 only)."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    B, Nsrc, H, D = q.shape
    per_head = 0
    if perm_q is not None:
        perm_q = np.ascontiguousarray(perm_q, dtype=np.int32)
    if perm_kv is not None:
        perm_kv = np.ascontiguousarray(perm_kv, dtype=np.int32)
        per_head = 1 if perm_kv.ndim == 3 else 0
    if n_layout is None:
        if perm_q is not None:
            n_layout = perm_q.shape[0]
        elif perm_kv is not None:
            n_layout = perm_kv.shape[-1]
        else:
            n_layout = Nsrc
    N = int(n_layout)
    NB = (N + 63) // 64
    N64 = NB * 64
    NB128 = (N + 127) // 128
    out = dict(
        q8=np.zeros((B, H, N64, D), np.uint8), k8=np.zeros((B, H, N64, D), np.uint8),
        v8t=np.zeros((B, H, D, N64), np.uint8), q_scale=np.zeros((B, H, NB), np.float32),
        k_scale=np.zeros((B, H, NB), np.float32), v_scale=np.zeros((B, H, D), np.float32),
        v_mean=np.zeros((B, H, NB128, D), np.uint16) if vsmooth else None,
        v_shift=np.zeros((B, H, D), np.float32) if smoothing == 2 else None,
        N=N, vsmooth=bool(vsmooth))
    rc = _load().orc_quantize(
        B, Nsrc, N, H, D, _p(q), _p(k), _p(v), _p(perm_q), _p(perm_kv), per_head,
        1 if vsmooth else 0, _p(out["q8"]), _p(out["k8"]), _p(out["v8t"]), _p(out["q_scale"]),
        _p(out["k_scale"]), _p(out["v_scale"]), _p(out["v_mean"]), int(smoothing),
        1 if v_bias_correction else 0, _p(out["v_shift"]))
    if rc != 0:
        raise ValueError("oracle quantize: invalid arguments")
    return out


def _sparse_args(sparse):
    if sparse is None:
        return 0, 0, None, None, None, None
    tl = np.ascontiguousarray(sparse["tile_len"], dtype=np.int32)
    rp = np.ascontiguousarray(sparse["row_ptr"], dtype=np.int32)
    ci = np.ascontiguousarray(sparse["col_idx"], dtype=np.int32)
    return int(sparse["tile_tokens"]), int(tl.shape[0]), tl, rp, ci, (tl, rp, ci)


class _OrcSol(ctypes.Structure):
    _fields_ = [("mask", ctypes.c_void_p), ("kq8", ctypes.c_void_p), ("kq_scale", ctypes.c_void_p),
                ("vsum", ctypes.c_void_p)]


def sol_prepare(qz, tau=1.0, estimator=0, sink_blocks=1, softmax_scale=1.0 / math.sqrt(128.0)):
    """Sol routing (TeleFuser "Sol Routing"): K/V block summaries, quantised K summaries, the
    per-Q-block threshold theta = mu + tau * sigma (estimator 0 diag, 1 exact) and the
    exact-block bitmask, on the output of ``quantize`` (layout order, no V-Smooth). Returns a dict:
    ksum f32 [B,H,NB,D], vsum uint16 bf16 [B,H,NB,D], kq8 uint8 [B,H,64*NBg,D], kq_scale f32
    [B,H,NBg], theta f64 [B,H,NB], mask and amb_mask uint64 [B,H,NB,W] (bit j%64 of word j//64:
    KV block j is exact for Q block u; amb_mask flags decisions within the device's evaluation
    error of theta, where either bit is correct)."""
    B, H, N64, D = qz["q8"].shape
    N = qz["N"]
    NB = -(-N // 64)
    NBg = W = -(-NB // 64)
    out = dict(ksum=np.zeros((B, H, NB, D), np.float32), vsum=np.zeros((B, H, NB, D), np.uint16),
               kq8=np.zeros((B, H, 64 * NBg, D), np.uint8), kq_scale=np.zeros((B, H, NBg), np.float32),
               theta=np.zeros((B, H, NB), np.float64), mask=np.zeros((B, H, NB, W), np.uint64),
               amb_mask=np.zeros((B, H, NB, W), np.uint64))
    rc = _load().orc_sol_prepare(
        B, N, H, D, _p(qz["q8"]), _p(qz["k8"]), _p(qz["v8t"]), _p(qz["q_scale"]), _p(qz["k_scale"]),
        _p(qz["v_scale"]), ctypes.c_double(tau), int(estimator), int(sink_blocks),
        ctypes.c_double(softmax_scale), _p(out["ksum"]), _p(out["vsum"]), _p(out["kq8"]),
        _p(out["kq_scale"]), _p(out["theta"]), _p(out["mask"]), _p(out["amb_mask"]))
    if rc != 0:
        raise ValueError("oracle sol_prepare: invalid arguments")
    return out


def mask_bits(mask, NB):
    """uint64 words [..., W] -> bool [..., NB]."""
    w = np.ascontiguousarray(mask, np.uint64)
    bits = ((w[..., :, None] >> np.arange(64, dtype=np.uint64)) & np.uint64(1)).astype(bool)
    return bits.reshape(*w.shape[:-1], -1)[..., :NB]


def attention_fp8(qz, rows=None, softmax_scale=1.0 / math.sqrt(128.0), p_scale=256.0,
                  kv_reverse=False, expcast=False, sparse=None, return_amb=False, kv_splits=1,
                  sol=None):
    """Full FP8 path (TeleFuser "SM90 CuTe Mainloop" + the P-cast paper's order/scale +
    VC-Attention's V-Smooth restore and ExpCast codes) on the output of ``quantize``.
    Returns (out f64 [B,H,R,D], out_bf16 uint16 [B,H,R,D], underflow int64 [B,H,R],
    row_valid uint8 [B,H,R]) and, with return_amb, amb_bound f64 [B,H,R,D]: per output element,
    the largest change that P codes lying within the evaluation error of a rounding boundary
    (FP32 and the E4M3 matrix-core contraction) and the contraction's own truncation can
    explain. kv_splits > 1: split-KV (TeleFuser long-sequence split-KV), dense rows only: the
    key blocks are cut at multiples of 2*ceil(NB/(2*kv_splits)) blocks, each piece runs its own
    online softmax and the pieces are merged by log-sum-exp. sol: the dict of ``sol_prepare``
    (its ``mask`` may be replaced by another valid mask): Sol routing. One running max, row sum
    and accumulator for both routes; the KV blocks are taken in route groups of 64, groups in KV
    order, and inside a group first its summary blocks, then its exact blocks (each in KV order).
    An exact block (mask bit set) takes the FP8 step; a summary block counts as n_j copies of its
    summary (kbar_j, vbar_j) scored by the route score r_j (m' = max(m, r_j), weight
    n_j exp(r_j - m'))."""
    B, H, N64, D = qz["q8"].shape
    N = qz["N"]
    rows = np.arange(N, dtype=np.int32) if rows is None else np.ascontiguousarray(rows, np.int32)
    R = rows.shape[0]
    out = np.zeros((B, H, R, D), np.float64)
    ob = np.zeros((B, H, R, D), np.uint16)
    uf = np.zeros((B, H, R), np.int64)
    rv = np.zeros((B, H, R), np.uint8)
    amb = np.zeros((B, H, R, D), np.float64) if return_amb else None
    tt, nt, tl, rp, ci, _keep = _sparse_args(sparse)
    sol_c = None
    if sol is not None:
        sol_keep = [np.ascontiguousarray(sol[k_]) for k_ in ("mask", "kq8", "kq_scale", "vsum")]
        sol_c = _OrcSol(*(a_.ctypes.data for a_ in sol_keep))
    rc = _load().orc_attention(
        MODE_FP8, B, N, H, D, None, None, None, _p(qz["q8"]), _p(qz["k8"]), _p(qz["v8t"]),
        _p(qz["q_scale"]), _p(qz["k_scale"]), _p(qz["v_scale"]),
        _p(qz["v_mean"]) if qz.get("vsmooth") else None, ctypes.c_double(softmax_scale),
        ctypes.c_double(p_scale), 1 if kv_reverse else 0, 1 if expcast else 0, tt, nt, _p(tl),
        _p(rp), _p(ci), _p(rows), ctypes.c_int64(R), _p(out), _p(ob), _p(uf), _p(rv), _p(amb),
        _p(qz.get("v_shift")), int(kv_splits), ctypes.byref(sol_c) if sol_c is not None else None)
    if rc != 0:
        raise ValueError("oracle attention: invalid arguments")
    return (out, ob, uf, rv, amb) if return_amb else (out, ob, uf, rv)


def attention_ref(mode, q, k, v, rows=None, softmax_scale=1.0 / math.sqrt(128.0),
                  p_scale=256.0, kv_reverse=False, expcast=False, sparse=None, kv_splits=1):
    """Unquantised modes on float64 [B, H, N, D] layout-order inputs: MODE_EXACT (two-pass
    FP64 softmax), MODE_NOQUANT (streaming loop, no casts), MODE_PCAST (only P cast to
    E4M3, the P-cast paper's kernel-faithful simulation). Returns (out, underflow, row_valid)."""
    q = np.ascontiguousarray(q, np.float64)
    k = np.ascontiguousarray(k, np.float64)
    v = np.ascontiguousarray(v, np.float64)
    B, H, N, D = q.shape
    rows = np.arange(N, dtype=np.int32) if rows is None else np.ascontiguousarray(rows, np.int32)
    R = rows.shape[0]
    out = np.zeros((B, H, R, D), np.float64)
    uf = np.zeros((B, H, R), np.int64)
    rv = np.zeros((B, H, R), np.uint8)
    tt, nt, tl, rp, ci, _keep = _sparse_args(sparse)
    rc = _load().orc_attention(
        int(mode), B, N, H, D, _p(q), _p(k), _p(v), None, None, None, None, None, None, None,
        ctypes.c_double(softmax_scale), ctypes.c_double(p_scale), 1 if kv_reverse else 0,
        1 if expcast else 0, tt, nt, _p(tl), _p(rp), _p(ci), _p(rows), ctypes.c_int64(R),
        _p(out), None, _p(uf), _p(rv), None, None, int(kv_splits), None)
    if rc != 0:
        raise ValueError("oracle attention_ref: invalid arguments")
    return out, uf, rv


# ----------------------------------------------------------------------------------------
# STA layout (FPSAttention 2.2 / 3.1) and V-Smooth clustering (VC-Attention 二).
# ----------------------------------------------------------------------------------------
def sta_layout(T, Hg, W, tt, th, tw, rt, rh, rw):
    nt, nh, nw = -(-T // tt), -(-Hg // th), -(-W // tw)
    n_tiles, tile = nt * nh * nw, tt * th * tw
    perm = np.zeros(n_tiles * tile, np.int32)
    tile_len = np.zeros(n_tiles, np.int32)
    row_ptr = np.zeros(n_tiles + 1, np.int32)
    col_idx = np.zeros(n_tiles * n_tiles, np.int32)
    nnz = ctypes.c_int32(0)
    rc = _load().orc_sta_layout(T, Hg, W, tt, th, tw, rt, rh, rw, _p(perm), _p(tile_len),
                                _p(row_ptr), _p(col_idx), ctypes.byref(nnz))
    if rc != 0:
        raise ValueError("oracle sta_layout: invalid arguments")
    return dict(perm=perm, tile_len=tile_len, row_ptr=row_ptr, col_idx=col_idx[:nnz.value].copy(),
                tile_tokens=tile, n_tiles=n_tiles)


def vsmooth_perm(v, n_clusters=16, n_feat=8, iters=10, return_labels=False):
    """v: uint16 bf16 [B, N, H, D] -> int32 perm [B, H, N] (cluster-contiguous order), and
    optionally the cluster id of every source token [B, H, N]."""
    v = np.ascontiguousarray(v, np.uint16)
    B, N, H, D = v.shape
    perm = np.zeros((B, H, N), np.int32)
    labels = np.zeros((B, H, N), np.int32)
    rc = _load().orc_vsmooth_perm(B, N, H, D, _p(v), n_clusters, n_feat, iters, _p(perm),
                                  _p(labels))
    if rc != 0:
        raise ValueError("oracle vsmooth_perm: invalid arguments")
    return (perm, labels) if return_labels else perm


# ----------------------------------------------------------------------------------------
# Closed forms of the P-cast paper, section 三.
# ----------------------------------------------------------------------------------------
def normal_cdf(x: float) -> float:
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def expected_max_normal(k: int) -> float:
    """delta_k = E[max of k i.i.d. N(0,1)] (the paper's delta_4 ~ 1.03), by quadrature of
    E[M] = integral m * k phi(m) Phi(m)^(k-1) dm."""
    m = np.linspace(-12.0, 12.0, 200001)
    phi = np.exp(-0.5 * m * m) / math.sqrt(2 * math.pi)
    Phi = 0.5 * np.vectorize(math.erfc)(-m / math.sqrt(2.0))
    f = m * k * phi * Phi ** (k - 1)
    return float(np.trapezoid(f, m))


def underflow_fraction(delta: float, S: float, k_sink: int = 4) -> float:
    """Proposition 1: F(Delta, S) = Phi(Delta + delta_k - 10 ln 2 - ln S) with the mean sink
    maximum plugged in (10 ln 2 = 6.93 is ln of the 2^-10 underflow threshold)."""
    return normal_cdf(delta + expected_max_normal(k_sink) - 10.0 * math.log(2.0) - math.log(S))


def underflow_fraction_rowwise(delta: float, S: float, k_sink: int = 4) -> float:
    """F(Delta, S) averaged over the row's own sink maximum M (density k phi Phi^(k-1)):
    the expectation of the forward-order Monte Carlo statistic."""
    m = np.linspace(-10.0, 10.0, 40001)
    phi = np.exp(-0.5 * m * m) / math.sqrt(2 * math.pi)
    erfc = np.vectorize(math.erfc)
    Phi = 0.5 * erfc(-m / math.sqrt(2.0))
    inner = 0.5 * erfc(-(delta + m - 10.0 * math.log(2.0) - math.log(S)) / math.sqrt(2.0))
    return float(np.trapezoid(inner * k_sink * phi * Phi ** (k_sink - 1), m))


def reverse_underflow_bound(n_tokens: float) -> float:
    """Theorem 4: with reverse order and S = 256, Pr[underflow] = Phi(m - 18 ln 2) with
    m = sqrt(2 ln N) (18 ln 2 = 12.48 = 10 ln 2 + ln 256)."""
    return normal_cdf(math.sqrt(2.0 * math.log(n_tokens)) - 18.0 * math.log(2.0))


def dp(S: float) -> float:
    """Quantisation-step sawtooth dp(S) (Theorem 6): the spacing of the E4M3 grid just below
    S, relative to S, i.e. the largest relative step that p in [0, 1] sees after scaling.
    Reading (the paper gives no formula): c* = smallest code with value >= S;
    dp(S) = (value(c*) - value(c* - 1)) / S."""
    vals = e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    idx = int(np.searchsorted(vals, S, side="left"))
    if idx >= len(vals) or idx == 0:
        raise ValueError("S outside (0, 448]")
    return float((vals[idx] - vals[idx - 1]) / S)
