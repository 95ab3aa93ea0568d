"""Python binding of libfp8attn (block-scaled FP8 attention forward for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP kernels of
``libfp8attn.so``; PyTorch supplies device memory and the current HIP stream. The entry points
mirror the C ABI in ``include/fp8attn.h``:

* ``quantize_qkv``  -> ``fp8attn_quantize_qkv``
* ``forward``       -> ``fp8attn_forward``
* ``sta_build``     -> ``fp8attn_sta_build`` (host helper)
* ``vsmooth_cluster`` -> ``fp8attn_vsmooth_cluster``
* ``vsmooth_prepare`` -> ``fp8attn_vsmooth_prepare``
* ``sol_forward``   -> ``fp8attn_sol_forward``

There is no fallback: if the library is missing or the device is not gfx950 these calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8attn.so")

FP8ATTN_KV_FORWARD, FP8ATTN_KV_REVERSE = 0, 1
FP8ATTN_PCAST_RNE, FP8ATTN_PCAST_EXPCAST = 0, 1
FP8ATTN_KV_SPLITS_AUTO, FP8ATTN_KV_SPLITS_MAX = -1, 16
HEAD_DIM = 128

_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape or device", 3: "HIP runtime error",
           4: "shape needs more scratch than the no-allocation entry point holds"}
FP8ATTN_ESCRATCH = 4


class Fp8AttnError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)} (status {status})")
        self.status = status


class _QuantArgs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("N_src", ctypes.c_int32), ("N", ctypes.c_int32),
                ("H", ctypes.c_int32), ("D", ctypes.c_int32), ("perm_q", ctypes.c_void_p),
                ("perm_kv", ctypes.c_void_p), ("perm_kv_per_head", ctypes.c_int32),
                ("vsmooth", ctypes.c_int32), ("smoothing", ctypes.c_int32),
                ("v_bias_correction", ctypes.c_int32), ("v_shift", ctypes.c_void_p)]


class _Sparse(ctypes.Structure):
    _fields_ = [("tile_tokens", ctypes.c_int32), ("n_tiles", ctypes.c_int32),
                ("tile_len", ctypes.c_void_p), ("row_ptr", ctypes.c_void_p),
                ("col_idx", ctypes.c_void_p)]


class _SolOpts(ctypes.Structure):
    _fields_ = [("softmax_scale", ctypes.c_float), ("p_scale", ctypes.c_float),
                ("kv_order", ctypes.c_int), ("pcast", ctypes.c_int), ("tau", ctypes.c_float),
                ("estimator", ctypes.c_int32), ("sink_blocks", ctypes.c_int32),
                ("v_shift", ctypes.c_void_p)]


class _FwdOpts(ctypes.Structure):
    _fields_ = [("softmax_scale", ctypes.c_float), ("p_scale", ctypes.c_float),
                ("kv_order", ctypes.c_int), ("pcast", ctypes.c_int),
                ("sparse", ctypes.POINTER(_Sparse)), ("out_rows", ctypes.c_void_p),
                ("n_out", ctypes.c_int32), ("underflow", ctypes.c_void_p),
                ("v_shift", ctypes.c_void_p), ("kv_splits", ctypes.c_int32)]


_lib = None

EXPORTED = ("fp8attn_quantize_qkv", "fp8attn_quantize_workspace_bytes", "fp8attn_forward",
            "fp8attn_forward_workspace_bytes", "fp8attn_sta_build", "fp8attn_status_string",
            "fp8attn_vsmooth_cluster", "fp8attn_vsmooth_cluster_workspace_bytes",
            "fp8attn_sol_forward", "fp8attn_sol_workspace_bytes", "fp8attn_diag_e4m3_encode",
            "fp8attn_diag_e4m3_decode", "fp8attn_diag_mfma_e4m3", "fp8attn_forward_noalloc", "fp8attn_vsmooth_prepare",
            "fp8attn_vsmooth_prepare_workspace_bytes")


def lib():
    """The loaded libfp8attn (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        L.fp8attn_quantize_qkv.restype = ctypes.c_int
        L.fp8attn_quantize_qkv.argtypes = [ctypes.POINTER(_QuantArgs)] + [ctypes.c_void_p] * 11 + [
            ctypes.c_size_t, ctypes.c_void_p]
        L.fp8attn_quantize_workspace_bytes.restype = ctypes.c_size_t
        L.fp8attn_quantize_workspace_bytes.argtypes = [ctypes.c_int32] * 5
        L.fp8attn_forward.restype = ctypes.c_int
        L.fp8attn_forward.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p] * 7 + [
            ctypes.POINTER(_FwdOpts), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
            ctypes.c_void_p]
        L.fp8attn_forward_workspace_bytes.restype = ctypes.c_size_t
        L.fp8attn_forward_workspace_bytes.argtypes = [ctypes.c_int32] * 6
        L.fp8attn_sta_build.restype = ctypes.c_int
        L.fp8attn_sta_build.argtypes = [ctypes.c_int32] * 9 + [ctypes.c_void_p] * 4 + [
            ctypes.c_int32, ctypes.c_void_p]
        L.fp8attn_status_string.restype = ctypes.c_char_p
        L.fp8attn_status_string.argtypes = [ctypes.c_int]
        L.fp8attn_vsmooth_cluster_workspace_bytes.restype = ctypes.c_size_t
        L.fp8attn_vsmooth_cluster_workspace_bytes.argtypes = [ctypes.c_int32] * 5
        L.fp8attn_vsmooth_cluster.restype = ctypes.c_int
        L.fp8attn_vsmooth_cluster.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p] + [ctypes.c_int32] * 3 + [
            ctypes.c_void_p] * 3 + [ctypes.c_size_t, ctypes.c_void_p]
        L.fp8attn_vsmooth_prepare_workspace_bytes.restype = ctypes.c_size_t
        L.fp8attn_vsmooth_prepare_workspace_bytes.argtypes = [ctypes.c_int32] * 5
        L.fp8attn_vsmooth_prepare.restype = ctypes.c_int
        L.fp8attn_vsmooth_prepare.argtypes = [ctypes.POINTER(_QuantArgs)] + [ctypes.c_void_p] * 3 + [
            ctypes.c_int32] * 3 + [ctypes.c_void_p] * 10 + [ctypes.c_size_t, ctypes.c_void_p]
        L.fp8attn_sol_workspace_bytes.restype = ctypes.c_size_t
        L.fp8attn_sol_workspace_bytes.argtypes = [ctypes.c_int32] * 4
        L.fp8attn_sol_forward.restype = ctypes.c_int
        L.fp8attn_sol_forward.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p] * 6 + [
            ctypes.POINTER(_SolOpts), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_size_t, ctypes.c_void_p]
        L.fp8attn_forward_noalloc.restype = ctypes.c_int
        L.fp8attn_forward_noalloc.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p] * 7 + [
            ctypes.POINTER(_FwdOpts), ctypes.c_void_p, ctypes.c_void_p]
        L.fp8attn_diag_e4m3_encode.restype = ctypes.c_int
        L.fp8attn_diag_e4m3_encode.argtypes = [ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        L.fp8attn_diag_e4m3_decode.restype = ctypes.c_int
        L.fp8attn_diag_e4m3_decode.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        L.fp8attn_diag_mfma_e4m3.restype = ctypes.c_int
        L.fp8attn_diag_mfma_e4m3.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int32, ctypes.c_void_p]
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(fn, status):
    if status != 0:
        raise Fp8AttnError(fn, status)


@dataclass
class Quantized:
    """Output of quantize_qkv (device tensors, layout described in include/fp8attn.h)."""
    q8: torch.Tensor
    k8: torch.Tensor
    v8t: torch.Tensor
    q_scale: torch.Tensor
    k_scale: torch.Tensor
    v_scale: torch.Tensor
    v_mean: torch.Tensor | None
    B: int
    N: int
    H: int
    v_shift: torch.Tensor | None = None  # FP32 [B, H, 128] from sequence-mean smoothing (V)


def alloc_quantized(B, N, H, vsmooth, device, smoothing=0):
    NB = (N + 63) // 64
    N64 = NB * 64
    NB128 = (N + 127) // 128
    u8 = dict(dtype=torch.uint8, device=device)
    f32 = dict(dtype=torch.float32, device=device)
    return Quantized(
        q8=torch.empty((B, H, N64, HEAD_DIM), **u8), k8=torch.empty((B, H, N64, HEAD_DIM), **u8),
        v8t=torch.empty((B, H, HEAD_DIM, N64), **u8), q_scale=torch.empty((B, H, NB), **f32),
        k_scale=torch.empty((B, H, NB), **f32), v_scale=torch.empty((B, H, HEAD_DIM), **f32),
        v_mean=torch.empty((B, H, NB128, HEAD_DIM), dtype=torch.int16, device=device) if vsmooth else None,
        B=B, N=N, H=H,
        v_shift=torch.empty((B, H, HEAD_DIM), **f32) if smoothing == 2 else None)


def quantize_workspace(B, N, H, vsmooth, device):
    n = lib().fp8attn_quantize_workspace_bytes(B, N, H, HEAD_DIM, 1 if vsmooth else 0)
    return torch.empty(max(int(n), 256), dtype=torch.uint8, device=device)


def quantize_qkv(q, k, v, perm_q=None, perm_kv=None, vsmooth=False, n_layout=None, out=None,
                 workspace=None, smoothing=0, v_bias_correction=False):
    """q, k, v: bf16 device tensors [B, N_src, H, 128]. perm_q: int32 device [N] or None;
    perm_kv: int32 device [N] (shared by heads) or [B, H, N] or None. smoothing: 0 none, 1 K,
    2 K and V sequence-mean smoothing (then Quantized.v_shift is set; v_bias_correction adds the
    rounding-bias compensation). Returns Quantized."""
    B, Nsrc, H, D = q.shape
    for t in (q, k, v):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.shape != q.shape:
            raise ValueError("q, k, v must be contiguous bf16 tensors of one shape")
    per_head = 0
    if perm_kv is not None:
        per_head = 1 if perm_kv.dim() == 3 else 0
    if n_layout is None:
        n_layout = perm_q.shape[0] if perm_q is not None else (
            perm_kv.shape[-1] if perm_kv is not None else Nsrc)
    N = int(n_layout)
    qz = out if out is not None else alloc_quantized(B, N, H, vsmooth, q.device, smoothing)
    ws = workspace if workspace is not None else quantize_workspace(B, N, H, vsmooth, q.device)
    args = _QuantArgs(B, Nsrc, N, H, D, _ptr(perm_q), _ptr(perm_kv), per_head, 1 if vsmooth else 0,
                      int(smoothing), 1 if v_bias_correction else 0,
                      _ptr(qz.v_shift) if smoothing == 2 else None)
    st = lib().fp8attn_quantize_qkv(
        ctypes.byref(args), _ptr(q), _ptr(k), _ptr(v), _ptr(qz.q8), _ptr(qz.k8), _ptr(qz.v8t),
        _ptr(qz.q_scale), _ptr(qz.k_scale), _ptr(qz.v_scale), _ptr(qz.v_mean) if vsmooth else None,
        _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(q.device))
    _check("fp8attn_quantize_qkv", st)
    return qz


@dataclass
class Sparse:
    """STA descriptor with device arrays (see fp8attn_sparse)."""
    tile_tokens: int
    n_tiles: int
    tile_len: torch.Tensor
    row_ptr: torch.Tensor
    col_idx: torch.Tensor

    def _c(self):
        return _Sparse(self.tile_tokens, self.n_tiles, self.tile_len.data_ptr(),
                       self.row_ptr.data_ptr(), self.col_idx.data_ptr())


def vsmooth_cluster(v, n_clusters=16, n_feat=8, iters=10, labels=False, workspace=None):
    """fp8attn_vsmooth_cluster: V-Smooth token permutation of bf16 V [B, N, H, 128] on its device.
    Returns perm int32 [B, H, N] (and labels int32 [B, H, N] when labels=True); pass perm as
    perm_kv to quantize_qkv."""
    B, N, H, D = v.shape
    dev = v.device
    perm = torch.empty((B, H, N), dtype=torch.int32, device=dev)
    lab = torch.empty((B, H, N), dtype=torch.int32, device=dev) if labels else None
    if workspace is None:
        n = lib().fp8attn_vsmooth_cluster_workspace_bytes(B, N, H, D, n_feat)
        workspace = torch.empty(max(int(n), 256), dtype=torch.uint8, device=dev)
    _check("fp8attn_vsmooth_cluster", lib().fp8attn_vsmooth_cluster(
        B, N, H, D, _ptr(v), n_clusters, n_feat, iters, _ptr(perm), _ptr(lab), _ptr(workspace),
        workspace.numel(), _stream(dev)))
    return (perm, lab) if labels else perm


def vsmooth_prepare_workspace(B, N, H, device, n_feat=8):
    n = lib().fp8attn_vsmooth_prepare_workspace_bytes(B, N, H, HEAD_DIM, n_feat)
    return torch.empty(max(int(n), 256), dtype=torch.uint8, device=device)


def vsmooth_prepare(q, k, v, n_clusters=16, n_feat=8, iters=10, perm_q=None, smoothing=0, labels=False,
                    out=None, workspace=None):
    """fp8attn_vsmooth_prepare: clustering and V-Smooth quantisation of one clustering step, the
    stable scatter fused into the V block statistics. q, k, v: bf16 [B, N, H, 128]; perm_q int32
    [N] or None; smoothing 0 or 1. Returns (Quantized, perm int32 [B, H, N]) and labels when
    labels=True; perm is the perm_kv of quantize_qkv on the reuse steps."""
    B, N, H, D = q.shape
    for t in (q, k, v):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.shape != q.shape:
            raise ValueError("q, k, v must be contiguous bf16 tensors of one shape")
    dev = q.device
    qz = out if out is not None else alloc_quantized(B, N, H, True, dev, smoothing)
    perm = torch.empty((B, H, N), dtype=torch.int32, device=dev)
    lab = torch.empty((B, H, N), dtype=torch.int32, device=dev) if labels else None
    if workspace is None:
        workspace = vsmooth_prepare_workspace(B, N, H, dev, n_feat)
    args = _QuantArgs(B, N, N, H, D, _ptr(perm_q), None, 0, 1, int(smoothing), 0, None)
    _check("fp8attn_vsmooth_prepare", lib().fp8attn_vsmooth_prepare(
        ctypes.byref(args), _ptr(q), _ptr(k), _ptr(v), n_clusters, n_feat, iters, _ptr(perm), _ptr(lab),
        _ptr(qz.q8), _ptr(qz.k8), _ptr(qz.v8t), _ptr(qz.q_scale), _ptr(qz.k_scale), _ptr(qz.v_scale),
        _ptr(qz.v_mean), _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(dev)))
    return (qz, perm, lab) if labels else (qz, perm)


def sta_build(T, Hg, W, tt, th, tw, rt, rh, rw):
    """Host layout helper -> dict of numpy int32 arrays (perm, tile_len, row_ptr, col_idx)."""
    gt, gh, gw = -(-T // tt), -(-Hg // th), -(-W // tw)
    n_tiles, tile = gt * gh * gw, tt * th * tw
    perm = np.zeros(n_tiles * tile, np.int32)
    tile_len = np.zeros(n_tiles, np.int32)
    row_ptr = np.zeros(n_tiles + 1, np.int32)
    nnz = ctypes.c_int32(0)
    L = lib()
    st = L.fp8attn_sta_build(T, Hg, W, tt, th, tw, rt, rh, rw, perm.ctypes.data, tile_len.ctypes.data,
                             row_ptr.ctypes.data, None, 0, ctypes.byref(nnz))
    col_idx = np.zeros(max(nnz.value, 1), np.int32)
    st = L.fp8attn_sta_build(T, Hg, W, tt, th, tw, rt, rh, rw, perm.ctypes.data, tile_len.ctypes.data,
                             row_ptr.ctypes.data, col_idx.ctypes.data, nnz.value, ctypes.byref(nnz))
    _check("fp8attn_sta_build", st)
    return dict(perm=perm, tile_len=tile_len, row_ptr=row_ptr, col_idx=col_idx[:nnz.value],
                tile_tokens=tile, n_tiles=n_tiles)


def sparse_to_device(layout, device):
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return Sparse(int(layout["tile_tokens"]), int(layout["n_tiles"]), to(layout["tile_len"]),
                  to(layout["row_ptr"]), to(layout["col_idx"]))


def forward_workspace(B, N, H, vsmooth, device, kv_splits=1):
    n = int(lib().fp8attn_forward_workspace_bytes(B, N, H, HEAD_DIM, 1 if vsmooth else 0, int(kv_splits)))
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def forward(qz: Quantized, softmax_scale=1.0 / math.sqrt(HEAD_DIM), p_scale=256.0,
            kv_order=FP8ATTN_KV_REVERSE, pcast=FP8ATTN_PCAST_RNE, sparse: Sparse | None = None,
            out_rows=None, n_out=None, underflow=None, out=None, workspace=None, kv_splits=1):
    """Attention forward on quantised operands. Returns bf16 [B, n_out, H, 128] (``out`` when
    given; rows the call does not own keep their previous contents). kv_splits: 1 (no split),
    2..16 or FP8ATTN_KV_SPLITS_AUTO (split-KV, dense only)."""
    B, N, H = qz.B, qz.N, qz.H
    dev = qz.q8.device
    if n_out is None:
        n_out = N
    if out is None:
        out = torch.zeros((B, n_out, H, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    vs = qz.v_mean is not None
    ks = 1 if sparse is not None else int(kv_splits)
    ws = workspace if workspace is not None else forward_workspace(B, N, H, vs, dev, ks)
    sp = sparse._c() if sparse is not None else None
    opts = _FwdOpts(float(softmax_scale), float(p_scale), int(kv_order), int(pcast),
                    ctypes.pointer(sp) if sp is not None else None, _ptr(out_rows), int(n_out),
                    _ptr(underflow), _ptr(qz.v_shift), int(kv_splits))
    st = lib().fp8attn_forward(
        B, N, H, HEAD_DIM, _ptr(qz.q8), _ptr(qz.k8), _ptr(qz.v8t), _ptr(qz.q_scale),
        _ptr(qz.k_scale), _ptr(qz.v_scale), _ptr(qz.v_mean), ctypes.byref(opts), _ptr(out),
        _ptr(ws), ctypes.c_size_t(0 if ws is None else ws.numel()), _stream(dev))
    _check("fp8attn_forward", st)
    return out


def forward_noalloc(qz: Quantized, softmax_scale=1.0 / math.sqrt(HEAD_DIM), p_scale=256.0,
                    kv_order=FP8ATTN_KV_REVERSE, pcast=FP8ATTN_PCAST_RNE, sparse: Sparse | None = None,
                    out_rows=None, n_out=None, underflow=None, out=None, kv_splits=1):
    """fp8attn_forward_noalloc: as ``forward``, with no workspace (the library's static scratch).
    ``out`` must be given when the caller cannot allocate."""
    B, N, H = qz.B, qz.N, qz.H
    dev = qz.q8.device
    if n_out is None:
        n_out = N
    if out is None:
        out = torch.zeros((B, n_out, H, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    sp = sparse._c() if sparse is not None else None
    opts = _FwdOpts(float(softmax_scale), float(p_scale), int(kv_order), int(pcast),
                    ctypes.pointer(sp) if sp is not None else None, _ptr(out_rows), int(n_out),
                    _ptr(underflow), _ptr(qz.v_shift), int(kv_splits))
    st = lib().fp8attn_forward_noalloc(
        B, N, H, HEAD_DIM, _ptr(qz.q8), _ptr(qz.k8), _ptr(qz.v8t), _ptr(qz.q_scale),
        _ptr(qz.k_scale), _ptr(qz.v_scale), _ptr(qz.v_mean), ctypes.byref(opts), _ptr(out), _stream(dev))
    _check("fp8attn_forward_noalloc", st)
    return out


def sol_workspace(B, N, H, device):
    n = int(lib().fp8attn_sol_workspace_bytes(B, N, H, HEAD_DIM))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def sol_forward(qz: Quantized, tau=3.0, estimator=0, sink_blocks=1,
                softmax_scale=1.0 / math.sqrt(HEAD_DIM), p_scale=256.0,
                kv_order=FP8ATTN_KV_REVERSE, pcast=FP8ATTN_PCAST_RNE, out=None, workspace=None,
                return_mask=False):
    """fp8attn_sol_forward: Sol routing attention on quantised operands (layout order, no
    V-Smooth). Returns bf16 [B, N, H, 128], and with return_mask the exact-block mask, uint64
    words [B, H, NB, ceil(NB / 64)] (bit j % 64 of word j // 64: KV block j exact)."""
    if qz.v_mean is not None:
        raise ValueError("Sol routing takes operands quantised without V-Smooth")
    B, N, H = qz.B, qz.N, qz.H
    dev = qz.q8.device
    NB = (N + 63) // 64
    W = (NB + 63) // 64
    if out is None:
        out = torch.empty((B, N, H, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    ws = workspace if workspace is not None else sol_workspace(B, N, H, dev)
    mask = torch.empty((B, H, NB, W), dtype=torch.int64, device=dev) if return_mask else None
    opts = _SolOpts(float(softmax_scale), float(p_scale), int(kv_order), int(pcast), float(tau),
                    int(estimator), int(sink_blocks), _ptr(qz.v_shift))
    st = lib().fp8attn_sol_forward(
        B, N, H, HEAD_DIM, _ptr(qz.q8), _ptr(qz.k8), _ptr(qz.v8t), _ptr(qz.q_scale),
        _ptr(qz.k_scale), _ptr(qz.v_scale), ctypes.byref(opts), _ptr(out), _ptr(mask), _ptr(ws),
        ctypes.c_size_t(ws.numel()), _stream(dev))
    _check("fp8attn_sol_forward", st)
    return (out, mask) if return_mask else out


def diag_e4m3_encode(first_bits, n, out):
    """fp8attn_diag_e4m3_encode: the quantiser's E4M3 codes of the FP32 bit patterns
    first_bits .. first_bits + n - 1 into the uint8 device tensor ``out`` (n a multiple of 4)."""
    if out.dtype != torch.uint8 or out.numel() < n:
        raise ValueError("out must be a uint8 tensor of at least n elements")
    _check("fp8attn_diag_e4m3_encode",
           lib().fp8attn_diag_e4m3_encode(int(first_bits), int(n), _ptr(out), _stream(out.device)))
    return out


def diag_e4m3_decode(codes):
    """fp8attn_diag_e4m3_decode: uint8 device tensor of n codes (n a multiple of 4) -> float32
    [2, n]: row 0 decoded two codes per conversion, row 1 one code per conversion."""
    if codes.dtype != torch.uint8 or codes.dim() != 1 or codes.numel() % 4 != 0:
        raise ValueError("codes must be a 1-D uint8 tensor whose length is a multiple of 4")
    codes = codes.contiguous()
    n = codes.numel()
    out = torch.empty((2, n), dtype=torch.float32, device=codes.device)
    _check("fp8attn_diag_e4m3_decode",
           lib().fp8attn_diag_e4m3_decode(_ptr(codes), n, _ptr(out), _stream(codes.device)))
    return out


def diag_mfma_e4m3(a, bt):
    """fp8attn_diag_mfma_e4m3: a, bt uint8 [T, 32, 64] device tensors (E4M3 codes; bt holds B
    transposed) -> float32 [T, 32, 32], C[t] = A[t] B[t] on the matrix cores."""
    if a.dtype != torch.uint8 or bt.dtype != torch.uint8 or a.shape != bt.shape or a.shape[1:] != (32, 64):
        raise ValueError("a and bt must be uint8 [T, 32, 64]")
    a, bt = a.contiguous(), bt.contiguous()
    c = torch.empty((a.shape[0], 32, 32), dtype=torch.float32, device=a.device)
    _check("fp8attn_diag_mfma_e4m3",
           lib().fp8attn_diag_mfma_e4m3(_ptr(a), _ptr(bt), _ptr(c), int(a.shape[0]), _stream(a.device)))
    return c
