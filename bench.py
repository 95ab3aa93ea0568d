"""Benchmark of the block-scaled FP8 attention forward on one MI355X.

One step = the whole hot path on one batch of synthetic inputs already resident in HBM:
QKV quantisation (fp8attn_quantize_qkv) + attention forward (fp8attn_forward). The metric is
the attention forward's dense-equivalent FLOP count 4 * N^2 * D * H * B divided by the step
time (TFLOP/s). The attention kernel's own time (HIP events around its launches on the stream
it runs on) gives the roofline fraction against the FP8 dense MFMA peak. The CPU oracle is
timed on a bounded sample of the same workload as a reported baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 attn fwd TFLOP/s (4·N²·D·H, dense-equiv) + % of MI355X FP8 MFMA peak"
FP8_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 MFMA (no sparsity)
HBM_PEAK_GBS = 8000.0     # MI355X HBM3E
ATTN_SRC = os.path.join(ROOT, "bit_attention_video_qkv_amd", "csrc", "fp8attn_attn.hip")
# HBM bytes per attention launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated) as measured by
# rocprofv3 for the attention source whose code (comments and blank lines dropped) has this
# sha256 prefix, per workload; see profiles/. Reported only while that code is unchanged.
MEASURED_TRAFFIC = {("e51e0f02b9d9", "wan14b"): 16029482546}


def code_sha(path):
    """sha256 prefix of a source file with // comments and blank lines removed."""
    import hashlib
    import re
    lines = []
    with open(path, encoding="utf-8") as fh:
        for ln in fh.read().splitlines():
            ln = re.sub(r"//.*$", "", ln).rstrip()
            if ln.strip():
                lines.append(ln)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:12]

WORKLOADS = {
    # name: (workloads.py config, sparse, vsmooth+expcast, description)
    "wan14b": ("wan14b", False, False,
               "Wan-14B-720p-shaped dense FP8 attention, B=1 H=40 N=75600 (21x45x80) D=128, "
               "Q/K E4M3 per-64-token block scales, V per-channel scale, S=256, reverse KV order"),
    "wan14b_sparse": ("wan14b", True, False,
                      "Wan-14B-720p-shaped STA block-sparse: grid 21x45x80 padded to 24x48x80, "
                      "tiles (6,8,8), Chebyshev radius 1, N'=92160, H=40, D=128, S=256, reverse"),
    "wan13b": ("wan13b", False, False,
               "Wan-1.3B-480p-shaped dense FP8 attention, B=1 H=12 N=32760 (21x30x52) D=128 with "
               "4 outlier channels x8 per head and tensor, S=256, reverse KV order"),
    "vsmooth": ("vsmooth", False, True,
                "V-Smooth + ExpCast, B=1 H=24 N=49152 D=128, 5% token outliers x20 in V, "
                "16-cluster k-means permutation (reused, not timed), S=256, reverse KV order"),
    "wan14b_local": ("wan14b_local", False, False,
                     "Wan-14B-720p-shaped dense FP8 attention on video-like inputs (logits falling "
                     "off with 3D distance on the 21x45x80 grid), B=1 H=40 N=75600 D=128, S=256, "
                     "reverse KV order"),
    "sink4096": ("sink4096", False, False,
                 "sink stress, B=1 H=8 N=4096 D=128, 4 sink keys with logit offset 9, S=256, "
                 "reverse KV order (256 query tiles: below the machine's width)"),
}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan14b", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=0, help="oracle sample rows (0 = auto)")
    ap.add_argument("--smoothing", type=int, default=0, choices=(0, 1, 2),
                    help="sequence-mean smoothing in the quantisation: 0 none, 1 K, 2 K and V")
    ap.add_argument("--bias-correction", action="store_true",
                    help="with --smoothing 2: the V rounding-bias correction")
    ap.add_argument("--heads", type=int, default=0,
                    help="run only this many heads of the workload (one GPU's share of a head-"
                         "sharded run); 0 = all")
    ap.add_argument("--kv-splits", default="1",
                    help="split-KV pieces: 1 (none), 2..16, or auto (dense workloads)")
    ap.add_argument("--sol-tau", type=float, default=None,
                    help="Sol routing with this threshold multiplier (dense workloads)")
    ap.add_argument("--sol-estimator", type=int, default=0, choices=(0, 1),
                    help="Sol threshold estimator: 0 diag, 1 exact")
    ap.add_argument("--sol-sinks", type=int, default=1, help="Sol: leading KV blocks always exact")
    ap.add_argument("--pcast", default="default", choices=("default", "rne", "expcast"),
                    help="P cast: the standard E4M3 RNE cast of S*exp, or the ExpCast codes "
                         "(default: ExpCast with V-Smooth, as the V-Smooth configuration, else RNE)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the path runs per GPU on its own heads with no "
              "communication, so only --gpus 1 is supported", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_attention_video_qkv_amd as fa
    import workloads

    if args.calibrate_copy:
        calibrate_copy(torch)
        return

    cfg_name, sparse, vs, desc = WORKLOADS[args.workload]
    expcast = vs if args.pcast == "default" else args.pcast == "expcast"
    if expcast != vs:
        desc += "; ExpCast P codes" if expcast else "; standard P cast"
    kv_splits = fa.FP8ATTN_KV_SPLITS_AUTO if args.kv_splits == "auto" else int(args.kv_splits)
    if sparse and kv_splits > 1:
        print("split-KV is for dense workloads", file=sys.stderr)
        sys.exit(2)
    sol = args.sol_tau is not None
    if sol and (sparse or vs or kv_splits != 1):
        print("Sol routing runs on dense workloads without V-Smooth or split-KV", file=sys.stderr)
        sys.exit(2)
    if sol:
        desc += (f"; Sol routing (tau {args.sol_tau}, {'exact' if args.sol_estimator else 'diag'} "
                 f"estimator, {args.sol_sinks} sink blocks)")
    if args.smoothing == 2 and vs:
        print("--smoothing 2 shifts V and cannot be combined with V-Smooth", file=sys.stderr)
        sys.exit(2)
    if args.bias_correction and args.smoothing != 2:
        print("--bias-correction needs --smoothing 2", file=sys.stderr)
        sys.exit(2)
    if args.smoothing:
        desc += (f"; sequence-mean smoothing of {'K' if args.smoothing == 1 else 'K and V'}"
                 + (" with the V bias correction" if args.bias_correction else ""))
    dev = torch.device("cuda:0")
    t0 = time.time()
    q, k, v = workloads.workload(cfg_name, delta=9 if cfg_name == "sink4096" else None,
                                 heads=args.heads or None)
    if args.heads:
        desc += f"; {args.heads} of its heads (one GPU's share)"
    B, N, H, D = q.shape
    log(f"inputs {args.workload} B={B} N={N} H={H} D={D} generated in {time.time() - t0:.1f}s")

    perm_q = perm_kv = sp = out_rows = None
    n_layout, n_out = N, N
    if sparse:
        lay = fa.sta_build(21, 45, 80, 6, 8, 8, 1, 1, 1)
        perm_q = torch.from_numpy(lay["perm"]).to(dev)
        perm_kv = perm_q
        sp = fa.sparse_to_device(lay, dev)
        out_rows = perm_q
        n_layout = lay["perm"].shape[0]
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    del q, k, v
    cluster_ms = prepare_ms = None
    if vs:
        # The V-Smooth cluster permutation is computed once and reused across steps (VC-Attention
        # section 二), so it is timed on its own and not inside the step.
        m_perm = fa.vsmooth_cluster(vd, n_clusters=16, n_feat=8, iters=10)
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        perm_kv = fa.vsmooth_cluster(vd, n_clusters=16, n_feat=8, iters=10)
        c1.record()
        torch.cuda.synchronize()
        cluster_ms = c0.elapsed_time(c1)
        assert torch.equal(perm_kv, m_perm)
        log(f"V-Smooth clustering (16 clusters, 8 channels, 10 rounds): {cluster_ms:.3f} ms, once")
        # the whole preparation of a clustering step in one call (clustering, then the
        # quantisation with the stable scatter fused into the V block statistics), also once
        qz_p = fa.alloc_quantized(B, N, H, True, dev)
        ws_p = fa.vsmooth_prepare_workspace(B, N, H, dev)
        fa.vsmooth_prepare(qd, kd, vd, out=qz_p, workspace=ws_p)
        torch.cuda.synchronize()
        c0.record()
        _, perm_p = fa.vsmooth_prepare(qd, kd, vd, out=qz_p, workspace=ws_p)
        c1.record()
        torch.cuda.synchronize()
        prepare_ms = c0.elapsed_time(c1)
        assert torch.equal(perm_p, perm_kv)
        del qz_p, ws_p
        log(f"V-Smooth clustering step, fused preparation (clustering + quantisation): {prepare_ms:.3f} ms, once")
    qz = fa.alloc_quantized(B, n_layout, H, vs, dev, smoothing=args.smoothing)
    ws_q = fa.quantize_workspace(B, n_layout, H, vs, dev)
    ws_f = fa.forward_workspace(B, n_layout, H, vs, dev, 1 if sparse else kv_splits)
    out = torch.zeros((B, n_out, H, D), dtype=torch.bfloat16, device=dev)
    pcast = fa.FP8ATTN_PCAST_EXPCAST if expcast else fa.FP8ATTN_PCAST_RNE

    ws_sol = fa.sol_workspace(B, n_layout, H, dev) if sol else None

    def step(ev=None):
        fa.quantize_qkv(qd, kd, vd, perm_q=perm_q, perm_kv=perm_kv, vsmooth=vs, n_layout=n_layout,
                        out=qz, workspace=ws_q, smoothing=args.smoothing,
                        v_bias_correction=args.bias_correction)
        if ev is not None:
            ev[0].record()
        if sol:
            fa.sol_forward(qz, tau=args.sol_tau, estimator=args.sol_estimator,
                           sink_blocks=args.sol_sinks, p_scale=256.0, kv_order=fa.FP8ATTN_KV_REVERSE,
                           pcast=pcast, out=out, workspace=ws_sol)
        else:
            fa.forward(qz, p_scale=256.0, kv_order=fa.FP8ATTN_KV_REVERSE, pcast=pcast, sparse=sp,
                       out_rows=out_rows, n_out=n_out, out=out, workspace=ws_f,
                       kv_splits=1 if sparse else kv_splits)
        if ev is not None:
            ev[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(evs[i])
    stop.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps
    ms_attn = sum(a.elapsed_time(b) for a, b in evs) / args.steps

    dense_flops = 4.0 * N * N * D * H * B
    value = dense_flops / (ms_step * 1e-3) / 1e12
    if sparse:
        tl = lay["tile_len"].astype(np.int64)
        rp, ci = lay["row_ptr"], lay["col_idx"]
        pairs = sum(int(tl[u]) * int(tl[ci[rp[u]:rp[u + 1]]].sum()) for u in range(len(tl)))
        attn_flops = 4.0 * pairs * D * H * B   # algorithmic work of the sparse kernel
    elif sol:
        # algorithmic work of Sol: exact-route pairs (4D each), the route QK of every query with
        # every summary (2D) and the summary PV over the non-exact summaries (2D)
        _, mask = fa.sol_forward(qz, tau=args.sol_tau, estimator=args.sol_estimator,
                                 sink_blocks=args.sol_sinks, p_scale=256.0, kv_order=fa.FP8ATTN_KV_REVERSE,
                                 pcast=pcast, out=out, workspace=ws_sol, return_mask=True)
        words = mask.cpu().numpy().view(np.uint64)
        NBk = -(-N // 64)
        bits = ((words[..., :, None] >> np.arange(64, dtype=np.uint64)) & np.uint64(1)).astype(bool)
        bits = bits.reshape(*words.shape[:-1], -1)[..., :NBk]          # [B, H, NB(q), NB(k)]
        rows_q = np.minimum(64, N - 64 * np.arange(NBk))
        keys_k = np.minimum(64, N - 64 * np.arange(NBk))
        exact_pairs = float(np.einsum("bhuj,u,j->", bits.astype(np.float64), rows_q, keys_k))
        summ_rows = float(np.einsum("bhuj,u->", (~bits).astype(np.float64), rows_q))
        attn_flops = 4.0 * exact_pairs * D + 2.0 * N * NBk * D * B * H + 2.0 * summ_rows * D
        sol_exact_frac = float(bits.mean())
        log(f"Sol: {100 * sol_exact_frac:.2f}% of (Q block, KV block) pairs exact")
    else:
        attn_flops = dense_flops
    achieved = attn_flops / (ms_attn * 1e-3) / 1e12
    ms_quant = ms_step - ms_attn
    # quantisation, algorithmic HBM bytes: each of Q, K, V read once as bf16 (2 B per source
    # token, head and channel) and written once as E4M3 (1 B per layout position), plus the FP32
    # scales and (V-Smooth) the bf16 means
    nb = -(-n_layout // 64)
    quant_bytes = (3 * 2 * B * N * H * D + 3 * B * n_layout * H * D + 4 * B * H * (2 * nb + D)
                   + (2 * B * H * -(-n_layout // 128) * D if vs else 0))
    log(f"step {ms_step:.3f} ms, attention kernel {ms_attn:.3f} ms, quantize {ms_quant:.3f} ms "
        f"({quant_bytes / (ms_quant * 1e-3) / 1e9:.0f} GB/s algorithmic)")

    # the counters were taken on the workload's default configuration only
    default_cfg = not (args.heads or sol or args.smoothing or args.kv_splits != "1")
    traffic = MEASURED_TRAFFIC.get((code_sha(ATTN_SRC), args.workload)) if default_cfg else None

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3",
        "data": "synthetic",
        "config": {"workload": desc, "global_batch": B, "seq_len": N, "heads": H, "head_dim": D,
                   "parallelism": "none (one GPU)", "name": args.workload,
                   "smoothing": args.smoothing, "v_bias_correction": args.bias_correction,
                   "kv_splits": args.kv_splits, "pcast": "expcast" if expcast else "rne",
                   "sol": None if not sol else {"tau": args.sol_tau, "estimator": args.sol_estimator,
                                                 "sink_blocks": args.sol_sinks}},
        "quantize_ms": round(ms_quant, 4),
        "quantize": {"ms": round(ms_quant, 4), "algorithmic_bytes": quant_bytes,
                     "achieved_GBps": round(quant_bytes / (ms_quant * 1e-3) / 1e9, 1),
                     "peak_GBps": HBM_PEAK_GBS,
                     "frac": round(quant_bytes / (ms_quant * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / FP8_PEAK_TFLOPS, 4),
                     "traffic": traffic,
                     "traffic_source": ("rocprofv3 FETCH_SIZE + WRITE_SIZE per launch, copy-calibrated, "
                                        "measured on this attention source; profiles/attn_fwd_wan14b_dense.md")
                     if traffic is not None else None,
                     "kernel": "attn_fwd", "kernel_ms": round(ms_attn, 4),
                     "algorithmic_flop_per_launch": attn_flops},
    }

    if cluster_ms is not None:
        result["vsmooth_cluster_ms_once"] = round(cluster_ms, 3)
        result["vsmooth_prepare_ms_once"] = round(prepare_ms, 3)
    if sol:
        result["sol_exact_fraction"] = round(sol_exact_frac, 5)
        result["roofline"]["kernel"] = "fp8attn_sol_forward (all kernels)"
        result["roofline"]["traffic"] = None
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(args, cfg_name, sparse, vs, expcast)
    print(json.dumps(result), flush=True)


def calibrate_copy(torch, nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of known size: its FETCH_SIZE / WRITE_SIZE readings per
    dispatch give the factor that turns those counters into HBM bytes for the other kernels."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    # (the copy's own rate, read + write bytes: what a plain streaming kernel reaches on this HBM)
    print(json.dumps({"calibrate_copy_bytes": nbytes, "reps": reps, "ms_per_copy": round(ms, 4),
                      "copy_GBps": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}), flush=True)


def cpu_baseline(args, cfg_name, sparse, vs, expcast):
    """The oracle as it stands on the host cores: quantisation of one head plus the attention
    of a bounded sample of that head's query rows, scaled to TFLOP/s."""
    import numpy as np

    import oracle
    import workloads

    oracle._load()
    q, k, v = workloads.workload(cfg_name, heads=1, delta=9 if cfg_name == "sink4096" else None)
    B, N, H, D = q.shape
    bq, bk, bv = workloads.bits(q), workloads.bits(k), workloads.bits(v)
    rows_n = args.cpu_rows or 16384
    t0 = time.time()
    if sparse:
        lay = oracle.sta_layout(21, 45, 80, 6, 8, 8, 1, 1, 1)
        qz = oracle.quantize(bq, bk, bv, perm_q=lay["perm"], perm_kv=lay["perm"],
                             smoothing=args.smoothing, v_bias_correction=args.bias_correction)
    else:
        lay = None
        perm_kv = oracle.vsmooth_perm(bv) if vs else None  # the head's cluster order
        qz = oracle.quantize(bq, bk, bv, vsmooth=vs, perm_kv=perm_kv, smoothing=args.smoothing,
                             v_bias_correction=args.bias_correction)
    t_quant = time.time() - t0
    Nl = qz["N"]
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(Nl, rows_n, replace=False)).astype(np.int32)
    t1 = time.time()
    oracle.attention_fp8(qz, rows=rows, kv_reverse=True, expcast=expcast, sparse=lay)
    t_attn = time.time() - t1
    flops = 4.0 * rows_n * N * D            # dense-equivalent work of the sampled rows
    return {"value": round(flops / t_attn / 1e12, 6), "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"sampled: 1 head of {cfg_name}: quantisation of the head ({t_quant:.2f} s, not "
                      f"in value) + attention of {rows_n} seeded random query rows over all {N} keys "
                      f"({t_attn:.2f} s); value = 4*rows*N*D / attention time"}


def cpu_model():
    """The host CPU's model name (Linux), or None."""
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
