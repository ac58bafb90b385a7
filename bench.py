#!/usr/bin/env python3
"""Throughput of the selected-block attention hot path on one MI355X.

Default workload (``bsa_window_128k``, the largest one-GPU configuration):
block-sparse attention forward + backward, BNSD, B=1, N1=N2=8, S=131072,
D=128, bf16, 128x128 blocks; each Q block selects its 8-block sliding
window plus 24 distinct random earlier blocks (258,176 selected pairs).
One step = the whole path over one batch: mask compaction + forward
attention, then dQ (with softmax_grad) + dK/dV reusing the lists.

Prints ONE JSON line.  ``value`` is effective TFLOP/s counted on the
selected blocks only (forward 4*rows*keys*D per selected block pair,
backward 2.5x that), i.e. algorithmic FLOPs / measured step time.  The same
run then times the further workloads named by ``--also`` (by default all
the others but bsa_small) and reports them under ``workloads``; only the
main workload carries the oracle CPU baseline.

Workloads (``--workload``): bsa_window_128k, bsa_causal_8k (B=2, N=16,
S=8192, causal block mask with p=0.25), bsa_small, bsa_tnd_varlen
(block-sparse in TND layout over sequences of 2048, 4096, 8192, 2048 tokens,
16 query / 4 KV heads), nsa_varlen (forward + backward), sfa_decode and
sfa_sharedkv_decode (forward; value in GB/s of algorithmic gathered bytes),
floyd_256 (FloydAttention forward + backward, B=1, H=8, N=M=K=256, D=64).
"""

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # enough untimed steps for the GPU clocks to settle (timing right after a
    # cold start reads several percent slow)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default="bsa_window_128k", choices=WORKLOADS)
    ap.add_argument("--also", default="bsa_causal_8k,bsa_tnd_varlen,nsa_varlen,sfa_decode,"
                    "sfa_sharedkv_decode,floyd_256",
                    help="comma-separated workloads timed after the main one in the same run "
                         "(same steps and warm-up) and reported under 'workloads'; 'none' = "
                         "only the main workload")
    ap.add_argument("--settle-seconds", type=float, default=1.0,
                    help="after the warm-up steps, further untimed steps until this much "
                         "warm-up time has passed (the GPU clocks need about a second of load "
                         "to settle); their count is reported as settle_steps")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured GEMM / copy peaks reported beside the published ones")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample (0 = skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain copy kernel of known size (HBM counter calibration)")
    ap.add_argument("--ingest-copy", metavar="DIR",
                    help="read the copy kernel's FETCH_SIZE / WRITE_SIZE runs (DIR/fetch, "
                         "DIR/write) into profiles/traffic.json (no GPU needed)")
    ap.add_argument("--ingest", metavar="DIR",
                    help="summarise rocprofv3 runs of --workload (DIR/trace, DIR/bench.json, "
                         "DIR/fetch, DIR/write) into profiles/ (no GPU needed)")
    return ap.parse_args()


WORKLOADS = ["bsa_window_128k", "bsa_causal_8k", "bsa_small", "bsa_tnd_varlen", "nsa_varlen",
             "sfa_decode", "sfa_sharedkv_decode", "floyd_256"]


def _warm(step, args):
    """args.warmup untimed steps, then more until args.settle_seconds of
    warm-up have passed.  Returns the number of the extra steps."""
    import torch
    t0 = time.perf_counter()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    extra = 0
    while time.perf_counter() - t0 < args.settle_seconds:
        for _ in range(8):
            step()
        extra += 8
        torch.cuda.synchronize()
    return extra


def _events(n):
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()          # materialise the underlying hipEvent_t
    return evs


def _ev_array(evs):
    arr = (ctypes.c_void_p * len(evs))(*[e.cuda_event for e in evs])
    return arr


# Sources that decide each kernel's memory traffic: a counter summary taken
# before any of them changed no longer describes the kernel.
KERNEL_SOURCES = {
    "bsa_fwd_kernel": ["bsa_fwd.hip"],
    "bsa_dq_kernel": ["bsa_bwd.hip"],
    "bsa_dkdv_kernel": ["bsa_bwd.hip"],
    "nsa_fwd_kernel": ["nsa.hip"],
    "nsa_dq_kernel": ["nsa.hip"],
    "nsa_fwd_grp_kernel": ["nsa.hip"],
    "nsa_dq_grp_kernel": ["nsa.hip"],
    "nsa_dkdv_seg_kernel": ["nsa.hip"],
    "sfa_split_kernel": ["sfa.hip"],
}
COMMON_SOURCES = ["tsa_device.h", "tsa_internal.h"]
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


def _src_hash(kernel):
    h = hashlib.sha256()
    for n in KERNEL_SOURCES[kernel] + COMMON_SOURCES:
        with open(os.path.join(ROOT, "top_selected_attention_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(workload, kernel):
    """HBM bytes per launch of ``kernel`` on ``workload`` from the committed
    rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or
    None when absent or when the kernel's sources changed since it was taken."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    with open(TRAFFIC_JSON) as f:
        ent = json.load(f).get(workload, {}).get(kernel)
    if not ent or kernel not in KERNEL_SOURCES or ent.get("src_hash") != _src_hash(kernel):
        return None
    return ent.get("bytes_per_launch")


# ----------------------------------------------------------------------------
# Block-sparse attention
# ----------------------------------------------------------------------------

CFG_OF = {"bsa_small": 1, "bsa_causal_8k": 2, "bsa_window_128k": 5}


def _pair_flops(mask, bq, bkv, Sq, Skv, D=128):
    """Sum over selected (Q block, KV block) pairs of rows * keys * D."""
    QB, KB = mask.shape[2], mask.shape[3]
    rows = np.minimum(bq, Sq - np.arange(QB) * bq)
    keys = np.minimum(bkv, Skv - np.arange(KB) * bkv)
    sel = (mask != 0).astype(np.float64)
    return float(np.einsum("bnqk,q,k->", sel, rows, keys)) * D


# the library's timed stages of a BSA forward (lists, attention) and backward
# (lists, dQ, the dK/dV kernel, the reduction of split tiles' partials)
BSA_STAGES = ["fwd_lists", "fwd_attention", "bwd_lists", "bwd_dq", "bwd_dkdv", "bwd_dkdv_reduce"]


def bench_bsa(args):
    import torch
    import workloads as W
    import top_selected_attention_amd as tsa

    cfg = CFG_OF[args.workload]
    w, q, k, v, do, mask, scale = W.bsa_inputs(cfg)
    unit = _pair_flops(mask, w["bq"], w["bkv"], w["S"], w["S"])
    fwd_flops, bwd_flops = 4.0 * unit, 10.0 * unit
    dev = torch.device("cuda", 0)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    md = torch.from_numpy(mask).to(dev)
    plan = tsa.BsaPlan(qd, kd, vd, md, w["bq"], w["bkv"], scale, 0)
    plan.set_dout(dod)

    Wm = args.warmup
    stl, ms_step, K, ms_ev = _timed_steps(args, plan, 2, 4)
    st = dict(zip(BSA_STAGES, stl))
    fwd_ms = st["fwd_lists"] + st["fwd_attention"]
    bwd_ms = st["bwd_lists"] + st["bwd_dq"] + st["bwd_dkdv"] + st["bwd_dkdv_reduce"]
    # Per-kernel algorithmic FLOPs per launch, in units of rows*keys*D per
    # selected pair: forward 2 GEMMs (S, PV) = 4; dQ kernel S, dP, dQ = 6;
    # dK/dV kernel S, dP, dV, dK = 8 (the split recomputes S and dP).
    kern = {
        "bsa_fwd_kernel": (st["fwd_attention"], 4.0 * unit),
        "bsa_dq_kernel": (st["bwd_dq"], 6.0 * unit),
        "bsa_dkdv_kernel": (st["bwd_dkdv"], 8.0 * unit),
    }
    dom = max(kern, key=lambda n: kern[n][0])
    dms, dfl = kern[dom]
    achieved = dfl / (dms * 1e-3) / 1e12
    value = (fwd_flops + bwd_flops) / (ms_step * 1e-3) / 1e12
    res = {
        "metric": "effective TFLOP/s on selected blocks (fwd, bwd) and % of bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w["dtype"],
        "data": "synthetic",
        "config": {"workload": w["name"], "layout": "BNSD", "B": w["B"], "N1": w["N1"],
                   "N2": w["N2"], "S": w["S"], "D": w["D"], "block": f"{w['bq']}x{w['bkv']}",
                   "selected_pairs": int((mask != 0).sum()), "sparse_mode": 0},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(fwd_flops / (fwd_ms * 1e-3) / 1e12, 2),
        "bwd_tflops": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 2),
        "stage_ms": {k_: round(v_, 4) for k_, v_ in st.items()},
        "ms_per_step_instrumented": round(ms_ev, 4),
        "step_ms_events": _step_stats(plan.step_ms),
        "ms_per_step_cold": round(plan.cold_ms, 4),
        "settle_steps": plan.settle_steps,
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": _traffic(w["name"], dom)},
    }
    return res, (w, q, k, v, do, mask, scale, unit)


def cpu_baseline_bsa(ctx, seconds):
    """Oracle (float64 numpy) fwd + bwd on a bounded sample of Q blocks."""
    import oracle
    w, q, k, v, do, mask, scale, _ = ctx
    bq, bkv = w["bq"], w["bkv"]
    qn, kn, vn, don = (t.float().numpy() for t in (q, k, v, do))
    QB = mask.shape[2]
    # every 37th Q block in head-major order (37 is prime to the block counts),
    # so the sample mixes heads, positions and list lengths like the workload
    allt = [(b, n, qb) for b in range(w["B"]) for n in range(w["N1"]) for qb in range(QB)]
    order = [allt[(i * 37) % len(allt)] for i in range(len(allt))]
    done, flops = 0, 0.0
    t0 = time.perf_counter()
    for tile in order:
        b, n, qb = tile
        out, _ = oracle.bsa_fwd(qn, kn, vn, mask, bq, bkv, scale, 0, q_tiles=[tile])
        oracle.bsa_bwd(qn, kn, vn, np.nan_to_num(out), don, mask, bq, bkv, scale, 0,
                       q_tiles=[tile])
        rows = min(bq, w["S"] - qb * bq)
        keys = oracle.bsa_keys(mask[b, n, qb], bkv, w["S"]).size
        flops += 14.0 * rows * keys * w["D"]
        done += 1
        if time.perf_counter() - t0 > seconds:
            break
    el = time.perf_counter() - t0
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": _threads(),
            "kind": "oracle",
            "sample": f"{done} of {len(order)} Q blocks (every 37th in head-major order; "
                      f"fwd + bwd, float64) of {w['name']}, {el:.1f} s"}


def _tnd_pair_flops(mask, seqlens, bq, bkv, D=128):
    """Sum over sequences of their selected pairs' rows * keys * D (each
    sequence's own blocks only)."""
    total = 0.0
    for b, L in enumerate(seqlens):
        QB, KB = -(-L // bq), -(-L // bkv)
        total += _pair_flops(mask[b:b + 1, :, :QB, :KB], bq, bkv, L, L, D)
    return total


def bench_bsa_tnd(args):
    import torch
    import workloads as W
    import top_selected_attention_amd as tsa

    w = W.bsa_tnd_workload()
    cu, q, k, v, do, mask = W.bsa_tnd_inputs()
    bq, bkv, scale = w["bq"], w["bkv"], 1.0 / math.sqrt(w["D"])
    unit = _tnd_pair_flops(mask, w["seqlens"], bq, bkv)
    fwd_flops, bwd_flops = 4.0 * unit, 10.0 * unit
    dev = torch.device("cuda", 0)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    plan = tsa.BsaPlan(qd, kd, vd, torch.from_numpy(mask).to(dev), bq, bkv, scale, 0,
                       cu_seqlens_q=cu, cu_seqlens_kv=cu)
    plan.set_dout(dod)
    stl, ms_step, K, ms_ev = _timed_steps(args, plan, 2, 4)
    st = dict(zip(BSA_STAGES, stl))
    fwd_ms = st["fwd_lists"] + st["fwd_attention"]
    bwd_ms = st["bwd_lists"] + st["bwd_dq"] + st["bwd_dkdv"] + st["bwd_dkdv_reduce"]
    kern = {"bsa_fwd_kernel": (st["fwd_attention"], 4.0 * unit),
            "bsa_dq_kernel": (st["bwd_dq"], 6.0 * unit),
            "bsa_dkdv_kernel": (st["bwd_dkdv"], 8.0 * unit)}
    dom = max(kern, key=lambda n: kern[n][0])
    dms, dfl = kern[dom]
    achieved = dfl / (dms * 1e-3) / 1e12
    value = (fwd_flops + bwd_flops) / (ms_step * 1e-3) / 1e12
    res = {
        "metric": "effective TFLOP/s on selected blocks (fwd, bwd) and % of bf16 MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w["dtype"], "data": "synthetic",
        "config": {"workload": w["name"], "layout": "TND", "seqlens": w["seqlens"],
                   "N1": w["N1"], "N2": w["N2"], "D": w["D"], "block": f"{bq}x{bkv}",
                   "selected_pairs": int((mask != 0).sum()), "sparse_mode": 0},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(fwd_flops / (fwd_ms * 1e-3) / 1e12, 2),
        "bwd_tflops": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 2),
        "stage_ms": {k_: round(v_, 4) for k_, v_ in st.items()},
        "ms_per_step_instrumented": round(ms_ev, 4),
        "step_ms_events": _step_stats(plan.step_ms),
        "ms_per_step_cold": round(plan.cold_ms, 4),
        "settle_steps": plan.settle_steps,
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": _traffic(w["name"], dom)},
    }
    return res, (w, cu, q, k, v, do, mask, scale)


def cpu_baseline_bsa_tnd(ctx, seconds):
    """Oracle (float64 numpy) fwd + bwd on a bounded sample of Q tiles."""
    import oracle
    w, cu, q, k, v, do, mask, scale = ctx
    bq, bkv = w["bq"], w["bkv"]
    qn, kn, vn, don = (t.float().numpy() for t in (q, k, v, do))
    tiles = [(b, n, qb) for b, L in enumerate(w["seqlens"]) for n in range(w["N1"])
             for qb in range(-(-L // bq))]
    done, flops = 0, 0.0
    t0 = time.perf_counter()
    for tile in tiles:
        b, n, qb = tile
        out, _ = oracle.bsa_fwd_tnd(qn, kn, vn, mask, cu, cu, bq, bkv, scale, 0, q_tiles=[tile])
        oracle.bsa_bwd_tnd(qn, kn, vn, np.nan_to_num(out), don, mask, cu, cu, bq, bkv, scale, 0,
                           q_tiles=[tile])
        L = w["seqlens"][b]
        rows = min(bq, L - qb * bq)
        keys = oracle.bsa_keys(mask[b, n, qb, :-(-L // bkv)], bkv, L).size
        flops += 14.0 * rows * keys * w["D"]
        done += 1
        if time.perf_counter() - t0 > seconds:
            break
    el = time.perf_counter() - t0
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": _threads(),
            "kind": "oracle",
            "sample": f"{done} of {len(tiles)} Q tiles (fwd + bwd, float64) of {w['name']}, "
                      f"{el:.1f} s"}


# ----------------------------------------------------------------------------
# NSA selected attention
# ----------------------------------------------------------------------------

def bench_nsa(args):
    import torch
    import workloads as W
    import top_selected_attention_amd as tsa

    w = W.nsa_workload()
    cu, q, k, v, do, topk = W.nsa_inputs()
    sbs, G, D = w["sbs"], w["N1"] // w["N2"], w["D"]
    scale = 1.0 / math.sqrt(D)
    # effective (token, KV head, block) triples: blocks not wholly after the token
    pos = np.arange(int(cu[-1])) - np.repeat(cu[:-1], np.diff(cu))
    start = topk.astype(np.int64) * sbs
    kept = start <= pos[:, None, None]
    triples = int(kept.sum())
    unit = float(triples) * G * sbs * D
    # the count above takes a token's own (diagonal) block in full, as the
    # metric's definition does; the keys the causal mask leaves there number
    # pos - start + 1, so the exact count of unmasked keys is a little lower
    exact_keys = float(np.where(kept, np.minimum(sbs, pos[:, None, None] - start + 1), 0).sum())
    fwd_flops, bwd_flops = 4.0 * unit, 10.0 * unit
    dev = torch.device("cuda", 0)
    plan = tsa.NsaPlan(q.to(dev), k.to(dev), v.to(dev), torch.from_numpy(topk).to(dev), cu, cu,
                       sbs, scale, w["sparse_mode"])
    plan.set_dout(do.to(dev))
    st, ms_step, K, ms_ev = _timed_steps(args, plan, 2, 4)
    fwd_ms = st[0] + st[1]
    bwd_ms = st[2] + st[3] + st[4] + st[5]
    # dK/dV: the partial kernel does the 4 GEMMs; the reduction is a separate stage
    # head groups of up to 16 heads of 128 dims run the token-group forward / dQ kernels
    sfx = "_grp" if G <= 16 and D == 128 else ""
    kern = {f"nsa_fwd{sfx}_kernel": (st[1], 4.0 * unit), f"nsa_dq{sfx}_kernel": (st[3], 6.0 * unit),
            "nsa_dkdv_seg_kernel": (st[4], 8.0 * unit)}
    dom = max(kern, key=lambda n: kern[n][0])
    dms, dfl = kern[dom]
    achieved = dfl / (dms * 1e-3) / 1e12
    gathered = triples * sbs * D * 2 * 2      # K and V rows of every kept (token, block)
    # K/V rows the token-group kernels stage per pass: each group of 16
    # consecutive tokens of a sequence loads the union of its tokens' kept
    # blocks once (a block listed twice by one token counted once here)
    T = int(cu[-1])
    seq = np.repeat(np.arange(len(cu) - 1), np.diff(cu))
    grp = (seq.astype(np.int64) << 32) | (pos // 16)
    n2i = np.broadcast_to(np.arange(w["N2"])[None, :, None], topk.shape)
    key = (np.broadcast_to(grp[:, None, None], topk.shape) * w["N2"] + n2i) * (1 << 20) + topk
    staged = int(np.unique(key[kept]).size) * sbs * D * 2 * 2
    value = (fwd_flops + bwd_flops) / (ms_step * 1e-3) / 1e12
    res = {
        "metric": "effective TFLOP/s on selected blocks (fwd, bwd) and % of bf16 MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w["dtype"], "data": "synthetic",
        "config": {"workload": w["name"], "layout": "TND", "seqlens": w["seqlens"],
                   "N1": w["N1"], "N2": w["N2"], "D": D, "sbs": sbs, "sbc": w["sbc"],
                   "sparse_mode": w["sparse_mode"], "effective_triples": triples,
                   "flop_count": "4*G*sbs*D per kept (token, KV head, block), the own block "
                                 "in full; value_unmasked_keys counts only keys the causal "
                                 "mask leaves"},
        "value_unmasked_keys": round(value * exact_keys / (triples * sbs), 2),
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(fwd_flops / (fwd_ms * 1e-3) / 1e12, 2),
        "bwd_tflops": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 2),
        "stage_ms": dict(zip(["fwd_lists", "fwd_attention", "bwd_lists", "bwd_dq", "bwd_dkdv",
                              "bwd_dkdv_reduce"], [round(x, 4) for x in st])),
        "ms_per_step_instrumented": round(ms_ev, 4),
        "step_ms_events": _step_stats(plan.step_ms),
        "ms_per_step_cold": round(plan.cold_ms, 4),
        "settle_steps": plan.settle_steps,
        "fwd_kv_rows_GBps": round(gathered / (st[1] * 1e-3) / 1e9, 1),
        "fwd_staged_GBps": round(staged / (st[1] * 1e-3) / 1e9, 1),
        "fwd_staged_bytes": staged,
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": _traffic(w["name"], dom)},
    }
    return res, (w, cu, q, k, v, do, topk, scale, sbs, G, D)


def cpu_baseline_nsa(ctx, seconds):
    import oracle
    w, cu, q, k, v, do, topk, scale, sbs, G, D = ctx
    qn, kn, vn, don = (t.float().numpy() for t in (q, k, v, do))
    T = int(cu[-1])
    done, flops = 0, 0.0
    t0 = time.perf_counter()
    step = 97                                   # tokens spread over all sequences
    for t in list(range(0, T, step)):
        out, _ = oracle.nsa_fwd(qn, kn, vn, topk, cu, cu, sbs, scale, 2, tokens=[t])
        oracle.nsa_bwd(qn, kn, vn, np.nan_to_num(out), don, topk, cu, cu, sbs, scale, 2,
                       tokens=[t])
        b = int(np.searchsorted(cu, t, side="right") - 1)
        p_ = t - int(cu[b])
        eff = int((topk[t].astype(np.int64) * sbs <= p_).sum())
        flops += 14.0 * eff * G * sbs * D
        done += 1
        if time.perf_counter() - t0 > seconds:
            break
    el = time.perf_counter() - t0
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": _threads(),
            "kind": "oracle",
            "sample": f"{done} tokens (every {step}th, both KV heads, fwd + bwd, float64) of "
                      f"{w['name']}, {el:.1f} s"}


# ----------------------------------------------------------------------------
# Paged sparse flash attention decode
# ----------------------------------------------------------------------------

def _sfa_bytes(idx, kv_lens, B, Sq, N1, D, Dr, Dv):
    """Algorithmic HBM bytes: per sequence the union of its tokens' selected rows
    (key row + rope row; the value row is the key row), plus Q, q_rope, O, LSE,
    indices and the page-table entries read."""
    rows = 0
    for b in range(B):
        sel = idx[b].reshape(-1)
        sel = sel[(sel >= 0) & (sel < kv_lens[b])]
        rows += np.unique(sel).size
    per_tok = N1 * (D + Dr) * 2 + N1 * Dv * 2 + N1 * 4 + idx.shape[-1] * 4 * 2
    return rows * (D + Dr) * 2 + B * Sq * per_tok


def _time_forward(plan, n_stages, args):
    """Warm-up, K plain forward calls timed by the wall clock between
    synchronisations (the throughput), then K more with events around each
    stage on the library's stream, then five cache-cold calls.  Returns (ms
    per plain step, ms per instrumented step, [mean ms of each stage], per-step
    event ms, median cold ms)."""
    import torch
    K = args.steps
    plan.settle_steps = _warm(plan.fwd, args)
    wall0 = time.perf_counter()
    for _ in range(K):
        plan.fwd()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - wall0) * 1e3 / K
    # a second run of K steps with stage events (kept out of the throughput)
    evs = [_events(2 * n_stages) for _ in range(K)]
    arrs = [_ev_array(e) for e in evs]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(K):
        plan.a.n_events = n_stages
        plan.a.events = ctypes.cast(arrs[i], ctypes.POINTER(ctypes.c_void_p))
        plan.fwd()
    torch.cuda.synchronize()
    ms_ev = (time.perf_counter() - wall0) * 1e3 / K
    plan.a.n_events = 0
    step_ms = [e[0].elapsed_time(e[2 * n_stages - 1]) for e in evs]
    stages = [sum(e[2 * j].elapsed_time(e[2 * j + 1]) for e in evs) / K for j in range(n_stages)]
    cold_ms = _cold_steps(plan.fwd)
    return ms_step, ms_ev, stages, step_ms, cold_ms


def bench_sfa(args):
    import torch
    import workloads as W
    import top_selected_attention_amd as tsa

    w = W.sfa_workload()
    q, qr, kc, krc, bt, kv_lens, idx = W.sfa_inputs()
    scale = 1.0 / math.sqrt(w["D"] + w["Dr"])
    dev = torch.device("cuda", 0)
    kcd = kc.to(dev)
    plan = tsa.SfaPlan(q.to(dev), qr.to(dev), kcd, krc.to(dev), kcd, torch.from_numpy(bt).to(dev),
                       torch.from_numpy(kv_lens).to(dev), torch.from_numpy(idx).to(dev), scale, 3)
    nbytes = _sfa_bytes(idx, kv_lens, w["B"], w["Sq"], w["N1"], w["D"], w["Dr"], w["D"])
    flops = 2.0 * w["B"] * w["Sq"] * w["N1"] * w["topk"] * ((w["D"] + w["Dr"]) + w["D"])
    K = args.steps
    ms_step, ms_ev, (split_ms, comb_ms), step_ms, cold_ms = _time_forward(plan, 2, args)
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    kgbs = nbytes / (split_ms * 1e-3) / 1e9
    res = {
        "metric": "GB/s of algorithmic HBM bytes (paged top-k gather) and % of HBM peak",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w["dtype"], "data": "synthetic",
        "config": {"workload": w["name"], "B": w["B"], "Sq": w["Sq"], "N1": w["N1"], "N2": 1,
                   "D": w["D"], "Dr": w["Dr"], "page": w["page"], "kv_len": w["kv_len"],
                   "topk": w["topk"]},
        "pct_of_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "effective_tflops": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "stage_ms": {"split_attention": round(split_ms, 4), "combine": round(comb_ms, 4)},
        "ms_per_step_instrumented": round(ms_ev, 4),
        "step_ms_events": _step_stats(step_ms),
        "ms_per_step_cold": round(cold_ms, 4),
        "settle_steps": plan.settle_steps,
        "algorithmic_bytes": int(nbytes),
        "roofline": {"kernel": "sfa_split_kernel", "bound": "hbm", "achieved": round(kgbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(kgbs / PEAK_HBM_GBS, 4),
                     "traffic": _traffic(w["name"], "sfa_split_kernel")},
    }
    return res, (w, q, qr, kc, krc, bt, kv_lens, idx, scale, nbytes)


def cpu_baseline_sfa(ctx, seconds):
    import oracle
    w, q, qr, kc, krc, bt, kv_lens, idx, scale, nbytes = ctx
    qn, qrn = q.float().numpy(), qr.float().numpy()
    kcn, krcn = kc.float().numpy(), krc.float().numpy()
    tokens = [(b, s) for b in range(w["B"]) for s in range(w["Sq"])]
    done = 0
    t0 = time.perf_counter()
    for tkn in tokens:
        oracle.sfa_fwd(qn, qrn, kcn, krcn, kcn, bt, kv_lens, idx, scale, 3, tokens=[tkn])
        done += 1
        if time.perf_counter() - t0 > seconds:
            break
    el = time.perf_counter() - t0
    per_tok = nbytes / len(tokens)
    return {"value": round(per_tok * done / el / 1e9, 4), "unit": "GB/s", "cores": _threads(),
            "kind": "oracle",
            "sample": f"{done} of {len(tokens)} decode tokens (float64) of {w['name']}, {el:.1f} s"}


def _skv_bytes_and_keys(cu, kv_lens, idx, w):
    """Algorithmic HBM bytes of the shared-KV decode: per sequence the union of
    its tokens' band rows and the union of their kept compressed rows (key +
    rope row each; the value row is the key row), plus per token Q, q_rope, O,
    LSE, the top-k ids and one page-table entry per slot.  Also the kept keys
    summed over tokens (for the FLOP count)."""
    D, Dr, N1, K = w["D"], w["Dr"], w["N1"], w["cmp_topk"]
    win = w["win_left"] + w["win_right"] + 1
    rows, kept = 0, 0
    for b in range(len(kv_lens)):
        n, sq = int(kv_lens[b]), int(cu[b + 1] - cu[b])
        cl = n // w["cmp_ratio"]
        band, ids = set(), set()
        for s in range(sq):
            p = n - sq + s
            pos = range(max(0, p - w["win_left"]), min(n, p + w["win_right"] + 1))
            band.update(pos)
            sel = idx[cu[b] + s, 0]
            sel = sel[(sel >= 0) & (sel < cl) & (sel <= cl - sq + s)]
            ids.update(sel.tolist())
            kept += len(pos) + sel.size
        rows += len(band) + len(ids)
    T = int(cu[-1])
    per_tok = N1 * (D + Dr) * 2 + N1 * D * 2 + N1 * 4 + K * 4 + (win + K) * 4
    return rows * (D + Dr) * 2 + T * per_tok, kept


def bench_sfa_skv(args):
    import torch
    import workloads as W
    import top_selected_attention_amd as tsa

    w = W.sfa_sharedkv_workload()
    cu, q, qr, kv_lens, ori, cmp = W.sfa_sharedkv_inputs()
    scale = 1.0 / math.sqrt(w["D"] + w["Dr"])
    dev = torch.device("cuda", 0)
    ori_d = tuple(torch.as_tensor(t).to(dev) for t in ori)
    cmp_d = tuple(torch.as_tensor(t).to(dev) for t in cmp)
    plan = tsa.SfaSharedkvPlan(q.to(dev), qr.to(dev), torch.from_numpy(kv_lens).to(dev), ori_d,
                               cmp_d, scale, w["win_left"], w["win_right"], w["cmp_ratio"],
                               cu_seqlens_q=cu)
    nbytes, kept = _skv_bytes_and_keys(cu, kv_lens, cmp[3], w)
    flops = 2.0 * w["N1"] * kept * ((w["D"] + w["Dr"]) + w["D"])
    K = args.steps
    ms_step, ms_ev, (task_ms, split_ms, comb_ms), step_ms, cold_ms = _time_forward(plan, 3, args)
    # every layer of a decode step after the first reuses one task list
    plan.metadata()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for _ in range(K):
        plan.fwd()
    torch.cuda.synchronize()
    ms_reuse = (time.perf_counter() - wall0) * 1e3 / K
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    kgbs = nbytes / (split_ms * 1e-3) / 1e9
    res = {
        "metric": "GB/s of algorithmic HBM bytes (band + compressed top-k gather) and % of HBM "
                  "peak",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w["dtype"], "data": "synthetic",
        "config": {"workload": w["name"], "layout_q": "TND", "B": w["B"], "Sq": w["Sq"],
                   "N1": w["N1"], "N2": 1, "D": w["D"], "Dr": w["Dr"], "page": w["page"],
                   "kv_len": w["kv_len"], "win_left": w["win_left"], "win_right": w["win_right"],
                   "cmp_ratio": w["cmp_ratio"], "cmp_topk": w["cmp_topk"]},
        "pct_of_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "effective_tflops": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "stage_ms": {"task_list": round(task_ms, 4), "split_attention": round(split_ms, 4),
                     "combine": round(comb_ms, 4)},
        "ms_per_step_reusing_task_list": round(ms_reuse, 4),
        "ms_per_step_instrumented": round(ms_ev, 4),
        "step_ms_events": _step_stats(step_ms),
        "ms_per_step_cold": round(cold_ms, 4),
        "settle_steps": plan.settle_steps,
        "algorithmic_bytes": int(nbytes),
        "roofline": {"kernel": "sfa_split_kernel", "bound": "hbm", "achieved": round(kgbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(kgbs / PEAK_HBM_GBS, 4),
                     "traffic": _traffic(w["name"], "sfa_split_kernel")},
    }
    return res, (w, cu, q, qr, kv_lens, ori, cmp, scale, nbytes)


def cpu_baseline_sfa_skv(ctx, seconds):
    import oracle
    w, cu, q, qr, kv_lens, ori, cmp, scale, nbytes = ctx
    f = lambda t: t.float().numpy() if hasattr(t, "float") else t  # noqa: E731
    qn, qrn = q.float().numpy(), qr.float().numpy()
    orin, cmpn = tuple(f(t) for t in ori), tuple(f(t) for t in cmp)
    T = int(cu[-1])
    done = 0
    t0 = time.perf_counter()
    for t in range(T):
        oracle.sfa_sharedkv_fwd(qn, qrn, cu, kv_lens, scale, ori=orin, cmp=cmpn,
                                win_left=w["win_left"], win_right=w["win_right"],
                                cmp_ratio=w["cmp_ratio"], tokens=[t])
        done += 1
        if time.perf_counter() - t0 > seconds:
            break
    el = time.perf_counter() - t0
    return {"value": round(nbytes / T * done / el / 1e9, 4), "unit": "GB/s", "cores": _threads(),
            "kind": "oracle",
            "sample": f"{done} of {T} decode tokens (float64) of {w['name']}, {el:.1f} s"}


# ----------------------------------------------------------------------------
# FloydAttention
# ----------------------------------------------------------------------------

def bench_floyd(args):
    import torch
    import workloads as W
    import top_selected_attention_amd as tsa

    w = W.floyd_workload()
    q, k1, v1, k2, v2, do = W.floyd_inputs()
    scale = 1.0 / math.sqrt(w["D"])
    dev = torch.device("cuda", 0)
    plan = tsa.FloydPlan(*(t.to(dev) for t in (q, k1, v1, k2, v2)), scale=scale)
    plan.set_dout(do.to(dev))
    # one GEMM term: 2 * N * M * K * D per head; forward 4 terms (S over n and
    # over m, P V1, P V2), backward the method's 10 (S, dP, dV, dQ, dK, each
    # over n and over m)
    term = 2.0 * w["B"] * w["H"] * w["N"] * w["M"] * w["K"] * w["D"]
    fwd_flops, bwd_flops = 4.0 * term, 10.0 * term
    st, ms_step, K, ms_ev = _timed_steps(args, plan, 3, 5)
    fwd_ms, bwd_ms = sum(st[:3]), sum(st[3:])
    names = ["fwd_scores", "fwd_softmax", "fwd_pv", "bwd_scores_dp", "bwd_p_ds", "bwd_dv",
             "bwd_dq", "bwd_dk"]
    stage = dict(zip(names, st))
    # dominant stage: the backward scores and dP (four GEMM terms).  With
    # D = 64 these products write 4 bytes of fp32 score per 2*D FLOP, so the
    # stage is bound by HBM: algorithmic bytes = its six operand tensors read
    # once (q, k1, k2, dY, v1, v2) + S and dP written once in fp32.
    rl_ms = stage["bwd_scores_dp"]
    elems_in = w["B"] * w["H"] * w["N"] * w["M"] * w["D"]        # q and dY
    elems_kv = w["B"] * w["H"] * (w["N"] + w["M"]) * w["K"] * w["D"]  # k1 + k2, v1 + v2
    scores = w["B"] * w["H"] * w["N"] * w["M"] * w["K"]
    rl_bytes = 2.0 * (2 * elems_in + 2 * elems_kv) + 2 * 4.0 * scores
    achieved = rl_bytes / (rl_ms * 1e-3) / 1e9
    value = (fwd_flops + bwd_flops) / (ms_step * 1e-3) / 1e12
    res = {
        "metric": "effective TFLOP/s on selected blocks (fwd, bwd) and % of bf16 MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w["dtype"], "data": "synthetic",
        "config": {"workload": w["name"], "B": w["B"], "H": w["H"], "N": w["N"], "M": w["M"],
                   "K": w["K"], "D": w["D"],
                   "flop_count": "2*N*M*K*D per GEMM term and head; forward 4 terms, backward 10"},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(fwd_flops / (fwd_ms * 1e-3) / 1e12, 2),
        "bwd_tflops": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 2),
        "stage_ms": {k_: round(v_, 4) for k_, v_ in stage.items()},
        "ms_per_step_instrumented": round(ms_ev, 4),
        "step_ms_events": _step_stats(plan.step_ms),
        "ms_per_step_cold": round(plan.cold_ms, 4),
        "settle_steps": plan.settle_steps,
        "roofline": {"kernel": "floyd_gemm_kernel", "stage": "backward scores and dP",
                     "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "bytes_per_launch": int(rl_bytes)},
    }
    return res, (w, q, k1, v1, k2, v2, do, scale, term)


def cpu_baseline_floyd(ctx, seconds):
    """Oracle (float64 numpy) fwd + bwd, one head at a time."""
    import oracle
    w, q, k1, v1, k2, v2, do, scale, term = ctx
    f = [t.float().numpy() for t in (q, k1, v1, k2, v2, do)]
    done = 0
    t0 = time.perf_counter()
    for h in range(w["H"]):
        s_ = (slice(0, 1), slice(h, h + 1))
        args = [x[s_] for x in f[:5]]
        y, _ = oracle.floyd_fwd(*args, scale)
        oracle.floyd_bwd(*args, y, f[5][s_], scale)
        done += 1
        if time.perf_counter() - t0 > seconds:
            break
    el = time.perf_counter() - t0
    per_head = 14.0 * term / (w["B"] * w["H"])
    return {"value": round(per_head * done / el / 1e12, 6), "unit": "TFLOP/s", "cores": _threads(),
            "kind": "oracle",
            "sample": f"{done} of {w['H']} heads (fwd + bwd, float64) of {w['name']}, {el:.1f} s"}


def _flush_buffer():
    """512 MiB that one write sweeps through L2 (8 x 4 MiB) and MALL (256 MiB)."""
    import torch
    return torch.empty(128 << 20, dtype=torch.float32, device="cuda")


def _cold_steps(step, n=5):
    """Median ms of ``n`` steps, each right after a 512 MiB write that evicts
    the caches (HIP events around the step only)."""
    import torch
    buf = _flush_buffer()
    ts = []
    for i in range(n):
        buf.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del buf
    return float(np.median(ts))


def _step_stats(ms):
    return {"median": round(float(np.median(ms)), 4), "min": round(float(np.min(ms)), 4)}


def measured_peaks():
    """What this machine sustains, beside the published peaks: the library's own
    MFMA issue and HBM copy / read kernels (libtsa_peaks.so; the read also of
    a buffer the memory-side cache holds), and
    torch.matmul (hipBLASLt) of two 8192 x 8192 bf16 matrices."""
    import torch
    from top_selected_attention_amd import peaks

    res = peaks.measure()
    a = torch.randn(8192, 8192, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(8192, 8192, dtype=torch.bfloat16, device="cuda")
    ms = peaks._timed(lambda: torch.matmul(a, b), 20)
    res["hipblaslt_bf16_gemm_tflops"] = round(2 * 8192 ** 3 / (ms * 1e-3) / 1e12, 1)
    res["how"] = ("MFMA: 4 independent 32x32x16 chains per wave, 2048 x 256 threads; "
                  "HBM: 1 GiB with nontemporal 16-byte loads / stores, 8192 x 256 threads, copy "
                  "counts read + write; MALL: 160 MiB read with plain 16-byte loads after "
                  "warm-up reads (past the L2s, inside the memory-side cache); GEMM: "
                  "torch.matmul 8192^3 bf16")
    return res


def _timed_steps(args, plan, nf, nb):
    """Warm up, time K plain fwd+bwd steps (the throughput), then time K more
    with HIP events recorded around every stage on the library's stream (the
    per-kernel durations): event records add host and device work per step,
    so they stay out of the throughput region.  Returns (stage ms list [fwd
    stages..., bwd stages...], wall ms per plain step, K, wall ms per
    instrumented step)."""
    import torch
    K = args.steps

    def fb():
        plan.fwd()
        plan.bwd()
    plan.settle_steps = _warm(fb, args)
    wall0 = time.perf_counter()
    for _ in range(K):
        plan.fwd()
        plan.bwd()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - wall0) * 1e3 / K

    fev = [_events(2 * nf) for _ in range(K)]
    bev = [_events(2 * nb) for _ in range(K)]
    farr = [_ev_array(e) for e in fev]
    barr = [_ev_array(e) for e in bev]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(K):
        plan.fa.n_events, plan.fa.events = nf, ctypes.cast(farr[i], ctypes.POINTER(ctypes.c_void_p))
        plan.ba.n_events, plan.ba.events = nb, ctypes.cast(barr[i], ctypes.POINTER(ctypes.c_void_p))
        plan.fwd()
        plan.bwd()
    torch.cuda.synchronize()
    ms_ev = (time.perf_counter() - wall0) * 1e3 / K
    plan.fa.n_events = plan.ba.n_events = 0
    st = [sum(e[2 * j].elapsed_time(e[2 * j + 1]) for e in fev) / K for j in range(nf)]
    st += [sum(e[2 * j].elapsed_time(e[2 * j + 1]) for e in bev) / K for j in range(nb)]
    # per-step GPU time from the first stage's start to the last stage's end
    plan.step_ms = [f[0].elapsed_time(b_[2 * nb - 1]) for f, b_ in zip(fev, bev)]

    def step():
        plan.fwd()
        plan.bwd()
    plan.cold_ms = _cold_steps(step)
    return st, ms_step, K, ms_ev


# ----------------------------------------------------------------------------
# rocprofv3 summaries under profiles/
# ----------------------------------------------------------------------------

COPY_BYTES = 256 << 20   # the calibration kernel reads and writes this many bytes per launch


def copy_calibration():
    """Three launches of a plain elementwise copy (torch.neg, float32) that
    read COPY_BYTES and write COPY_BYTES each: what FETCH_SIZE / WRITE_SIZE
    report for a kernel of known HBM traffic."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_BYTES, "launches": 3}), flush=True)


def _csv_rows(d, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _short(name):
    """'void tsa::bsa_dkdv_kernel<tsa::BF16, 4>(...)' -> 'bsa_dkdv_kernel'."""
    n = name.split("(")[0].replace("void ", "").strip().split("<")[0]
    return n.split("::")[-1]


def _counter_means(d, counter, match=None):
    """Kernel short name (or the kernels whose full name contains ``match``)
    -> mean counter value per dispatch, in the counter's unit (KiB)."""
    acc = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        name = r["Kernel_Name"]
        if match is not None:
            if match not in name:
                continue
            key = match
        else:
            key = _short(name)
        acc.setdefault(key, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def _load_traffic():
    if os.path.exists(TRAFFIC_JSON):
        with open(TRAFFIC_JSON) as f:
            return json.load(f)
    return {}


def _save_traffic(t):
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(t, f, indent=1, sort_keys=True)
        f.write("\n")


def ingest_copy(d):
    """FETCH_SIZE / WRITE_SIZE calibration factors from the copy kernel's
    counter runs under d/fetch and d/write."""
    fk = _counter_means(os.path.join(d, "fetch"), "FETCH_SIZE", "neg_kernel")["neg_kernel"]
    wk = _counter_means(os.path.join(d, "write"), "WRITE_SIZE", "neg_kernel")["neg_kernel"]
    t = _load_traffic()
    t["_calibration"] = {
        "copy_bytes": COPY_BYTES, "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
        "fetch_factor": COPY_BYTES / (fk * 1024.0), "write_factor": COPY_BYTES / (wk * 1024.0)}
    _save_traffic(t)
    print(json.dumps(t["_calibration"]))


def ingest(d, workload):
    """Writes profiles/<dominant kernel>_<workload>.md from the kernel trace
    under d/trace (with the bench line the traced run printed, d/bench.json)
    and the counter runs under d/fetch, d/write (and, when present, the MFMA
    counter run under d/mfma); records each library kernel's calibrated HBM
    bytes per launch in profiles/traffic.json."""
    tr = {}
    for r in _csv_rows(os.path.join(d, "trace"), "kernel_trace.csv"):
        name = r["Kernel_Name"]
        if "tsa::" not in name:
            continue
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        tr.setdefault(_short(name), []).append(us)
    bench = None
    with open(os.path.join(d, "bench.json")) as f:
        for line in f:
            if line.startswith("{"):
                bench = json.loads(line)
    fetch = _counter_means(os.path.join(d, "fetch"), "FETCH_SIZE")
    write = _counter_means(os.path.join(d, "write"), "WRITE_SIZE")
    t = _load_traffic()
    cal = t["_calibration"]
    total = sum(sum(v) for v in tr.values())
    dom = bench["roofline"]["kernel"]
    entries = t.setdefault(workload, {})
    lines = []
    for k in sorted(tr, key=lambda k: -sum(tr[k])):
        v = tr[k]
        fb = fetch.get(k, 0.0) * 1024 * cal["fetch_factor"]
        wb = write.get(k, 0.0) * 1024 * cal["write_factor"]
        lines.append(f"| `{k}` | {len(v)} | {sum(v) / len(v):.1f} | {min(v):.1f} | {max(v):.1f} | "
                     f"{100 * sum(v) / total:.1f} | {fetch.get(k, 0.0):.0f} | {write.get(k, 0.0):.0f} | "
                     f"{(fb + wb) / 1e6:.2f} |")
        if k in KERNEL_SOURCES:
            entries[k] = {"src_hash": _src_hash(k), "fetch_kib": round(fetch.get(k, 0.0), 1),
                          "write_kib": round(write.get(k, 0.0), 1),
                          "bytes_per_launch": int(round(fb + wb)),
                          "avg_us_kernel_trace": round(sum(v) / len(v), 1)}
    _save_traffic(t)
    mdir = os.path.join(d, "mfma")
    mlines = []
    if os.path.isdir(mdir):
        util = _counter_means(mdir, "MfmaUtil")
        fbf = _counter_means(mdir, "MfmaFlopsBF16")
        ffp = _counter_means(mdir, "MfmaFlopsF16")
        for k in sorted(tr, key=lambda k: -sum(tr[k])):
            fl = fbf.get(k, 0.0) + ffp.get(k, 0.0)
            if fl > 0:
                mlines.append(f"| `{k}` | {util.get(k, 0.0):.1f} | {fl / 1e9:.2f} |")
    rl = bench["roofline"]
    cmd = (f"python3 bench.py --workload {workload} --also none --steps {bench['steps']} "
           f"--warmup {bench['warmup']} --settle-seconds 0 --cpu-seconds 0 --no-peaks")
    pcmd = (f"python3 bench.py --workload {workload} --also none --steps 2 --warmup 1 "
            f"--settle-seconds 0 --cpu-seconds 0 --no-peaks")
    d = os.path.normpath(d)
    cdir = os.path.join(os.path.dirname(d), "copy")   # the copy calibration beside it
    out = [
        f"# {dom} on {workload}: rocprofv3 kernel trace and HBM counters",
        "",
        f"Workload: `{json.dumps(bench['config'])}`.",
        "",
        "Commands (repository root, one MI355X; `cd /tmp && export TMPDIR=/tmp` first, then back):",
        "",
        "```",
        f"rocprofv3 --kernel-trace --stats --output-format csv -d {d}/trace -o run -- {cmd} > {d}/bench.json",
        f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/fetch -o run -- {pcmd}",
        f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/write -o run -- {pcmd}",
    ] + ([f"rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 MfmaFlopsF16 --output-format csv -d {d}/mfma "
          f"-o run -- {pcmd}"] if mlines else []) + [
        f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {cdir}/fetch -o run -- python3 bench.py --copy-calibration",
        f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {cdir}/write -o run -- python3 bench.py --copy-calibration",
        f"python3 bench.py --ingest-copy {cdir}",
        f"python3 bench.py --ingest {d} --workload {workload}",
        "```",
        "",
        "Kernel trace: every call of the traced run (warm-up included).  FETCH / WRITE: mean "
        "KiB per dispatch from the two counter runs; HBM MB = FETCH x "
        f"{cal['fetch_factor']:.4f} + WRITE x {cal['write_factor']:.4f} (the factors make a "
        f"plain copy of {COPY_BYTES >> 20} MiB read as {COPY_BYTES >> 20} MiB each way: it "
        f"reads {cal['fetch_kib']:.0f} / {cal['write_kib']:.0f} KiB).",
        "",
        "| kernel | calls | avg (us) | min (us) | max (us) | % of library GPU time | FETCH (KiB) | WRITE (KiB) | HBM MB / launch |",
        "|---|---|---|---|---|---|---|---|---|",
    ] + lines + [
        "",
        f"bench.py's own HIP-event stage times in the traced run (ms): `{json.dumps(bench['stage_ms'])}`.",
        "",
        f"Dominant kernel `{dom}`: {rl['achieved']} {rl['unit']} by the bench's events "
        f"(roofline fraction {rl['frac']} of {rl['peak']} {rl['unit']}); its kernel-trace average "
        f"above is the duration to compare.",
        "",
        f"Bench line of the traced run: value {bench['value']} {bench['unit']}, "
        f"{bench['ms_per_step']} ms per step.",
        "",
    ]
    if mlines:
        out += [
            "MFMA counters (mean per dispatch): MfmaUtil = MFMA-busy cycles summed over the "
            "SIMDs / (GPU-active cycles x SIMD count) x 100; MFMA GFLOP = the issued MFMA "
            "operations (SQ_INSTS_VALU_MFMA_MOPS_BF16 + _F16, 512 FLOP each), masked and "
            "padded work included.",
            "",
            "| kernel | MfmaUtil (%) | MFMA GFLOP / launch |",
            "|---|---|---|",
        ] + mlines + [""]
    path = os.path.join(ROOT, "profiles", f"{dom}_{workload}.md")
    with open(path, "w") as f:
        f.write("\n".join(out))
    print(path)


def _threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return 1


def _host():
    """The host the oracle baseline ran on: CPU model and the cores this
    process may use."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0))}


def main():
    args = parse()
    if args.ingest_copy:
        ingest_copy(args.ingest_copy)
        return
    if args.ingest:
        ingest(args.ingest, args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path shards by KV head / batch with no exchange, so per-GPU throughput "
              "is the single-GPU figure", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    res, ctx = run_workload(args.workload, args)
    if args.cpu_seconds > 0:
        res["cpu_baseline"] = CPU_BASELINE[_kind(args.workload)](ctx, args.cpu_seconds)
        res["cpu_baseline"].update(_host())
    del ctx
    also = [] if args.also in ("", "none") else [x for x in args.also.split(",") if x]
    for name in also:
        if name not in WORKLOADS:
            print(f"unknown workload {name!r} in --also", file=sys.stderr)
            sys.exit(2)
    extra = {}
    for name in also:
        if name == args.workload:
            continue
        torch.cuda.empty_cache()
        r, c = run_workload(name, args)
        del c
        extra[name] = {k_: r[k_] for k_ in EXTRA_KEYS if k_ in r}
        print(f"# {name}: {r['value']} {r['unit']}", file=sys.stderr, flush=True)
    if extra:
        res["workloads"] = extra
    if not args.no_peaks:
        res["measured_peaks"] = measured_peaks()
    print(json.dumps(res), flush=True)


# what the line carries for each further workload
EXTRA_KEYS = ["metric", "value", "unit", "ms_per_step", "dtype", "config", "pct_of_bf16_peak",
              "pct_of_hbm_peak", "fwd_tflops", "bwd_tflops", "effective_tflops", "stage_ms",
              "ms_per_step_cold", "settle_steps", "roofline"]


def _kind(name):
    return "bsa" if name in CFG_OF else name


BENCH = {"bsa": bench_bsa, "bsa_tnd_varlen": bench_bsa_tnd, "nsa_varlen": bench_nsa,
         "sfa_decode": bench_sfa, "sfa_sharedkv_decode": bench_sfa_skv, "floyd_256": bench_floyd}
CPU_BASELINE = {"bsa": cpu_baseline_bsa, "bsa_tnd_varlen": cpu_baseline_bsa_tnd,
                "nsa_varlen": cpu_baseline_nsa, "sfa_decode": cpu_baseline_sfa,
                "sfa_sharedkv_decode": cpu_baseline_sfa_skv, "floyd_256": cpu_baseline_floyd}


def run_workload(name, args):
    """Times one workload; returns (bench line dict, context for the oracle baseline)."""
    import argparse
    a = argparse.Namespace(**vars(args))
    a.workload = name
    return BENCH[_kind(name)](a)


if __name__ == "__main__":
    main()
