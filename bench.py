#!/usr/bin/env python3
"""GDPA throughput on one MI355X: forward + backward TFLOP/s on the jagged
self-attention workload (64 sequences, lengths uniform in [1, 1024], 4 heads,
head dim 128, FastGELU (tanh GELU), bf16 inputs, fp32 outputs).

One step = the whole hot path over one batch: gdpa_varlen_fwd (O) followed by
gdpa_varlen_bwd (dQ, dK, dV), all launched through the C ABI on one stream,
with every input already resident in HBM.  Prints ONE JSON line.

Flops are algorithmic: only allowed (query, key) pairs count, 4*D per pair and
query head for the forward (Q K^T and P V) and 10*D for the backward (the five
products S, dP, dV, dK, dQ); activation math is not counted.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME] [--cold]
  python bench.py --calibrate-copy 1024     # plain 1 GiB device copy, for PMC scaling
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gdpa_inputs as gi  # noqa: E402

BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def allowed_pairs(lq, lk, wl, wr):
    """Number of allowed (query, key) pairs of one sequence (bottom-right aligned window)."""
    lq, lk = int(lq), int(lk)
    if lq == 0 or lk == 0:
        return 0
    i = np.arange(lq, dtype=np.int64) + (lk - lq)
    lo = np.zeros(lq, np.int64) if wl < 0 else np.maximum(0, i - wl)
    hi = np.full(lq, lk - 1, np.int64) if wr < 0 else np.minimum(lk - 1, i + wr)
    return int(np.maximum(0, hi - lo + 1).sum())


def workload_pairs(bt: gi.Batch):
    wl = bt.wl
    left, right = {"none": (-1, -1), "causal": (-1, 0), "window": (wl.window_left, wl.window_right)}[wl.mask]
    per_seq = [allowed_pairs(a, b, left, right) for a, b in zip(bt.seqlens_q, bt.seqlens_k)]
    return np.array(per_seq, np.int64) * wl.heads_q


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "generalized_attention_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


# parity bars (max |err| / rms(reference)): bf16/fp16 forward, gradients, FP8 forward
TOL = {"o": 2e-2, "dq": 3e-2, "dk": 3e-2, "dv": 3e-2}
TOL_FP8 = 6e-2


def cpu_baseline(bt: gi.Batch, budget_s: float, gpu=None):
    """Time the fp64 oracle (forward + backward) on leading sequences of the same
    batch until about `budget_s` seconds of CPU work; report TFLOP/s on the
    algorithmic flops of the sequences processed.

    With `gpu` (host copies of the outputs the timed kernels wrote: o, and dq,
    dk, dv for a backward workload) it also returns max |gpu - oracle| /
    rms(oracle) per output over the same sequences, outside the timed region."""
    import oracle
    from threadpoolctl import threadpool_info
    wl = bt.wl
    pairs = workload_pairs(bt)
    DV = wl.head_dim_v or wl.head_dim
    with_bwd = not wl.fp8_qk and DV == wl.head_dim and bt.do is not None
    dec = oracle.decode_f16 if wl.fp16 else oracle.decode_bf16
    if wl.fp8_qk:
        q, k = oracle.decode_e4m3(bt.q, bt.q_scale), oracle.decode_e4m3(bt.k, bt.k_scale)
    else:
        q, k = dec(bt.q), dec(bt.k)
    v = dec(bt.v)
    do = dec(bt.do) if with_bwd else None
    cq, ck = bt.cu_seqlens_q, bt.cu_seqlens_k
    t_total, flops, nseq = 0.0, 0, 0
    err = {}  # output -> [max |diff|, sum of ref^2, element count]
    for b in range(wl.batch):
        sq, sk = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
        lcq, lck = [0, cq[b + 1] - cq[b]], [0, ck[b + 1] - ck[b]]
        kw = dict(act_param=wl.act_param, mask=wl.mask, window_left=wl.window_left, window_right=wl.window_right)
        t0 = time.perf_counter()
        refs = {"o": oracle.gdpa_forward(q[sq], k[sk], v[sk], lcq, lck, wl.scale, wl.act, **kw)}
        if with_bwd:
            refs["dq"], refs["dk"], refs["dv"] = oracle.gdpa_backward(q[sq], k[sk], v[sk], do[sq], lcq, lck,
                                                                     wl.scale, wl.act, **kw)
        t_total += time.perf_counter() - t0
        if gpu is not None:
            for name, ref in refs.items():
                got = gpu[name][sq if name in ("o", "dq") else sk]
                e = err.setdefault(name, [0.0, 0.0, 0])
                if ref.size:
                    e[0] = max(e[0], float(np.abs(got.astype(np.float64) - ref).max()))
                    e[1] += float((ref * ref).sum())
                    e[2] += ref.size
        flops += (14 * wl.head_dim if with_bwd else 2 * (wl.head_dim + DV)) * int(pairs[b])
        nseq += 1
        if t_total >= budget_s:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    sample = f"the first {nseq} of {wl.batch} sequences"
    base = {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 NumPy oracle, {'forward+backward' if with_bwd else 'forward'} of {sample} "
                      f"({flops / 1e9:.1f} GFLOP algorithmic) in {t_total:.1f} s"}
    if gpu is None:
        return base, None
    tol = {n: (TOL_FP8 if wl.fp8_qk else t) for n, t in TOL.items()}
    err_rms = {n: e[0] / np.sqrt(e[1] / e[2]) if e[2] and e[1] > 0 else 0.0 for n, e in err.items()}
    parity = {"sample": sample + " against the fp64 oracle, all elements",
              "err_rms": {n: float(f"{x:.3g}") for n, x in err_rms.items()},
              "tol": {n: tol[n] for n in err_rms},
              "pass": bool(all(err_rms[n] <= tol[n] for n in err_rms))}
    return base, parity


def measured_peaks(torch):
    """Sustained dense MFMA rates (bf16 32x32x16, FP8 32x32x64, TFLOP/s) and
    v_exp_f32 rate (lane results per second, in 1e12) over the whole chip from
    the probe kernels in generalized_attention_amd/probe, and the device-copy
    bandwidth (bytes read + written) of a 1 GiB torch copy; best of 5 runs
    each."""
    import ctypes
    path = os.path.join(ROOT, "generalized_attention_amd", "libgdpa_probe.so")
    lib = ctypes.CDLL(path)
    lib.gdpa_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.gdpa_probe_mfma.restype = ctypes.c_double
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 2 * cus  # two 4-wave workgroups per CU: two waves per SIMD
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    for kind, name, iters in ((0, "bf16_tflops", 20000), (1, "fp8_tflops", 10000), (2, "exp2_tops", 4000)):
        best = 0.0
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            flops = lib.gdpa_probe_mfma(kind, ctypes.c_void_p(out.data_ptr()), blocks, iters, stream)
            e1.record()
            torch.cuda.synchronize()
            if flops <= 0:
                raise RuntimeError("probe launch failed")
            best = max(best, flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        res[name] = round(best, 1)
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    best = 0.0
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, 2 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    res["copy_gbs"] = round(best, 1)
    del src, dst
    return res


def calibrate_copy(mib: int, reps: int):
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"calibrate_copy_bytes_read": n, "bytes_written": n, "reps": reps, "ms": ms,
                      "GBps_read_plus_write": 2 * n / ms / 1e6}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="jagged_self", choices=sorted(gi.WORKLOADS))
    ap.add_argument("--kernel-reps", type=int, default=20, help="launches per kernel for per-kernel timing")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold", action="store_true",
                    help="also time each kernel after evicting L2 / MALL (512 MiB write before every launch)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the GDPA kernels here run on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); "
              "GDPA work units are independent per (sequence, head), so more GPUs would each run this "
              "kernel on their own share with no collective.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, 20)
        return

    import generalized_attention_amd as g

    wl = gi.WORKLOADS[args.workload]
    DV = wl.head_dim_v or wl.head_dim
    # FP8 Q/K and distinct V head dims are forward-only paths (the README's FP8
    # support is inference); every other workload is timed forward + backward
    with_bwd = not wl.fp8_qk and DV == wl.head_dim
    if with_bwd and not wl.backward:
        wl = gi.dataclasses.replace(wl, backward=True)
    print(f"[bench] drawing {wl.name} (seed {wl.seed})", file=sys.stderr, flush=True)
    bt = gi.make_batch(wl)
    pairs = workload_pairs(bt)
    P = int(pairs.sum())
    D = wl.head_dim
    fwd_flops, bwd_flops = 2 * (D + DV) * P, (10 * D * P if with_bwd else 0)

    def dev(a, kind):
        t = torch.from_numpy(np.ascontiguousarray(a))
        views = {"bf16": torch.bfloat16, "fp16": torch.float16}
        t = t.view(torch.int16).view(views[kind]) if kind in views else t.view(torch.float8_e4m3fn)
        return t.cuda()

    e16 = "fp16" if wl.fp16 else "bf16"
    qk = "fp8" if wl.fp8_qk else e16
    q, k, v = dev(bt.q, qk), dev(bt.k, qk), dev(bt.v, e16)
    do = dev(bt.do, e16) if with_bwd else None
    cu_q, cu_k = torch.from_numpy(bt.cu_seqlens_q).cuda(), torch.from_numpy(bt.cu_seqlens_k).cuda()
    o = torch.empty(q.shape[0], wl.heads_q, DV, dtype=torch.float32, device="cuda")
    dq = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    dk = torch.empty(k.shape, dtype=torch.float32, device="cuda")
    dv = torch.empty(v.shape, dtype=torch.float32, device="cuda")
    mq, mk = bt.max_seqlen_q, bt.max_seqlen_k
    kw = dict(act=wl.act, act_param=wl.act_param, mask=wl.mask, window_left=wl.window_left,
              window_right=wl.window_right)

    def fwd():
        g.gdpa_varlen_fwd(q, k, v, o, cu_q, cu_k, mq, mk, wl.scale, q_descale=bt.q_scale, k_descale=bt.k_scale,
                          **kw)

    def bwd(want_dq=True, want_dkv=True):
        g.gdpa_varlen_bwd(q, k, v, do, dq if want_dq else None, dk if want_dkv else None,
                          dv if want_dkv else None, cu_q, cu_k, mq, mk, wl.scale, **kw)

    def step():
        fwd()
        if with_bwd:
            bwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done; timing {args.steps} steps", file=sys.stderr, flush=True)

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # per-kernel launch durations (HIP events on the stream the kernels run on):
    # back to back (inputs may stay in L2 / MALL between launches), and with
    # --cold also with a 512 MiB buffer written before every launch, so that
    # the inputs come from HBM
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda") if args.cold else None
    stats = {}

    def launch_ms(fn, reps, cold=False):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i, (a, b) in enumerate(evs):
            if cold:
                flush.fill_(i & 0xFF)
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in evs])

    def avg_ms(fn, reps, name):
        warm = launch_ms(fn, reps)
        stats[name] = {"mean": round(float(warm.mean()), 4), "median": round(float(np.median(warm)), 4),
                       "min": round(float(warm.min()), 4)}
        if args.cold:
            cold = launch_ms(fn, reps, cold=True)
            stats[name].update(cold_median=round(float(np.median(cold)), 4), cold_min=round(float(cold.min()), 4))
        return float(warm.mean())

    # algorithmic work per launch: flops of the products the gradient needs
    # (S, dP, dV, dK in the dK/dV kernel, dQ in the dQ kernel; the dQ kernel's
    # recomputed S and dP are not counted) and the bytes each kernel must move
    # at least (every input read once, every output written once)
    isz = {"q": q.element_size(), "k": k.element_size(), "v": 2, "do": 2, "out": 4}
    tq, tk = q.shape[0], k.shape[0]
    nq, nkv = tq * wl.heads_q * D, tk * wl.heads_kv * D
    nqv, nkvv = tq * wl.heads_q * DV, tk * wl.heads_kv * DV  # V- and O-shaped tensors
    kern = {"gdpa_fwd_kernel": (avg_ms(fwd, args.kernel_reps, "gdpa_fwd_kernel"), 2 * (D + DV) * P,
                                nq * isz["q"] + nkv * isz["k"] + nkvv * isz["v"] + nqv * isz["out"])}
    if with_bwd:
        kern["gdpa_bwd_dkdv_kernel"] = (avg_ms(lambda: bwd(False, True), args.kernel_reps, "gdpa_bwd_dkdv_kernel"),
                                        8 * D * P,
                                        nq * (isz["q"] + isz["do"]) + nkv * (isz["k"] + isz["v"]) + 2 * nkv * isz["out"])
        kern["gdpa_bwd_dq_kernel"] = (avg_ms(lambda: bwd(True, False), args.kernel_reps, "gdpa_bwd_dq_kernel"),
                                      2 * D * P,
                                      nq * (isz["q"] + isz["do"]) + nkv * (isz["k"] + isz["v"]) + nq * isz["out"])
    dom = max(kern, key=lambda n: kern[n][0])
    dom_ms, dom_flops, dom_bytes = kern[dom]
    # the roof that binds: the larger of the MFMA and HBM fractions
    mfma_tf = dom_flops / (dom_ms * 1e-3) / 1e12
    hbm_gbs = dom_bytes / (dom_ms * 1e-3) / 1e9
    if hbm_gbs / HBM_PEAK_GBS > mfma_tf / BF16_PEAK_TFLOPS:
        bound, achieved, peak, unit = "hbm", hbm_gbs, HBM_PEAK_GBS, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", mfma_tf, BF16_PEAK_TFLOPS, "TFLOP/s"
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        ent = rec.get("kernels", {}).get(dom)
        if ent and rec.get("source_hash") == kernel_source_hash() and rec.get("workload") == wl.name:
            traffic = ent["hbm_bytes_per_launch"]

    total_flops = fwd_flops + bwd_flops
    value = total_flops / (ms_step * 1e-3) / 1e12
    result = {
        "metric": "GDPA fwd/bwd TFLOP/s and % of bf16 MFMA peak on one MI355X (jagged)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f8" if wl.fp8_qk else e16,
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: B={wl.batch} sequences, lengths U[{wl.lq_range[0]},{wl.lq_range[1]}] "
                               f"(drawn total {int(bt.seqlens_q.sum())} tokens), Hq={wl.heads_q}, "
                               f"Hkv={wl.heads_kv}, D={D}, act={wl.act}, mask={wl.mask}, "
                               f"{'fwd+bwd' if with_bwd else 'fwd'}, fp32 outputs",
                   "global_batch": wl.batch, "seq_len": int(bt.max_seqlen_q), "parallelism": "none (1 GPU)"},
        "pct_of_bf16_peak": round(100 * value / BF16_PEAK_TFLOPS, 2),
        "fwd_tflops": round(fwd_flops / (kern["gdpa_fwd_kernel"][0] * 1e-3) / 1e12, 2),
        "bwd_tflops": (round(bwd_flops / ((kern["gdpa_bwd_dkdv_kernel"][0] + kern["gdpa_bwd_dq_kernel"][0]) * 1e-3)
                             / 1e12, 2) if with_bwd else None),
        "kernel_ms": {n: round(t[0], 4) for n, t in kern.items()},
        "kernel_ms_stats": stats,
        "roofline": {"kernel": dom, "bound": bound, "achieved": round(achieved, 2), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic},
    }
    # sustained peaks on this GPU, measured after the timed work (context for the
    # published peaks the roofline uses)
    peaks = measured_peaks(torch)
    result["measured_peak"] = peaks
    result["pct_of_measured_bf16_peak"] = round(100 * value / peaks["bf16_tflops"], 2)
    if not args.no_cpu_baseline:
        # the outputs the timed launches wrote (every launch computes the same values)
        torch.cuda.synchronize()
        gpu = {"o": o.cpu().numpy()}
        if with_bwd:
            gpu.update(dq=dq.cpu().numpy(), dk=dk.cpu().numpy(), dv=dv.cpu().numpy())
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"], result["parity"] = cpu_baseline(bt, args.cpu_budget, gpu)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
