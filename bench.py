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

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME] [--out-dtype fp32|bf16]
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


def pool_size():
    """Host cores for the oracle leg: this process's CPU affinity, capped at 16
    (the host-core share of one GPU on an 8-GPU MI355X node)."""
    return max(1, min(len(os.sched_getaffinity(0)), 16))


# Decoded inputs of the batch under test, set before the worker processes are
# forked (they inherit it and receive only (sequence, head) indices).
_ORACLE_INPUTS = {}


def _one_thread():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def _oracle_task(task):
    """Forward (and backward) of one (sequence b, query head h) in the fp64
    oracle: per-sequence outputs, dK/dV as head h's share of its KV group."""
    import oracle
    b, h = task
    st = _ORACLE_INPUTS
    wl = st["wl"]
    cq, ck = st["cq"], st["ck"]
    g = h // (wl.heads_q // wl.heads_kv)
    sq, sk = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
    lcq, lck = [0, cq[b + 1] - cq[b]], [0, ck[b + 1] - ck[b]]
    kw = dict(act_param=wl.act_param, mask=wl.mask, window_left=wl.window_left, window_right=wl.window_right)
    q, k, v = st["q"][sq, h:h + 1], st["k"][sk, g:g + 1], st["v"][sk, g:g + 1]
    t0 = time.perf_counter()
    out = {"o": oracle.gdpa_forward(q, k, v, lcq, lck, wl.scale, wl.act, **kw)}
    t1 = time.perf_counter()
    if st["with_bwd"]:
        out["dq"], out["dk"], out["dv"] = oracle.gdpa_backward(q, k, v, st["do"][sq, h:h + 1], lcq, lck, wl.scale,
                                                               wl.act, **kw)
    return b, h, t1 - t0, time.perf_counter() - t1, out


def cpu_baseline(bt: gi.Batch, budget_s: float, gpu=None, workers=None):
    """Time the fp64 oracle (forward + backward) on the batch's leading
    sequences, each (sequence, query head) a task in a pool of `workers`
    single-threaded processes (default pool_size()), until about `budget_s`
    seconds of wall time; report TFLOP/s on the algorithmic flops of the
    sequences processed.

    Returns (baseline record, oracle outputs of the sample).  parity_record()
    compares them with the GPU's outputs."""
    import multiprocessing
    import oracle
    wl = bt.wl
    workers = workers or pool_size()
    pairs = workload_pairs(bt) // max(wl.heads_q, 1)  # per sequence and head
    DV = wl.head_dim_v or wl.head_dim
    with_bwd = bt.do is not None
    dec = oracle.decode_f16 if wl.fp16 else oracle.decode_bf16
    if wl.mx4_qk:
        q, k = oracle.decode_mxfp4(bt.q, bt.q_mx), oracle.decode_mxfp4(bt.k, bt.k_mx)
    elif wl.mx_qk:
        q, k = oracle.decode_mxfp8(bt.q, bt.q_mx), oracle.decode_mxfp8(bt.k, bt.k_mx)
    elif wl.fp8_qk:
        q, k = oracle.decode_e4m3(bt.q, bt.q_scale), oracle.decode_e4m3(bt.k, bt.k_scale)
    else:
        q, k = dec(bt.q), dec(bt.k)
    _ORACLE_INPUTS.clear()
    _ORACLE_INPUTS.update(wl=wl, q=q, k=k, v=dec(bt.v), do=dec(bt.do) if with_bwd else None,
                          cq=bt.cu_seqlens_q, ck=bt.cu_seqlens_k, with_bwd=with_bwd)
    D = wl.head_dim
    per_pair = 2 * (D + DV) + (2 * (3 * D + 2 * DV) if with_bwd else 0)
    wall, t_fwd, t_bwd, flops, nseq = 0.0, 0.0, 0.0, 0, 0
    results = []
    ctx = multiprocessing.get_context("fork")
    with ctx.Pool(workers, initializer=_one_thread) as pool:
        b = 0
        while b < wl.batch and (wall < budget_s or nseq == 0):
            # whole sequences, at least one task per worker
            tasks = []
            while b < wl.batch and len(tasks) < workers:
                tasks += [(b, h) for h in range(wl.heads_q)]
                flops += per_pair * int(pairs[b]) * wl.heads_q
                b += 1
                nseq += 1
            t0 = time.perf_counter()
            res = pool.map(_oracle_task, tasks, chunksize=1)
            wall += time.perf_counter() - t0
            for _, _, tf, tb, _ in res:
                t_fwd += tf
                t_bwd += tb
            results += res
    _ORACLE_INPUTS.clear()
    decoded = {"q": q, "k": k, "v": dec(bt.v), "do": dec(bt.do) if with_bwd else None}
    base = {"value": flops / wall / 1e12, "unit": "TFLOP/s", "cores": int(workers), "kind": "oracle",
            "sample": f"fp64 NumPy oracle, {'forward+backward' if with_bwd else 'forward'} of the first {nseq} "
                      f"of {wl.batch} sequences ({flops / 1e9:.1f} GFLOP algorithmic), one task per "
                      f"(sequence, head) on {workers} single-threaded processes: {wall:.1f} s wall "
                      f"(task time forward {t_fwd:.1f} s, backward {t_bwd:.1f} s)"}
    return base, {"nseq": nseq, "results": results, "decoded": decoded}


def parity_record(bt: gi.Batch, sample, gpu):
    """max |gpu - oracle| / rms(oracle) per output over the oracle leg's
    sequences (all elements); gpu holds host copies of o (and dq, dk, dv).
    For activations whose derivative jumps (ReLU, LeakyReLU, HardSwish), dQ
    and dK errors get the per-element allowance the GPU parity tests give
    scores within rounding of a kink, where the kernel's fp32 score and the
    oracle's fp64 score may fall on different sides."""
    wl = bt.wl
    cq, ck = bt.cu_seqlens_q, bt.cu_seqlens_k
    allow = {}
    if "dq" in gpu:
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        from helpers import kink_allowance, kink_jumps
        if kink_jumps(wl.act, wl.act_param):
            d = sample["decoded"]
            allow["dq"], allow["dk"] = kink_allowance(bt, d["q"], d["k"], d["v"], d["do"])
    group = wl.heads_q // wl.heads_kv
    refs = {}
    for b, h, _, _, out in sample["results"]:
        for name, x in out.items():
            if name in ("o", "dq"):
                refs.setdefault(name, {})[(b, h)] = x[:, 0]
            else:  # dK, dV: sum the group's query heads in head order
                key = (b, h // group)
                acc = refs.setdefault(name, {})
                acc[key] = x[:, 0] if key not in acc else acc[key] + x[:, 0]
    err_rms = {}
    for name, parts in refs.items():
        mx, ss, n = 0.0, 0.0, 0
        for (b, j), ref in parts.items():
            rows = slice(cq[b], cq[b + 1]) if name in ("o", "dq") else slice(ck[b], ck[b + 1])
            got = gpu[name][rows, j].astype(np.float64)
            if ref.size:
                err = np.abs(got - ref)
                if name in allow:
                    err = np.maximum(err - allow[name][rows, j], 0.0)
                mx = max(mx, float(err.max()))
                ss += float((ref * ref).sum())
                n += ref.size
        err_rms[name] = mx / np.sqrt(ss / n) if n and ss > 0 else 0.0
    # 8- and 4-bit Q/K: the forward's bar is the FP8 one; the gradients keep theirs
    tol = {n: (TOL_FP8 if n == "o" and lowp_format(wl) else t) for n, t in TOL.items()}
    return {"sample": f"the first {sample['nseq']} of {wl.batch} sequences against the fp64 oracle, all elements"
                      + (" (dQ, dK: kink allowance)" if allow else ""),
            "err_rms": {n: float(f"{x:.3g}") for n, x in err_rms.items()},
            "tol": {n: tol[n] for n in err_rms},
            "pass": bool(all(err_rms[n] <= tol[n] for n in err_rms))}


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


def lowp_format(wl):
    """The 8- or 4-bit format of Q/K ("fp8", "mxfp8", "mxfp4"), or None."""
    return "mxfp4" if wl.mx4_qk else "mxfp8" if wl.mx_qk else "fp8" if wl.fp8_qk else None


def bwd_dq_path(max_seqlen_k):
    """The backward kernels a call takes (the library's default choice, or
    GDPA_BWD_DQ): dQ inside the dK/dV pass when every sequence's keys fit one
    128-key block, else a separate dQ kernel."""
    mode = os.environ.get("GDPA_BWD_DQ", "")
    if mode == "fused" or (mode != "separate" and max_seqlen_k <= 128):
        return "fused"
    return "separate"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="jagged_self", choices=sorted(gi.WORKLOADS))
    ap.add_argument("--out-dtype", default="fp32", choices=["fp32", "bf16"], help="dtype of O, dQ, dK, dV")
    ap.add_argument("--kernel-reps", type=int, default=20, help="launches per kernel for per-kernel timing")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle wall time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the GDPA kernels here run on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); "
              "GDPA work units are independent per (sequence, head), so more GPUs would each run this "
              "kernel on their own share with no collective.", file=sys.stderr)
        sys.exit(2)

    wl = gi.WORKLOADS[args.workload]
    DV = wl.head_dim_v or wl.head_dim
    # 16-bit workloads are timed forward + backward; 8- and 4-bit Q/K ones
    # forward + backward when the workload asks for it (the FP8 workload of the
    # windowed shape is the README's inference case, forward only)
    fmt = lowp_format(wl)
    with_bwd = wl.backward or fmt is None
    if with_bwd and not wl.backward:
        wl = gi.dataclasses.replace(wl, backward=True)
    if not args.calibrate_copy:
        print(f"[bench] drawing {wl.name} (seed {wl.seed})", file=sys.stderr, flush=True)
        bt = gi.make_batch(wl)
        oracle_sample = None
        if not args.no_cpu_baseline:
            # the oracle leg runs first, in forked worker processes, before
            # this process touches the GPU
            print(f"[bench] timing the CPU oracle baseline ({pool_size()} processes)", file=sys.stderr, flush=True)
            base, oracle_sample = cpu_baseline(bt, args.cpu_budget)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, 20)
        return

    import generalized_attention_amd as g

    pairs = workload_pairs(bt)
    P = int(pairs.sum())
    D = wl.head_dim
    # S and dK, dQ contract or produce Q/K's head dim D, dP and dV V's DV
    fwd_flops, bwd_flops = 2 * (D + DV) * P, (2 * (3 * D + 2 * DV) * P if with_bwd else 0)

    def dev(a, kind):
        t = torch.from_numpy(np.ascontiguousarray(a))
        views = {"bf16": torch.bfloat16, "fp16": torch.float16}
        if kind in views:
            t = t.view(torch.int16).view(views[kind])
        elif kind == "fp8":
            t = t.view(torch.float8_e4m3fn)
        return t.cuda()  # "u8": bytes as they are (MXFP4 pairs, E8M0 scales)

    e16 = "fp16" if wl.fp16 else "bf16"
    qk = {None: e16, "fp8": "fp8", "mxfp8": "fp8", "mxfp4": "u8"}[fmt]
    q, k, v = dev(bt.q, qk), dev(bt.k, qk), dev(bt.v, e16)
    q_mx = dev(bt.q_mx, "u8") if fmt in ("mxfp8", "mxfp4") else None
    k_mx = dev(bt.k_mx, "u8") if fmt in ("mxfp8", "mxfp4") else None
    do = dev(bt.do, e16) if with_bwd else None
    cu_q, cu_k = torch.from_numpy(bt.cu_seqlens_q).cuda(), torch.from_numpy(bt.cu_seqlens_k).cuda()
    odt = torch.float32 if args.out_dtype == "fp32" else torch.bfloat16
    o = torch.empty(q.shape[0], wl.heads_q, DV, dtype=odt, device="cuda")
    dq = torch.empty(q.shape[0], wl.heads_q, D, dtype=odt, device="cuda")
    dk = torch.empty(k.shape[0], wl.heads_kv, D, dtype=odt, device="cuda")
    dv = torch.empty(v.shape, dtype=odt, device="cuda")
    mq, mk = bt.max_seqlen_q, bt.max_seqlen_k
    kw = dict(act=wl.act, act_param=wl.act_param, mask=wl.mask, window_left=wl.window_left,
              window_right=wl.window_right)
    path = bwd_dq_path(mk) if with_bwd else None

    def fwd():
        if fmt == "mxfp4":
            g.gdpa_varlen_fwd_mxfp4(q, q_mx, k, k_mx, v, o, cu_q, cu_k, mq, mk, wl.scale, **kw)
        elif fmt == "mxfp8":
            g.gdpa_varlen_fwd_mxfp8(q, q_mx, k, k_mx, v, o, cu_q, cu_k, mq, mk, wl.scale, **kw)
        else:
            g.gdpa_varlen_fwd(q, k, v, o, cu_q, cu_k, mq, mk, wl.scale, q_descale=bt.q_scale,
                              k_descale=bt.k_scale, **kw)

    def bwd(want_dq=True, want_dkv=True):
        grads = (dq if want_dq else None, dk if want_dkv else None, dv if want_dkv else None)
        if fmt is not None:
            # decodes Q/K to bf16 in the workspace (inside the timing), then the 16-bit kernels
            g.gdpa_varlen_bwd_lowp(q, q_mx, k, k_mx, v, do, *grads, cu_q, cu_k, mq, mk, wl.scale, fmt,
                                   q_descale=bt.q_scale, k_descale=bt.k_scale, **kw)
        else:
            g.gdpa_varlen_bwd(q, k, v, do, *grads, cu_q, cu_k, mq, mk, wl.scale, **kw)

    def step():
        fwd()
        if with_bwd:
            bwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # a 512 MiB write evicts the inputs from L2 and the 256 MB MALL, so that a
    # flushed launch reads them from HBM
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    print(f"[bench] warmup done; timing {args.steps} steps, flushed and warm", file=sys.stderr, flush=True)

    # flushed: the 512 MiB write before every step, outside the timed region
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        flush.fill_(i & 0xFF)
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    flushed = np.array([a.elapsed_time(b) for a, b in evs])
    # warm: the same number of steps back to back
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms_warm = e0.elapsed_time(e1) / args.steps
    ms_step = float(np.median(flushed))

    # per-kernel launch durations (HIP events on the stream the kernels run
    # on), flushed like the steps and warm beside
    stats = {}

    def launch_ms(fn, reps, cold):
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
        cold = launch_ms(fn, reps, True)
        warm = launch_ms(fn, reps, False)
        stats[name] = {"mean": round(float(cold.mean()), 4), "median": round(float(np.median(cold)), 4),
                       "min": round(float(cold.min()), 4), "warm_mean": round(float(warm.mean()), 4),
                       "warm_median": round(float(np.median(warm)), 4)}
        return float(cold.mean())

    # algorithmic work per launch: flops of the products the gradient needs
    # (S, dP, dV, dK in the dK/dV kernel, dQ in the dQ kernel; the dQ kernel's
    # recomputed S and dP are not counted) and the bytes each kernel must move
    # at least (every input read once, every output written once)
    osz = 4 if args.out_dtype == "fp32" else 2
    # bytes per Q/K element: 16-bit, FP8 codes, MX codes plus one E8M0 scale per 32
    qk_b = {None: 2, "fp8": 1, "mxfp8": 1 + 1 / 32, "mxfp4": 0.5 + 1 / 32}[fmt]
    isz = {"q": qk_b, "k": qk_b, "v": 2, "do": 2, "out": osz}
    tq, tk = q.shape[0], k.shape[0]
    nq, nkv = tq * wl.heads_q * D, tk * wl.heads_kv * D
    nqv, nkvv = tq * wl.heads_q * DV, tk * wl.heads_kv * DV  # V- and O-shaped tensors
    kern = {"gdpa_fwd_kernel": (avg_ms(fwd, args.kernel_reps, "gdpa_fwd_kernel"), 2 * (D + DV) * P,
                                nq * isz["q"] + nkv * isz["k"] + nkvv * isz["v"] + nqv * isz["out"])}
    if path == "fused":
        # one kernel: dK, dV and dQ (the call's small schedule and clear kernels are inside the timing)
        kern["gdpa_bwd_fused_kernel"] = (avg_ms(bwd, args.kernel_reps, "gdpa_bwd_fused_kernel"), bwd_flops,
                                         nq * (isz["q"] + isz["out"]) + nqv * isz["do"]
                                         + nkv * (isz["k"] + isz["out"]) + nkvv * (isz["v"] + isz["out"]))
        bwd_ms = kern["gdpa_bwd_fused_kernel"][0]
    elif path == "separate":
        kern["gdpa_bwd_dkdv_kernel"] = (avg_ms(lambda: bwd(False, True), args.kernel_reps, "gdpa_bwd_dkdv_kernel"),
                                        2 * (2 * D + 2 * DV) * P,
                                        nq * isz["q"] + nqv * isz["do"] + nkv * (isz["k"] + isz["out"])
                                        + nkvv * (isz["v"] + isz["out"]))
        kern["gdpa_bwd_dq_kernel"] = (avg_ms(lambda: bwd(True, False), args.kernel_reps, "gdpa_bwd_dq_kernel"),
                                      2 * D * P,
                                      nq * (isz["q"] + isz["out"]) + nqv * isz["do"] + nkv * isz["k"]
                                      + nkvv * isz["v"])
        bwd_ms = kern["gdpa_bwd_dkdv_kernel"][0] + kern["gdpa_bwd_dq_kernel"][0]
    dom = max(kern, key=lambda n: kern[n][0])
    dom_ms, dom_flops, dom_bytes = kern[dom]
    # the roof that binds: the larger of the MFMA and HBM fractions
    mfma_tf = dom_flops / (dom_ms * 1e-3) / 1e12
    hbm_gbs = dom_bytes / (dom_ms * 1e-3) / 1e9
    if hbm_gbs / HBM_PEAK_GBS > mfma_tf / BF16_PEAK_TFLOPS:
        bound, achieved, peak, unit = "hbm", hbm_gbs, HBM_PEAK_GBS, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", mfma_tf, BF16_PEAK_TFLOPS, "TFLOP/s"
    # HBM bytes the counters measured for this kernel, workload and output
    # type with the same kernel sources (profiles/traffic.json); None otherwise
    traffic, traffic_source = None, None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        wrec = rec.get("workloads", {}).get(wl.name, {})
        ent = wrec.get("kernels", {}).get(dom)
        if ent and rec.get("source_hash") == kernel_source_hash() and wrec.get("out_dtype") == args.out_dtype:
            traffic = round(ent["hbm_bytes_per_launch"])
            traffic_source = ("profiles/traffic.json: rocprofv3 FETCH_SIZE and WRITE_SIZE per launch of this kernel "
                              "(bench.py, this workload, the same kernel sources), scaled by the counters of a "
                              "plain 1 GiB device copy")

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
        "dtype": {None: e16, "fp8": "f8", "mxfp8": "mxfp8", "mxfp4": "mxfp4"}[fmt],
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: B={wl.batch} sequences, lengths U[{wl.lq_range[0]},{wl.lq_range[1]}] "
                               f"(drawn total {int(bt.seqlens_q.sum())} tokens), Hq={wl.heads_q}, "
                               f"Hkv={wl.heads_kv}, D={D}, Q/K {fmt or e16}, act={wl.act}, mask={wl.mask}, "
                               f"{'fwd+bwd' if with_bwd else 'fwd'}, {args.out_dtype} outputs",
                   "global_batch": wl.batch, "seq_len": int(bt.max_seqlen_q), "parallelism": "none (1 GPU)"},
        "timing": ("ms_per_step is the median over the timed steps, each after a 512 MiB write outside the "
                   "timed region (inputs read from HBM); ms_per_step_warm runs the same steps back to back"),
        "ms_per_step_warm": round(ms_warm, 4),
        "value_warm": round(total_flops / (ms_warm * 1e-3) / 1e12, 2),
        "ms_per_step_min": round(float(flushed.min()), 4),
        "pct_of_bf16_peak": round(100 * value / BF16_PEAK_TFLOPS, 2),
        "fwd_tflops": round(fwd_flops / (kern["gdpa_fwd_kernel"][0] * 1e-3) / 1e12, 2),
        "bwd_tflops": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 2) if with_bwd else None,
        "bwd_dq_path": path,
        "kernel_ms": {n: round(t[0], 4) for n, t in kern.items()},
        "kernel_ms_stats": stats,
        "roofline": {"kernel": dom, "bound": bound, "achieved": round(achieved, 2), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic,
                     "traffic_source": traffic_source,
                     "achieved_from": f"algorithmic {'bytes' if bound == 'hbm' else 'flops'} per launch / mean "
                                      f"flushed launch time ({args.kernel_reps} launches)"},
    }
    if bound == "mfma" and hbm_gbs > 0:
        result["roofline"]["hbm_gbs"] = round(hbm_gbs, 1)
    # sustained peaks on this GPU, measured after the timed work (context for the
    # published peaks the roofline uses)
    peaks = measured_peaks(torch)
    result["measured_peak"] = peaks
    result["pct_of_measured_bf16_peak"] = round(100 * value / peaks["bf16_tflops"], 2)
    if not args.no_cpu_baseline:
        # the outputs the timed launches wrote (every launch computes the same values)
        torch.cuda.synchronize()
        gpu = {"o": o.float().cpu().numpy()}
        if with_bwd:
            gpu.update(dq=dq.float().cpu().numpy(), dk=dk.float().cpu().numpy(), dv=dv.float().cpu().numpy())
        result["cpu_baseline"] = base
        result["parity"] = parity_record(bt, oracle_sample, gpu)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
