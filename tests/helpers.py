"""Shared helpers for the GPU parity tests: move seeded inputs to the device,
run the HIP path through the C-ABI binding, and compare with the fp64 oracle."""
from __future__ import annotations

import numpy as np

import gdpa_inputs as gi
import oracle

TOL_FWD_BF16 = 2e-2   # max|err| <= tol * rms(ref), bf16 inputs
TOL_BWD = 3e-2        # dQ, dK, dV
TOL_FWD_FP8 = 6e-2    # FP8 E4M3 Q/K


def to_dev(arr, dtype_name):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(arr))
    if dtype_name == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    elif dtype_name == "fp16":
        t = t.view(torch.int16).view(torch.float16)
    elif dtype_name == "fp8":
        t = t.view(torch.float8_e4m3fn)
    return t.cuda()


def oracle_inputs(bt: gi.Batch):
    """fp64 values the kernels consume (decoded bf16 / fp16 / E4M3 codes x scale)."""
    dec = oracle.decode_f16 if bt.wl.fp16 else oracle.decode_bf16
    if bt.wl.fp8_qk:
        q = oracle.decode_e4m3(bt.q, bt.q_scale)
        k = oracle.decode_e4m3(bt.k, bt.k_scale)
    else:
        q = dec(bt.q)
        k = dec(bt.k)
    v = dec(bt.v)
    do = dec(bt.do) if bt.do is not None else None
    return q, k, v, do


def mask_kw(wl: gi.Workload):
    return dict(act_param=wl.act_param, mask=wl.mask, window_left=wl.window_left, window_right=wl.window_right)


def device_batch(bt: gi.Batch):
    import torch
    wl = bt.wl
    e16 = "fp16" if wl.fp16 else "bf16"
    qk = "fp8" if wl.fp8_qk else e16
    d = dict(q=to_dev(bt.q, qk), k=to_dev(bt.k, qk), v=to_dev(bt.v, e16),
             cu_q=torch.from_numpy(bt.cu_seqlens_q).cuda(), cu_k=torch.from_numpy(bt.cu_seqlens_k).cuda())
    if bt.do is not None:
        d["do"] = to_dev(bt.do, e16)
    return d


def run_forward(g, bt: gi.Batch, dev=None, out_dtype=None, poison=True):
    """HIP forward through the C ABI; returns the output tensor (on device)."""
    import torch
    wl = bt.wl
    dev = dev or device_batch(bt)
    out_dtype = out_dtype or torch.float32
    tq, H, D = bt.q.shape
    DV = bt.v.shape[2]
    o = torch.full((tq, H, DV), float("nan"), dtype=out_dtype, device="cuda") if poison else \
        torch.empty((tq, H, DV), dtype=out_dtype, device="cuda")
    kw = dict(act=wl.act, act_param=wl.act_param, mask=wl.mask, window_left=wl.window_left,
              window_right=wl.window_right, q_descale=bt.q_scale, k_descale=bt.k_scale)
    if wl.varlen:
        g.gdpa_varlen_fwd(dev["q"], dev["k"], dev["v"], o, dev["cu_q"], dev["cu_k"], bt.max_seqlen_q,
                          bt.max_seqlen_k, wl.scale, **kw)
    else:
        B = wl.batch
        Lq, Lk = int(bt.seqlens_q[0]), int(bt.seqlens_k[0])
        o4 = o.view(B, Lq, H, DV)
        g.gdpa_fwd(dev["q"].view(B, Lq, H, D), dev["k"].view(B, Lk, wl.heads_kv, D),
                   dev["v"].view(B, Lk, wl.heads_kv, DV), o4, wl.scale, **kw)
    return o


def run_backward(g, bt: gi.Batch, dev=None, grad_dtype=None, poison=True):
    import torch
    wl = bt.wl
    dev = dev or device_batch(bt)
    grad_dtype = grad_dtype or torch.float32
    fill = (lambda s: torch.full(s, float("nan"), dtype=grad_dtype, device="cuda")) if poison else \
        (lambda s: torch.empty(s, dtype=grad_dtype, device="cuda"))
    dq, dk, dv = fill(bt.q.shape), fill(bt.k.shape), fill(bt.v.shape)
    kw = dict(act=wl.act, act_param=wl.act_param, mask=wl.mask, window_left=wl.window_left,
              window_right=wl.window_right)
    if wl.varlen:
        g.gdpa_varlen_bwd(dev["q"], dev["k"], dev["v"], dev["do"], dq, dk, dv, dev["cu_q"], dev["cu_k"],
                          bt.max_seqlen_q, bt.max_seqlen_k, wl.scale, **kw)
    else:
        B, H, G, D = wl.batch, wl.heads_q, wl.heads_kv, wl.head_dim
        Lq, Lk = int(bt.seqlens_q[0]), int(bt.seqlens_k[0])
        g.gdpa_bwd(dev["q"].view(B, Lq, H, D), dev["k"].view(B, Lk, G, D), dev["v"].view(B, Lk, G, D),
                   dev["do"].view(B, Lq, H, D), dq.view(B, Lq, H, D), dk.view(B, Lk, G, D), dv.view(B, Lk, G, D),
                   wl.scale, **kw)
    return dq, dk, dv


def err_ratio(got, ref):
    """max|got - ref| / rms(ref); NaN-safe (NaN counts as infinite error)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    if ref.size == 0:
        return 0.0
    if not np.all(np.isfinite(got)):
        return float("inf")
    err = float(np.max(np.abs(got - ref)))
    if rms == 0.0:
        return 0.0 if err == 0.0 else float("inf")
    return err / rms


def sample_rows(cu, heads, n, seed):
    """Deterministic (token, head) sample: first/last token of sampled sequences plus random ones."""
    rng = np.random.default_rng(seed)
    cu = np.asarray(cu, np.int64)
    B = len(cu) - 1
    rows = []
    nonempty = [b for b in range(B) if cu[b + 1] > cu[b]]
    for b in rng.choice(nonempty, size=min(len(nonempty), max(1, n // 4)), replace=False):
        rows.append((int(cu[b]), int(rng.integers(heads))))
        rows.append((int(cu[b + 1] - 1), int(rng.integers(heads))))
    total = int(cu[-1])
    while len(rows) < n and total > 0:
        rows.append((int(rng.integers(total)), int(rng.integers(heads))))
    return rows
