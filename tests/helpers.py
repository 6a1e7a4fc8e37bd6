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
    """fp64 values the kernels consume (decoded bf16 / fp16 / E4M3 codes x scale
    / MXFP8 codes x block scale)."""
    dec = oracle.decode_f16 if bt.wl.fp16 else oracle.decode_bf16
    if bt.wl.mx4_qk:
        q = oracle.decode_mxfp4(bt.q, bt.q_mx)
        k = oracle.decode_mxfp4(bt.k, bt.k_mx)
    elif bt.wl.mx_qk:
        q = oracle.decode_mxfp8(bt.q, bt.q_mx)
        k = oracle.decode_mxfp8(bt.k, bt.k_mx)
    elif bt.wl.fp8_qk:
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
    qk = "fp8" if (wl.fp8_qk or wl.mx_qk) else "u8" if wl.mx4_qk else e16
    d = dict(q=to_dev(bt.q, qk), k=to_dev(bt.k, qk), v=to_dev(bt.v, e16),
             cu_q=torch.from_numpy(bt.cu_seqlens_q).cuda(), cu_k=torch.from_numpy(bt.cu_seqlens_k).cuda())
    if wl.mx_qk or wl.mx4_qk:
        d["q_mx"] = torch.from_numpy(np.ascontiguousarray(bt.q_mx)).cuda()
        d["k_mx"] = torch.from_numpy(np.ascontiguousarray(bt.k_mx)).cuda()
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
    if wl.mx_qk or wl.mx4_qk:
        kw.pop("q_descale"), kw.pop("k_descale")
        fwd_mx = g.gdpa_varlen_fwd_mxfp4 if wl.mx4_qk else g.gdpa_varlen_fwd_mxfp8
        fwd_mx(dev["q"], dev["q_mx"], dev["k"], dev["k_mx"], dev["v"], o, dev["cu_q"], dev["cu_k"],
               bt.max_seqlen_q, bt.max_seqlen_k, wl.scale, **kw)
    elif wl.varlen:
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
    D = wl.head_dim
    dq = fill((bt.q.shape[0], bt.q.shape[1], D))
    dk, dv = fill((bt.k.shape[0], bt.k.shape[1], D)), fill(bt.v.shape)
    kw = dict(act=wl.act, act_param=wl.act_param, mask=wl.mask, window_left=wl.window_left,
              window_right=wl.window_right)
    if wl.fp8_qk or wl.mx_qk or wl.mx4_qk:
        # 8- and 4-bit q/k: the jagged low-precision entry point
        fmt = "mxfp4" if wl.mx4_qk else "mxfp8" if wl.mx_qk else "fp8"
        g.gdpa_varlen_bwd_lowp(dev["q"], dev.get("q_mx"), dev["k"], dev.get("k_mx"), dev["v"], dev["do"], dq, dk, dv,
                               dev["cu_q"], dev["cu_k"], bt.max_seqlen_q, bt.max_seqlen_k, wl.scale, fmt,
                               q_descale=bt.q_scale, k_descale=bt.k_scale, **kw)
    elif wl.varlen:
        g.gdpa_varlen_bwd(dev["q"], dev["k"], dev["v"], dev["do"], dq, dk, dv, dev["cu_q"], dev["cu_k"],
                          bt.max_seqlen_q, bt.max_seqlen_k, wl.scale, **kw)
    else:
        B, H, G, D = wl.batch, wl.heads_q, wl.heads_kv, wl.head_dim
        DV = bt.v.shape[2]
        Lq, Lk = int(bt.seqlens_q[0]), int(bt.seqlens_k[0])
        g.gdpa_bwd(dev["q"].view(B, Lq, H, D), dev["k"].view(B, Lk, G, D), dev["v"].view(B, Lk, G, DV),
                   dev["do"].view(B, Lq, H, DV), dq.view(B, Lq, H, D), dk.view(B, Lk, G, D), dv.view(B, Lk, G, DV),
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


# ------------------------------------------------------------------ kinks
# ReLU, LeakyReLU and HardSwish have derivatives that jump at kinks (0, and
# +-3 for HardSwish).  A score S = scale * q.k computed in fp32 by any
# implementation may land on the other side of a kink from the fp64 value
# when it lies within the fp32 accumulation error of that kink; both one-sided
# derivatives are then correct results of the method in the precision it is
# computed in.  The backward comparisons therefore allow, for each output
# element, the sum over such pairs of |jump| * |dP| times the other operand
# (|K| for dQ, |Q| for dK); dV depends on the activation itself, which is
# continuous, and gets no allowance.  The error bound of a length-D fp32 dot
# product of exactly representable products is gamma_D * sum_d |q_d k_d| with
# gamma_D = D u / (1 - D u), u = 2^-24 (Higham, Accuracy and Stability of
# Numerical Algorithms, 2nd ed., section 3.1); it is doubled here, plus two
# roundings of |S|, for the scaling and the activation's argument.
U32 = 2.0 ** -24


def kink_jumps(act, alpha):
    """(kink, |act'(kink+) - act'(kink-)|) of the activations whose
    derivative is discontinuous."""
    if act == "relu":
        return [(0.0, 1.0)]
    if act == "leaky_relu":
        return [(0.0, abs(1.0 - alpha))]
    if act == "hardswish":
        return [(-3.0, 0.5), (3.0, 0.5)]
    return []


def kink_allowance(bt, q, k, v, do):
    """Per-element extra absolute error (dq, dk) allowed for pairs whose score
    lies within fp32 rounding of a derivative kink (zeros for smooth
    activations).  q, k, v, do: fp64 [tokens, heads, D] as the oracle sees them."""
    wl = bt.wl
    aq, ak = np.zeros(q.shape), np.zeros(k.shape)
    jumps = kink_jumps(wl.act, wl.act_param)
    if not jumps:
        return aq, ak
    D = q.shape[2]
    gamma = D * U32 / (1.0 - D * U32)
    group = wl.heads_q // wl.heads_kv
    cq, ck = bt.cu_seqlens_q, bt.cu_seqlens_k
    for b in range(len(cq) - 1):
        sq, sk = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
        lq, lk = cq[b + 1] - cq[b], ck[b + 1] - ck[b]
        if lq == 0 or lk == 0:
            continue
        allowed = oracle.allowed_mask(lq, lk, wl.mask, wl.window_left, wl.window_right)
        for h in range(wl.heads_q):
            g = h // group
            Q, K, V, dO = q[sq, h], k[sk, g], v[sk, g], do[sq, h]
            s = wl.scale * (Q @ K.T)
            bound = 2.0 * abs(wl.scale) * gamma * (np.abs(Q) @ np.abs(K).T) + 2.0 * U32 * np.abs(s) + 1e-30
            near = np.zeros_like(s)
            for kink, jump in jumps:
                near += np.where(np.abs(s - kink) <= bound, jump, 0.0)
            w = np.where(allowed, near * np.abs(dO @ V.T), 0.0)   # |jump * dP| per ambiguous pair
            if not w.any():
                continue
            aq[sq, h] += abs(wl.scale) * (w @ np.abs(K))
            ak[sk, g] += abs(wl.scale) * (w.T @ np.abs(Q))
    return aq, ak


def err_ratio_allow(got, ref, allow):
    """err_ratio with `allow` (absolute, per element) subtracted from each
    element's error first."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    if not np.all(np.isfinite(got)):
        return float("inf")
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.maximum(np.abs(got - ref) - allow, 0.0)))
    if rms == 0.0:
        return 0.0 if err == 0.0 else float("inf")
    return err / rms


def seq_ratios(got, ref, cu, allow=None):
    """Per sequence b: max|err| / rms(ref) over rows cu[b]:cu[b+1] (each
    sequence against its own rms; empty sequences skipped), with an optional
    per-element allowance."""
    out = {}
    for b in range(len(cu) - 1):
        sl = slice(int(cu[b]), int(cu[b + 1]))
        if cu[b + 1] > cu[b]:
            a = 0.0 if allow is None else allow[sl]
            out[b] = err_ratio_allow(got[sl], ref[sl], a)
    return out


def backward_ratios(bt, dq, dk, dv, refs=None, per_seq=None):
    """max|err| / rms(ref) of dQ, dK, dV against the oracle, with the kink
    allowance above (dV none).  per_seq (a dict) receives the per-sequence
    ratios of each gradient."""
    q, k, v, do = oracle_inputs(bt)
    wl = bt.wl
    if refs is None:
        refs = oracle.gdpa_backward(q, k, v, do, bt.cu_seqlens_q, bt.cu_seqlens_k, wl.scale, wl.act, **mask_kw(wl))
    aq, ak = kink_allowance(bt, q, k, v, do)
    rq, rk, rv = refs
    as_np = lambda t: t if isinstance(t, np.ndarray) else t.float().cpu().double().numpy()
    gq, gk, gv = as_np(dq).reshape(rq.shape), as_np(dk).reshape(rk.shape), as_np(dv).reshape(rv.shape)
    if per_seq is not None:
        per_seq["dq"] = seq_ratios(gq, rq, bt.cu_seqlens_q, aq)
        per_seq["dk"] = seq_ratios(gk, rk, bt.cu_seqlens_k, ak)
        per_seq["dv"] = seq_ratios(gv, rv, bt.cu_seqlens_k)
    return dict(dq=err_ratio_allow(gq, rq, aq), dk=err_ratio_allow(gk, rk, ak), dv=err_ratio(gv, rv))
