"""GDPA forward and backward, written out as the plain definition in fp64.

Test infrastructure (see the package docstring).

Layout (FlashAttention's varlen convention, which the GDPA README's
"CUTE-DSL" usage example follows with cu_seqlens_q/k and max_seqlen_q/k):
q [total_q, Hq, D], k/v [total_k, Hkv, D], cu_seqlens int prefix sums [B+1].
Sequence b owns rows cu[b]..cu[b+1]-1.  Fixed-length [B, L, H, D] tensors are
the special case cu[b] = b*L, reshaped.

Readings of points the pages leave open (each is listed in the design notes):
  * masked pairs contribute exactly zero: P = M * act(S) (an additive -inf
    would give act(-inf) = -inf for identity/LeakyReLU and NaN for GELU/SiLU);
  * no row normalisation of any kind (the README replaces softmax by the
    activation and names nothing else);
  * the scale multiplies Q K^T inside the activation, act(scale * Q K^T);
  * GQA: query head h reads KV head h // (Hq // Hkv);
  * causal masks align bottom-right: query i of a sequence with Lq queries and
    Lk keys may see key j iff j <= i + (Lk - Lq);
  * a sliding window (window_left, window_right) allows
    i' - window_left <= j <= i' + window_right with i' = i + Lk - Lq;
    -1 means unbounded on that side; causal = (-1, 0), none = (-1, -1).
"""
from __future__ import annotations

import numpy as np

from .activations import act, act_grad


def window_bounds(mask: str, window_left: int = -1, window_right: int = -1):
    if mask == "none":
        return -1, -1
    if mask == "causal":
        return -1, 0
    if mask == "window":
        return int(window_left), int(window_right)
    raise ValueError(f"unknown mask {mask!r}")


def allowed_mask(lq: int, lk: int, mask: str = "none", window_left: int = -1,
                 window_right: int = -1) -> np.ndarray:
    """Boolean [lq, lk]: True where query i may attend key j."""
    wl, wr = window_bounds(mask, window_left, window_right)
    i = np.arange(lq)[:, None] + (lk - lq)
    j = np.arange(lk)[None, :]
    ok = np.ones((lq, lk), dtype=bool)
    if wl >= 0:
        ok &= j >= i - wl
    if wr >= 0:
        ok &= j <= i + wr
    return ok


def _check(q, k, v, cu_q, cu_k, hq, hkv):
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3:
        raise ValueError("q, k, v must be [tokens, heads, dim]")
    if q.shape[1] != hq or k.shape[1] != hkv or v.shape[1] != hkv:
        raise ValueError("head counts do not match tensor shapes")
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if len(cu_q) != len(cu_k):
        raise ValueError("cu_seqlens_q and cu_seqlens_k differ in length")


def gdpa_forward(q, k, v, cu_seqlens_q, cu_seqlens_k, scale, act_name,
                 act_param=0.01, mask="none", window_left=-1, window_right=-1):
    """O[total_q, Hq, D] = per sequence and head, M*act(scale Q K^T) V (fp64)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    hq, hkv = q.shape[1], k.shape[1]
    cu_q = np.asarray(cu_seqlens_q, np.int64)
    cu_k = np.asarray(cu_seqlens_k, np.int64)
    _check(q, k, v, cu_q, cu_k, hq, hkv)
    group = hq // hkv
    o = np.zeros((q.shape[0], hq, v.shape[2]), np.float64)
    for b in range(len(cu_q) - 1):
        qs, qe, ks, ke = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        if qe == qs:
            continue
        m = allowed_mask(qe - qs, ke - ks, mask, window_left, window_right)
        for h in range(hq):
            g = h // group
            s = scale * (q[qs:qe, h, :] @ k[ks:ke, g, :].T)
            p = np.where(m, act(act_name, s, act_param), 0.0)
            o[qs:qe, h, :] = p @ v[ks:ke, g, :]
    return o


def gdpa_backward(q, k, v, do, cu_seqlens_q, cu_seqlens_k, scale, act_name,
                  act_param=0.01, mask="none", window_left=-1, window_right=-1):
    """(dQ, dK, dV) of L = sum(O * dO) for the forward above (fp64).

    dP = dO V^T, dS = M * act'(S) * dP, dQ = scale dS K, dK = scale dS^T Q
    (summed over the query heads of a KV group), dV = P^T dO (same sum).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    hq, hkv = q.shape[1], k.shape[1]
    cu_q = np.asarray(cu_seqlens_q, np.int64)
    cu_k = np.asarray(cu_seqlens_k, np.int64)
    _check(q, k, v, cu_q, cu_k, hq, hkv)
    group = hq // hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(len(cu_q) - 1):
        qs, qe, ks, ke = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        if qe == qs or ke == ks:
            continue
        m = allowed_mask(qe - qs, ke - ks, mask, window_left, window_right)
        for h in range(hq):
            g = h // group
            qh, kg, vg, doh = q[qs:qe, h, :], k[ks:ke, g, :], v[ks:ke, g, :], do[qs:qe, h, :]
            s = scale * (qh @ kg.T)
            p = np.where(m, act(act_name, s, act_param), 0.0)
            dp = doh @ vg.T
            ds = np.where(m, act_grad(act_name, s, act_param) * dp, 0.0)
            dq[qs:qe, h, :] = scale * (ds @ kg)
            dk[ks:ke, g, :] += scale * (ds.T @ qh)
            dv[ks:ke, g, :] += p.T @ doh
    return dq, dk, dv


def _seq_of(cu, t):
    return int(np.searchsorted(cu, t, side="right") - 1)


def gdpa_forward_rows(q, k, v, cu_seqlens_q, cu_seqlens_k, scale, act_name, rows,
                      act_param=0.01, mask="none", window_left=-1, window_right=-1):
    """O[t, h, :] for each (t, h) in `rows`, one row at a time (for large problems)."""
    cu_q = np.asarray(cu_seqlens_q, np.int64)
    cu_k = np.asarray(cu_seqlens_k, np.int64)
    hq, hkv = q.shape[1], k.shape[1]
    group = hq // hkv
    out = np.zeros((len(rows), v.shape[2]), np.float64)
    for r, (t, h) in enumerate(rows):
        b = _seq_of(cu_q, t)
        i = t - cu_q[b]
        lq, ks, ke = cu_q[b + 1] - cu_q[b], cu_k[b], cu_k[b + 1]
        g = h // group
        kg = np.asarray(k[ks:ke, g, :], np.float64)
        vg = np.asarray(v[ks:ke, g, :], np.float64)
        s = scale * (kg @ np.asarray(q[t, h, :], np.float64))
        m = allowed_mask(lq, ke - ks, mask, window_left, window_right)[i]
        p = np.where(m, act(act_name, s, act_param), 0.0)
        out[r] = p @ vg
    return out


def gdpa_backward_q_rows(q, k, v, do, cu_seqlens_q, cu_seqlens_k, scale, act_name, rows,
                         act_param=0.01, mask="none", window_left=-1, window_right=-1):
    """dQ[t, h, :] for each (t, h) in `rows`, one row at a time."""
    cu_q = np.asarray(cu_seqlens_q, np.int64)
    cu_k = np.asarray(cu_seqlens_k, np.int64)
    hq, hkv = q.shape[1], k.shape[1]
    group = hq // hkv
    out = np.zeros((len(rows), q.shape[2]), np.float64)
    for r, (t, h) in enumerate(rows):
        b = _seq_of(cu_q, t)
        i = t - cu_q[b]
        lq, ks, ke = cu_q[b + 1] - cu_q[b], cu_k[b], cu_k[b + 1]
        g = h // group
        kg = np.asarray(k[ks:ke, g, :], np.float64)
        vg = np.asarray(v[ks:ke, g, :], np.float64)
        s = scale * (kg @ np.asarray(q[t, h, :], np.float64))
        dp = vg @ np.asarray(do[t, h, :], np.float64)
        m = allowed_mask(lq, ke - ks, mask, window_left, window_right)[i]
        ds = np.where(m, act_grad(act_name, s, act_param) * dp, 0.0)
        out[r] = scale * (ds @ kg)
    return out


def gdpa_backward_k_rows(q, k, v, do, cu_seqlens_q, cu_seqlens_k, scale, act_name, rows,
                         act_param=0.01, mask="none", window_left=-1, window_right=-1):
    """(dK[t, g, :], dV[t, g, :]) for each KV row (t, g) in `rows`, one at a time."""
    cu_q = np.asarray(cu_seqlens_q, np.int64)
    cu_k = np.asarray(cu_seqlens_k, np.int64)
    hq, hkv = q.shape[1], k.shape[1]
    group = hq // hkv
    dk = np.zeros((len(rows), k.shape[2]), np.float64)
    dv = np.zeros((len(rows), v.shape[2]), np.float64)
    for r, (t, g) in enumerate(rows):
        b = _seq_of(cu_k, t)
        j = t - cu_k[b]
        qs, qe, lk = cu_q[b], cu_q[b + 1], cu_k[b + 1] - cu_k[b]
        m = allowed_mask(qe - qs, lk, mask, window_left, window_right)[:, j]
        kj = np.asarray(k[t, g, :], np.float64)
        vj = np.asarray(v[t, g, :], np.float64)
        for h in range(g * group, (g + 1) * group):
            qh = np.asarray(q[qs:qe, h, :], np.float64)
            doh = np.asarray(do[qs:qe, h, :], np.float64)
            s = scale * (qh @ kj)
            p = np.where(m, act(act_name, s, act_param), 0.0)
            dp = doh @ vj
            ds = np.where(m, act_grad(act_name, s, act_param) * dp, 0.0)
            dk[r] += scale * (ds @ qh)
            dv[r] += p @ doh
    return dk, dv
