"""Full-size parity: the four large reference workloads at their real sizes (and
the jagged one with fp16 inputs, with head dim 96 and with head dims (192, 128);
the windowed one with FP8, MXFP8 and MXFP4 Q/K forward and backward), in
the launch configuration the benchmark uses (same C entry points, same
shapes).  Every output element is checked to have been written (outputs are
NaN-poisoned before the call); sampled rows are recomputed one by one by the
fp64 oracle and compared at the stated tolerances."""
import numpy as np
import pytest

import gdpa_inputs as gi
import oracle
from helpers import (TOL_BWD, TOL_FWD_BF16, TOL_FWD_FP8, device_batch, err_ratio, run_backward, run_forward,
                     sample_rows)

pytestmark = pytest.mark.gpu

FULL = ["jagged_self", "full_self", "short_kv_cross", "window_gqa_fp8", "jagged_self_fp16", "jagged_self_d96",
        "jagged_self_d192"]
N_ROWS = 96


@pytest.fixture(scope="module")
def g():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import generalized_attention_amd
    return generalized_attention_amd


def _decode16(bt, arr):
    return oracle.decode_f16(arr) if bt.wl.fp16 else oracle.decode_bf16(arr)


def _decode_qk(bt, arr, scale, blocks=None):
    if bt.wl.mx4_qk:
        return oracle.decode_mxfp4(arr, blocks)
    if bt.wl.mx_qk:
        return oracle.decode_mxfp8(arr, blocks)
    return oracle.decode_e4m3(arr, scale) if bt.wl.fp8_qk else _decode16(bt, arr)


def _seq(bt, b):
    """fp64 views of sequence b: q [Lq,Hq,D], k/v [Lk,Hkv,D], do [Lq,Hq,D] (or None)."""
    cq, ck = bt.cu_seqlens_q, bt.cu_seqlens_k
    sq, sk = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
    mx = bt.wl.mx_qk or bt.wl.mx4_qk
    q = _decode_qk(bt, bt.q[sq], bt.q_scale, bt.q_mx[sq] if mx else None)
    k = _decode_qk(bt, bt.k[sk], bt.k_scale, bt.k_mx[sk] if mx else None)
    v = _decode16(bt, bt.v[sk])
    do = _decode16(bt, bt.do[sq]) if bt.do is not None else None
    return q, k, v, do


def _kw(wl):
    return dict(act_param=wl.act_param, mask=wl.mask, window_left=wl.window_left, window_right=wl.window_right)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_full_size_workload(g, name):
    _check_workload(g, gi.WORKLOADS[name], None, N_ROWS)


# Robustness sweep: the same full-size check on other draws of the workloads
# whose structure the seed changes (jagged lengths, short-KV query lengths,
# windowed FP8 lengths), with fewer sampled rows each.
SWEEP_SEEDS = [101, 102, 103, 104, 105, 201, 202, 203, 204, 205]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("seed", SWEEP_SEEDS)
@pytest.mark.parametrize("name", ["jagged_self", "short_kv_cross", "window_gqa_fp8"])
def test_full_size_seed_sweep(g, name, seed):
    _check_workload(g, gi.WORKLOADS[name], seed, 32)


# bf16 outputs (O, dQ, dK, dV rounded to bf16 on the device) at the
# jagged, full-length and short-KV workloads
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["jagged_self", "full_self", "short_kv_cross"])
def test_full_size_bf16_outputs(g, name):
    import torch
    _check_workload(g, gi.WORKLOADS[name], None, 48, out_dtype=torch.bfloat16)


def _check_workload(g, wl, seed, n_rows, out_dtype=None):
    import torch
    name = wl.name if seed is None else f"{wl.name} seed {seed}"
    if out_dtype is not None:
        name += f" ({str(out_dtype).replace('torch.', '')} outputs)"
    print(f"[fullsize] {name}: drawing inputs", flush=True)
    bt = gi.make_batch(wl, seed=seed)
    base_seed = wl.seed if seed is None else seed
    dev = device_batch(bt)
    print(f"[fullsize] {name}: forward", flush=True)
    o = run_forward(g, bt, dev, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any(), "forward left unwritten (NaN-poisoned) outputs"
    cq, ck = bt.cu_seqlens_q, bt.cu_seqlens_k
    rows = sample_rows(cq, wl.heads_q, n_rows, seed=1000 + base_seed)
    idx_t = torch.tensor([t for t, _ in rows], device="cuda")
    idx_h = torch.tensor([h for _, h in rows], device="cuda")
    got = o[idx_t, idx_h].double().cpu().numpy()
    ref = np.zeros_like(got)
    for r, (t, h) in enumerate(rows):
        b = int(np.searchsorted(cq, t, side="right") - 1)
        q, k, v, _ = _seq(bt, b)
        ref[r] = oracle.gdpa_forward_rows(q, k, v, [0, q.shape[0]], [0, k.shape[0]], wl.scale, wl.act,
                                          [(t - cq[b], h)], **_kw(wl))[0]
    tol = TOL_FWD_FP8 if (wl.fp8_qk or wl.mx_qk or wl.mx4_qk) else TOL_FWD_BF16
    ratio = err_ratio(got, ref)
    print(f"[fullsize] {name}: forward err/rms {ratio:.3e} over {len(rows)} rows", flush=True)
    assert ratio <= tol
    del o
    if not wl.backward:
        return

    print(f"[fullsize] {name}: backward", flush=True)
    dq, dk, dv = run_backward(g, bt, dev, grad_dtype=out_dtype)
    torch.cuda.synchronize()
    for t_ in (dq, dk, dv):
        assert not torch.isnan(t_).any(), "backward left unwritten (NaN-poisoned) outputs"
    got_q = dq[idx_t, idx_h].double().cpu().numpy()
    ref_q = np.zeros_like(got_q)
    for r, (t, h) in enumerate(rows):
        b = int(np.searchsorted(cq, t, side="right") - 1)
        q, k, v, do = _seq(bt, b)
        ref_q[r] = oracle.gdpa_backward_q_rows(q, k, v, do, [0, q.shape[0]], [0, k.shape[0]], wl.scale, wl.act,
                                               [(t - cq[b], h)], **_kw(wl))[0]
    krows = sample_rows(ck, wl.heads_kv, n_rows, seed=2000 + base_seed)
    kt = torch.tensor([t for t, _ in krows], device="cuda")
    kg = torch.tensor([h for _, h in krows], device="cuda")
    got_k = dk[kt, kg].double().cpu().numpy()
    got_v = dv[kt, kg].double().cpu().numpy()
    ref_k = np.zeros_like(got_k)
    ref_v = np.zeros_like(got_v)
    for r, (t, gg) in enumerate(krows):
        b = int(np.searchsorted(ck, t, side="right") - 1)
        q, k, v, do = _seq(bt, b)
        a_, b_ = oracle.gdpa_backward_k_rows(q, k, v, do, [0, q.shape[0]], [0, k.shape[0]], wl.scale, wl.act,
                                             [(t - ck[b], gg)], **_kw(wl))
        ref_k[r], ref_v[r] = a_[0], b_[0]
    errs = dict(dq=err_ratio(got_q, ref_q), dk=err_ratio(got_k, ref_k), dv=err_ratio(got_v, ref_v))
    print(f"[fullsize] {name}: backward err/rms {errs}", flush=True)
    assert max(errs.values()) <= TOL_BWD, errs


# The windowed GQA workload's real shape (16 sequences of 1024-4096 tokens,
# Hq = 16, Hkv = 4, D = 64, LeakyReLU, causal window 512) with Q/K in each 8-
# and 4-bit format, forward and backward (the backward through the
# low-precision entry point)
@pytest.mark.timeout(900)
@pytest.mark.parametrize("fmt", ["fp8", "mxfp8", "mxfp4"])
def test_full_size_low_precision_formats(g, fmt):
    import dataclasses
    wl = dataclasses.replace(gi.WORKLOADS["window_gqa_fp8"], name=f"window_gqa_{fmt}", fp8_qk=fmt == "fp8",
                             mx_qk=fmt == "mxfp8", mx4_qk=fmt == "mxfp4", backward=True)
    _check_workload(g, wl, None, 48)


@pytest.mark.timeout(600)
def test_tensors_beyond_2gib(g):
    """Four 300k-token sequences (H = 8, D = 128): q, k, v, dO are 2.46 GB each and
    the last sequence starts beyond 2^31 bytes of o, dq, dk, dv (and its tail beyond
    2^31 bytes of q, k, v).  Causal window of 512 keys keeps the GPU work small; a
    2048-query block at the end of the last sequence is recomputed by the oracle
    with its 511 preceding keys, which holds every key its queries see and every
    query that sees its first 1537 keys."""
    import torch
    B, L, H, D, W = 4, 300_000, 8, 128, 512
    act, scale = "silu", D ** -0.5
    total = B * L
    print("[fullsize] beyond 2 GiB: drawing inputs on the GPU", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(7)
    def draw():
        return torch.randn((total, H, D), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    q, k, v, do = draw(), draw(), draw(), draw()
    cu = torch.arange(0, total + 1, L, dtype=torch.int32, device="cuda")
    kw = dict(act=act, mask="window", window_left=W - 1, window_right=0)
    o = torch.full((total, H, D), float("nan"), device="cuda")
    print("[fullsize] beyond 2 GiB: forward", flush=True)
    g.gdpa_varlen_fwd(q, k, v, o, cu, cu, L, L, scale, **kw)
    dq, dk, dv = (torch.full((total, H, D), float("nan"), device="cuda") for _ in range(3))
    print("[fullsize] beyond 2 GiB: backward", flush=True)
    g.gdpa_varlen_bwd(q, k, v, do, dq, dk, dv, cu, cu, L, L, scale, **kw)
    torch.cuda.synchronize()
    assert q.numel() * 2 > 2 ** 31 and 3 * L * H * D * 4 > 2 ** 31
    for t_ in (o, dq, dk, dv):
        assert not torch.isnan(t_).any(), "unwritten (NaN-poisoned) outputs"
    t1 = total - 5
    t0 = t1 - 2048                       # queries [t0, t1) of the last sequence
    k0 = t0 - (W - 1)                     # keys [k0, t1)
    assert (total - L) * H * D * 4 > 2 ** 31 and t0 * H * D * 2 > 2 ** 31
    dec = lambda t: t.float().cpu().double().numpy()
    qs, ks, vs, dos = dec(q[t0:t1]), dec(k[k0:t1]), dec(v[k0:t1]), dec(do[t0:t1])
    cq, ck = [0, t1 - t0], [0, t1 - k0]
    okw = dict(mask="window", window_left=W - 1, window_right=0)
    ref_o = oracle.gdpa_forward(qs, ks, vs, cq, ck, scale, act, **okw)
    rq, rk, rv = oracle.gdpa_backward(qs, ks, vs, dos, cq, ck, scale, act, **okw)
    nk = t1 - W + 1 - t0                  # keys [t0, t1 - 511) see all their queries in the block
    errs = dict(o=err_ratio(dec(o[t0:t1]), ref_o), dq=err_ratio(dec(dq[t0:t1]), rq),
                dk=err_ratio(dec(dk[t0:t0 + nk]), rk[W - 1:W - 1 + nk]),
                dv=err_ratio(dec(dv[t0:t0 + nk]), rv[W - 1:W - 1 + nk]))
    print(f"[fullsize] beyond 2 GiB: err/rms {errs}", flush=True)
    assert errs["o"] <= TOL_FWD_BF16
    assert max(errs["dq"], errs["dk"], errs["dv"]) <= TOL_BWD


@pytest.mark.timeout(600)
@pytest.mark.parametrize("mode", ["fused", "separate"])
@pytest.mark.parametrize("name", ["jagged_self", "full_self"])
def test_full_size_backward_is_bitwise_repeatable(g, monkeypatch, name, mode):
    """Three backward calls at full size give bitwise the same dQ, dK and dV,
    with dQ from the dK/dV pass (per-XCD work queues, the ordered dQ
    reduction) and from the separate dQ kernel (the dK/dV work queue)."""
    import torch
    monkeypatch.setenv("GDPA_BWD_DQ", mode)
    wl = gi.WORKLOADS[name]
    print(f"[fullsize] {name}: drawing inputs (repeatability)", flush=True)
    bt = gi.make_batch(wl)
    dev = device_batch(bt)
    first = run_backward(g, bt, dev)
    for rep in range(2):
        again = run_backward(g, bt, dev)
        torch.cuda.synchronize()
        for a, b in zip(first, again):
            assert torch.equal(a, b), f"{name} ({mode}): backward run {rep + 2} differs"
        del again
    print(f"[fullsize] {name} ({mode}): backward repeatable", flush=True)


@pytest.mark.timeout(600)
def test_full_self_whole_slice(g):
    """Full-length workload (32 x 2048, 8 heads): every element of one whole
    (sequence, head) slice of O, dQ, dK and dV against the fp64 oracle."""
    import torch
    wl = gi.WORKLOADS["full_self"]
    print("[fullsize] full_self: drawing inputs (whole slice)", flush=True)
    bt = gi.make_batch(wl)
    dev = device_batch(bt)
    o = run_forward(g, bt, dev)
    dq, dk, dv = run_backward(g, bt, dev)
    torch.cuda.synchronize()
    b, h = 21, 5
    q, k, v, do = _seq(bt, b)
    L = q.shape[0]
    sl = slice(int(bt.cu_seqlens_q[b]), int(bt.cu_seqlens_q[b + 1]))
    qh, kh, vh, doh = q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], do[:, h:h + 1]
    ref_o = oracle.gdpa_forward(qh, kh, vh, [0, L], [0, L], wl.scale, wl.act, **_kw(wl))
    rq, rk, rv = oracle.gdpa_backward(qh, kh, vh, doh, [0, L], [0, L], wl.scale, wl.act, **_kw(wl))
    errs = dict(o=err_ratio(o[sl, h:h + 1].double().cpu().numpy(), ref_o),
                dq=err_ratio(dq[sl, h:h + 1].double().cpu().numpy(), rq),
                dk=err_ratio(dk[sl, h:h + 1].double().cpu().numpy(), rk),
                dv=err_ratio(dv[sl, h:h + 1].double().cpu().numpy(), rv))
    print(f"[fullsize] full_self slice (b={b}, h={h}): err/rms {errs}", flush=True)
    assert errs["o"] <= TOL_FWD_BF16
    assert max(errs["dq"], errs["dk"], errs["dv"]) <= TOL_BWD
