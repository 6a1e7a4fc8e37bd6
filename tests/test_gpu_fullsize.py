"""Full-size parity: the four large reference workloads at their real sizes (and
the jagged one with fp16 inputs and with head dim 96), in
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

FULL = ["jagged_self", "full_self", "short_kv_cross", "window_gqa_fp8", "jagged_self_fp16", "jagged_self_d96"]
N_ROWS = 96


@pytest.fixture(scope="module")
def g():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import generalized_attention_amd
    return generalized_attention_amd


def _decode16(bt, arr):
    return oracle.decode_f16(arr) if bt.wl.fp16 else oracle.decode_bf16(arr)


def _decode_qk(bt, arr, scale):
    return oracle.decode_e4m3(arr, scale) if bt.wl.fp8_qk else _decode16(bt, arr)


def _seq(bt, b):
    """fp64 views of sequence b: q [Lq,Hq,D], k/v [Lk,Hkv,D], do [Lq,Hq,D] (or None)."""
    cq, ck = bt.cu_seqlens_q, bt.cu_seqlens_k
    sq, sk = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
    q = _decode_qk(bt, bt.q[sq], bt.q_scale)
    k = _decode_qk(bt, bt.k[sk], bt.k_scale)
    v = _decode16(bt, bt.v[sk])
    do = _decode16(bt, bt.do[sq]) if bt.do is not None else None
    return q, k, v, do


def _kw(wl):
    return dict(act_param=wl.act_param, mask=wl.mask, window_left=wl.window_left, window_right=wl.window_right)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_full_size_workload(g, name):
    import torch
    wl = gi.WORKLOADS[name]
    print(f"[fullsize] {name}: drawing inputs", flush=True)
    bt = gi.make_batch(wl)
    dev = device_batch(bt)
    print(f"[fullsize] {name}: forward", flush=True)
    o = run_forward(g, bt, dev)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any(), "forward left unwritten (NaN-poisoned) outputs"
    cq, ck = bt.cu_seqlens_q, bt.cu_seqlens_k
    rows = sample_rows(cq, wl.heads_q, N_ROWS, seed=1000 + wl.seed)
    idx_t = torch.tensor([t for t, _ in rows], device="cuda")
    idx_h = torch.tensor([h for _, h in rows], device="cuda")
    got = o[idx_t, idx_h].double().cpu().numpy()
    ref = np.zeros_like(got)
    for r, (t, h) in enumerate(rows):
        b = int(np.searchsorted(cq, t, side="right") - 1)
        q, k, v, _ = _seq(bt, b)
        ref[r] = oracle.gdpa_forward_rows(q, k, v, [0, q.shape[0]], [0, k.shape[0]], wl.scale, wl.act,
                                          [(t - cq[b], h)], **_kw(wl))[0]
    tol = TOL_FWD_FP8 if wl.fp8_qk else TOL_FWD_BF16
    ratio = err_ratio(got, ref)
    print(f"[fullsize] {name}: forward err/rms {ratio:.3e} over {len(rows)} rows", flush=True)
    assert ratio <= tol
    del o
    if not wl.backward:
        return

    print(f"[fullsize] {name}: backward", flush=True)
    dq, dk, dv = run_backward(g, bt, dev)
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
    krows = sample_rows(ck, wl.heads_kv, N_ROWS, seed=2000 + wl.seed)
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
