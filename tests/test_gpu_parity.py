"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Inputs are seeded (gdpa_inputs); the oracle consumes exactly the values the
kernels consume (decoded bf16, E4M3 code x scale).  Bar: max|err| <= tol *
rms(ref) with tol = 2e-2 (bf16 forward), 3e-2 (dQ/dK/dV), 6e-2 (FP8 forward).
Outputs are NaN-poisoned before each call, so an unwritten element fails.
"""
import dataclasses

import numpy as np
import pytest

import gdpa_inputs as gi
import oracle
from helpers import (TOL_BWD, TOL_FWD_BF16, TOL_FWD_FP8, backward_ratios, device_batch, err_ratio, mask_kw,
                     oracle_inputs, run_backward, run_forward, seq_ratios)

pytestmark = pytest.mark.gpu

# The bar (max|err| <= tol * rms(ref)) is stated for a whole output.  Per
# sequence, against that sequence's own rms, the tests require PER_SEQ_FACTOR
# times the bar: a short sequence's rms can sit well below the batch's, and
# the 16-bit rounding of P or dS over its few keys does not average out (the
# hi + lo split is chosen from the batch's max_seqlen), while a misplaced or
# unwritten sequence still fails by orders of magnitude.
PER_SEQ_FACTOR = 2.0

ALL_ACTS = gi.ACTIVATIONS


@pytest.fixture(scope="module")
def g():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import generalized_attention_amd
    return generalized_attention_amd


def _wl(**kw):
    base = dict(name="t", batch=4, heads_q=4, heads_kv=2, head_dim=128, lq_range=(1, 300), lk_range=None,
                act="silu", backward=True, seed=11)
    base.update(kw)
    return gi.Workload(**base)


def check_forward(g, bt, tol=None):
    wl = bt.wl
    tol = tol or (TOL_FWD_FP8 if (wl.fp8_qk or wl.mx_qk or wl.mx4_qk) else TOL_FWD_BF16)
    o = run_forward(g, bt).cpu().double().numpy()
    q, k, v, _ = oracle_inputs(bt)
    ref = oracle.gdpa_forward(q, k, v, bt.cu_seqlens_q, bt.cu_seqlens_k, wl.scale, wl.act, **mask_kw(wl))
    r = err_ratio(o, ref)
    assert r <= tol, f"{wl} forward err/rms {r:.4g} > {tol}"
    # every sequence against its own rms as well (reported; bounded by
    # PER_SEQ_FACTOR times the bar, see there)
    per = seq_ratios(o, ref, bt.cu_seqlens_q)
    worst = max(per, key=per.get) if per else None
    if worst is not None:
        print(f"forward err/rms {r:.3e}; worst sequence {worst} (len {bt.seqlens_q[worst]}) {per[worst]:.3e}")
        assert per[worst] <= PER_SEQ_FACTOR * tol, f"{wl} forward, sequence {worst}: err/rms {per[worst]:.4g}"
    return r


def check_backward(g, bt, tol=TOL_BWD):
    wl = bt.wl
    dq, dk, dv = [t.cpu().double().numpy() for t in run_backward(g, bt)]
    per = {}
    errs = backward_ratios(bt, dq, dk, dv, per_seq=per)
    assert max(errs.values()) <= tol, f"{wl} backward {errs}"
    # every sequence against its own rms as well (reported; bounded by
    # PER_SEQ_FACTOR times the bar)
    for name, ratios in per.items():
        if ratios:
            worst = max(ratios, key=ratios.get)
            print(f"{name} err/rms {errs[name]:.3e}; worst sequence {worst} {ratios[worst]:.3e}")
            assert ratios[worst] <= PER_SEQ_FACTOR * tol, f"{wl} {name}, sequence {worst}: {ratios[worst]:.4g}"
    return errs


# ------------------------------------------------------------- reference workload 1
def test_tiny_fixed_length_forward(g):
    bt = gi.make_batch(gi.WORKLOADS["tiny"])
    check_forward(g, bt)


# ------------------------------------------------------------ activation x head dim
@pytest.mark.parametrize("D", [64, 96, 128])
@pytest.mark.parametrize("act", ALL_ACTS)
def test_forward_every_activation(g, act, D):
    # jagged lengths incl. 0, 1 and ragged tails across several 128-row / KV tiles; GQA 4:2
    bt = gi.make_batch(_wl(act=act, head_dim=D, act_param=0.05), seqlens_q=[37, 0, 300, 1, 129],
                       seqlens_k=[37, 0, 300, 1, 129])
    check_forward(g, bt)


@pytest.mark.parametrize("D", [64, 96, 128])
@pytest.mark.parametrize("act", ALL_ACTS)
def test_backward_every_activation(g, act, D):
    bt = gi.make_batch(_wl(act=act, head_dim=D, act_param=0.05), seqlens_q=[37, 0, 300, 1, 129],
                       seqlens_k=[37, 0, 300, 1, 129])
    check_backward(g, bt)


@dataclasses.dataclass(frozen=True)
class _ScaledWorkload(gi.Workload):
    scale_value: float = 1.0

    @property
    def scale(self) -> float:
        return self.scale_value


# the activations whose score scale the kernels fold into the output factor
# (ReLU, LeakyReLU at slopes below, at and above 1, identity) and two that keep
# it inside, at a negative and a zero scale, with a window mask
@pytest.mark.parametrize("act,alpha", [("relu", 0.0), ("leaky_relu", 0.05), ("leaky_relu", 0.0),
                                       ("leaky_relu", 2.5), ("leaky_relu", -0.5), ("identity", 0.0),
                                       ("relu2", 0.0), ("gelu_tanh", 0.0)])
@pytest.mark.parametrize("scale", [-0.2, 0.0])
def test_negative_and_zero_scale(g, act, alpha, scale):
    base = dict(name="t", batch=3, heads_q=4, heads_kv=2, head_dim=64, lq_range=(1, 300), lk_range=None, act=act,
                act_param=alpha, mask="window", window_left=70, window_right=5, backward=True, seed=13)
    bt = gi.make_batch(_ScaledWorkload(**base, scale_value=scale), seqlens_q=[37, 130, 1], seqlens_k=[50, 130, 9])
    check_forward(g, bt)
    check_backward(g, bt)


# ---------------------------------------------------------------------- masks
MASK_CASES = [
    ("causal", -1, -1, [200, 77, 256], [200, 77, 256]),
    ("causal", -1, -1, [50, 130, 1], [300, 140, 64]),      # Lq < Lk: bottom-right alignment
    ("causal", -1, -1, [300, 20], [100, 3]),               # Lq > Lk: leading rows fully masked
    ("window", 63, 0, [400, 129], [400, 129]),
    ("window", 17, 5, [333, 64], [333, 80]),
    ("window", 0, 0, [150], [150]),
    ("window", -1, 40, [260], [260]),
    ("window", 100, -1, [260], [300]),
]


@pytest.mark.parametrize("D", [64, 96, 128])
@pytest.mark.parametrize("case", range(len(MASK_CASES)))
def test_masks_forward_backward(g, case, D):
    mask, wl_, wr_, lq, lk = MASK_CASES[case]
    wl = _wl(act="gelu_tanh", head_dim=D, mask=mask, window_left=wl_, window_right=wr_, batch=len(lq))
    bt = gi.make_batch(wl, seqlens_q=lq, seqlens_k=lk)
    check_forward(g, bt)
    check_backward(g, bt)


@pytest.mark.parametrize("hq,hkv", [(8, 1), (6, 3), (2, 2)])
def test_head_configs(g, hq, hkv):
    # MQA (Hkv = 1), GQA 2:1, MHA
    bt = gi.make_batch(_wl(heads_q=hq, heads_kv=hkv, act="relu2"), seqlens_q=[90, 257], seqlens_k=[90, 257])
    check_forward(g, bt)
    check_backward(g, bt)


def test_cross_attention_short_kv(g):
    wl = dataclasses.replace(gi.WORKLOADS["short_kv_cross"], batch=6)
    bt = gi.make_batch(wl)
    check_forward(g, bt)
    check_backward(g, bt)


@pytest.mark.parametrize("D", [64, 96, 128])
def test_fp8_forward(g, D):
    wl = _wl(head_dim=D, fp8_qk=True, act="leaky_relu", mask="window", window_left=127, window_right=0,
             heads_q=8, heads_kv=2, backward=False)
    bt = gi.make_batch(wl, seqlens_q=[300, 45, 513], seqlens_k=[300, 45, 513])
    check_forward(g, bt)


@pytest.mark.parametrize("mask", ["none", "causal"])
@pytest.mark.parametrize("act", ["silu", "gelu_tanh", "relu2", "identity"])
@pytest.mark.parametrize("D", [64, 96, 128])
def test_fp8_forward_activations_masks(g, D, act, mask):
    # Q K^T on the K = 64 FP8 MFMA (at 96 followed by two K = 16 MFMAs): every
    # activation path and the unmasked / causal tile kinds, with ragged lengths
    # (tail tiles) and MQA
    wl = _wl(head_dim=D, fp8_qk=True, act=act, mask=mask, heads_q=4, heads_kv=1, backward=False)
    bt = gi.make_batch(wl, seqlens_q=[129, 1, 64, 250], seqlens_k=[129, 7, 64, 250])
    check_forward(g, bt)


# ---------------------------------------------------------------- fp16 inputs
# Q, K, V, dO in IEEE binary16; P and dS rounded to fp16 for the products.
# Same bars as bf16 (the oracle consumes the decoded fp16 values).
FP16_LENS = [37, 0, 300, 1, 129]


@pytest.mark.parametrize("D", [64, 96, 128])
@pytest.mark.parametrize("act", ["identity", "gelu", "fast_gelu", "relu", "relu2", "leaky_relu", "silu",
                                 "hardswish"])
def test_fp16_forward(g, act, D):
    bt = gi.make_batch(_wl(act=act, head_dim=D, fp16=True, backward=False), seqlens_q=FP16_LENS,
                       seqlens_k=FP16_LENS)
    check_forward(g, bt)


@pytest.mark.parametrize("D", [64, 96, 128])
@pytest.mark.parametrize("act", ["gelu", "fast_gelu", "relu2", "silu", "hardswish"])
def test_fp16_backward(g, act, D):
    bt = gi.make_batch(_wl(act=act, head_dim=D, fp16=True), seqlens_q=FP16_LENS, seqlens_k=FP16_LENS)
    check_backward(g, bt)


@pytest.mark.parametrize("case", [0, 1, 3, 4])
def test_fp16_masks_gqa(g, case):
    mask, wl_, wr_, lq, lk = MASK_CASES[case]
    wl = _wl(act="silu", fp16=True, mask=mask, window_left=wl_, window_right=wr_, batch=len(lq), heads_q=8,
             heads_kv=2)
    bt = gi.make_batch(wl, seqlens_q=lq, seqlens_k=lk)
    check_forward(g, bt)
    check_backward(g, bt)


def test_fp16_short_kv(g):
    # few products per output row: fp16 keeps P and dS in one word (no hi/lo split)
    wl = dataclasses.replace(gi.WORKLOADS["short_kv_cross"], batch=4, fp16=True)
    bt = gi.make_batch(wl)
    check_forward(g, bt)
    check_backward(g, bt)


def test_fp16_outputs(g):
    import torch
    bt = gi.make_batch(_wl(act="gelu", fp16=True), seqlens_q=[300, 65], seqlens_k=[300, 65])
    o = run_forward(g, bt, out_dtype=torch.float16).float().cpu().double().numpy()
    q, k, v, do = oracle_inputs(bt)
    wl = bt.wl
    ref = oracle.gdpa_forward(q, k, v, bt.cu_seqlens_q, bt.cu_seqlens_k, wl.scale, wl.act)
    assert err_ratio(o, ref) <= TOL_FWD_BF16
    grads = [t.float().cpu().double().numpy() for t in run_backward(g, bt, grad_dtype=torch.float16)]
    refs = oracle.gdpa_backward(q, k, v, do, bt.cu_seqlens_q, bt.cu_seqlens_k, wl.scale, wl.act)
    for a, b in zip(grads, refs):
        assert err_ratio(a, b) <= TOL_BWD


def test_empty_kv_gives_zero_output(g):
    import torch
    bt = gi.make_batch(_wl(act="identity"), seqlens_q=[5, 70], seqlens_k=[0, 0])
    o = run_forward(g, bt).cpu()
    assert torch.all(o == 0)
    dq, dk, dv = run_backward(g, bt)
    assert torch.all(dq.cpu() == 0) and dk.numel() == 0


def test_bf16_outputs(g):
    import torch
    bt = gi.make_batch(_wl(act="silu"), seqlens_q=[300, 65], seqlens_k=[300, 65])
    o = run_forward(g, bt, out_dtype=torch.bfloat16).float().cpu().double().numpy()
    q, k, v, do = oracle_inputs(bt)
    wl = bt.wl
    ref = oracle.gdpa_forward(q, k, v, bt.cu_seqlens_q, bt.cu_seqlens_k, wl.scale, wl.act)
    assert err_ratio(o, ref) <= TOL_FWD_BF16
    grads = [t.float().cpu().double().numpy() for t in run_backward(g, bt, grad_dtype=torch.bfloat16)]
    refs = oracle.gdpa_backward(q, k, v, do, bt.cu_seqlens_q, bt.cu_seqlens_k, wl.scale, wl.act)
    for a, b in zip(grads, refs):
        assert err_ratio(a, b) <= TOL_BWD


def test_deterministic(g):
    import torch
    bt = gi.make_batch(_wl(act="fast_gelu", mask="causal"), seqlens_q=[300, 129, 5], seqlens_k=[300, 129, 5])
    dev = device_batch(bt)
    o1 = run_forward(g, bt, dev)
    o2 = run_forward(g, bt, dev)
    assert torch.equal(o1, o2)
    g1 = run_backward(g, bt, dev)
    g2 = run_backward(g, bt, dev)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_fixed_length_equals_varlen(g):
    import torch
    wl = _wl(act="hardswish", varlen=False, lq_range=(200, 200), batch=3)
    bt = gi.make_batch(wl)
    o_fixed = run_forward(g, bt)
    bt_var = dataclasses.replace(bt, wl=dataclasses.replace(wl, varlen=True))
    o_var = run_forward(g, bt_var)
    assert torch.equal(o_fixed, o_var)
    for a, b in zip(run_backward(g, bt), run_backward(g, bt_var)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("mode", ["fused", "separate"])
def test_partial_gradients(g, monkeypatch, mode):
    # dq alone (separate dQ kernel) and dk/dv alone (dK/dV kernel) against the
    # full call (fused: dQ reduced in another fixed order inside the dK/dV
    # pass): dK and dV take the same products in the same order, bitwise; dQ
    # matches the oracle
    import torch
    monkeypatch.setenv("GDPA_BWD_DQ", mode)
    bt = gi.make_batch(_wl(act="silu", mask="causal"), seqlens_q=[200, 70], seqlens_k=[200, 70])
    dev = device_batch(bt)
    dq, dk, dv = run_backward(g, bt, dev)
    wl = bt.wl
    common = (dev["cu_q"], dev["cu_k"], bt.max_seqlen_q, bt.max_seqlen_k, wl.scale)
    kw = dict(act=wl.act, mask=wl.mask)
    dq2 = torch.full_like(dq, float("nan"))
    g.gdpa_varlen_bwd(dev["q"], dev["k"], dev["v"], dev["do"], dq2, None, None, *common, **kw)
    dk2, dv2 = torch.full_like(dk, float("nan")), torch.full_like(dv, float("nan"))
    g.gdpa_varlen_bwd(dev["q"], dev["k"], dev["v"], dev["do"], None, dk2, dv2, *common, **kw)
    assert torch.equal(dk, dk2) and torch.equal(dv, dv2)
    for t in (dq, dq2):
        assert backward_ratios(bt, t, dk, dv)["dq"] <= TOL_BWD


# -------------------------------------------- fused backward (ordered dQ sums)
FUSED_CASES = [
    dict(act="silu"),
    dict(act="gelu_tanh", mask="causal"),
    dict(act="relu2", mask="window", window_left=130, window_right=70),
    dict(act="leaky_relu", heads_q=8, heads_kv=2),                 # GQA 4:1: a step loop over the group's heads
    dict(act="hardswish", heads_q=4, heads_kv=1, mask="causal"),   # MQA
    dict(act="gelu"),
]


@pytest.mark.parametrize("D", [64, 96, 128])
@pytest.mark.parametrize("case", range(len(FUSED_CASES)))
def test_fused_and_separate_dq_match_the_oracle(g, monkeypatch, case, D):
    # long sequences (several key blocks per tile, up to 12 contributors per
    # dQ tile), ragged tails, an empty sequence; dK/dV bitwise equal between
    # the two paths, dQ within the bar for both
    import torch
    lens = [700, 1, 0, 1537, 64, 129]
    bt = gi.make_batch(_wl(head_dim=D, batch=len(lens), act_param=0.05, **FUSED_CASES[case]), seqlens_q=lens,
                       seqlens_k=lens)
    dev = device_batch(bt)
    monkeypatch.setenv("GDPA_BWD_DQ", "fused")
    fused = run_backward(g, bt, dev)
    monkeypatch.setenv("GDPA_BWD_DQ", "separate")
    sep = run_backward(g, bt, dev)
    assert torch.equal(fused[1], sep[1]) and torch.equal(fused[2], sep[2])
    errs = backward_ratios(bt, *fused)
    assert max(errs.values()) <= TOL_BWD, errs
    assert backward_ratios(bt, *sep)["dq"] <= TOL_BWD


SHORT_KV_CASES = [
    dict(act="relu2"),                                          # dS split into hi + lo words (few keys)
    dict(act="gelu_tanh", mask="causal"),
    dict(act="silu", heads_q=8, heads_kv=2),                    # GQA 4:1
    dict(act="relu2", heads_q=2, heads_kv=1, fp16=True),        # fp16: one word
]


@pytest.mark.parametrize("D", [64, 96, 128])
@pytest.mark.parametrize("case", range(len(SHORT_KV_CASES)))
def test_short_kv_fused_and_separate_match_the_oracle(g, monkeypatch, case, D):
    # keys fit one block (the fused pass is the default): each query tile has
    # one contributor, so dQ is written directly; empty and one-key sequences,
    # ragged query tails; dK/dV bitwise equal between the paths
    import torch
    lq, lk = [700, 1, 0, 300, 64, 129, 5], [64, 64, 64, 1, 0, 33, 128]
    bt = gi.make_batch(_wl(head_dim=D, batch=len(lq), **SHORT_KV_CASES[case]), seqlens_q=lq, seqlens_k=lk)
    dev = device_batch(bt)
    default = run_backward(g, bt, dev)
    monkeypatch.setenv("GDPA_BWD_DQ", "fused")
    fused = run_backward(g, bt, dev)
    monkeypatch.setenv("GDPA_BWD_DQ", "separate")
    sep = run_backward(g, bt, dev)
    for a, b in zip(default, fused):
        assert torch.equal(a, b)
    assert torch.equal(fused[1], sep[1]) and torch.equal(fused[2], sep[2])
    errs = backward_ratios(bt, *fused)
    assert max(errs.values()) <= TOL_BWD, errs
    assert backward_ratios(bt, *sep)["dq"] <= TOL_BWD


def test_fused_cross_attention_lengths(g, monkeypatch):
    # Lq != Lk in both directions, causal (bottom-right) and a window: query
    # tiles no key block reaches are written as zeros by the first block item
    monkeypatch.setenv("GDPA_BWD_DQ", "fused")
    lq, lk = [300, 40, 900, 129], [100, 600, 900, 1000]
    for mask, wl_, wr_ in (("causal", -1, -1), ("window", 200, 10), ("none", -1, -1)):
        bt = gi.make_batch(_wl(head_dim=128, batch=4, act="silu", mask=mask, window_left=wl_, window_right=wr_),
                           seqlens_q=lq, seqlens_k=lk)
        check_backward(g, bt)


def test_fused_backward_16bit_gradients(g, monkeypatch):
    # bf16 and fp16 dQ: fp32 sums in the workspace, the last contributor
    # rounds; compared with fp32 dQ of the same call at the output's precision
    import torch
    monkeypatch.setenv("GDPA_BWD_DQ", "fused")
    lens = [700, 1537, 64]
    for fp16 in (False, True):
        bt = gi.make_batch(_wl(head_dim=128, batch=3, act="gelu_tanh", mask="causal", fp16=fp16), seqlens_q=lens,
                           seqlens_k=lens)
        dev = device_batch(bt)
        ref = run_backward(g, bt, dev)
        got = run_backward(g, bt, dev, grad_dtype=torch.float16 if fp16 else torch.bfloat16)
        for a, b in zip(got, ref):
            assert torch.isfinite(a).all()
            err = (a.float() - b).abs().max().item()
            assert err <= 2 ** -7 * b.abs().max().item(), err


def test_fused_wait_flag_in_debug_mode(g, monkeypatch):
    # GDPA_DEBUG_CHECKS makes the call wait for the kernel and report a dQ turn
    # wait that gave up; the default limit never trips, and a negative limit
    # (forced from the host) gives up every wait at once, so the error path is
    # taken while every kernel still runs to its end
    lens = [1537, 700]
    bt = gi.make_batch(_wl(head_dim=128, batch=2, act="silu"), seqlens_q=lens, seqlens_k=lens)
    dev = device_batch(bt)
    monkeypatch.setenv("GDPA_BWD_DQ", "fused")
    monkeypatch.setenv("GDPA_DEBUG_CHECKS", "1")
    check = run_backward(g, bt, dev)
    monkeypatch.setenv("GDPA_DEBUG_SPIN_LIMIT", "-1")
    with pytest.raises(g.GDPAError) as e:
        run_backward(g, bt, dev)
    assert e.value.status == 5
    monkeypatch.delenv("GDPA_DEBUG_SPIN_LIMIT")
    import torch
    again = run_backward(g, bt, dev)
    for a, b in zip(check, again):
        assert torch.equal(a, b)


# ------------------------------------------------------- longest-first schedule
def test_sequence_order_does_not_change_results(g):
    # jagged calls process sequences longest first; reversing the batch must
    # give each sequence bitwise the same output and gradients
    import torch
    lens = [5, 300, 1, 129, 64, 0, 257]
    bt = gi.make_batch(_wl(act="gelu_tanh", mask="causal", batch=len(lens)), seqlens_q=lens, seqlens_k=lens)
    rev = list(reversed(range(len(lens))))
    cq = bt.cu_seqlens_q

    def seq_rows(arr, order):
        return np.concatenate([arr[cq[b]:cq[b + 1]] for b in order])

    bt_rev = dataclasses.replace(bt, seqlens_q=np.asarray(lens)[rev], seqlens_k=np.asarray(lens)[rev],
                                 cu_seqlens_q=np.concatenate([[0], np.cumsum(np.asarray(lens)[rev])]).astype(np.int32),
                                 cu_seqlens_k=np.concatenate([[0], np.cumsum(np.asarray(lens)[rev])]).astype(np.int32),
                                 q=seq_rows(bt.q, rev), k=seq_rows(bt.k, rev), v=seq_rows(bt.v, rev),
                                 do=seq_rows(bt.do, rev))
    o = run_forward(g, bt).cpu().numpy()
    o_rev = run_forward(g, bt_rev).cpu().numpy()
    assert np.array_equal(seq_rows(o, rev), o_rev)
    for a, b in zip(run_backward(g, bt), run_backward(g, bt_rev)):
        assert np.array_equal(seq_rows(a.cpu().numpy(), rev), b.cpu().numpy())


def test_batch_beyond_schedule_limit(g):
    # more sequences than the on-device sort handles: index order, no workspace
    rng = np.random.default_rng(5)
    lens = rng.integers(0, 6, size=4100)
    wl = _wl(act="relu2", head_dim=64, heads_q=2, heads_kv=1, batch=len(lens))
    bt = gi.make_batch(wl, seqlens_q=lens, seqlens_k=lens)
    assert g._lib.gdpa_varlen_fwd_workspace_size(len(lens), 5, 5, 2, 1, 64) == 0
    check_forward(g, bt)
    check_backward(g, bt)


def test_batch_sorted_in_lds(g):
    # 65..4096 sequences take the schedule's LDS sort (64 or fewer sort across one wave)
    rng = np.random.default_rng(9)
    lens = rng.integers(0, 41, size=300)
    wl = _wl(act="silu", head_dim=64, heads_q=2, heads_kv=1, batch=len(lens))
    bt = gi.make_batch(wl, seqlens_q=lens, seqlens_k=lens)
    check_forward(g, bt)
    check_backward(g, bt)


def _mask_blocks(lq, lk, mask, wl_, wr_):
    # 64 x 64 blocks holding an allowed pair, counted from the oracle's mask
    if lq == 0 or lk == 0:
        return 0
    ok = oracle.allowed_mask(lq, lk, mask, wl_, wr_)
    mt, nt = -(-lq // 64), -(-lk // 64)
    pad = np.zeros((mt * 64, nt * 64), dtype=bool)
    pad[:lq, :lk] = ok
    return int(pad.reshape(mt, 64, nt, 64).any(axis=(1, 3)).sum())


@pytest.mark.parametrize("batch,maxlen", [(40, 400), (300, 300), (1500, 150)])
@pytest.mark.parametrize("case", [("none", -1, -1), ("causal", -1, 0), ("window", 100, 0), ("window", 50, 30)])
def test_schedule_orders_by_masked_blocks(g, batch, maxlen, case):
    # the jagged schedule (one wave, one thread per sequence, and LDS sorts)
    # orders sequences by the 64 x 64 blocks their mask leaves work in, then
    # by lq + lk, then by index; the order sits in the first batch words of
    # the forward's workspace
    import torch
    mask, wl_, wr_ = case
    rng = np.random.default_rng(batch + 7 * wl_ + wr_)
    lq = rng.integers(0, maxlen + 1, size=batch)
    lk = rng.integers(0, maxlen + 1, size=batch)
    dev = torch.device("cuda:0")
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum(lq)]), dtype=torch.int32, device=dev)
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum(lk)]), dtype=torch.int32, device=dev)
    tq, tk = int(lq.sum()), int(lk.sum())
    q = torch.randn(tq, 1, 64, device=dev).to(torch.bfloat16)
    k = torch.randn(tk, 1, 64, device=dev).to(torch.bfloat16)
    v = torch.randn(tk, 1, 64, device=dev).to(torch.bfloat16)
    o = torch.empty(tq, 1, 64, device=dev)
    nws = g._lib.gdpa_varlen_fwd_workspace_size(batch, int(lq.max()), int(lk.max()), 1, 1, 64)
    assert nws >= 4 * batch
    ws = torch.zeros(nws, dtype=torch.uint8, device=dev)
    st = g._lib.gdpa_varlen_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), cu_q.data_ptr(),
                                cu_k.data_ptr(), batch, int(lq.max()), int(lk.max()), tq, tk, 1, 1, 64, 64, 0.125,
                                g._mask(mask), wl_, wr_, g._act("relu"), 0.0, g.DTYPE_BF16, g.DTYPE_BF16,
                                g.DTYPE_FP32, 1.0, 1.0, ws.data_ptr(), nws, g._stream(dev))
    assert st == 0, g._lib.gdpa_status_string(st)
    torch.cuda.synchronize()
    perm = ws[:4 * batch].cpu().view(torch.int32).numpy()
    cost = [_mask_blocks(int(lq[i]), int(lk[i]), mask, wl_, wr_) for i in range(batch)]
    want = sorted(range(batch), key=lambda i: (-cost[i], -(int(lq[i]) + int(lk[i])), i))
    assert perm.tolist() == want


# ------------------------------------------------------ autograd and call forms
def _oracle_check(bt, o, grads, mask="none", wl_=-1, wr_=-1):
    wl = bt.wl
    q, k, v, do = oracle_inputs(bt)
    kw = dict(act_param=wl.act_param, mask=mask, window_left=wl_, window_right=wr_)
    ref = oracle.gdpa_forward(q, k, v, bt.cu_seqlens_q, bt.cu_seqlens_k, wl.scale, wl.act, **kw)
    assert err_ratio(o.detach().float().cpu().double().numpy().reshape(ref.shape), ref) <= TOL_FWD_BF16
    refs = oracle.gdpa_backward(q, k, v, do, bt.cu_seqlens_q, bt.cu_seqlens_k, wl.scale, wl.act, **kw)
    for name, a, b in zip("qkv", grads, refs):
        r = err_ratio(a.float().cpu().double().numpy().reshape(b.shape), b)
        assert r <= TOL_BWD, f"d{name} err/rms {r:.4g}"


def test_autograd_varlen(g):
    import torch
    bt = gi.make_batch(_wl(act="silu", heads_q=4, heads_kv=2), seqlens_q=[300, 0, 65], seqlens_k=[300, 0, 65])
    dev = device_batch(bt)
    q, k, v = [dev[n].clone().requires_grad_() for n in ("q", "k", "v")]
    o, lse = g.flash_attn_varlen_func(q, k, v, dev["cu_q"], dev["cu_k"], bt.max_seqlen_q, bt.max_seqlen_k,
                                      activation="silu", out_dtype=torch.float32)
    assert lse is None and o.dtype == torch.float32
    (o * dev["do"].float()).sum().backward()
    assert q.grad.dtype == q.dtype and k.grad.shape == k.shape
    _oracle_check(bt, o, (q.grad, k.grad, v.grad))


def test_autograd_fixed_length_causal(g):
    import torch
    wl = _wl(act="gelu", varlen=False, batch=2, heads_q=4, heads_kv=4, mask="causal", lq_range=(200, 200))
    bt = gi.make_batch(wl)
    dev = device_batch(bt)
    B, L, H, D = 2, 200, 4, 128
    q, k, v = [dev[n].view(B, L, H, D).clone().requires_grad_() for n in ("q", "k", "v")]
    # fp32 output: the bf16 rounding of O alone takes most of the 2e-2 budget
    o, _ = g.flash_attn_func(q, k, v, causal=True, activation="gelu", out_dtype=torch.float32)
    assert o.shape == q.shape
    (o.float() * dev["do"].view(B, L, H, D).float()).sum().backward()
    _oracle_check(bt, o, (q.grad, k.grad, v.grad), mask="causal")


def test_triton_call_form_equals_c_call(g):
    import torch
    bt = gi.make_batch(_wl(act="fast_gelu"), seqlens_q=[129, 7], seqlens_k=[129, 7])
    dev = device_batch(bt)
    o1 = g.generalized_dot_product_attention(dev["q"], dev["k"], dev["v"], query_offset=dev["cu_q"],
                                             key_offset=dev["cu_k"], max_seq_len_q=bt.max_seqlen_q,
                                             max_seq_len_kv=bt.max_seqlen_k, activation="fast_gelu",
                                             out_dtype=torch.float32)
    o2 = run_forward(g, bt, dev)
    assert torch.equal(o1, o2)


# ------------------------------------------------------------ long sequences
# (several KV tiles per query block, window edges inside tiles, one 1-row sequence)
@pytest.mark.parametrize("D", [64, 96, 128])
@pytest.mark.parametrize("mask,wl_,wr_", [("none", -1, -1), ("causal", -1, -1), ("window", 300, 0)])
def test_long_sequence_forward(g, D, mask, wl_, wr_):
    lens = [1100, 1500, 1030, 1]
    wl = _wl(act="silu", head_dim=D, mask=mask, window_left=wl_, window_right=wr_, batch=len(lens),
             backward=False)
    check_forward(g, gi.make_batch(wl, seqlens_q=lens, seqlens_k=lens))


def test_long_sequence_forward_fp16_gqa(g):
    lens = [2048, 1000]
    wl = _wl(act="fast_gelu", fp16=True, heads_q=8, heads_kv=2, batch=2, backward=False)
    check_forward(g, gi.make_batch(wl, seqlens_q=lens, seqlens_k=lens))


# ------------------------------------------- head dims (192, 128): Q/K 192, V/O 128
@pytest.mark.parametrize("act", ["identity", "fast_gelu", "silu", "relu2", "leaky_relu", "gelu"])
def test_head_dims_192_128_forward(g, act):
    bt = gi.make_batch(_wl(act=act, head_dim=192, head_dim_v=128, backward=False, act_param=0.05),
                       seqlens_q=FP16_LENS, seqlens_k=FP16_LENS)
    check_forward(g, bt)


@pytest.mark.parametrize("case", [0, 1, 3, 4])
def test_head_dims_192_128_masks_gqa(g, case):
    mask, wl_, wr_, lq, lk = MASK_CASES[case]
    wl = _wl(act="silu", head_dim=192, head_dim_v=128, mask=mask, window_left=wl_, window_right=wr_,
             batch=len(lq), heads_q=8, heads_kv=2, backward=False)
    check_forward(g, gi.make_batch(wl, seqlens_q=lq, seqlens_k=lk))


def test_head_dims_192_128_fp16_and_fixed_length(g):
    check_forward(g, gi.make_batch(_wl(act="fast_gelu", head_dim=192, head_dim_v=128, fp16=True,
                                       backward=False), seqlens_q=[1100, 33], seqlens_k=[1100, 33]))
    wl = _wl(act="silu", head_dim=192, head_dim_v=128, varlen=False, batch=2, lq_range=(300, 300),
             backward=False)
    check_forward(g, gi.make_batch(wl))


@pytest.mark.parametrize("act", ["identity", "fast_gelu", "silu", "relu2", "leaky_relu", "gelu", "hardswish"])
def test_head_dims_192_128_backward(g, act):
    # S and dK over the 192 head dims of Q and K, dP and dV over V's 128:
    # jagged lengths with empty, one-token and ragged sequences, GQA 4:2
    bt = gi.make_batch(_wl(act=act, head_dim=192, head_dim_v=128, act_param=0.05), seqlens_q=FP16_LENS,
                       seqlens_k=FP16_LENS)
    check_backward(g, bt)


@pytest.mark.parametrize("case", [0, 1, 3, 4])
def test_head_dims_192_128_backward_masks_gqa(g, case):
    mask, wl_, wr_, lq, lk = MASK_CASES[case]
    wl = _wl(act="silu", head_dim=192, head_dim_v=128, mask=mask, window_left=wl_, window_right=wr_,
             batch=len(lq), heads_q=8, heads_kv=2)
    check_backward(g, gi.make_batch(wl, seqlens_q=lq, seqlens_k=lk))


def test_head_dims_192_128_backward_fp16_short_kv_and_fixed_length(g):
    # fp16 inputs; few keys (dS carried as hi + lo for dQ, still the separate
    # dQ kernel: the fused pass needs equal head dims); fixed-length entry point
    check_backward(g, gi.make_batch(_wl(act="fast_gelu", head_dim=192, head_dim_v=128, fp16=True),
                                    seqlens_q=[1100, 33], seqlens_k=[1100, 33]))
    check_backward(g, gi.make_batch(_wl(act="relu2", head_dim=192, head_dim_v=128), seqlens_q=[300, 50, 7],
                                    seqlens_k=[64, 100, 1]))
    wl = _wl(act="silu", head_dim=192, head_dim_v=128, varlen=False, batch=2, lq_range=(300, 300))
    check_backward(g, gi.make_batch(wl))


# ------------------------------------------------ MXFP8 Q/K (E8M0 block scales)
MX_CASES = [
    dict(act="fast_gelu"),
    dict(act="leaky_relu", act_param=0.01, mask="window", window_left=100, window_right=0, heads_q=8, heads_kv=2),
    dict(act="silu", mask="causal"),
    dict(act="relu2", heads_q=4, heads_kv=1),
]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("case", range(len(MX_CASES)))
def test_mxfp8_forward(g, case, D):
    # per-block E8M0 scales of Q and K (the quantiser gives every 32-element
    # block its own exponent) enter the block-scaled MFMA; jagged lengths with
    # empty, one-token and ragged sequences over several KV tiles
    lens = [700, 1, 0, 300, 64, 129]
    bt = gi.make_batch(_wl(head_dim=D, batch=len(lens), mx_qk=True, backward=False, **MX_CASES[case]),
                       seqlens_q=lens, seqlens_k=lens)
    # spread the block scales (a seeded offset in [-3, 3] per block): any
    # block taking another block's scale then fails by factors of up to 2^6
    rng = np.random.default_rng(77 + case)
    bt = dataclasses.replace(bt, q_mx=(bt.q_mx.astype(np.int64) + rng.integers(-3, 4, bt.q_mx.shape)).astype(np.uint8),
                             k_mx=(bt.k_mx.astype(np.int64) + rng.integers(-3, 4, bt.k_mx.shape)).astype(np.uint8))
    assert len(np.unique(bt.q_mx)) >= 7 and len(np.unique(bt.k_mx)) >= 7
    check_forward(g, bt)


def test_mxfp8_scales_are_applied(g):
    # raising every q scale by 2 and every k scale by 1 multiplies the scores
    # by 8; checked against the oracle on the changed scales, and the output
    # differs from the unchanged one
    import torch
    lens = [200, 77]
    bt = gi.make_batch(_wl(head_dim=128, batch=2, mx_qk=True, backward=False, act="silu"), seqlens_q=lens,
                       seqlens_k=lens)
    o1 = run_forward(g, bt)
    bt2 = dataclasses.replace(bt, q_mx=(bt.q_mx + 2).astype(np.uint8), k_mx=(bt.k_mx + 1).astype(np.uint8))
    check_forward(g, bt2)
    assert not torch.equal(o1, run_forward(g, bt2))


def test_mxfp8_unsupported_head_dim_and_missing_scales(g):
    import torch
    bt = gi.make_batch(_wl(head_dim=96, batch=1, mx_qk=True, backward=False), seqlens_q=[40], seqlens_k=[40])
    with pytest.raises(g.GDPAError) as e:
        run_forward(g, bt)
    assert e.value.status == 2
    bt = gi.make_batch(_wl(head_dim=64, batch=1, mx_qk=True, backward=False), seqlens_q=[40], seqlens_k=[40])
    dev = device_batch(bt)
    o = torch.empty(40, 4, 64, device="cuda")
    with pytest.raises(g.GDPAError) as e:
        g.gdpa_varlen_fwd_mxfp8(dev["q"], None, dev["k"], dev["k_mx"], dev["v"], o, dev["cu_q"], dev["cu_k"], 40, 40,
                                0.1)
    assert e.value.status == 1


# --------------------------------------------------- MXFP4 (E2M1, E8M0 per 32)
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("case", range(len(MX_CASES)))
def test_mxfp4_forward(g, case, D):
    # the MXFP8 cases with FP4 elements: per-block scales spread by a seeded
    # offset, jagged lengths with empty, one-token and ragged sequences
    lens = [700, 1, 0, 300, 64, 129]
    bt = gi.make_batch(_wl(head_dim=D, batch=len(lens), mx4_qk=True, backward=False, **MX_CASES[case]),
                       seqlens_q=lens, seqlens_k=lens)
    rng = np.random.default_rng(97 + case)
    bt = dataclasses.replace(bt, q_mx=(bt.q_mx.astype(np.int64) + rng.integers(-3, 4, bt.q_mx.shape)).astype(np.uint8),
                             k_mx=(bt.k_mx.astype(np.int64) + rng.integers(-3, 4, bt.k_mx.shape)).astype(np.uint8))
    assert len(np.unique(bt.q_mx)) >= 7 and len(np.unique(bt.k_mx)) >= 7
    check_forward(g, bt)


def test_mxfp4_scales_and_nibble_order_matter(g):
    # raising the q scales by 2 multiplies the scores by 4 (checked against the
    # oracle); swapping the two nibbles of every q byte changes the result
    import torch
    lens = [200, 77]
    bt = gi.make_batch(_wl(head_dim=128, batch=2, mx4_qk=True, backward=False, act="silu"), seqlens_q=lens,
                       seqlens_k=lens)
    o1 = run_forward(g, bt)
    bt2 = dataclasses.replace(bt, q_mx=(bt.q_mx + 2).astype(np.uint8))
    check_forward(g, bt2)
    assert not torch.equal(o1, run_forward(g, bt2))
    bt3 = dataclasses.replace(bt, q=((bt.q >> 4) | (bt.q << 4)).astype(np.uint8))
    check_forward(g, bt3)
    assert not torch.equal(o1, run_forward(g, bt3))


def test_mxfp4_unsupported_head_dim_and_missing_scales(g):
    import torch
    bt = gi.make_batch(_wl(head_dim=96, batch=1, mx4_qk=True, backward=False), seqlens_q=[40], seqlens_k=[40])
    with pytest.raises(g.GDPAError) as e:
        run_forward(g, bt)
    assert e.value.status == 2
    bt = gi.make_batch(_wl(head_dim=64, batch=1, mx4_qk=True, backward=False), seqlens_q=[40], seqlens_k=[40])
    dev = device_batch(bt)
    o = torch.empty(40, 4, 64, device="cuda")
    with pytest.raises(g.GDPAError) as e:
        g.gdpa_varlen_fwd_mxfp4(dev["q"], dev["q_mx"], dev["k"], None, dev["v"], o, dev["cu_q"], dev["cu_k"], 40, 40,
                                0.1)
    assert e.value.status == 1


# ------------------------------- backward from 8- and 4-bit Q/K (decoded to bf16)
def _lowp(fmt):
    return dict(fp8_qk=fmt == "fp8", mx_qk=fmt == "mxfp8", mx4_qk=fmt == "mxfp4")


@pytest.mark.parametrize("fmt,D", [("fp8", 64), ("fp8", 96), ("fp8", 128), ("mxfp8", 64), ("mxfp8", 128),
                                   ("mxfp4", 64), ("mxfp4", 128)])
def test_lowp_backward(g, fmt, D):
    # FP8 codes carry per-tensor descales (amax / 448, not 1: S, dQ and dK
    # fold them in differently); MX codes block scales.  Jagged lengths with
    # empty and one-token sequences over several key blocks (separate dQ)
    lens = [300, 1, 0, 129, 64]
    bt = gi.make_batch(_wl(head_dim=D, batch=len(lens), act="silu", **_lowp(fmt)), seqlens_q=lens, seqlens_k=lens)
    if fmt == "fp8":
        assert abs(bt.q_scale - 1) > 0.5 and abs(bt.k_scale - 1) > 0.5 and bt.q_scale != bt.k_scale
    check_backward(g, bt)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp8", "mxfp4"])
@pytest.mark.parametrize("case", [0, 1, 3])
def test_lowp_backward_masks_gqa(g, fmt, case):
    mask, wl_, wr_, lq, lk = MASK_CASES[case]
    wl = _wl(act="gelu_tanh", mask=mask, window_left=wl_, window_right=wr_, batch=len(lq), heads_q=8, heads_kv=2,
             **_lowp(fmt))
    check_backward(g, gi.make_batch(wl, seqlens_q=lq, seqlens_k=lk))


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_lowp_backward_short_kv_and_bf16_gradients(g, fmt):
    # 64 keys per sequence: dQ comes from the fused pass (written from the
    # single key block), with its own dQ factor; then bf16 gradients
    import torch
    wl = dataclasses.replace(gi.WORKLOADS["short_kv_cross"], batch=4, act="relu2", **_lowp(fmt))
    bt = gi.make_batch(wl)
    check_backward(g, bt)
    dq, dk, dv = [t.cpu().double().numpy() for t in run_backward(g, bt, grad_dtype=torch.bfloat16)]
    errs = backward_ratios(bt, dq, dk, dv)
    assert max(errs.values()) <= TOL_BWD, errs


# ---------------------------------------- short key/value: hi/lo-split dS and P
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("act", ["silu", "fast_gelu", "gelu", "hardswish"])
def test_short_kv_backward(g, act, D):
    # at most 128 keys per sequence: dQ carries dS as a bf16 hi/lo pair
    bt = gi.make_batch(_wl(act=act, head_dim=D), seqlens_q=[300, 50, 7], seqlens_k=[64, 100, 1])
    check_forward(g, bt)
    check_backward(g, bt)
