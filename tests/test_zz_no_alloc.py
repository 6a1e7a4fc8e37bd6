"""The allocation-free backward (gdpa_varlen_bwd_noalloc) against the
workspace entry point (gdpa_varlen_bwd) through the C ABI: bitwise the same
dQ, dK and dV on consecutive calls that share the library's per-GPU scratch
array (the later calls smaller), on the separate-dQ path, the fused pass with
one key block, and the fused pass with ordered multi-block dQ sums; a call
whose workspace exceeds the scratch size is refused before anything runs."""
import pytest

import gdpa_inputs as gi
from helpers import TOL_BWD, backward_ratios, device_batch, run_backward

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import generalized_attention_amd
    return generalized_attention_amd


def _wl(**kw):
    base = dict(name="t", batch=2, heads_q=4, heads_kv=2, head_dim=128, lq_range=(1, 300), lk_range=None,
                act="silu", backward=True, seed=23)
    base.update(kw)
    return gi.Workload(**base)


def _noalloc(g, bt, dev, grad_dtype):
    import torch
    wl = bt.wl
    fill = lambda s: torch.full(s, float("nan"), dtype=grad_dtype, device="cuda")
    dq, dk, dv = fill(bt.q.shape), fill(bt.k.shape), fill(bt.v.shape)
    g.gdpa_varlen_bwd_noalloc(dev["q"], dev["k"], dev["v"], dev["do"], dq, dk, dv, dev["cu_q"], dev["cu_k"],
                              bt.max_seqlen_q, bt.max_seqlen_k, wl.scale, act=wl.act, act_param=wl.act_param,
                              mask=wl.mask, window_left=wl.window_left, window_right=wl.window_right)
    return dq, dk, dv


# (dQ mode, grad dtype, lq, lk, workload options): each later case smaller
# than the one before it in the same mode
CASES = [
    ("auto", "fp32", [700, 1, 0, 1537, 64, 129], None, dict(mask="causal")),   # several key blocks: separate dQ
    ("auto", "fp32", [300, 65], None, dict()),
    ("auto", "bf16", [900, 7, 300], [64, 100, 1], dict(act="relu2")),           # one key block: fused, direct dQ
    ("auto", "bf16", [129, 3], [33, 64], dict(act="relu2")),
    ("fused", "fp32", [1100, 40, 700], None, dict(act="gelu_tanh")),            # ordered multi-block dQ sums
    ("fused", "fp32", [260, 9], None, dict(act="gelu_tanh", mask="window", window_left=100, window_right=20)),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_noalloc_backward_matches_the_workspace_entry_point(g, monkeypatch, case):
    import torch
    mode, gd, lq, lk, opts = CASES[case]
    if mode != "auto":
        monkeypatch.setenv("GDPA_BWD_DQ", mode)
    grad_dtype = torch.float32 if gd == "fp32" else torch.bfloat16
    bt = gi.make_batch(_wl(batch=len(lq), **opts), seqlens_q=lq, seqlens_k=lk or lq)
    dev = device_batch(bt)
    print(f"[noalloc] case {case}: mode {mode}, {gd}, lq {lq}, lk {lk or lq}", flush=True)
    ref = run_backward(g, bt, dev, grad_dtype=grad_dtype)
    for rep in range(2):
        got = _noalloc(g, bt, dev, grad_dtype)
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"case {case}, call {rep + 1}"
    if gd == "fp32":
        errs = backward_ratios(bt, *got)
        assert max(errs.values()) <= TOL_BWD, errs


def test_noalloc_refuses_a_workspace_beyond_its_scratch(g, monkeypatch):
    # bf16 dQ summed over several key blocks inside the dK/dV pass needs an
    # fp32 accumulator of total_q x Hq x D values: 5000 x 4 x 128 x 4 B > 8 MiB
    import torch
    monkeypatch.setenv("GDPA_BWD_DQ", "fused")
    lens = [2500, 2500]
    bt = gi.make_batch(_wl(batch=2), seqlens_q=lens, seqlens_k=lens)
    need = g.lib().gdpa_varlen_bwd_workspace_size(2, 2500, 2500, 5000, 4, 2, 128, 0)  # bf16 grads
    assert need > 8 << 20
    dev = device_batch(bt)
    dq = torch.full(bt.q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    dk = torch.full(bt.k.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    dv = torch.full(bt.v.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(g.GDPAError) as e:
        g.gdpa_varlen_bwd_noalloc(dev["q"], dev["k"], dev["v"], dev["do"], dq, dk, dv, dev["cu_q"], dev["cu_k"],
                                  2500, 2500, bt.wl.scale, act=bt.wl.act)
    assert e.value.status == 3                       # GDPA_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.isnan(dq.float()).all() and torch.isnan(dk.float()).all()   # nothing ran
