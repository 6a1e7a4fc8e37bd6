"""Host-side logic of bench.py (CPU): the allowed-pair count behind the flop
figures, and the parity record that the oracle leg attaches to a bench line."""
import dataclasses

import numpy as np
import pytest

import bench
import gdpa_inputs as gi
import oracle
from helpers import oracle_inputs


@pytest.mark.parametrize("lq,lk,wl,wr", [(7, 7, -1, -1), (7, 7, -1, 0), (5, 9, -1, 0), (9, 5, -1, 0),
                                         (12, 12, 3, 0), (6, 10, 2, 1), (10, 6, 0, 0), (0, 4, -1, -1)])
def test_allowed_pairs_matches_mask(lq, lk, wl, wr):
    # the bench's closed-form count equals the oracle's mask summed element by element
    mask = "none" if wl < 0 and wr < 0 else ("causal" if wl < 0 else "window")
    want = int(oracle.allowed_mask(lq, lk, mask, wl, wr).sum()) if lq and lk else 0
    assert bench.allowed_pairs(lq, lk, wl, wr) == want


def _oracle_outputs(bt):
    wl = bt.wl
    q, k, v, do = (oracle.decode_bf16(x) for x in (bt.q, bt.k, bt.v, bt.do))
    kw = dict(act_param=wl.act_param, mask=wl.mask, window_left=wl.window_left, window_right=wl.window_right)
    cu = (bt.cu_seqlens_q, bt.cu_seqlens_k)
    o = oracle.gdpa_forward(q, k, v, *cu, wl.scale, wl.act, **kw)
    dq, dk, dv = oracle.gdpa_backward(q, k, v, do, *cu, wl.scale, wl.act, **kw)
    return {n: x.astype(np.float32) for n, x in dict(o=o, dq=dq, dk=dk, dv=dv).items()}


def test_parity_record_passes_on_oracle_outputs_and_flags_a_wrong_one():
    wl = dataclasses.replace(gi.WORKLOADS["tiny"], backward=True)
    bt = gi.make_batch(wl)
    out = _oracle_outputs(bt)
    base, sample = bench.cpu_baseline(bt, 1.0, workers=2)
    assert base["kind"] == "oracle" and base["value"] > 0 and base["cores"] == 2
    parity = bench.parity_record(bt, sample, out)
    assert parity["pass"] and set(parity["err_rms"]) == {"o", "dq", "dk", "dv"}
    assert max(parity["err_rms"].values()) < 1e-6  # fp32 storage of the fp64 result
    out["dv"] = out["dv"].copy()
    out["dv"][3, 1, 5] += 0.5 * np.sqrt(np.mean(out["dv"].astype(np.float64) ** 2)) / 0.01  # one element off
    bad = bench.parity_record(bt, sample, out)
    assert not bad["pass"] and bad["err_rms"]["dv"] > bad["tol"]["dv"]


def test_cpu_baseline_pool_size_and_gqa_sums():
    # GQA: dK/dV of a KV head sum the group's query heads, computed as
    # separate tasks; the pool record states its process count
    wl = dataclasses.replace(gi.WORKLOADS["tiny"], heads_q=4, heads_kv=2, backward=True)
    bt = gi.make_batch(wl)
    out = _oracle_outputs(bt)
    base, sample = bench.cpu_baseline(bt, 0.5, workers=3)
    assert base["unit"] == "TFLOP/s" and base["cores"] == 3
    assert bench.parity_record(bt, sample, out)["pass"]
    assert 1 <= bench.pool_size() <= 16


def test_cpu_baseline_decodes_the_low_precision_formats():
    # the oracle leg of the 8- and 4-bit workloads consumes the decoded codes
    # (codes x per-tensor or block scale); the forward takes the FP8 bar, the
    # gradients their own
    for fmt in ("fp8", "mxfp8", "mxfp4"):
        wl = dataclasses.replace(gi.WORKLOADS["tiny"], backward=True, fp8_qk=fmt == "fp8", mx_qk=fmt == "mxfp8",
                                 mx4_qk=fmt == "mxfp4")
        assert bench.lowp_format(wl) == fmt
        bt = gi.make_batch(wl)
        q, k, v, do = oracle_inputs(bt)
        kw = dict(act_param=wl.act_param, mask=wl.mask, window_left=wl.window_left, window_right=wl.window_right)
        cu = (bt.cu_seqlens_q, bt.cu_seqlens_k)
        o = oracle.gdpa_forward(q, k, v, *cu, wl.scale, wl.act, **kw)
        dq, dk, dv = oracle.gdpa_backward(q, k, v, do, *cu, wl.scale, wl.act, **kw)
        out = {n: x.astype(np.float32) for n, x in dict(o=o, dq=dq, dk=dk, dv=dv).items()}
        base, sample = bench.cpu_baseline(bt, 0.5, workers=2)
        parity = bench.parity_record(bt, sample, out)
        assert parity["pass"] and max(parity["err_rms"].values()) < 1e-6, (fmt, parity)
        assert parity["tol"]["o"] == bench.TOL_FP8 and parity["tol"]["dq"] == bench.TOL["dq"]
    assert bench.lowp_format(gi.WORKLOADS["jagged_self"]) is None


def test_parity_record_kink_allowance_for_piecewise_linear_activations():
    # LeakyReLU gradients: the record subtracts the tests' per-element kink
    # allowance from dQ/dK errors (zero away from the kink, so oracle outputs
    # still pass exactly and a gross error still fails)
    wl = dataclasses.replace(gi.WORKLOADS["tiny"], act="leaky_relu", act_param=0.01, backward=True)
    bt = gi.make_batch(wl)
    out = _oracle_outputs(bt)
    base, sample = bench.cpu_baseline(bt, 0.5, workers=2)
    parity = bench.parity_record(bt, sample, out)
    assert parity["pass"] and "kink allowance" in parity["sample"]
    assert max(parity["err_rms"].values()) < 1e-6
    out["dq"] = out["dq"] * 1.5
    assert not bench.parity_record(bt, sample, out)["pass"]


def test_more_than_one_gpu_exits_with_a_message():
    # the path runs on one GPU; a multi-GPU request is refused before any
    # GPU or oracle work, with exit status 2 and a message saying so
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=root)
    assert r.returncode == 2 and r.stdout == ""
    assert "one GPU" in r.stderr or "1 GPU" in r.stderr, r.stderr
