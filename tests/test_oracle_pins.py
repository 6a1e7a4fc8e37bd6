"""Pins of the fp64 CPU oracle against things other than itself.

Each test checks the oracle against a fact the pages or mathematics fix:
hand-derived fixtures, textbook activation values, library routines, closed
forms, brute force on tiny inputs, and finite differences.  A plausible
mistake in the oracle (a dropped term, wrong sign, wrong index, transposed
operand, wrong mask alignment or head mapping) fails at least one of them.
"""
import json
import math
import os
import statistics

import numpy as np
import pytest

import oracle
from oracle import act, act_grad, decode_bf16, decode_e4m3, decode_f16, gdpa_forward, gdpa_backward
from oracle.gdpa import allowed_mask, gdpa_forward_rows, gdpa_backward_q_rows, gdpa_backward_k_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ACTS = oracle.ACT_NAMES
# act(x) - act(-x) = c x  (odd part); ReLU^2 has none of this form
ODD_C = {"identity": 2.0, "gelu": 1.0, "gelu_tanh": 1.0, "fast_gelu": 1.0, "fast_gelu_bf16": 1.0,
         "relu": 1.0, "leaky_relu": 1.0 + 0.01, "silu": 1.0, "fast_silu": 1.0, "hardswish": 1.0}


def _cu(lens):
    cu = np.zeros(len(lens) + 1, np.int64)
    cu[1:] = np.cumsum(lens)
    return cu


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ----------------------------------------------------------------- activations
def test_activation_textbook_values():
    with open(os.path.join(GOLDEN, "activation_values.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        y = act(c["act"], c["x"], c.get("alpha", 0.01))
        assert abs(float(y) - c["y"]) <= 1e-12 * max(1.0, abs(c["y"])), c


def test_gelu_is_x_times_normal_cdf():
    nd = statistics.NormalDist()
    for x in np.linspace(-6, 6, 97):
        assert abs(act("gelu", x) - x * nd.cdf(x)) < 1e-13


def test_silu_via_tanh_identity():
    # sigmoid(x) = (1 + tanh(x/2)) / 2
    for x in np.linspace(-20, 20, 81):
        ref = x * 0.5 * (1.0 + math.tanh(x / 2.0))
        assert abs(act("silu", x) - ref) < 1e-13 * max(1, abs(x))
        assert act("fast_silu", x) == act("silu", x)


def test_tanh_gelu_approximates_gelu():
    # the tanh form is within 4.74e-4 of the erf form everywhere (max near x=-2.70)
    x = np.linspace(-12, 12, 240001)
    d = np.abs(act("gelu_tanh", x) - act("gelu", x))
    assert d.max() < 4.74e-4
    assert d.max() > 4.7e-4   # the published constants give exactly this peak deviation
    for n in ("fast_gelu", "fast_gelu_bf16"):
        assert np.array_equal(act(n, x), act("gelu_tanh", x))


@pytest.mark.parametrize("name", ACTS)
def test_activation_zero_at_zero(name):
    assert act(name, 0.0) == 0.0


@pytest.mark.parametrize("name", ACTS)
def test_activation_derivative_matches_finite_differences(name):
    x = np.linspace(-7.3, 7.3, 1461)
    kinks = {"relu": [0.0], "relu2": [0.0], "leaky_relu": [0.0], "hardswish": [-3.0, 3.0]}.get(name, [])
    for k in kinks:
        x = x[np.abs(x - k) > 1e-3]
    h = 1e-6
    fd = (act(name, x + h, 0.01) - act(name, x - h, 0.01)) / (2 * h)
    assert np.max(np.abs(fd - act_grad(name, x, 0.01))) < 5e-8


@pytest.mark.parametrize("name", [a for a in ACTS if a != "relu2"])
def test_activation_odd_part(name):
    x = np.linspace(-9, 9, 721)
    assert np.max(np.abs(act(name, x) - act(name, -x) - ODD_C[name] * x)) < 1e-12


def test_leaky_relu_limits():
    x = np.linspace(-5, 5, 101)
    assert np.array_equal(act("leaky_relu", x, 1.0), x)
    assert np.array_equal(act("leaky_relu", x, 0.0), act("relu", x))


# ------------------------------------------------------------------- formats
def test_bf16_decode_matches_torch():
    import torch
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy().astype(np.float64)
    got = decode_bf16(bits)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_f16_decode_matches_numpy():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = decode_f16(bits)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    # binary16 landmarks: 1, -2, largest finite, smallest subnormal, infinity
    assert list(decode_f16([0x3C00, 0xC000, 0x7BFF, 0x0001, 0x7C00])) == [1.0, -2.0, 65504.0, 2.0 ** -24, np.inf]


def test_e4m3_decode_matches_torch():
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = decode_e4m3(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.nanmax(got) == 448.0 and decode_e4m3([0x01])[0] == 2.0 ** -9
    assert decode_e4m3([0x38], 0.5)[0] == 0.5   # 1.0 * scale


# -------------------------------------------------------------- hand fixture
def test_hand_fixture():
    with open(os.path.join(GOLDEN, "hand_relu_cross.json")) as f:
        g = json.load(f)
    q = np.array(g["q"], float)[:, None, :]
    k = np.array(g["k"], float)[:, None, :]
    v = np.array(g["v"], float)[:, None, :]
    cq, ck = [0, 2], [0, 3]
    o = gdpa_forward(q, k, v, cq, ck, 1.0, "relu")[:, 0]
    assert np.array_equal(o, np.array(g["relu_none"], float))
    o = gdpa_forward(q, k, v, cq, ck, 1.0, "relu", mask="causal")[:, 0]
    assert np.array_equal(o, np.array(g["relu_causal"], float))
    o = gdpa_forward(q, k, v, cq, ck, 1.0, "relu", mask="window", window_left=0, window_right=0)[:, 0]
    assert np.array_equal(o, np.array(g["relu_window_0_0"], float))
    o = gdpa_forward(q, k, v, cq, ck, 1.0, "identity")[:, 0]
    assert np.array_equal(o, np.array(g["identity_none"], float))
    do = np.ones((2, 1, 2))
    dq, dk, dv = gdpa_backward(q, k, v, do, cq, ck, 1.0, "identity")
    gg = g["identity_none_grad_do_ones"]
    assert np.array_equal(dq[:, 0], np.array(gg["dq"], float))
    assert np.array_equal(dk[:, 0], np.array(gg["dk"], float))
    assert np.array_equal(dv[:, 0], np.array(gg["dv"], float))


# ---------------------------------------------------------------- brute force
def _brute_forward(q, k, v, lq, lk, scale, name, alpha, mask, wl, wr):
    """Pure-Python loops, one (sequence, head, i, j, d) at a time."""
    B = len(lq)
    hq, hkv, D = q.shape[1], k.shape[1], v.shape[2]
    o = [[[0.0] * D for _ in range(hq)] for _ in range(q.shape[0])]
    qoff = koff = 0
    for b in range(B):
        for h in range(hq):
            g = (h * hkv) // hq
            for i in range(lq[b]):
                ip = i + lk[b] - lq[b]
                for j in range(lk[b]):
                    if mask == "causal" and j > ip:
                        continue
                    if mask == "window" and ((wl >= 0 and j < ip - wl) or (wr >= 0 and j > ip + wr)):
                        continue
                    s = 0.0
                    for d in range(q.shape[2]):
                        s += q[qoff + i, h, d] * k[koff + j, g, d]
                    p = float(act(name, scale * s, alpha))
                    for d in range(D):
                        o[qoff + i][h][d] += p * v[koff + j, g, d]
        qoff += lq[b]
        koff += lk[b]
    return np.array(o)


BRUTE_CASES = [
    # lq, lk, hq, hkv, mask, wl, wr
    ([3, 0, 5], [4, 2, 5], 2, 1, "none", -1, -1),
    ([4, 6], [4, 6], 4, 2, "causal", -1, -1),
    ([2, 7], [5, 7], 2, 2, "causal", -1, -1),
    ([6, 3], [6, 8], 4, 1, "window", 2, 0),
    ([5], [7], 1, 1, "window", 1, 2),
]


@pytest.mark.parametrize("case", range(len(BRUTE_CASES)))
@pytest.mark.parametrize("name", ["gelu", "fast_gelu", "relu2", "leaky_relu", "silu", "hardswish", "identity"])
def test_forward_matches_brute_force(case, name):
    lq, lk, hq, hkv, mask, wl, wr = BRUTE_CASES[case]
    rng = np.random.default_rng(100 + case)
    D = 3
    q = _rand(rng, sum(lq), hq, D)
    k = _rand(rng, sum(lk), hkv, D)
    v = _rand(rng, sum(lk), hkv, D)
    o = gdpa_forward(q, k, v, _cu(lq), _cu(lk), 0.7, name, 0.05, mask, wl, wr)
    ref = _brute_forward(q, k, v, lq, lk, 0.7, name, 0.05, mask, wl, wr)
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", [0, 1, 3])
@pytest.mark.parametrize("name", ["fast_gelu", "silu", "relu2"])
def test_forward_matches_brute_force_distinct_v_dim(case, name):
    # head dim of V (and O) differs from that of Q and K (the README's "(192, 128)")
    lq, lk, hq, hkv, mask, wl, wr = BRUTE_CASES[case]
    rng = np.random.default_rng(200 + case)
    q = _rand(rng, sum(lq), hq, 3)
    k = _rand(rng, sum(lk), hkv, 3)
    v = _rand(rng, sum(lk), hkv, 5)
    o = gdpa_forward(q, k, v, _cu(lq), _cu(lk), 0.7, name, 0.05, mask, wl, wr)
    assert o.shape == (sum(lq), hq, 5)
    ref = _brute_forward(q, k, v, lq, lk, 0.7, name, 0.05, mask, wl, wr)
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- closed forms
def test_identity_closed_form_associativity():
    # identity act, no mask: O = scale Q (K^T V) per (b, h)
    rng = np.random.default_rng(7)
    lq, lk, hq, hkv, D = [5, 9, 1], [6, 3, 4], 6, 3, 8
    q, k, v = _rand(rng, sum(lq), hq, D), _rand(rng, sum(lk), hkv, D), _rand(rng, sum(lk), hkv, D)
    cq, ck = _cu(lq), _cu(lk)
    o = gdpa_forward(q, k, v, cq, ck, 0.3, "identity")
    for b in range(3):
        for h in range(hq):
            g = h // 2
            kv = k[ck[b]:ck[b + 1], g].T @ v[ck[b]:ck[b + 1], g]           # [D, D]
            ref = 0.3 * q[cq[b]:cq[b + 1], h] @ kv
            assert np.allclose(o[cq[b]:cq[b + 1], h], ref, rtol=1e-12, atol=1e-12)


def test_identity_causal_and_window_prefix_sums():
    # O_i = scale q_i (sum_{allowed j} k_j v_j^T), allowed set a contiguous range -> prefix sums
    rng = np.random.default_rng(8)
    lq, lk, D = 7, 10, 4
    q, k, v = _rand(rng, lq, 1, D), _rand(rng, lk, 1, D), _rand(rng, lk, 1, D)
    outer = np.einsum("jd,je->jde", k[:, 0], v[:, 0])
    pref = np.concatenate([np.zeros((1, D, D)), np.cumsum(outer, axis=0)])   # pref[n] = sum_{j<n}
    for mask, wl, wr in [("causal", -1, -1), ("window", 3, 1), ("window", 0, 0), ("window", -1, 2)]:
        o = gdpa_forward(q, k, v, [0, lq], [0, lk], 1.25, "identity", mask=mask, window_left=wl, window_right=wr)
        for i in range(lq):
            ip = i + lk - lq
            lo = 0 if (mask == "causal" or wl < 0) else max(0, ip - wl)
            hi = ip if mask == "causal" else (lk - 1 if wr < 0 else min(lk - 1, ip + wr))
            m = pref[hi + 1] - pref[lo] if hi >= lo else np.zeros((D, D))
            assert np.allclose(o[i, 0], 1.25 * q[i, 0] @ m, rtol=1e-11, atol=1e-12)


def test_relu2_feature_map():
    # Q, K >= 0 elementwise -> s >= 0 and relu2(s) = s^2 = (q (x) q) . (k (x) k)
    rng = np.random.default_rng(9)
    lq, lk, D = 6, 5, 3
    q, k, v = np.abs(_rand(rng, lq, 1, D)), np.abs(_rand(rng, lk, 1, D)), _rand(rng, lk, 1, D)
    o = gdpa_forward(q, k, v, [0, lq], [0, lk], 0.5, "relu2")
    phi_q = np.einsum("id,ie->ide", q[:, 0], q[:, 0]).reshape(lq, D * D)
    phi_k = np.einsum("jd,je->jde", k[:, 0], k[:, 0]).reshape(lk, D * D)
    ref = 0.25 * phi_q @ (phi_k.T @ v[:, 0])
    assert np.allclose(o[:, 0], ref, rtol=1e-12, atol=1e-12)
    # homogeneity of degree 2 in Q
    o2 = gdpa_forward(3.0 * q, k, v, [0, lq], [0, lk], 0.5, "relu2")
    assert np.allclose(o2, 9.0 * o, rtol=1e-12)


def test_relu_on_nonnegative_scores_is_identity():
    rng = np.random.default_rng(10)
    q, k, v = np.abs(_rand(rng, 4, 2, 3)), np.abs(_rand(rng, 6, 2, 3)), _rand(rng, 6, 2, 3)
    a = gdpa_forward(q, k, v, [0, 4], [0, 6], 0.9, "relu")
    b = gdpa_forward(q, k, v, [0, 4], [0, 6], 0.9, "identity")
    assert np.allclose(a, b, rtol=1e-13)


@pytest.mark.parametrize("name", [a for a in ACTS if a != "relu2"])
@pytest.mark.parametrize("mask", ["none", "causal", "window"])
def test_odd_part_identity_through_attention(name, mask):
    # O_act(Q) - O_act(-Q) = c * O_identity(Q) under any mask
    rng = np.random.default_rng(11)
    lq, lk, hq, hkv, D = [5, 3], [5, 6], 2, 1, 4
    q, k, v = _rand(rng, 8, hq, D), _rand(rng, 11, hkv, D), _rand(rng, 11, hkv, D)
    kw = dict(mask=mask, window_left=2, window_right=1)
    a = gdpa_forward(q, k, v, _cu(lq), _cu(lk), 0.6, name, 0.01, **kw)
    b = gdpa_forward(-q, k, v, _cu(lq), _cu(lk), 0.6, name, 0.01, **kw)
    c = gdpa_forward(q, k, v, _cu(lq), _cu(lk), 0.6, "identity", **kw)
    assert np.allclose(a - b, ODD_C[name] * c, rtol=1e-11, atol=1e-11)


# ---------------------------------------------------------- structural checks
def test_jagged_equals_concatenation_of_dense():
    rng = np.random.default_rng(12)
    lq, lk, hq, hkv, D = [4, 0, 7, 2], [3, 5, 7, 1], 4, 2, 5
    q, k, v = _rand(rng, sum(lq), hq, D), _rand(rng, sum(lk), hkv, D), _rand(rng, sum(lk), hkv, D)
    do = _rand(rng, sum(lq), hq, D)
    cq, ck = _cu(lq), _cu(lk)
    o = gdpa_forward(q, k, v, cq, ck, 0.4, "silu", mask="causal")
    dq, dk, dv = gdpa_backward(q, k, v, do, cq, ck, 0.4, "silu", mask="causal")
    for b in range(4):
        sq, sk = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
        ob = gdpa_forward(q[sq], k[sk], v[sk], [0, lq[b]], [0, lk[b]], 0.4, "silu", mask="causal")
        assert np.array_equal(o[sq], ob)
        g = gdpa_backward(q[sq], k[sk], v[sk], do[sq], [0, lq[b]], [0, lk[b]], 0.4, "silu", mask="causal")
        assert np.array_equal(dq[sq], g[0]) and np.array_equal(dk[sk], g[1]) and np.array_equal(dv[sk], g[2])


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(13)
    lq, lk, hq, hkv, D = [5, 6], [4, 6], 6, 2, 3
    q, k, v = _rand(rng, 11, hq, D), _rand(rng, 10, hkv, D), _rand(rng, 10, hkv, D)
    do = _rand(rng, 11, hq, D)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)   # head h -> kv head h // 3
    cq, ck = _cu(lq), _cu(lk)
    a = gdpa_forward(q, k, v, cq, ck, 0.5, "gelu", mask="window", window_left=2, window_right=0)
    b = gdpa_forward(q, kr, vr, cq, ck, 0.5, "gelu", mask="window", window_left=2, window_right=0)
    assert np.allclose(a, b, rtol=1e-14, atol=1e-14)
    ga = gdpa_backward(q, k, v, do, cq, ck, 0.5, "gelu", mask="causal")
    gb = gdpa_backward(q, kr, vr, do, cq, ck, 0.5, "gelu", mask="causal")
    assert np.allclose(ga[0], gb[0], rtol=1e-13, atol=1e-13)
    for i in (1, 2):
        summed = gb[i].reshape(gb[i].shape[0], hkv, 3, D).sum(axis=2)
        assert np.allclose(ga[i], summed, rtol=1e-12, atol=1e-12)


def test_mask_reductions():
    L = 9
    assert np.array_equal(allowed_mask(L, L, "causal"), np.tril(np.ones((L, L), bool)))
    assert np.array_equal(allowed_mask(L, L, "window", L - 1, 0), allowed_mask(L, L, "causal"))
    assert np.array_equal(allowed_mask(L, L, "window", -1, -1), np.ones((L, L), bool))
    # bottom-right alignment: a single query (decode step) sees every key under causal
    assert allowed_mask(1, 6, "causal").all()
    # Lq > Lk: the first Lq-Lk queries see nothing
    m = allowed_mask(5, 3, "causal")
    assert not m[:2].any() and np.array_equal(m[2:], np.tril(np.ones((3, 3), bool)))
    # window 512 incl. the diagonal: each full row has window_left + 1 keys
    m = allowed_mask(600, 600, "window", 511, 0)
    assert m.sum(axis=1)[-1] == 512 and m.sum(axis=1)[0] == 1


def test_fully_masked_rows_are_zero():
    rng = np.random.default_rng(14)
    q, k, v = _rand(rng, 5, 1, 3), _rand(rng, 3, 1, 3), _rand(rng, 3, 1, 3)
    o = gdpa_forward(q, k, v, [0, 5], [0, 3], 1.0, "identity", mask="causal")
    assert np.all(o[:2] == 0.0) and np.all(o[2:] != 0.0)
    do = _rand(rng, 5, 1, 3)
    dq, _, _ = gdpa_backward(q, k, v, do, [0, 5], [0, 3], 1.0, "identity", mask="causal")
    assert np.all(dq[:2] == 0.0)


@pytest.mark.parametrize("name", ACTS)
def test_zero_padding_invariance(name):
    # act(0) = 0: extra zero K/V rows change nothing; zero Q/dO rows leave dK/dV unchanged
    rng = np.random.default_rng(15)
    q, k, v, do = _rand(rng, 4, 1, 3), _rand(rng, 5, 1, 3), _rand(rng, 5, 1, 3), _rand(rng, 4, 1, 3)
    o = gdpa_forward(q, k, v, [0, 4], [0, 5], 0.8, name)
    kz, vz = np.concatenate([k, np.zeros((3, 1, 3))]), np.concatenate([v, np.zeros((3, 1, 3))])
    assert np.allclose(gdpa_forward(q, kz, vz, [0, 4], [0, 8], 0.8, name), o, rtol=1e-14, atol=1e-14)
    qz, doz = np.concatenate([q, np.zeros((2, 1, 3))]), np.concatenate([do, np.zeros((2, 1, 3))])
    g1 = gdpa_backward(q, k, v, do, [0, 4], [0, 5], 0.8, name)
    g2 = gdpa_backward(qz, k, v, doz, [0, 6], [0, 5], 0.8, name)
    assert np.allclose(g1[1], g2[1], rtol=1e-13, atol=1e-13) and np.allclose(g1[2], g2[2], rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ backward
FD_CASES = [
    ([3, 0, 2], [2, 3, 4], 2, 1, "none", -1, -1),
    ([4, 3], [4, 5], 4, 2, "causal", -1, -1),
    ([5], [6], 2, 2, "window", 2, 1),
]


@pytest.mark.parametrize("case", range(len(FD_CASES)))
@pytest.mark.parametrize("name", ACTS)
def test_backward_matches_finite_differences(case, name):
    lq, lk, hq, hkv, mask, wl, wr = FD_CASES[case]
    rng = np.random.default_rng(200 + case)
    D = 3
    q, k, v = _rand(rng, sum(lq), hq, D), _rand(rng, sum(lk), hkv, D), _rand(rng, sum(lk), hkv, D)
    G = _rand(rng, sum(lq), hq, D)
    cq, ck = _cu(lq), _cu(lk)
    kw = dict(act_param=0.05, mask=mask, window_left=wl, window_right=wr)

    def loss(qq, kk, vv):
        return float(np.sum(gdpa_forward(qq, kk, vv, cq, ck, 0.9, name, **kw) * G))

    # keep scores away from the kinks of the piecewise activations
    kinks = {"relu": [0.0], "relu2": [0.0], "leaky_relu": [0.0], "hardswish": [-3.0, 3.0]}.get(name, [])
    if kinks:
        for _ in range(50):
            o_s = [0.9 * q[cq[b]:cq[b + 1], h] @ k[ck[b]:ck[b + 1], h * hkv // hq].T
                   for b in range(len(lq)) for h in range(hq)]
            mind = min([np.min(np.abs(s - kk)) for s in o_s if s.size for kk in kinks] + [1.0])
            if mind > 1e-2:
                break
            q = q + 0.05 * _rand(rng, *q.shape)
    dq, dk, dv = gdpa_backward(q, k, v, G, cq, ck, 0.9, name, **kw)
    h = 1e-6
    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = loss(q, k, v)
            arr[idx] = old - h
            lm = loss(q, k, v)
            arr[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        assert np.allclose(grad, fd, rtol=1e-6, atol=1e-6), (name, np.max(np.abs(grad - fd)))


@pytest.mark.parametrize("name", ["silu", "fast_gelu", "relu2"])
def test_backward_distinct_value_head_dim_matches_finite_differences(name):
    # V and dO narrower than Q and K (the pages' head dims (192, 128)), here
    # 5 and 3: dP contracts over V's head dim, S over Q's
    rng = np.random.default_rng(321)
    lq, lk, hq, hkv = [4, 2], [3, 5], 2, 1
    q, k = _rand(rng, sum(lq), hq, 5), _rand(rng, sum(lk), hkv, 5)
    v, G = _rand(rng, sum(lk), hkv, 3), _rand(rng, sum(lq), hq, 3)
    cq, ck = _cu(lq), _cu(lk)

    def loss(qq, kk, vv):
        return float(np.sum(gdpa_forward(qq, kk, vv, cq, ck, 0.7, name, act_param=0.05) * G))

    dq, dk, dv = gdpa_backward(q, k, v, G, cq, ck, 0.7, name, act_param=0.05)
    assert dq.shape == q.shape and dk.shape == k.shape and dv.shape == v.shape
    h = 1e-6
    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = loss(q, k, v)
            arr[idx] = old - h
            lm = loss(q, k, v)
            arr[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        assert np.allclose(grad, fd, rtol=1e-6, atol=1e-6), (name, np.max(np.abs(grad - fd)))


def test_backward_identity_closed_forms():
    # identity, no mask: dV = scale K (Q^T dO), dQ = scale dO (V^T K), dK = scale V (dO^T Q)
    rng = np.random.default_rng(16)
    lq, lk, D = 6, 4, 5
    q, k, v, do = _rand(rng, lq, 1, D), _rand(rng, lk, 1, D), _rand(rng, lk, 1, D), _rand(rng, lq, 1, D)
    dq, dk, dv = gdpa_backward(q, k, v, do, [0, lq], [0, lk], 0.7, "identity")
    Q, K, V, G = q[:, 0], k[:, 0], v[:, 0], do[:, 0]
    assert np.allclose(dv[:, 0], 0.7 * K @ (Q.T @ G), rtol=1e-12)
    assert np.allclose(dq[:, 0], 0.7 * G @ (V.T @ K), rtol=1e-12)
    assert np.allclose(dk[:, 0], 0.7 * V @ (G.T @ Q), rtol=1e-12)


# ----------------------------------------------------- single-row evaluators
def test_row_evaluators_match_full():
    rng = np.random.default_rng(17)
    lq, lk, hq, hkv, D = [5, 7, 3], [6, 7, 2], 4, 2, 4
    q, k, v, do = (_rand(rng, 15, hq, D), _rand(rng, 15, hkv, D), _rand(rng, 15, hkv, D),
                   _rand(rng, 15, hq, D))
    cq, ck = _cu(lq), _cu(lk)
    kw = dict(act_param=0.02, mask="window", window_left=3, window_right=1)
    o = gdpa_forward(q, k, v, cq, ck, 0.5, "hardswish", **kw)
    dq, dk, dv = gdpa_backward(q, k, v, do, cq, ck, 0.5, "hardswish", **kw)
    rows = [(0, 0), (4, 3), (6, 1), (12, 2), (14, 3)]
    assert np.allclose(gdpa_forward_rows(q, k, v, cq, ck, 0.5, "hardswish", rows, **kw),
                       np.array([o[t, h] for t, h in rows]), rtol=1e-13, atol=1e-13)
    assert np.allclose(gdpa_backward_q_rows(q, k, v, do, cq, ck, 0.5, "hardswish", rows, **kw),
                       np.array([dq[t, h] for t, h in rows]), rtol=1e-13, atol=1e-13)
    krows = [(0, 0), (5, 1), (6, 0), (13, 1), (14, 0)]
    a, b = gdpa_backward_k_rows(q, k, v, do, cq, ck, 0.5, "hardswish", krows, **kw)
    assert np.allclose(a, np.array([dk[t, g] for t, g in krows]), rtol=1e-13, atol=1e-13)
    assert np.allclose(b, np.array([dv[t, g] for t, g in krows]), rtol=1e-13, atol=1e-13)


def test_output_rms_statistics():
    # N(0,1) inputs, scale 1/sqrt(D): S ~ N(0,1), so E[O^2] = Lk * E[act(z)^2]
    rng = np.random.default_rng(18)
    L, D = 512, 64
    q, k, v = _rand(rng, L, 1, D), _rand(rng, L, 1, D), _rand(rng, L, 1, D)
    z = np.random.default_rng(19).standard_normal(2_000_000)
    for name in ("gelu", "silu", "relu2"):
        o = gdpa_forward(q, k, v, [0, L], [0, L], 1 / np.sqrt(D), name)
        pred = np.sqrt(L * np.mean(act(name, z) ** 2))
        assert abs(np.sqrt(np.mean(o ** 2)) / pred - 1) < 0.1, name
