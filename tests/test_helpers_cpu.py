"""CPU checks of the test-side kink allowance (tests/helpers.py)."""
import numpy as np

import gdpa_inputs as gi
from helpers import kink_allowance, kink_jumps


def _batch(act, q, k):
    wl = gi.Workload("k", 1, 1, 1, q.shape[-1], (q.shape[0], q.shape[0]), (k.shape[0], k.shape[0]), act,
                     act_param=0.05, backward=True)
    lq, lk = q.shape[0], k.shape[0]
    return gi.Batch(wl, np.array([lq]), np.array([lk]), np.array([0, lq], np.int32), np.array([0, lk], np.int32),
                    None, None, None, None)


def test_jump_sizes():
    assert kink_jumps("relu", 0.01) == [(0.0, 1.0)]
    assert kink_jumps("leaky_relu", 0.05) == [(0.0, 0.95)]
    assert kink_jumps("hardswish", 0.0) == [(-3.0, 0.5), (3.0, 0.5)]
    for smooth in ("silu", "gelu", "gelu_tanh", "relu2", "identity"):
        assert kink_jumps(smooth, 0.01) == []


def test_allowance_marks_only_pairs_on_a_kink():
    rng = np.random.default_rng(3)
    D = 8
    q = rng.standard_normal((3, 1, D))
    k = rng.standard_normal((4, 1, D))
    k[2, 0] = 0.0
    k[2, 0, 0], k[2, 0, 1] = q[1, 0, 1], -q[1, 0, 0]     # q1 . k2 = 0 exactly
    v = rng.standard_normal((4, 1, D))
    do = rng.standard_normal((3, 1, D))
    for act in ("leaky_relu", "relu"):
        aq, ak = kink_allowance(_batch(act, q, k), q, k, v, do)
        assert np.all(aq[[0, 2]] == 0) and aq[1].any()
        assert np.all(ak[[0, 1, 3]] == 0) and np.all(ak[2] > 0)
        jump = kink_jumps(act, 0.05)[0][1]
        scale = 1 / np.sqrt(D)
        dp = do[1, 0] @ v[2, 0]
        assert np.allclose(aq[1, 0], scale * jump * abs(dp) * np.abs(k[2, 0]))
    aq, ak = kink_allowance(_batch("silu", q, k), q, k, v, do)
    assert not aq.any() and not ak.any()
