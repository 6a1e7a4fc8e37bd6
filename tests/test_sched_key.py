"""The jagged schedule's sort key on the host (CPU only): the block count of
each sequence against the oracle's mask, and the order the keys sort into
(larger cost, then larger lq + lk, then smaller index), the index decoded back
from the key.  The device sort of the same keys is checked in
test_gpu_parity.py."""
import os
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"


def _blocks(lq, lk, mask, wl, wr):
    if lq == 0 or lk == 0:
        return 0
    ok = oracle.allowed_mask(lq, lk, mask, wl, wr)
    mt, nt = -(-lq // 64), -(-lk // 64)
    pad = np.zeros((mt * 64, nt * 64), dtype=bool)
    pad[:lq, :lk] = ok
    return int(pad.reshape(mt, 64, nt, 64).any(axis=(1, 3)).sum())


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not installed")
    exe = str(tmp_path_factory.mktemp("sched") / "sched_key")
    subprocess.run([HIPCC, "-x", "hip", "-O1", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "generalized_attention_amd", "csrc"),
                    os.path.join(ROOT, "tests", "sched_key_driver.cpp"), "-o", exe], check=True, capture_output=True)
    return exe


CASES = [("none", -1, -1), ("causal", -1, 0), ("window", 100, 0), ("window", 50, 30), ("window", 0, 0),
         ("window", -1, 40), ("window", 200, -1)]


@pytest.mark.parametrize("case", CASES)
def test_sort_key_matches_the_mask(driver, case):
    mask, wl, wr = case
    rng = np.random.default_rng(17 + wl + 3 * wr)
    n = 700
    lq = rng.integers(0, 600, size=n)
    lk = rng.integers(0, 600, size=n)
    lq[:5], lk[:5] = [0, 1, 64, 65, 300], [5, 0, 64, 700, 1]  # empty, single, tile edges
    lq[-4:], lk[-4:] = lq[10], lk[10]  # ties: equal lengths sort by index
    wl_, wr_ = (-1, 0) if mask == "causal" else (wl, wr)
    text = f"{wl_} {wr_} {n}\n" + "".join(f"{a} {b}\n" for a, b in zip(lq, lk))
    r = subprocess.run([driver], input=text, capture_output=True, text=True, check=True)
    out = [int(x) for x in r.stdout.split()]
    cost = [_blocks(int(a), int(b), mask, wl, wr) for a, b in zip(lq, lk)]
    assert out[:n] == cost
    want = sorted(range(n), key=lambda i: (-cost[i], -(int(lq[i]) + int(lk[i])), i))
    assert out[n:] == want


def test_sort_key_extremes(driver):
    # index 4095 survives beside the largest lengths; lengths past 2^20 keep the cost order
    n = 4096
    lens = [(1 << 20, 1 << 20)] + [(3, 3)] * (n - 2) + [(2000000, 64)]
    text = f"-1 -1 {n}\n" + "".join(f"{a} {b}\n" for a, b in lens)
    r = subprocess.run([driver], input=text, capture_output=True, text=True, check=True)
    out = [int(x) for x in r.stdout.split()]
    assert out[0] == (1 << 14) * (1 << 14) and out[n - 1] == 31250
    assert out[n:n + 3] == [0, n - 1, 1] and sorted(out[n:]) == list(range(n))
