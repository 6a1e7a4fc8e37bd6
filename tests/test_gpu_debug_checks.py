"""GDPA_DEBUG_CHECKS=1: jagged calls validate cu_seqlens on the host and refuse
bad device data before queuing any kernel.  Every bad case here would also stay
inside the tensors if it reached the kernels (no decreasing entries)."""
import pytest
import torch

pytestmark = pytest.mark.gpu

H, D, TOTAL = 2, 64, 100
INVALID_ARG = 1  # GDPA_ERR_INVALID_ARG in include/gdpa.h


@pytest.fixture(scope="module")
def g():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import generalized_attention_amd
    return generalized_attention_amd


def _inputs():
    gen = torch.Generator(device="cuda").manual_seed(3)
    q, k, v, do = (torch.randn((TOTAL, H, D), generator=gen, device="cuda").to(torch.bfloat16) for _ in range(4))
    return q, k, v, do


def _cu(vals):
    return torch.tensor(vals, dtype=torch.int32, device="cuda")


def _fwd(g, q, k, v, cu, max_len):
    o = torch.empty((TOTAL, H, D), device="cuda")
    g.gdpa_varlen_fwd(q, k, v, o, cu, cu, max_len, max_len, D ** -0.5, act="silu")
    return o


def _bwd(g, q, k, v, do, cu, max_len):
    dq, dk, dv = (torch.empty((TOTAL, H, D), device="cuda") for _ in range(3))
    g.gdpa_varlen_bwd(q, k, v, do, dq, dk, dv, cu, cu, max_len, max_len, D ** -0.5, act="silu")
    return dq, dk, dv


def test_valid_batch_passes_and_matches_unchecked(g, monkeypatch):
    q, k, v, do = _inputs()
    cu = _cu([0, 37, 37, 100])
    ref_o, ref_g = _fwd(g, q, k, v, cu, 63), _bwd(g, q, k, v, do, cu, 63)
    monkeypatch.setenv("GDPA_DEBUG_CHECKS", "1")
    o, grads = _fwd(g, q, k, v, cu, 63), _bwd(g, q, k, v, do, cu, 63)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o)
    for a, b in zip(grads, ref_g):
        assert torch.equal(a, b)


@pytest.mark.parametrize("vals,max_len,why", [
    ([0, 50, 90], 64, "cu[B] != total"),
    ([10, 60, 100], 64, "cu[0] != 0"),
    ([0, 30, 100], 64, "a length above max_seqlen"),
])
def test_bad_cu_seqlens_are_refused(g, monkeypatch, vals, max_len, why):
    q, k, v, do = _inputs()
    monkeypatch.setenv("GDPA_DEBUG_CHECKS", "1")
    cu = _cu(vals)
    with pytest.raises(g.GDPAError) as e:
        _fwd(g, q, k, v, cu, max_len)
    assert e.value.status == INVALID_ARG, why
    with pytest.raises(g.GDPAError) as e:
        _bwd(g, q, k, v, do, cu, max_len)
    assert e.value.status == INVALID_ARG, why
