"""CPU-only checks of the C-ABI library: it loads, exports every function
include/gdpa.h declares, and rejects invalid arguments before any HIP call."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdpa.h")
LIB = os.path.join(ROOT, "generalized_attention_amd", "libgdpa.so")

OK, INVALID, UNSUPPORTED, WS_SMALL, HIPERR = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        subprocess.run([sys.executable, os.path.join(ROOT, "generalized_attention_amd", "build.py")], check=True)
    import generalized_attention_amd as g
    return g.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(gdpa_\w+)\s*\(", text, re.M)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("gdpa_fwd", "gdpa_varlen_fwd", "gdpa_bwd", "gdpa_varlen_bwd"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (gdpa_\w+)$", out, re.M))
    assert set(declared_functions()) <= exported


def test_probe_library_is_separate_and_exports_its_probe(lib):
    # bench.py's peak probes live in their own library, outside the GDPA ABI
    probe = os.path.join(ROOT, "generalized_attention_amd", "libgdpa_probe.so")
    assert os.path.exists(probe)
    out = subprocess.run(["nm", "-D", "--defined-only", probe], capture_output=True, text=True, check=True).stdout
    assert re.search(r" T gdpa_probe_mfma$", out, re.M)
    main = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    assert "gdpa_probe_mfma" not in main


def test_abi_version_and_status_strings(lib):
    ver = int(re.search(r"#define GDPA_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert lib.gdpa_abi_version() == ver
    for code, name in [(0, b"GDPA_OK"), (1, b"GDPA_ERR_INVALID_ARG"), (2, b"GDPA_ERR_UNSUPPORTED"),
                       (3, b"GDPA_ERR_WORKSPACE_TOO_SMALL"), (4, b"GDPA_ERR_HIP"), (5, b"GDPA_ERR_DEVICE_WAIT"),
                       (99, b"GDPA_ERR_UNKNOWN")]:
        assert lib.gdpa_status_string(code) == name


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def fwd(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=2, Lq=128, Lk=128, Hq=4, Hkv=2, D=128, Dv=None, scale=0.1, mask=0,
             wl=-1, wr=-1, act=3, ap=0.01, qk=0, vd=0, od=3, qd=1.0, kd=1.0, ws=None, nws=0, stream=None)
    a.update(over)
    if a["Dv"] is None:
        a["Dv"] = a["D"]
    return lib.gdpa_fwd(*a.values())


def varlen_fwd(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, cq=FAKE, ck=FAKE, B=2, mq=128, mk=128, tq=200, tk=200, Hq=4, Hkv=4,
             D=64, Dv=None, scale=0.1, mask=0, wl=-1, wr=-1, act=3, ap=0.01, qk=0, vd=0, od=3, qd=1.0, kd=1.0, ws=None,
             nws=0, stream=None)
    a.update(over)
    if a["Dv"] is None:
        a["Dv"] = a["D"]
    return lib.gdpa_varlen_fwd(*a.values())


def varlen_fwd_mx(lib, name, **over):
    a = dict(q=FAKE, qs=FAKE, k=FAKE, ks=FAKE, v=FAKE, o=FAKE, cq=FAKE, ck=FAKE, B=2, mq=128, mk=128, tq=200, tk=200,
             Hq=4, Hkv=4, D=128, scale=0.1, mask=0, wl=-1, wr=-1, act=3, ap=0.01, od=3, ws=None, nws=0, stream=None)
    a.update(over)
    return getattr(lib, name)(*a.values())


def bwd(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=2, Lq=128, Lk=128, Hq=4, Hkv=2, D=128,
             Dv=None, scale=0.1, mask=0, wl=-1, wr=-1, act=8, ap=0.01, ind=0, gd=3, ws=None, nws=0, stream=None)
    a.update(over)
    if a["Dv"] is None:
        a["Dv"] = a["D"]
    return lib.gdpa_bwd(*a.values())


def varlen_bwd(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, cq=FAKE, ck=FAKE, B=2, mq=128, mk=128,
             tq=200, tk=200, Hq=4, Hkv=2, D=128, Dv=None, scale=0.1, mask=0, wl=-1, wr=-1, act=8, ap=0.01, ind=0, gd=3,
             ws=None, nws=0, stream=None)
    a.update(over)
    if a["Dv"] is None:
        a["Dv"] = a["D"]
    return lib.gdpa_varlen_bwd(*a.values())


@pytest.mark.parametrize("over,expect", [
    (dict(Hq=3, Hkv=2), INVALID),            # Hq % Hkv != 0
    (dict(Hkv=0), INVALID),
    (dict(D=192, Dv=192), UNSUPPORTED),      # built: (192, 128) only
    (dict(D=128, Dv=64), UNSUPPORTED),
    (dict(D=80), UNSUPPORTED),
    (dict(Dv=0), INVALID),
    (dict(D=192, Dv=128, B=0), OK),          # the README's (192, 128)
    (dict(D=0), INVALID),
    (dict(B=-1), INVALID),
    (dict(Lq=-5), INVALID),
    (dict(act=11), INVALID),
    (dict(act=-1), INVALID),
    (dict(mask=3), INVALID),
    (dict(mask=2, wl=-2), INVALID),
    (dict(qk=1), UNSUPPORTED),               # fp16 Q/K with bf16 V (P takes V's type)
    (dict(vd=1), UNSUPPORTED),               # bf16 Q/K with fp16 V
    (dict(qk=2, vd=1), UNSUPPORTED),         # FP8 Q/K with fp16 V
    (dict(qk=1, vd=1, B=0), OK),             # fp16 throughout
    (dict(od=1, B=0), OK),                   # fp16 output
    (dict(od=4), INVALID),
    (dict(vd=2), UNSUPPORTED),               # fp8 V
    (dict(od=2), INVALID),                   # fp8 output
    (dict(q=None), INVALID),
    (dict(o=None), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(qk=2, qd=float("inf")), INVALID),
    (dict(B=0), OK),                         # empty problem: no launch
    (dict(Lq=0), OK),
])
def test_fwd_validation(lib, over, expect):
    assert fwd(lib, **over) == expect


@pytest.mark.parametrize("over,expect", [
    (dict(cq=None), INVALID),
    (dict(tq=-1), INVALID),
    (dict(tq=2 ** 31, B=2 ** 24), UNSUPPORTED),   # rows past 32-bit token indices
    (dict(tq=257), INVALID),                  # more tokens than batch x max_seqlen_q
    (dict(tk=257), INVALID),
    (dict(B=0), OK),
    (dict(tq=0), OK),
    (dict(D=256), UNSUPPORTED),
])
def test_varlen_fwd_validation(lib, over, expect):
    assert varlen_fwd(lib, **over) == expect


@pytest.mark.parametrize("name", ["gdpa_varlen_fwd_mxfp8", "gdpa_varlen_fwd_mxfp4"])
@pytest.mark.parametrize("over,expect", [
    (dict(D=96), UNSUPPORTED),               # 32-wide blocks on the K = 64 MFMA: head dims 64 and 128
    (dict(D=192), UNSUPPORTED),
    (dict(qs=None), INVALID),                # the block scales are required
    (dict(ks=None), INVALID),
    (dict(B=0), OK),
    (dict(od=2), INVALID),
    (dict(tq=257), INVALID),
])
def test_mx_forward_validation(lib, name, over, expect):
    assert varlen_fwd_mx(lib, name, **over) == expect


def varlen_bwd_lowp(lib, **over):
    a = dict(q=FAKE, qs=None, k=FAKE, ks=None, v=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, cq=FAKE, ck=FAKE, B=2,
             mq=128, mk=128, tq=200, tk=200, Hq=4, Hkv=2, D=128, scale=0.1, mask=0, wl=-1, wr=-1, act=8, ap=0.01,
             qk=2, qd=1.0, kd=1.0, gd=3, ws=None, nws=0, stream=None)
    a.update(over)
    return lib.gdpa_varlen_bwd_lowp(*a.values())


@pytest.mark.parametrize("over,expect", [
    (dict(), WS_SMALL),                      # FP8 needs the workspace (decoded copies)
    (dict(qk=0), INVALID),                    # bf16 q/k take gdpa_varlen_bwd
    (dict(qk=3), INVALID),
    (dict(D=192), UNSUPPORTED),
    (dict(D=96, qk=4, qs=FAKE, ks=FAKE), UNSUPPORTED),   # MX: head dims 64 and 128
    (dict(qs=FAKE), INVALID),                 # FP8 has no block scales
    (dict(qk=4), INVALID),                    # MX without its block scales
    (dict(qk=5, qs=FAKE), INVALID),
    (dict(qd=float("nan")), INVALID),
    (dict(dk=None), INVALID),                 # dk and dv together
    (dict(gd=2), INVALID),
    (dict(cq=None), INVALID),
    (dict(B=0), OK),
    (dict(tq=0, tk=0), OK),
    (dict(tq=257), INVALID),
])
def test_lowp_backward_validation(lib, over, expect):
    assert varlen_bwd_lowp(lib, **over) == expect


def test_lowp_backward_workspace(lib):
    base = lib.gdpa_varlen_bwd_workspace_size(2, 128, 128, 200, 4, 2, 128, 3)
    need = lib.gdpa_varlen_bwd_lowp_workspace_size(2, 128, 128, 200, 150, 4, 2, 128, 2, 3)
    # the 16-bit backward's part, then bf16 Q (200 x 4 rows) and K (150 x 2 rows)
    assert need == (base + 255) // 256 * 256 + 200 * 4 * 128 * 2 + (150 * 2 * 128 * 2 + 255) // 256 * 256
    assert lib.gdpa_varlen_bwd_lowp(*[FAKE, None, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 128, 128,
                                      200, 150, 4, 2, 128, 0.1, 0, -1, -1, 8, 0.01, 2, 1.0, 1.0, 3, FAKE, need - 1,
                                      None]) == WS_SMALL
    assert lib.gdpa_varlen_bwd_lowp_workspace_size(2, 2 ** 30, 128, 2 ** 43, 150, 1024, 2, 128, 2, 3) == 2 ** 64 - 1


def test_mx_dtypes_need_their_entry_points(lib):
    # the MX dtypes through the plain entry point carry no scales
    assert varlen_fwd(lib, qk=4) == INVALID
    assert varlen_fwd(lib, qk=5) == INVALID
    assert varlen_fwd(lib, qk=6) == INVALID


@pytest.mark.parametrize("over,expect", [
    (dict(ind=2), UNSUPPORTED),              # FP8 is forward-only (README "Features")
    (dict(ind=1, B=0), OK),                  # fp16 inputs
    (dict(D=192, Dv=128, B=0), OK),          # the README's (192, 128)
    (dict(D=192, Dv=192), UNSUPPORTED),
    (dict(D=192, Dv=128, ind=2), UNSUPPORTED),   # FP8 is forward-only
    (dict(ind=3), INVALID),                  # fp32 inputs
    (dict(gd=1, B=0), OK),                   # fp16 gradients
    (dict(gd=2), INVALID),
    (dict(dk=None), INVALID),                # dk and dv must be requested together
    (dict(dq=None, dk=None, dv=None), INVALID),
    (dict(Hq=5), INVALID),
    (dict(B=0), OK),
])
def test_bwd_validation(lib, over, expect):
    assert bwd(lib, **over) == expect


@pytest.mark.parametrize("over,expect", [
    (dict(ck=None), INVALID),
    (dict(dv=None), INVALID),
    (dict(tq=0, tk=0), OK),
    (dict(act=42), INVALID),
])
def test_varlen_bwd_validation(lib, over, expect):
    assert varlen_bwd(lib, **over) == expect


def test_workspace_queries(lib):
    # forward: fixed-length calls need none; jagged calls of up to 4096
    # sequences hold the longest-first order (one int32 per sequence) and 8
    # work-queue counters, rounded up to 256 bytes
    assert lib.gdpa_fwd_workspace_size(64, 1024, 1024, 4, 4, 128) == 0
    f = lib.gdpa_varlen_fwd_workspace_size
    assert f(56, 1024, 1024, 4, 4, 128) == 256
    assert f(57, 1024, 1024, 4, 4, 128) == 512
    assert f(4096, 1024, 1024, 4, 4, 128) == 16640
    assert f(4097, 1024, 1024, 4, 4, 128) == 0
    assert f(0, 1024, 1024, 4, 4, 128) == 0


FP32, BF16, FP16 = 3, 0, 1


def test_backward_workspace_layout(lib):
    # fixed length: queue state (256 B) + one turn counter per (64-row query
    # tile, head): 64 sequences x 16 tiles x 4 heads x 4 B = 16 KiB
    fx = lib.gdpa_bwd_workspace_size
    assert fx(64, 1024, 1024, 4, 4, 128, FP32) == 256 + 16384
    assert fx(64, 1000, 1024, 4, 4, 128, FP32) == 256 + 16384       # 16 tiles of 64 rows
    # 16-bit dQ adds an fp32 accumulator of total_q x Hq x D values only when
    # the dK/dV pass reduces several key blocks' partial sums (forced with
    # GDPA_BWD_DQ=fused; by default several key blocks take the separate dQ
    # kernel, and one key block writes dQ directly)
    assert fx(64, 1024, 1024, 4, 4, 128, BF16) == 256 + 16384
    assert fx(0, 1024, 1024, 4, 4, 128, FP32) == 0
    # jagged: sequence order (batch int32) + queue state + (total_q / 64 +
    # batch + 1) tiles per head, each part rounded up to 256 bytes
    vb = lib.gdpa_varlen_bwd_workspace_size
    turns = (34868 // 64 + 64 + 1) * 4 * 4
    assert vb(64, 1024, 1024, 34868, 4, 4, 128, FP32) == 256 + 256 + (turns + 255) // 256 * 256
    assert vb(64, 1024, 1024, 34868, 4, 4, 128, BF16) == vb(64, 1024, 1024, 34868, 4, 4, 128, FP32)
    # beyond 4096 sequences no order is kept
    assert vb(5000, 8, 8, 5000, 1, 1, 64, FP32) == 256 + ((5000 // 64 + 5001) * 4 + 255) // 256 * 256
    for n in (vb(64, 1024, 1024, 34868, 4, 4, 128, FP32), fx(3, 77, 77, 2, 1, 96, FP32)):
        assert n % 256 == 0


def test_backward_accumulator_follows_the_dq_mode(lib, monkeypatch):
    fx, vb = lib.gdpa_bwd_workspace_size, lib.gdpa_varlen_bwd_workspace_size
    base = fx(64, 1024, 1024, 4, 4, 128, FP32)
    monkeypatch.setenv("GDPA_BWD_DQ", "fused")
    assert fx(64, 1024, 1024, 4, 4, 128, BF16) == base + 64 * 1024 * 4 * 128 * 4
    assert fx(64, 1024, 1024, 4, 4, 128, FP16) == fx(64, 1024, 1024, 4, 4, 128, BF16)
    assert fx(64, 1024, 1024, 4, 4, 128, FP32) == base
    assert fx(64, 1024, 128, 4, 4, 128, BF16) == base        # one key block: no partial sums to keep
    assert (vb(64, 1024, 1024, 34868, 4, 4, 128, BF16) - vb(64, 1024, 1024, 34868, 4, 4, 128, FP32)
            == (34868 * 4 * 128 * 4 + 255) // 256 * 256)
    monkeypatch.setenv("GDPA_BWD_DQ", "separate")
    assert fx(64, 1024, 1024, 4, 4, 128, BF16) == base


def test_backward_needs_its_workspace(lib):
    # every backward call with work to do needs the queried workspace
    assert bwd(lib) == WS_SMALL
    nws = lib.gdpa_bwd_workspace_size(2, 128, 128, 4, 2, 128, FP32)
    assert bwd(lib, ws=FAKE, nws=nws - 1) == WS_SMALL
    assert bwd(lib, B=0) == OK


def test_jagged_calls_check_the_workspace_before_launching(lib):
    # valid arguments, no workspace: refused on the host, nothing launched
    assert varlen_fwd(lib) == WS_SMALL
    assert varlen_fwd(lib, ws=FAKE, nws=255) == WS_SMALL
    assert varlen_bwd(lib) == WS_SMALL
    assert varlen_bwd(lib, ws=FAKE, nws=8) == WS_SMALL


def test_python_binding_names_match_c_names():
    import generalized_attention_amd as g
    for n in ("gdpa_fwd", "gdpa_varlen_fwd", "gdpa_bwd", "gdpa_varlen_bwd"):
        assert callable(getattr(g, n))
    assert set(g.EXPORTED) == set(declared_functions())


def test_binding_modules_do_not_import_the_oracle():
    pkg = os.path.join(ROOT, "generalized_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in re.sub(r"(#|//).*", "", text), f


@pytest.mark.parametrize("causal,window,expect", [
    (False, (-1, -1), ("none", -1, -1)),
    (True, (-1, -1), ("causal", -1, -1)),
    (True, (511, -1), ("window", 511, 0)),     # causal window of 512 keys
    (False, (3, 4), ("window", 3, 4)),
    (False, (-1, 40), ("window", -1, 40)),
])
def test_flash_attn_mask_arguments(causal, window, expect):
    # the README's call form (causal, window_size) -> the C ABI's mask arguments
    import generalized_attention_amd as g
    assert g._mask_args(causal, window) == expect


# ------------------------------------------------ binding-side argument checks
# The C entry points take raw pointers on trust; the binding checks dtypes,
# shapes, contiguity and devices first.  Every case below is invalid, so it
# must raise before any library call (the tensors live on the CPU).
def _cpu(shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


def _bwd_case(name):
    import torch
    B, L, H, D = 2, 16, 2, 64
    a = dict(q=_cpu((B, L, H, D)), k=_cpu((B, L, H, D)), v=_cpu((B, L, H, D)), dout=_cpu((B, L, H, D)),
             dq=_cpu((B, L, H, D), torch.float32), dk=_cpu((B, L, H, D), torch.float32),
             dv=_cpu((B, L, H, D), torch.float32))
    if name == "mixed_grad_dtypes":
        a["dk"] = _cpu((B, L, H, D), torch.bfloat16)
    elif name == "dq_wrong_shape":
        a["dq"] = _cpu((B, L, H, 2 * D), torch.float32)
    elif name == "dv_not_contiguous":
        a["dv"] = _cpu((B, L, H, 2 * D), torch.float32)[..., :D]
    elif name == "dout_other_dtype":
        a["dout"] = _cpu((B, L, H, D), torch.float16)
    elif name == "k_other_dtype":
        a["k"] = _cpu((B, L, H, D), torch.float16)
    elif name == "dk_without_dv":
        a["dv"] = None
    elif name == "int_grads":
        a["dq"] = a["dk"] = a["dv"] = _cpu((B, L, H, D), torch.int32)
    return a


@pytest.mark.parametrize("name,exc", [
    ("mixed_grad_dtypes", TypeError), ("dq_wrong_shape", ValueError), ("dv_not_contiguous", ValueError),
    ("dout_other_dtype", TypeError), ("k_other_dtype", TypeError), ("dk_without_dv", ValueError),
    ("int_grads", TypeError),
])
def test_binding_rejects_bad_backward_tensors(lib, name, exc):
    import generalized_attention_amd as g
    a = _bwd_case(name)
    with pytest.raises(exc):
        g.gdpa_bwd(a["q"], a["k"], a["v"], a["dout"], a["dq"], a["dk"], a["dv"], 0.125)


@pytest.mark.parametrize("name,exc", [
    ("o_wrong_shape", ValueError), ("o_not_contiguous", ValueError), ("o_int", TypeError),
    ("v_wrong_heads", ValueError), ("q_fp32", TypeError),
])
def test_binding_rejects_bad_forward_tensors(lib, name, exc):
    import torch
    import generalized_attention_amd as g
    B, L, H, D = 2, 16, 2, 64
    q, k, v = _cpu((B, L, H, D)), _cpu((B, L, H, D)), _cpu((B, L, H, D))
    o = _cpu((B, L, H, D), torch.float32)
    if name == "o_wrong_shape":
        o = _cpu((B, L + 1, H, D), torch.float32)
    elif name == "o_not_contiguous":
        o = _cpu((B, L, H, 2 * D), torch.float32)[..., ::2]
    elif name == "o_int":
        o = _cpu((B, L, H, D), torch.int32)
    elif name == "v_wrong_heads":
        v = _cpu((B, L, H + 1, D))
    elif name == "q_fp32":
        q = _cpu((B, L, H, D), torch.float32)
    with pytest.raises(exc):
        g.gdpa_fwd(q, k, v, o, 0.125)


def test_binding_rejects_bad_cu_seqlens(lib):
    import torch
    import generalized_attention_amd as g
    q, k, v = _cpu((10, 2, 64)), _cpu((10, 2, 64)), _cpu((10, 2, 64))
    o = _cpu((10, 2, 64), torch.float32)
    cu64 = torch.tensor([0, 4, 10], dtype=torch.int64)
    cu32 = torch.tensor([0, 4, 10], dtype=torch.int32)
    with pytest.raises(ValueError):
        g.gdpa_varlen_fwd(q, k, v, o, cu64, cu32, 6, 6, 0.125)
    with pytest.raises(ValueError):
        g.gdpa_varlen_fwd(q, k, v, o, cu32, cu32[:2], 6, 6, 0.125)
