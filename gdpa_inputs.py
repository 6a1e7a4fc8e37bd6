"""Seeded synthetic inputs for GDPA workloads.

This module is shared by the CPU oracle tests, the GPU parity tests and the
benchmark.  It holds no attention arithmetic: it draws sequence lengths and
N(0,1) tensors from a seeded PCG64 generator and encodes them into the storage
formats the kernels consume (bf16 bit patterns, OCP FP8 E4M3 codes with a
per-tensor fp32 scale).  Decoding those formats back to numbers is done by each
consumer on its own.

Workload families follow the GDPA README (page "gdpa/README.md",
"Benchmark Results"): self-attention at sparsity (mean fill) 1.0 and 0.5 and
cross-attention with a short KV sequence, and its "Features" list (jagged
sequences, MHA/GQA, causal/sliding-window masks, FP8 E4M3 forward).
The production traffic the README measures on is not public; these seeded
draws stand in for it.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# activation names (strings) in the order of the C enum gdpa_act_t
ACTIVATIONS = (
    "identity", "gelu", "gelu_tanh", "fast_gelu", "fast_gelu_bf16",
    "relu", "relu2", "leaky_relu", "silu", "fast_silu", "hardswish",
)
MASKS = ("none", "causal", "window")


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and structure of one GDPA problem."""
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    head_dim: int            # of Q and K
    lq_range: tuple          # (lo, hi) inclusive; lo == hi means fixed length
    lk_range: Optional[tuple]  # None: KV lengths equal Q lengths (self-attention)
    act: str
    act_param: float = 0.01
    mask: str = "none"       # "none" | "causal" | "window"
    window_left: int = -1    # -1 = unbounded
    window_right: int = -1
    fp8_qk: bool = False
    mx_qk: bool = False               # Q and K in MXFP8 (E4M3 elements, E8M0 scale per 32 head dims)
    mx4_qk: bool = False              # Q and K in MXFP4 (E2M1 element pairs per byte, E8M0 scale per 32)
    fp16: bool = False       # fp16 Q/K/V/dO instead of bf16
    head_dim_v: Optional[int] = None  # of V and O (None: head_dim)
    backward: bool = False
    varlen: bool = True      # False: fixed-length [B, L, H, D] API
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))


# The five reference workloads (tiny parity case, jagged self-attention at
# fill ~0.5, full-length self-attention fwd+bwd, short-KV cross-attention
# fwd+bwd, causal sliding-window GQA with FP8 Q/K).
WORKLOADS = {
    "tiny": Workload("tiny", 2, 2, 2, 64, (128, 128), None, "gelu_tanh",
                     varlen=False, seed=1),
    "jagged_self": Workload("jagged_self", 64, 4, 4, 128, (1, 1024), None,
                            "fast_gelu", backward=True, seed=2),
    "full_self": Workload("full_self", 32, 8, 8, 128, (2048, 2048), None,
                          "silu", backward=True, varlen=False, seed=3),
    "short_kv_cross": Workload("short_kv_cross", 512, 4, 4, 128, (256, 2048),
                               (64, 64), "relu2", backward=True, seed=4),
    "jagged_self_fp16": Workload("jagged_self_fp16", 64, 4, 4, 128, (1, 1024), None,
                                 "fast_gelu", fp16=True, backward=True, seed=2),
    "jagged_self_d96": Workload("jagged_self_d96", 64, 4, 4, 96, (1, 1024), None,
                                "fast_gelu", backward=True, seed=2),
    "jagged_self_d192": Workload("jagged_self_d192", 64, 4, 4, 192, (1, 1024), None,
                                 "fast_gelu", head_dim_v=128, backward=True, seed=2),
    "window_gqa_fp8": Workload("window_gqa_fp8", 16, 16, 4, 64, (1024, 4096),
                               None, "leaky_relu", act_param=0.01,
                               mask="window", window_left=511, window_right=0,
                               fp8_qk=True, seed=5),
    # the same shape with the 8- and 4-bit Q/K formats forward and backward
    # (the README lists MXFP8 and MXFP4 forward and backward as coming; the
    # backward from FP8 Q/K is read the same way)
    "window_gqa_fp8_bwd": Workload("window_gqa_fp8_bwd", 16, 16, 4, 64, (1024, 4096),
                                   None, "leaky_relu", act_param=0.01,
                                   mask="window", window_left=511, window_right=0,
                                   fp8_qk=True, backward=True, seed=5),
    "window_gqa_mxfp8": Workload("window_gqa_mxfp8", 16, 16, 4, 64, (1024, 4096),
                                 None, "leaky_relu", act_param=0.01,
                                 mask="window", window_left=511, window_right=0,
                                 mx_qk=True, backward=True, seed=5),
    "window_gqa_mxfp4": Workload("window_gqa_mxfp4", 16, 16, 4, 64, (1024, 4096),
                                 None, "leaky_relu", act_param=0.01,
                                 mask="window", window_left=511, window_right=0,
                                 mx4_qk=True, backward=True, seed=5),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest even) and return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16 encoding expects finite values")
    u = x.view(np.uint32)
    r = (u >> 16) & 1          # finite patterns are <= 0xff7fffff, so the sum below cannot wrap
    r += u
    r += 0x7FFF
    r >>= 16
    return r.astype(np.uint16)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE binary16 (round to nearest even) and return uint16 bits."""
    return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def quantize_e4m3(x: np.ndarray):
    """Per-tensor OCP FP8 E4M3 quantisation: scale = max|x|/448, code = RNE(x/scale).

    Returns (uint8 codes, float32 scale).  Uses torch's float8_e4m3fn cast
    (round to nearest even); x/scale never exceeds 448 in magnitude by more
    than rounding, and 448 is the largest finite E4M3 value.
    """
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    scale = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
    y = torch.from_numpy(x / scale).clamp_(-448.0, 448.0)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, float(scale)


def quantize_mxfp8(x: np.ndarray, block: int = 32):
    """OCP MX quantisation to MXFP8 (E4M3 elements) along the last axis: for
    every block of 32 elements, shared exponent e = floor(log2(max|x|)) - 8
    (8 = the largest E4M3 exponent; 0 for an all-zero block), clamped to
    [-127, 127], scale code e + 127 (E8M0), element code = RNE(x / 2^e)
    saturated to +-448 (torch's float8_e4m3fn cast).

    Returns (uint8 codes of x's shape, uint8 scale codes [..., D / block])."""
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    blocks = x.reshape(*x.shape[:-1], x.shape[-1] // block, block)
    amax = np.max(np.abs(blocks), axis=-1)
    e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8, 0)
    e = np.clip(e, -127, 127).astype(np.int64)
    y = blocks / np.exp2(e.astype(np.float64))[..., None]
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32)).clamp_(-448.0, 448.0)
    codes = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(x.shape).copy()
    return codes, (e + 127).astype(np.uint8)


# E2M1 magnitudes by code (OCP MX specification, FP4 E2M1)
_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def quantize_mxfp4(x: np.ndarray, block: int = 32):
    """OCP MX quantisation to MXFP4 (E2M1 elements) along the last axis: for
    every block of 32 elements, shared exponent e = floor(log2(max|x|)) - 2
    (2 = the largest E2M1 exponent; 0 for an all-zero block), clamped to
    [-127, 127], scale code e + 127 (E8M0); element = the nearest E2M1 value
    of x / 2^e (ties to the even code), saturated to +-6.

    Returns (uint8 bytes [..., D / 2] holding element 2 i in the low nibble
    of byte i and element 2 i + 1 in the high nibble, uint8 scale codes
    [..., D / block])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    blocks = x.reshape(*x.shape[:-1], x.shape[-1] // block, block).astype(np.float64)
    amax = np.max(np.abs(blocks), axis=-1)
    e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, 0)
    e = np.clip(e, -127, 127).astype(np.int64)
    y = np.minimum(np.abs(blocks / np.exp2(e.astype(np.float64))[..., None]), 6.0)
    dist = np.abs(y[..., None] - _E2M1_GRID)
    best = dist.min(-1, keepdims=True)
    # among the nearest grid points take the even code (ties to even)
    cand = np.where(dist == best, np.arange(8), 99)
    even = np.where(cand % 2 == 0, cand, 99).min(-1)
    mag = np.where(even < 99, even, cand.min(-1)).astype(np.uint8)
    codes = (mag | np.where(blocks < 0, 8, 0).astype(np.uint8)).reshape(x.shape)
    codes[(codes & 0x7) == 0] = 0   # -0 stored as +0
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)


@dataclasses.dataclass
class Batch:
    """One drawn problem instance.  Tensors are storage-format numpy arrays."""
    wl: Workload
    seqlens_q: np.ndarray     # int64 [B]
    seqlens_k: np.ndarray     # int64 [B]
    cu_seqlens_q: np.ndarray  # int32 [B+1]
    cu_seqlens_k: np.ndarray  # int32 [B+1]
    q: np.ndarray             # uint16 bf16/fp16 bits, uint8 E4M3 codes [total_q, Hq, D], or MXFP4 bytes [.., D / 2]
    k: np.ndarray             # same format as q                             [total_k, Hkv, D]
    v: np.ndarray             # uint16 bf16/fp16 bits                        [total_k, Hkv, D]
    do: Optional[np.ndarray]  # uint16, same format as v                     [total_q, Hq, D]
    q_scale: float = 1.0      # per-tensor scale of q codes (fp8 only)
    k_scale: float = 1.0
    q_mx: Optional[np.ndarray] = None  # uint8 E8M0 block scales of q codes [total_q, Hq, D / 32] (MXFP8, MXFP4)
    k_mx: Optional[np.ndarray] = None  #                          of k codes [total_k, Hkv, D / 32]

    @property
    def max_seqlen_q(self) -> int:
        return int(self.seqlens_q.max()) if len(self.seqlens_q) else 0

    @property
    def max_seqlen_k(self) -> int:
        return int(self.seqlens_k.max()) if len(self.seqlens_k) else 0


def draw_lengths(rng, batch, rng_range):
    lo, hi = rng_range
    if lo == hi:
        return np.full(batch, lo, dtype=np.int64)
    return rng.integers(lo, hi + 1, size=batch).astype(np.int64)


def draw_seqlens(wl: Workload, seed: Optional[int] = None):
    """The (Q lengths, KV lengths) that make_batch draws for `wl`, without the
    tensors (same generator, same draw order)."""
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    lq = draw_lengths(rng, wl.batch, wl.lq_range)
    lk = lq.copy() if wl.lk_range is None else draw_lengths(rng, wl.batch, wl.lk_range)
    return lq, lk


def make_batch(wl: Workload, seed: Optional[int] = None, with_do: Optional[bool] = None,
               seqlens_q=None, seqlens_k=None) -> Batch:
    """Draw one instance of `wl`.

    Draw order: Q lengths, KV lengths (if drawn), then Q, K, V, dO as float32
    N(0,1).  Q/K are quantised to E4M3 for FP8 workloads, everything else is
    rounded to bf16 (fp16 for fp16 workloads).  Explicit `seqlens_q`/`seqlens_k` override the draws.
    """
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    lq = draw_lengths(rng, wl.batch, wl.lq_range) if seqlens_q is None else np.asarray(seqlens_q, np.int64)
    if seqlens_k is not None:
        lk = np.asarray(seqlens_k, np.int64)
    elif wl.lk_range is None:
        lk = lq.copy()
    else:
        lk = draw_lengths(rng, wl.batch, wl.lk_range)
    B = len(lq)
    cu_q = np.zeros(B + 1, np.int32)
    cu_k = np.zeros(B + 1, np.int32)
    cu_q[1:] = np.cumsum(lq)
    cu_k[1:] = np.cumsum(lk)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    H, G, D = wl.heads_q, wl.heads_kv, wl.head_dim
    DV = wl.head_dim_v or D
    qf = rng.standard_normal((tq, H, D), dtype=np.float32)
    kf = rng.standard_normal((tk, G, D), dtype=np.float32)
    vf = rng.standard_normal((tk, G, DV), dtype=np.float32)
    want_do = wl.backward if with_do is None else with_do
    dof = rng.standard_normal((tq, H, DV), dtype=np.float32) if want_do else None
    qs = ks = 1.0
    qmx = kmx = None
    enc = f32_to_f16_bits if wl.fp16 else f32_to_bf16_bits
    if wl.mx4_qk:
        q, qmx = quantize_mxfp4(qf)
        k, kmx = quantize_mxfp4(kf)
    elif wl.mx_qk:
        q, qmx = quantize_mxfp8(qf)
        k, kmx = quantize_mxfp8(kf)
    elif wl.fp8_qk:
        q, qs = quantize_e4m3(qf)
        k, ks = quantize_e4m3(kf)
    else:
        q, k = enc(qf), enc(kf)
    v = enc(vf)
    do = enc(dof) if dof is not None else None
    return Batch(wl, lq, lk, cu_q, cu_k, q, k, v, do, qs, ks, qmx, kmx)


def small_variant(wl: Workload, batch: int, lq_range, lk_range=None, **kw) -> Workload:
    """Same activation/mask/heads/dtype as `wl` at a size the oracle finishes quickly."""
    return dataclasses.replace(wl, batch=batch, lq_range=lq_range,
                               lk_range=lk_range if lk_range is not None else wl.lk_range,
                               **kw)
