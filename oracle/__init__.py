"""Plain fp64 CPU oracle for Generalized Dot Product Attention (GDPA).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only the test suite, the smoke check and the benchmark's CPU-baseline leg do.
It shares no code with the HIP library; both read only the seeded inputs
module (`gdpa_inputs`).

What it computes follows the GDPA README (page "gdpa/README.md" of
facebookresearch/ads_model_kernel_library, intro paragraph): dot-product
attention whose softmax is replaced by a pointwise activation.  With no
softmax there is no row normaliser, so the result is the plain definition

    S = scale * Q K^T,   P = M * act(S),   O = P V

per sequence and query head, and its gradients.  Masks, head layouts, jagged
sequences and the activation list come from the README's "Features" section;
scale/cu_seqlens/max_seqlen conventions from its "CUTE-DSL" usage example.

Every function is pinned by tests under tests/ (test_oracle_*.py) against
closed forms, library routines, brute force and finite differences.
"""
from .activations import act, act_grad, ACT_NAMES
from .formats import (decode_bf16, decode_e2m1, decode_e4m3, decode_e8m0, decode_f16, decode_mxfp4,
                      decode_mxfp8, unpack_fp4)
from .gdpa import (
    allowed_mask,
    gdpa_forward,
    gdpa_backward,
    gdpa_forward_rows,
    gdpa_backward_q_rows,
    gdpa_backward_k_rows,
)

__all__ = [
    "act", "act_grad", "ACT_NAMES", "decode_bf16", "decode_e4m3", "decode_e8m0", "decode_f16", "decode_mxfp8",
    "allowed_mask",
    "gdpa_forward", "gdpa_backward", "gdpa_forward_rows", "gdpa_backward_q_rows",
    "gdpa_backward_k_rows",
]
