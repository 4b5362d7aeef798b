"""CPU oracle for the routed MoE layer forward over block-quantised experts.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library.

It is written for obviousness, not speed: NumPy in float64, exact decoding of
every code, a literal per-token loop over the selected experts, and a grouped
mode that performs the same arithmetic with one matmul per expert.

Sources.  The FreeToken README ("Broad MoE & Ecosystem Support") names the
weight formats MXFP4, NVFP4, FP8 and BF16 and describes a Mixture-of-Experts
serving engine, but never writes the layer's arithmetic down.  The readings
used here (router GEMM, softmax over the k selected logits, SwiGLU experts,
weighted combine, sigmoid-gated shared expert, per-tensor E4M3 activations)
are the standard routed-MoE layer, and the MXFP8 activation mode follows
the OCP Microscaling v1.0 conversion rule; each is listed with its justification in
the design notes.  Code tables follow the public OCP Microscaling v1.0 (E2M1,
E8M0), OCP OFP8 (E4M3FN) and NVIDIA NVFP4 definitions.

Pinning.  Every function here is checked by ``tests/test_oracle_*.py`` against
something other than itself: exhaustive code tables versus the bit-field
definitions and torch's independent float8 dtypes, closed forms (E=1, k=1 is
a dense SwiGLU MLP; k=E is the full softmax), invariants (token permutation,
weights summing to one, counts summing to T*k) and brute force over all
experts on tiny shapes.
"""
from .codecs import (  # noqa: F401
    E2M1_VALUES,
    e2m1_decode,
    e8m0_decode,
    e4m3_decode,
    e4m3_encode_nearest,
    dequant_mxfp4,
    dequant_nvfp4,
    dequant_fp8,
    dequant_bf16,
    dequant,
)
from .moe import (  # noqa: F401
    bf16_to_f64,
    router_logits,
    selection_scores,
    route,
    select_topk,
    topk_softmax,
    shared_gate,
    align,
    align_max_padded,
    quant_act_per_tensor,
    quant_act_mxfp8,
    swiglu_expert,
    forward,
    forward_grouped,
    forward_tokens,
    dense_swiglu,
    forward_all_experts_masked,
)
