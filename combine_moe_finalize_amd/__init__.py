"""MI355X (gfx950) deferred MoE finalize.

Python face of libmoe_finalize.so (C ABI in include/moe_finalize.h). The
entry points carry the C names; ``_binding`` holds the marshalling rules.
``workloads`` draws the seeded synthetic inputs; ``build`` compiles the
library in-tree.
"""
from ._binding import (  # noqa: F401
    DEVERR_INDEX_OUT_OF_RANGE,
    MoeFinalizeError,
    OP_FINALIZE,
    OP_QUANT_UE8M0,
    OP_RESIDUAL_RMSNORM,
    abi_version,
    load_library,
    moe_act_quant_fp8_amax,
    moe_act_quant_fp8_ue8m0,
    moe_allreduce_residual_rmsnorm,
    moe_finalize,
    moe_finalize_describe_launch,
    moe_finalize_ep_combine,
    moe_finalize_quant_ue8m0,
    moe_finalize_residual_rmsnorm,
    moe_topk_packed_decode,
    moe_topk_sigmoid_gate,
    status_string,
)
