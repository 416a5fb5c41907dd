"""MI355X-native GPTQ (and AWQ) post-training quantization of linear layers
(hand-written HIP for gfx950).

The C ABI (include/gptq.h, libgptq.so) holds every step; this package is the
thin ctypes binding (names as in the C ABI) plus drivers that allocate outputs
and chain the calls: one layer with GPTQ or AWQ, and one decoder block layer
by layer.
"""
from ._lib import (  # noqa: F401
    EXPORTED, GPTQError, LIB_PATH, NotPositiveDefinite, gptq_abi_version, gptq_config,
    gptq_hessian_accumulate, gptq_hessian_accumulate_noalloc, gptq_hessian_noalloc_scratch_bytes,
    gptq_hessian_workspace_size, gptq_layer_error,
    gptq_layer_error_workspace_size, gptq_pack_dense, gptq_pack_int4, gptq_prepare_hinv,
    gptq_w4a16_gemm, AWQ_DEFAULT_GRID, gptq_awq_act_sumsq, gptq_awq_quantize, gptq_awq_search,
    gptq_awq_search_workspace_size, gptq_awq_sumsq_workspace_size, gptq_block_attention,
    gptq_block_attention_workspace_size, gptq_linear, gptq_linear_workspace_size, gptq_rmsnorm,
    gptq_swiglu,
    gptq_prepare_hinv_workspace_size, gptq_quantize_layer, gptq_quantize_workspace_size,
    gptq_status_string, lib, make_config,
)
from .layer import AWQLayerResult, GPTQLayerResult, awq_quantize_layer, quantize_layer_outputs  # noqa: F401
from .block import BlockResult, BlockShape, quantize_block_sequential  # noqa: F401
