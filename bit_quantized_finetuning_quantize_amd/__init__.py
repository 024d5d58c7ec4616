"""MI355X (gfx950) NF4 linear layer with a LoRA adapter: a C-ABI HIP library
(libqlora.so, header include/qlora.h) and a thin Python binding."""

from .api import (  # noqa: F401
    BLOCK,
    GROUP,
    STORE_DQ_FP8,
    STORE_FP4,
    STORE_NF4,
    Nf4Store,
    QloraError,
    adamw8_state,
    adamw_state,
    empty_store,
    qlora_adamw8_step,
    qlora_adamw_step,
    qlora_dropout_mask,
    qlora_linear_bwd,
    qlora_linear_bwd_dropout,
    qlora_linear_fwd,
    qlora_linear_fwd_dropout,
    qlora_linear_fwd_noalloc,
    qlora_linear_workspace_bytes,
    qlora_nf4_codebook,
    qlora_nf4_codes_bytes,
    qlora_nf4_dequantize,
    qlora_nf4_dequantize_bf16,
    qlora_nf4_merge,
    qlora_nf4_num_blocks,
    qlora_nf4_num_groups,
    qlora_nf4_quantize,
    workspace,
)
from ._lib import LIB_PATH  # noqa: F401
