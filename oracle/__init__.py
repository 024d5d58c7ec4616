"""CPU oracle for the QLoRA NF4 linear layer.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, obviously correct
definition that the HIP library is checked against. Only the test suite, the
smoke check and the CPU-baseline leg of the benchmark may import it; the
product path never does. It shares no code, tables or constants with the HIP
library under ``bit_quantized_finetuning_quantize_amd/``.

Sources (the pages are cited by address, title and section):

* [P1] ai360xpert.com/papers/qlora, "QLoRA"
* [P2] crackai.dev/papers/qlora, "QLoRA: Efficient Finetuning of Quantized LLMs"
* [P3] narrativegoldmine.com/notes/pages/QLoRA, "QLoRA"
* [P4] ozercemkelahmet.com/tools/qlora, "QLoRA"
* [P5] fanfani.net/articles/qlora, "QLoRA"

Pinning status of each function is stated in its module docstring.
"""

from .nf4 import (  # noqa: F401
    BLOCK,
    GROUP,
    P_MAX,
    codebook,
    codebook_fp64,
    level8,
    nearest_level,
    quantize,
    dequantize,
    dequantize_nodq,
    unpack_codes,
    pack_codes,
    num_blocks,
    num_groups,
    codes_bytes,
    store_bytes,
    bits_per_param,
)
from .bf16 import bf16_round, bf16_bits_to_f32, f32_to_bf16_bits  # noqa: F401
from .linear import linear_fwd, linear_bwd  # noqa: F401
from .merge import merge  # noqa: F401
from .adamw import adamw_step  # noqa: F401
from .philox import philox4x32_10  # noqa: F401
from .dropout import (  # noqa: F401
    dropout_keep,
    keep_scale,
    keep_threshold,
    pack_keep,
    unpack_keep,
)
from . import fp8  # noqa: F401
from . import fp4  # noqa: F401
from . import store  # noqa: F401
from .adamw8 import BLOCK8, adamw8_step, dequantize_state, num_blocks8, quantize_state  # noqa: F401
