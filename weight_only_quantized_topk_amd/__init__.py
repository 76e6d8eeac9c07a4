"""MI355X (gfx950) fused MoE layer with weight-only quantized experts
(W4A16 GPTQ-style with act-order, W8A16 per-column) and the 2:4-sparse W4A16
linear layer.  The compute lives in libwqmoe.so (hand-written HIP); this
package is its thin ctypes binding plus the layer composition."""
from ._lib import (WQ_BF16, WQ_ERR_DEVICE, WQ_ERR_HIP, WQ_ERR_INVALID, WQ_ERR_UNSUPPORTED, WQ_F16, WQ_OK,  # noqa
                   WQ_PACK_INTERLEAVE_GATE_UP, WQ_STAGE_DOWN, WQ_STAGE_GATE_UP, WQ_STAGE_RAW, WqError, load)
from .ops import *  # noqa: F401,F403
from .layer import (Fp8MoERunner, MoERunner, PackedFp8MoE, PackedMoE, choose_block_size, fused_moe,  # noqa: F401
                    fused_moe_fp8, pack_moe, pack_moe_fp8)
