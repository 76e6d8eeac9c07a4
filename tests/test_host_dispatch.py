"""Host-side batch-size dispatch of the MoE layer (no GPU): the token block
size chosen for each workload's batch sizes, as measured on MI355X."""
from weight_only_quantized_topk_amd.layer import choose_block_size

import gen


def test_block_size_per_workload():
    want = {  # (config, M) -> block size
        (2, 1): 16, (2, 4): 16, (2, 8): 16, (2, 64): 16, (2, 1024): 128,
        (3, 1): 16, (3, 16): 16, (3, 256): 128, (3, 4096): 128,
        (5, 64): 16, (5, 4096): 128,
        (1, 16): 16,
    }
    for (cid, M), bs in want.items():
        spec = gen.CONFIGS[cid]
        assert choose_block_size(M, spec.topk, spec.E, spec.bits) == bs, (cid, M)


def test_block_size_regimes():
    # eight experts: small-batch up to 16 rows per expert, 64-row tiles up to
    # 32 (int8) / 48 (int4), 128 above
    assert choose_block_size(80, 2, 8, 8) == 64
    assert choose_block_size(128, 2, 8, 8) == 64
    assert choose_block_size(160, 2, 8, 8) == 128
    assert choose_block_size(192, 2, 8, 4) == 64
    # many experts (skewed routing): 64-row tiles from 6 mean rows per expert
    assert choose_block_size(128, 6, 160, 8) == 16
    assert choose_block_size(256, 6, 160, 8) == 64
    assert choose_block_size(1024, 6, 160, 8) == 64
    assert choose_block_size(2048, 6, 160, 8) == 128
    assert choose_block_size(0, 2, 8, 8) == 16
