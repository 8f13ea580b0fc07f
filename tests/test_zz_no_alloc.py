"""GPU check of the allocation-free chain entry point (bl_ffn_chain_noalloc)
through the C ABI: two calls in a row, the second with fewer rows, each
bit-identical to bl_ffn_chain with a caller workspace; sizes beyond the fixed
scratch are rejected before anything is enqueued."""
import numpy as np
import pytest
import torch

import oracle
from bit_ternary_weight_amd import synth
from gpu_helpers import bf16_dev, dev, guarded, host, requires_gpu, to_dev

pytestmark = [pytest.mark.gpu, requires_gpu]


def _weights(seed, H, I):
    pg, wg, _ = oracle.ternarize_pack(synth.master_weight(seed, I, H))
    pu, wu, _ = oracle.ternarize_pack(synth.master_weight(seed + 1, I, H))
    pd, wd, _ = oracle.ternarize_pack(synth.master_weight(seed + 2, H, I))
    return (to_dev(np.concatenate([pg, pu])), to_dev(np.array([wg, wu], np.float32)), to_dev(pd),
            to_dev(np.array([wd], np.float32)))


def test_noalloc_chain_matches_the_workspace_chain_twice():
    from bit_ternary_weight_amd import binding as bl
    H, I = 2560, 6912
    pgu, wgu, pd, wd = _weights(400, H, I)
    for M, ydt in ((300, torch.float32), (4, torch.bfloat16)):     # prefill path, then a smaller decode call
        h = bf16_dev(synth.act_outliers_bf16(410 + M, M, H))
        ref = bl.ffn_chain(h, pgu, wgu, pd, wd, y_dtype=ydt)
        out = guarded((M, H), ydt)
        bl.ffn_chain_noalloc(h, pgu, wgu, pd, wd, out.t)
        torch.cuda.synchronize()
        out.check("noalloc y")
        assert torch.equal(out.t.view(torch.int16) if ydt == torch.bfloat16 else out.t,
                           ref.view(torch.int16) if ydt == torch.bfloat16 else ref), M


def test_noalloc_chain_rejects_sizes_beyond_its_scratch():
    from bit_ternary_weight_amd import binding as bl
    H, I = 2560, 6912
    limit = bl.raw.bl_ffn_chain_noalloc_max_bytes()
    assert limit == 32 << 20
    M = 1000                                        # 1000 rows need about 37 MB at this shape
    assert bl.raw.bl_ffn_chain_workspace_bytes(M, H, I) > limit
    pgu, wgu, pd, wd = _weights(420, H, I)
    h = torch.zeros((M, H), dtype=torch.float32, device=dev())
    y = torch.empty((M, H), dtype=torch.float32, device=dev())
    with pytest.raises(bl.BitLinearError) as e:
        bl.ffn_chain_noalloc(h, pgu, wgu, pd, wd, y)
    assert e.value.status == bl.BL_ERR_WORKSPACE
    assert bl.raw.bl_ffn_chain_workspace_bytes(903, H, I) <= limit < bl.raw.bl_ffn_chain_workspace_bytes(904, H, I)
