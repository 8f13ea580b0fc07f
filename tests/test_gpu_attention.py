"""GPU parity of the decode-step attention (bl_attn_decode) against the oracle.

The oracle rotates and attends in fp64; the kernels work in fp32 (RoPE from
the fp32 table, fp32 scores, exponentials and sums).  Acceptance, derived
from fp32 rounding over a 128-term dot product and a softmax over at most
2048 positions: max |out - ref| <= 1e-4 * max(1, max |ref|) per call; the
cached value at pos is bit-exact (a copy) and the cached key within 1e-6 of
the fp64 rotation (relative to its row's maximum).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import dev, host, requires_gpu, to_dev

pytestmark = [pytest.mark.gpu, requires_gpu]

ATTN_TOL = 1e-4


def _bl():
    from bit_ternary_weight_amd import binding
    return binding


def _inputs(seed, H, KVH, S, D=128):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(H * D).astype(np.float32)
    kn = rng.standard_normal(KVH * D).astype(np.float32)
    vn = rng.standard_normal(KVH * D).astype(np.float32)
    kc = rng.standard_normal((KVH, S, D)).astype(np.float32)
    vc = rng.standard_normal((KVH, S, D)).astype(np.float32)
    return q, kn, vn, kc, vc


def _run(q, kn, vn, pos, kc, vc, base, H, KVH):
    bl = _bl()
    S = kc.shape[1]
    rc, rs = bl.rope_table(S, 128, base, device=dev())
    kcd, vcd = to_dev(kc), to_dev(vc)
    out = bl.attn_decode(to_dev(q), to_dev(kn), to_dev(vn), pos, kcd, vcd, rc, rs, H, KVH)
    torch.cuda.synchronize()
    return host(out).reshape(H, 128), host(kcd), host(vcd)


def _check(seed, H, KVH, S, positions, base=500000.0):
    q, kn, vn, kc, vc = _inputs(seed, H, KVH, S)
    for pos in positions:
        out, kcg, vcg = _run(q, kn, vn, pos, kc, vc, base, H, KVH)
        ref = oracle.attn_decode(q, kn, vn, pos, kc, vc, base, H, KVH)
        err = np.abs(out - ref).max()
        assert err <= ATTN_TOL * max(1.0, np.abs(ref).max()), (pos, err)
        # the token's value copied and its rotated key written at pos; the rest untouched
        assert np.array_equal(vcg[:, pos], vn.reshape(KVH, 128))
        kr = oracle.rope(kn.reshape(KVH, 128), pos, base)
        assert np.abs(kcg[:, pos] - kr).max() <= 1e-6 * max(1.0, np.abs(kr).max())
        mask = np.ones(S, bool)
        mask[pos] = False
        assert np.array_equal(kcg[:, mask], kc[:, mask]) and np.array_equal(vcg[:, mask], vc[:, mask])


@pytest.mark.parametrize("H,KVH", [(4, 1), (4, 4), (6, 3), (8, 2)])
def test_attn_decode_small(H, KVH):
    # chunk edges (64 positions), a single position, the last one
    _check(11, H, KVH, 200, [0, 1, 63, 64, 65, 127, 128, 199])


def test_attn_decode_model_shape():
    # 20 query heads, 5 key/value heads, 128 dimensions, 2048 positions
    _check(12, 20, 5, 2048, [0, 700, 2047], base=500000.0)


def test_attn_decode_many_chunks():
    # 79 and 512 chunks of 64 positions: merges over several batches, and the
    # longest cache the kernel serves
    _check(15, 8, 2, 5000, [4999, 4160])
    _check(16, 4, 1, 32768, [32767])


def test_attn_decode_other_base_and_peaked_scores():
    H, KVH, S, pos = 20, 5, 300, 257
    q, kn, vn, kc, vc = _inputs(13, H, KVH, S)
    # one cached key per group nearly parallel to the group's rotated queries:
    # a sharply peaked softmax
    qr = oracle.rope(q.reshape(H, 128), pos, 10000.0)
    for g in range(KVH):
        kc[g, 42] = (6.0 * qr[4 * g] / np.linalg.norm(qr[4 * g]) * np.sqrt(128)).astype(np.float32)
    out, _, _ = _run(q, kn, vn, pos, kc, vc, 10000.0, H, KVH)
    ref = oracle.attn_decode(q, kn, vn, pos, kc, vc, 10000.0, H, KVH)
    assert np.abs(out - ref).max() <= ATTN_TOL * max(1.0, np.abs(ref).max())


def test_attn_decode_sequence_from_empty_cache():
    """Decode 70 tokens from an empty cache; the oracle keeps its own cache
    (its fp64 rotations rounded to fp32), so no GPU value feeds it."""
    bl = _bl()
    H, KVH, S, base = 8, 2, 96, 500000.0
    rng = np.random.default_rng(14)
    rc, rs = bl.rope_table(S, 128, base, device=dev())
    kcd = torch.zeros((KVH, S, 128), dtype=torch.float32, device=dev())
    vcd = torch.zeros_like(kcd)
    kc_ref = np.zeros((KVH, S, 128), np.float32)
    vc_ref = np.zeros((KVH, S, 128), np.float32)
    for pos in range(70):
        q = rng.standard_normal(H * 128).astype(np.float32)
        kn = rng.standard_normal(KVH * 128).astype(np.float32)
        vn = rng.standard_normal(KVH * 128).astype(np.float32)
        out = host(bl.attn_decode(to_dev(q), to_dev(kn), to_dev(vn), pos, kcd, vcd, rc, rs, H, KVH)).reshape(H, 128)
        ref = oracle.attn_decode(q, kn, vn, pos, kc_ref, vc_ref, base, H, KVH)
        assert np.abs(out - ref).max() <= ATTN_TOL * max(1.0, np.abs(ref).max()), pos
        kc_ref[:, pos] = oracle.rope(kn.reshape(KVH, 128), pos, base).astype(np.float32)
        vc_ref[:, pos] = vn.reshape(KVH, 128)
