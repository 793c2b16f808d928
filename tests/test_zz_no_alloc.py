"""attn_decode_paged_noalloc: paged decode with the library's own device
workspace, for callers that cannot allocate.

The GPU test calls it through the C ABI twice in a row, the second time with
a smaller input, and checks each result against attn_decode_paged on the
same input with a workspace of its own: the same kernels with the same split
count, so the outputs must be bit-identical (and therefore within the bf16
tolerances of the oracle parity tests).  The CPU test checks that a shape
needing more than the array holds is refused before the device is touched.
"""
import math
import sys

import numpy as np
import pytest

from attention_flash_fwd_amd import _lib

torch = pytest.importorskip("torch")

WORKSPACE = 6


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_noalloc_rejects_shapes_beyond_the_array():
    lib = _lib.load()
    fake = ctypes_ptr(0x10000)
    B, Hq, Hkv, D, mb = 64, 32, 8, 128, 2048
    assert lib.attn_decode_workspace_bytes(B, Hq, Hkv, D, mb, 16, 64) > _lib.STATIC_SCRATCH_BYTES
    st = lib.attn_decode_paged_noalloc(fake, fake, fake, fake, fake, fake, fake, B, Hq, Hkv, D, 100000,
                                       16, mb, 64, 0.1, ctypes_ptr(0))
    assert st == WORKSPACE
    # 31 splits still fit for this shape; 32 do not.
    assert lib.attn_decode_workspace_bytes(B, Hq, Hkv, D, mb, 16, 31) <= _lib.STATIC_SCRATCH_BYTES
    assert lib.attn_decode_workspace_bytes(B, Hq, Hkv, D, mb, 16, 32) > _lib.STATIC_SCRATCH_BYTES


def ctypes_ptr(x):
    import ctypes
    return ctypes.c_void_p(x)


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point_on_consecutive_calls(cuda):
    import attention_flash_fwd_amd as afa
    from attention_flash_fwd_amd import inputs
    _lib.load()
    cases = [
        # (context lengths, Hq, Hkv, D, splits): the second call is smaller
        (inputs.decode_context_lengths(16, 512, 32768, seed=61), 32, 8, 128, 16),
        ([1000, 37, 4097], 32, 8, 128, 0),
    ]
    for i, (ctx, Hq, Hkv, D, splits) in enumerate(cases):
        say(f"case noalloc call {i}: batch {len(ctx)} max ctx {max(ctx)} Hq{Hq} Hkv{Hkv} D{D} splits {splits}")
        inp = inputs.decode_inputs(ctx, Hq, Hkv, D, seed=60 + i, device="cuda", spare_blocks=3, table_pad=1)
        scale = 1 / math.sqrt(D)
        o_ref, l_ref = afa.decode_paged(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                                        num_splits=splits, scale=scale)
        o = torch.full_like(inp.q, float("nan"))
        lse = torch.full((len(ctx), Hq), float("nan"), dtype=torch.float32, device="cuda")
        o2, l2 = afa.decode_paged_noalloc(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                                          num_splits=splits, scale=scale, out=o, lse_out=lse)
        torch.cuda.synchronize()
        assert o2.data_ptr() == o.data_ptr() and l2.data_ptr() == lse.data_ptr()
        assert torch.isfinite(o).all() and torch.isfinite(lse).all()
        err = (o.float() - o_ref.float()).abs()
        say(f"  max |o - o_workspace| = {err.max().item():.3e}, "
            f"max |lse - lse_workspace| = {(lse - l_ref).abs().max().item():.3e}")
        assert err.max().item() <= 2e-2 and err.mean().item() <= 2e-3
        assert (lse - l_ref).abs().max().item() <= 1e-4
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), "not bit-identical to attn_decode_paged"
        del inp
        torch.cuda.empty_cache()
