"""Parity of the HIP path with the fp64 oracle on seeded random shapes.

The hand-picked cases of test_parity_gpu.py cover the edges one at a time;
these draw batch, lengths (ragged and unaligned), head layout, head_dim,
causality and split counts from a seeded generator, so that combinations
nobody picked are exercised too.  Same tolerances as the other parity tests
(bf16 output max-abs 2e-2, mean-abs 2e-3; lse max-abs 1e-4).  Sizes are
capped so that the oracle finishes each case in well under a second.
"""
import math
import sys

import numpy as np
import pytest

import oracle
from tests.helpers import BF16_LSE_ABS, BF16_MAX_ABS, BF16_MEAN_ABS, check_lse, check_o, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MAX_PAIRS = 20_000_000      # (query row, key, query head) triples per case


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def afa(cuda):
    import attention_flash_fwd_amd as afa_mod
    from attention_flash_fwd_amd import _lib
    _lib.load()
    return afa_mod


def heads(rng, max_hq=32):
    # Group sizes that are odd, even but not a multiple of 4, and multiples
    # of 4 (the prefill kernel takes 1, 2 or 4 query heads per work item).
    while True:
        hkv = int(rng.choice([1, 2, 3, 4, 8]))
        g = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16]))
        if hkv * g <= max_hq:
            return hkv * g, hkv


def oracle_paged(inp, q, causal, scale):
    qn = to_np(q)
    os_, ls_ = [], []
    for b in range(len(inp.ctx)):
        kb, vb = inp.logical_kv(b, device="cpu")
        o, l = oracle.attention(qn[b:b + 1], kb.float().numpy()[None], vb.float().numpy()[None], causal, scale)
        os_.append(o[0])
        ls_.append(l[0])
    return np.stack(os_), np.stack(ls_)


@pytest.mark.parametrize("seed", range(12))
def test_prefill_random(afa, seed):
    from attention_flash_fwd_amd import inputs
    rng = np.random.default_rng(9100 + seed)
    B = int(rng.integers(1, 4))
    Hq, Hkv = heads(rng)
    D = int(rng.choice([64, 128]))
    causal = bool(rng.random() < 0.7)
    Sq = int(rng.integers(1, 700))
    Sk = Sq if rng.random() < 0.5 else int(rng.integers(1, 700))
    while B * Hq * Sq * Sk > MAX_PAIRS:
        Sq, Sk = max(1, Sq * 3 // 4), max(1, Sk * 3 // 4)
    say(f"case random prefill seed{seed}: B{B} Sq{Sq} Sk{Sk} Hq{Hq} Hkv{Hkv} D{D} causal{causal}")
    q, k, v = inputs.prefill_inputs(B, Sq, Sk, Hq, Hkv, D, torch.bfloat16, 500 + seed, device="cpu")
    scale = 1 / math.sqrt(D)
    o, lse = afa.prefill(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(to_np(q), to_np(k), to_np(v), causal, scale)
    check_o(to_np(o), o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    check_lse(to_np(lse), l_ref, BF16_LSE_ABS)


@pytest.mark.parametrize("seed", range(8))
def test_prefill_paged_random(afa, seed):
    from attention_flash_fwd_amd import inputs
    rng = np.random.default_rng(9200 + seed)
    nseq = int(rng.integers(1, 5))
    Hq, Hkv = heads(rng)
    D = int(rng.choice([64, 128]))
    causal = bool(rng.random() < 0.7)
    ctx = [int(rng.integers(0, 900)) for _ in range(nseq)]
    Sq = int(rng.integers(1, 400))
    while nseq * Hq * Sq * max(max(ctx), 1) > MAX_PAIRS:
        Sq = max(1, Sq * 3 // 4)
        ctx = [c * 3 // 4 for c in ctx]
    say(f"case random prefill_paged seed{seed}: ctx{ctx} Sq{Sq} Hq{Hq} Hkv{Hkv} D{D} causal{causal}")
    inp = inputs.decode_inputs(ctx, Hq, Hkv, D, seed=600 + seed, device="cuda", spare_blocks=2)
    q = inputs.chunk_queries(nseq, Sq, Hq, D, seed=600 + seed, device="cuda")
    scale = 1 / math.sqrt(D)
    o, lse = afa.prefill_paged(q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                               causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_paged(inp, q, causal, scale)
    check_o(to_np(o), o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    check_lse(to_np(lse), l_ref, BF16_LSE_ABS)


@pytest.mark.parametrize("seed", range(8))
def test_decode_random(afa, seed):
    from attention_flash_fwd_amd import inputs
    rng = np.random.default_rng(9300 + seed)
    nseq = int(rng.integers(1, 9))
    Hq, Hkv = heads(rng, max_hq=64)
    D = int(rng.choice([64, 128]))
    T = int(rng.integers(1, 5)) if rng.random() < 0.5 else int(rng.integers(5, 17))
    while (Hq // Hkv) * T > 256:
        T -= 1
    ctx = [int(rng.integers(1, 3000)) for _ in range(nseq)]
    splits = int(rng.choice([0, 1, 2, 3, 5, 8, 13, 32]))
    say(f"case random decode seed{seed}: ctx{ctx} T{T} Hq{Hq} Hkv{Hkv} D{D} splits{splits}")
    inp = inputs.decode_inputs(ctx, Hq, Hkv, D, seed=700 + seed, device="cuda", spare_blocks=2)
    q = inputs.chunk_queries(nseq, T, Hq, D, seed=700 + seed, device="cuda")
    scale = 1 / math.sqrt(D)
    o, lse = afa.decode_paged_multi(q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                                    num_splits=splits, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_paged(inp, q, True, scale)
    check_o(to_np(o), o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    check_lse(to_np(lse), l_ref, BF16_LSE_ABS)


@pytest.mark.parametrize("seed", range(6))
def test_decode_random_many_items(afa, seed):
    # More (chunk, KV head, sequence) items than the GPU holds split
    # workgroups at once, with one or two column tiles (G T <= 32), so that
    # most items are handed out by the split kernel's work counter; the
    # ragged lengths (some empty) make items of very different cost.  Odd
    # seeds read an fp8 cache.
    from attention_flash_fwd_amd import inputs
    rng = np.random.default_rng(9500 + seed)
    fp8 = seed % 2 == 1
    nseq = int(rng.integers(32, 49))
    Hkv = int(rng.choice([4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hq = Hkv * G
    T = 1 if seed < 2 else int(rng.integers(1, 32 // G + 1))
    D = int(rng.choice([64, 128]))
    ctx = [0 if rng.random() < 0.1 else int(rng.integers(1, 2500)) for _ in range(nseq)]
    splits = int(rng.choice([24, 32]))
    ks, vs = (0.03, 0.05) if fp8 else (1.0, 1.0)
    say(f"case random decode, many items, seed{seed}: nseq{nseq} T{T} Hq{Hq} Hkv{Hkv} D{D} "
        f"splits{splits} {'fp8' if fp8 else 'bf16'} ctx[:6]{ctx[:6]}")
    inp = inputs.decode_inputs(ctx, Hq, Hkv, D, seed=800 + seed, device="cuda", spare_blocks=2,
                               kv_format="fp8" if fp8 else "bf16", k_scale=ks, v_scale=vs)
    q = inputs.chunk_queries(nseq, T, Hq, D, seed=800 + seed, device="cuda")
    scale = 1 / math.sqrt(D)
    if fp8:
        o, lse = afa.decode_paged_fp8(q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens, ks, vs,
                                      num_splits=splits, scale=scale)
    else:
        o, lse = afa.decode_paged_multi(q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                                        num_splits=splits, scale=scale)
    torch.cuda.synchronize()
    if fp8:
        qn = to_np(q)
        os_, ls_ = [], []
        for b in range(nseq):
            kb, vb = inp.logical_kv(b, device="cpu")
            k = oracle.e4m3_decode(kb.numpy()).astype(np.float32)[None]
            v = oracle.e4m3_decode(vb.numpy()).astype(np.float32)[None]
            ob, lb = oracle.attention(qn[b:b + 1], k, v, True, scale * ks)
            os_.append(ob[0] * vs)
            ls_.append(lb[0])
        o_ref, l_ref = np.stack(os_), np.stack(ls_)
    else:
        o_ref, l_ref = oracle_paged(inp, q, True, scale)
    check_o(to_np(o), o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    check_lse(to_np(lse), l_ref, BF16_LSE_ABS)


@pytest.mark.parametrize("seed", range(40))
def test_decode_random_sweep(afa, seed):
    # Wider draws than test_decode_random: up to 48 sequences (some empty),
    # every column-tile count up to 16 (G T <= 256 with T <= 32), explicit
    # or automatic split counts, bf16 or fp8 caches with random scales.
    from attention_flash_fwd_amd import inputs
    rng = np.random.default_rng(12000 + seed)
    fp8 = bool(rng.random() < 0.4)
    nseq = int(rng.integers(1, 49))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
    Hq = Hkv * G
    T = int(rng.integers(1, 256 // G + 1)) if rng.random() < 0.3 else int(rng.integers(1, 5))
    T = min(T, 32)
    D = int(rng.choice([64, 128]))
    ctx = [0 if rng.random() < 0.08 else int(rng.integers(1, 2000)) for _ in range(nseq)]
    splits = int(rng.choice([0, 1, 7, 16, 32, 64]))
    ks, vs = (float(rng.uniform(0.02, 0.06)), float(rng.uniform(0.02, 0.06))) if fp8 else (1.0, 1.0)
    say(f"case random decode sweep seed{seed}: nseq{nseq} T{T} Hq{Hq} Hkv{Hkv} D{D} splits{splits} "
        f"{'fp8' if fp8 else 'bf16'}")
    inp = inputs.decode_inputs(ctx, Hq, Hkv, D, seed=900 + seed, device="cuda", spare_blocks=2,
                               kv_format="fp8" if fp8 else "bf16", k_scale=ks, v_scale=vs)
    q = inputs.chunk_queries(nseq, T, Hq, D, seed=900 + seed, device="cuda")
    scale = 1 / math.sqrt(D)
    if fp8:
        o, lse = afa.decode_paged_fp8(q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens, ks, vs,
                                      num_splits=splits, scale=scale)
    else:
        o, lse = afa.decode_paged_multi(q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                                        num_splits=splits, scale=scale)
    torch.cuda.synchronize()
    qn = to_np(q)
    os_, ls_ = [], []
    for b in range(nseq):
        kb, vb = inp.logical_kv(b, device="cpu")
        if fp8:
            k = oracle.e4m3_decode(kb.numpy()).astype(np.float32)[None]
            v = oracle.e4m3_decode(vb.numpy()).astype(np.float32)[None]
            ob, lb = oracle.attention(qn[b:b + 1], k, v, True, scale * ks)
            ob = ob * vs
        else:
            ob, lb = oracle.attention(qn[b:b + 1], kb.float().numpy()[None], vb.float().numpy()[None], True, scale)
        os_.append(ob[0])
        ls_.append(lb[0])
    check_o(to_np(o), np.stack(os_), BF16_MAX_ABS, BF16_MEAN_ABS)
    check_lse(to_np(lse), np.stack(ls_), BF16_LSE_ABS)


@pytest.mark.parametrize("seed", range(30))
def test_prefill_random_sweep(afa, seed):
    # Wider draws than test_prefill_random / test_prefill_paged_random:
    # lengths up to about 1100, contiguous or paged keys.
    from attention_flash_fwd_amd import inputs
    rng = np.random.default_rng(15000 + seed)
    Hq, Hkv = heads(rng)
    D = int(rng.choice([64, 128]))
    causal = bool(rng.random() < 0.7)
    scale = 1 / math.sqrt(D)
    if rng.random() >= 0.4:
        B = int(rng.integers(1, 4))
        Sq = int(rng.integers(1, 1100))
        Sk = Sq if rng.random() < 0.5 else int(rng.integers(1, 1100))
        while B * Hq * Sq * Sk > MAX_PAIRS:
            Sq, Sk = max(1, Sq * 3 // 4), max(1, Sk * 3 // 4)
        say(f"case random prefill sweep seed{seed}: B{B} Sq{Sq} Sk{Sk} Hq{Hq} Hkv{Hkv} D{D} causal{causal}")
        q, k, v = inputs.prefill_inputs(B, Sq, Sk, Hq, Hkv, D, torch.bfloat16, 3000 + seed, device="cpu")
        o, lse = afa.prefill(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attention(to_np(q), to_np(k), to_np(v), causal, scale)
    else:
        nseq = int(rng.integers(1, 6))
        ctx = [int(rng.integers(0, 1200)) for _ in range(nseq)]
        Sq = int(rng.integers(1, 600))
        while nseq * Hq * Sq * max(max(ctx), 1) > MAX_PAIRS:
            Sq = max(1, Sq * 3 // 4)
            ctx = [c * 3 // 4 for c in ctx]
        say(f"case random prefill_paged sweep seed{seed}: ctx{ctx} Sq{Sq} Hq{Hq} Hkv{Hkv} D{D} causal{causal}")
        inp = inputs.decode_inputs(ctx, Hq, Hkv, D, seed=4000 + seed, device="cuda", spare_blocks=2)
        q = inputs.chunk_queries(nseq, Sq, Hq, D, seed=4000 + seed, device="cuda")
        o, lse = afa.prefill_paged(q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                                   causal=causal, scale=scale)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle_paged(inp, q, causal, scale)
    check_o(to_np(o), o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    check_lse(to_np(lse), l_ref, BF16_LSE_ABS)


@pytest.mark.parametrize("seed", range(6))
def test_decode_random_head_groups(afa, seed):
    # Single-token decode in the four-KV-head regime (KV heads a multiple of
    # four, at least one item per compute unit, chunks of at most 2048
    # tokens), where items are handed out longest sequence first: random
    # batch (the last seed past the 256 sequences the length ranking holds,
    # so unranked), heads, group size, head_dim, lengths (some empty), split
    # counts; odd seeds read an fp8 cache.
    from attention_flash_fwd_amd import inputs
    rng = np.random.default_rng(9700 + seed)
    fp8 = seed % 2 == 1
    nseq = 300 if seed == 5 else int(rng.integers(64, 257))
    Hkv = int(rng.choice([4, 8, 12]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    while Hkv * G > 64:
        G //= 2
    Hq = Hkv * G
    D = int(rng.choice([64, 128]))
    ctx = [0 if rng.random() < 0.05 else int(rng.integers(1, 1500)) for _ in range(nseq)]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    splits = int(rng.choice([1, 2, 3, 5]))
    while nseq * (Hkv // 4) * splits < cus:
        splits += 1
    ks, vs = (float(rng.uniform(0.02, 0.06)), float(rng.uniform(0.02, 0.06))) if fp8 else (1.0, 1.0)
    say(f"case random decode, four-head items, seed{seed}: nseq{nseq} Hq{Hq} Hkv{Hkv} D{D} splits{splits} "
        f"{'fp8' if fp8 else 'bf16'}")
    inp = inputs.decode_inputs(ctx, Hq, Hkv, D, seed=1000 + seed, device="cuda", spare_blocks=2,
                               kv_format="fp8" if fp8 else "bf16", k_scale=ks, v_scale=vs)
    max_tokens = inp.block_table.shape[1] * 16
    assert -(-max_tokens // splits) <= 2048
    scale = 1 / math.sqrt(D)
    if fp8:
        o, lse = afa.decode_paged_fp8(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens, ks, vs,
                                      num_splits=splits, scale=scale)
    else:
        o, lse = afa.decode_paged(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                                  num_splits=splits, scale=scale)
    torch.cuda.synchronize()
    qn = to_np(inp.q)
    kv = [inp.logical_kv(b, device="cpu") for b in range(nseq)]
    if fp8:
        o_ref, l_ref = oracle.decode_fp8(qn, [x[0].numpy() for x in kv], [x[1].numpy() for x in kv], scale, ks, vs)
    else:
        o_ref, l_ref = oracle.decode(qn, [x[0].float().numpy() for x in kv], [x[1].float().numpy() for x in kv],
                                     scale)
    check_o(to_np(o), o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    fin = np.isfinite(l_ref)
    assert np.array_equal(fin, np.isfinite(to_np(lse)))
    check_lse(to_np(lse)[fin], l_ref[fin], BF16_LSE_ABS)
