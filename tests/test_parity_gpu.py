"""Parity of the HIP path with the fp64 oracle, on the GPU.

Every case draws seeded inputs from attention_flash_fwd_amd.inputs, runs the
library through its C ABI (the Python binding only marshals pointers), and
compares with the oracle on the same bytes:
  bf16 output  max-abs <= 2e-2, mean-abs <= 2e-3; lse max-abs <= 1e-4
  fp32 path    max-abs <= 1e-5 (output and lse)
Small shapes are compared in full; the full-size workloads are compared on
sampled rows (prefill) or sampled sequences (decode) that the oracle computes
one by one, plus properties that hold at any size.
"""
import math
import sys

import numpy as np
import pytest

import oracle
from tests.helpers import (BF16_LSE_ABS, BF16_MAX_ABS, BF16_MEAN_ABS, F32_MAX_ABS, check_lse,
                           check_o, to_np)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def afa(cuda):
    import attention_flash_fwd_amd as afa_mod
    from attention_flash_fwd_amd import _lib
    _lib.load()
    return afa_mod


def gen_prefill(B, Sq, Sk, Hq, Hkv, D, dtype, seed):
    from attention_flash_fwd_amd import inputs
    return inputs.prefill_inputs(B, Sq, Sk, Hq, Hkv, D, dtype, seed, device="cpu")


def run_prefill(afa, q, k, v, causal, scale):
    o, lse = afa.prefill(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return to_np(o), to_np(lse)


# ------------------------------------------------------------- prefill ---
def test_tiny_noncausal_f32_config(afa):
    from attention_flash_fwd_amd import inputs
    cfg = inputs.TINY_F32
    say(f"case {cfg.name}")
    q, k, v = inputs.prefill_config_inputs(cfg)
    o, lse = run_prefill(afa, q, k, v, cfg.causal, cfg.scale)
    o_ref, lse_ref = oracle.attention(q.numpy(), k.numpy(), v.numpy(), cfg.causal, cfg.scale)
    check_o(o, o_ref, F32_MAX_ABS)
    check_lse(lse, lse_ref, F32_MAX_ABS)


@pytest.mark.parametrize("B,Sq,Sk,Hq,Hkv,D,causal", [
    (1, 200, 200, 4, 2, 128, True),
    (2, 129, 129, 2, 1, 64, True),
    (1, 100, 300, 2, 2, 128, True),
    (1, 77, 33, 2, 1, 64, False),
])
def test_prefill_f32(afa, B, Sq, Sk, Hq, Hkv, D, causal):
    say(f"case f32 B{B} Sq{Sq} Sk{Sk} Hq{Hq} Hkv{Hkv} D{D} causal{causal}")
    q, k, v = gen_prefill(B, Sq, Sk, Hq, Hkv, D, torch.float32, 7)
    scale = 1 / math.sqrt(D)
    o, lse = run_prefill(afa, q, k, v, causal, scale)
    o_ref, lse_ref = oracle.attention(q.numpy(), k.numpy(), v.numpy(), causal, scale)
    check_o(o, o_ref, F32_MAX_ABS)
    check_lse(lse, lse_ref, F32_MAX_ABS)


PREFILL_BF16_CASES = [
    (1, 1, 1, 1, 1, 128, True),
    (1, 17, 17, 2, 1, 128, True),
    (1, 127, 127, 4, 4, 64, False),
    (1, 129, 129, 8, 2, 128, True),
    (2, 200, 200, 4, 2, 128, True),
    (1, 257, 257, 8, 8, 64, True),
    (1, 1000, 1000, 4, 1, 128, True),
    (2, 100, 300, 4, 2, 128, True),     # Sq < Sk: bottom-right causal alignment
    (1, 300, 100, 2, 1, 128, True),     # Sq > Sk: leading rows see no key
    (3, 333, 333, 6, 3, 64, False),
    (2, 300, 300, 16, 4, 128, True),    # (batch, KV head) pairs a multiple of 8
    (1, 384, 384, 32, 8, 128, True),
    (1, 130, 70, 4, 2, 128, False),
    (1, 512, 512, 8, 8, 64, True),      # two full 256-row workgroups, D = 64
    (2, 5, 1000, 4, 2, 128, False),     # few queries, many keys: one busy wave per workgroup
    (4, 520, 520, 32, 8, 64, True),     # 384 items: a second, partial round of the resident grid
    (3, 520, 520, 36, 12, 64, False),   # 324 items, (batch, KV head) pairs not a multiple of 8
    (2, 300, 300, 9, 3, 128, True),     # causal, group size 3: one query head per item
    (1, 400, 400, 12, 2, 64, True),     # causal, group size 6: two query heads per item
]


@pytest.mark.parametrize("B,Sq,Sk,Hq,Hkv,D,causal", PREFILL_BF16_CASES)
def test_prefill_bf16(afa, B, Sq, Sk, Hq, Hkv, D, causal):
    say(f"case bf16 B{B} Sq{Sq} Sk{Sk} Hq{Hq} Hkv{Hkv} D{D} causal{causal}")
    q, k, v = gen_prefill(B, Sq, Sk, Hq, Hkv, D, torch.bfloat16, 11 + Sq)
    scale = 1 / math.sqrt(D)
    o, lse = run_prefill(afa, q, k, v, causal, scale)
    o_ref, lse_ref = oracle.attention(to_np(q), to_np(k), to_np(v), causal, scale)
    check_o(o, o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    check_lse(lse, lse_ref, BF16_LSE_ABS)


def test_prefill_empty_keys(afa):
    say("case bf16 Sk=0")
    q = torch.randn(1, 64, 2, 128).to(torch.bfloat16).cuda()
    k = torch.zeros(1, 0, 1, 128, dtype=torch.bfloat16, device="cuda")
    o, lse = afa.prefill(q, k, k.clone(), causal=False)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_prefill_empty_batch(afa):
    q = torch.zeros(0, 8, 2, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(0, 8, 1, 128, dtype=torch.bfloat16, device="cuda")
    o, lse = afa.prefill(q, k, k.clone())
    assert o.shape == q.shape and lse.shape == (0, 2, 8)


def sample_rows(B, S, Hq, n, seed):
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(B):
        for h in (0, Hq - 1):
            for i in (0, 1, 127, 128, 129, S // 2, S - 2, S - 1):
                rows.add((b, h, i))
    while len(rows) < n:
        rows.add((int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(S))))
    return sorted(rows)


@pytest.mark.parametrize("cfg_name", ["causal_gqa_prefill_b4_h32kv8_s2048_d128_bf16",
                                      "causal_gqa_prefill_b2_h32kv8_s8192_d128_bf16"])
def test_prefill_full_size_sampled(afa, cfg_name):
    from attention_flash_fwd_amd import inputs
    cfg = inputs.CONFIGS[cfg_name]
    say(f"case {cfg.name} (sampled rows)")
    q, k, v = inputs.prefill_config_inputs(cfg, device="cuda")
    o, lse = afa.prefill(q, k, v, causal=cfg.causal, scale=cfg.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    # Causal row 0 of every head is exactly V[0] of its KV head.
    G = cfg.n_q_heads // cfg.n_kv_heads
    v0 = v[:, 0].repeat_interleave(G, dim=1)
    assert torch.equal(o[:, 0], v0)
    rows = sample_rows(cfg.batch, cfg.seqlen, cfg.n_q_heads, 400, 123)
    o_ref, lse_ref = oracle.attention_rows(to_np(q), to_np(k), to_np(v), cfg.causal, cfg.scale, rows)
    on, ln = to_np(o), to_np(lse)
    got_o = np.stack([on[b, i, h] for (b, h, i) in rows])
    got_l = np.array([ln[b, h, i] for (b, h, i) in rows])
    check_o(got_o, o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    check_lse(got_l, lse_ref, BF16_LSE_ABS)


def test_prefill_invariants(afa):
    say("case prefill invariants")
    B, S, Hq, Hkv, D = 2, 300, 8, 2, 128
    q, k, v = gen_prefill(B, S, S, Hq, Hkv, D, torch.bfloat16, 99)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    o1, l1 = afa.prefill(qc, kc, vc, causal=True)
    o2, l2 = afa.prefill(qc, kc, vc, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "repeat run differs"
    # GQA == MHA with each KV head repeated for its query heads (same arithmetic).
    G = Hq // Hkv
    o3, l3 = afa.prefill(qc, kc.repeat_interleave(G, 2).contiguous(),
                         vc.repeat_interleave(G, 2).contiguous(), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o3) and torch.equal(l1, l3), "GQA differs from repeated-KV MHA"
    # Causal row 0 is V[0] exactly.
    assert torch.equal(o1[:, 0], vc[:, 0].repeat_interleave(G, 1))
    # Constant V per KV head -> every output row equals that constant (to bf16 rounding of P).
    cst = torch.randn(B, 1, Hkv, D).to(torch.bfloat16).cuda()
    o4, _ = afa.prefill(qc, kc, cst.expand(B, S, Hkv, D).contiguous(), causal=True)
    torch.cuda.synchronize()
    want = cst.expand(B, S, Hkv, D).repeat_interleave(G, 2).float()
    assert (o4.float() - want).abs().max().item() <= 2e-2
    # scale = 0: mean of the visible values (closed form), lse = ln(#visible).
    o5, l5 = afa.prefill(qc, kc, vc, causal=True, scale=0.0)
    torch.cuda.synchronize()
    cnt = torch.arange(1, S + 1, device="cuda", dtype=torch.float32)
    mean = vc.float().cumsum(1) / cnt[None, :, None, None]
    assert (o5.float() - mean.repeat_interleave(G, 2)).abs().max().item() <= 2e-2
    assert (l5 - cnt.log()[None, None, :]).abs().max().item() <= 1e-5


@pytest.mark.parametrize("dtype,scale_mul,q_mul", [
    ("bf16", -1.0, 1.0),        # negative scale: the kernel flips Q's sign bits
    ("bf16", 1.0, 16.0),        # large logits: Q x 16 (exact in bf16)
    ("f32", -1.0, 1.0),
])
def test_prefill_negative_scale_and_large_logits(afa, dtype, scale_mul, q_mul):
    say(f"case prefill {dtype} scale x{scale_mul} q x{q_mul}")
    B, S, Hq, Hkv, D = 1, 260, 4, 2, 128
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v = gen_prefill(B, S, S, Hq, Hkv, D, tdt, 31)
    q = q * q_mul
    scale = scale_mul / math.sqrt(D)
    o, lse = run_prefill(afa, q, k, v, True, scale)
    o_ref, lse_ref = oracle.attention(to_np(q), to_np(k), to_np(v), True, scale)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    if dtype == "bf16":
        check_o(o, o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
        check_lse(lse, lse_ref, BF16_LSE_ABS)
    else:
        check_o(o, o_ref, F32_MAX_ABS)
        check_lse(lse, lse_ref, F32_MAX_ABS)


@pytest.mark.parametrize("causal,D,profile,Hq,Hkv", [
    (True, 128, "ramp", 4, 2),      # key norms grow 1x -> 6x along the keys: the reference moves often
    (False, 128, "ramp", 4, 2),
    (True, 64, "bump", 4, 2),       # one 3x tile in the middle, then back to 1x
    (False, 128, "bump", 4, 2),
    (True, 128, "ramp", 8, 2),      # four query heads per work item
    (True, 128, "bump", 3, 1),      # odd group: one query head per work item
])
def test_prefill_scores_growing_along_keys(afa, causal, D, profile, Hq, Hkv):
    """Scores that grow from tile to tile, so that the exponent reference
    has to move after a row's first tile: by a little (where the tile sums
    exceed the bound although the growth is small) or by a lot."""
    say(f"case prefill growing scores causal{causal} D{D} {profile} Hq{Hq} Hkv{Hkv}")
    B, S = 1, 700
    q, k, v = gen_prefill(B, S, S, Hq, Hkv, D, torch.bfloat16, 53)
    j = torch.arange(S, dtype=torch.float32)
    if profile == "ramp":
        r = 1.0 + 5.0 * j / (S - 1)
    else:
        r = torch.where((j >= 320) & (j < 384), torch.tensor(3.0), torch.tensor(1.0))
    k = (k.float() * r[None, :, None, None]).to(torch.bfloat16)
    scale = 1 / math.sqrt(D)
    o, lse = run_prefill(afa, q, k, v, causal, scale)
    o_ref, lse_ref = oracle.attention(to_np(q), to_np(k), to_np(v), causal, scale)
    check_o(o, o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    check_lse(lse, lse_ref, BF16_LSE_ABS)


def test_decode_negative_scale_and_large_logits(afa):
    say("case decode scale < 0 and q x 16")
    inp = gen_decode([700, 33], 8, 2, 128, seed=41)
    for scale, qm in ((-1 / math.sqrt(128), 1.0), (1 / math.sqrt(128), 16.0)):
        q = (inp.q * qm).contiguous()
        o, lse = afa.decode_paged(q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                                  num_splits=3, scale=scale)
        torch.cuda.synchronize()
        qn = to_np(q)
        ref = [oracle.decode(qn[b:b + 1], [to_np(inp.logical_kv(b)[0])], [to_np(inp.logical_kv(b)[1])], scale)
               for b in range(2)]
        o_ref = np.concatenate([r[0] for r in ref])
        l_ref = np.concatenate([r[1] for r in ref])
        check_o(to_np(o), o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
        check_lse(to_np(lse), l_ref, BF16_LSE_ABS)


# -------------------------------------------------------------- decode ---
def gen_decode(ctx, Hq, Hkv, D, seed, device="cuda", spare_blocks=3, table_pad=2):
    from attention_flash_fwd_amd import inputs
    return inputs.decode_inputs(ctx, Hq, Hkv, D, seed=seed, device=device,
                                spare_blocks=spare_blocks, table_pad=table_pad)


def decode_oracle(inp, scale, seqs=None):
    seqs = range(inp.batch) if seqs is None else seqs
    q = to_np(inp.q)
    o_all, l_all = [], []
    for b in seqs:
        kb, vb = inp.logical_kv(b, device="cpu")
        o, l = oracle.decode(q[b:b + 1], [to_np(kb)], [to_np(vb)], scale)
        o_all.append(o[0])
        l_all.append(l[0])
    return np.stack(o_all), np.stack(l_all)


def run_decode(afa, inp, splits, scale=None):
    o, lse = afa.decode_paged(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                              num_splits=splits, scale=scale)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("ctx,Hq,Hkv,D,splits", [
    ([1, 15, 16, 17, 513], 8, 2, 128, 1),
    ([1, 15, 16, 17, 513], 8, 2, 128, 2),
    ([1, 15, 16, 17, 513], 8, 2, 128, 7),
    ([1, 15, 16, 17, 513], 8, 2, 128, 64),
    ([33, 700, 1024, 5], 8, 8, 128, 3),      # G = 1
    ([100, 2000], 32, 8, 128, 16),           # G = 4
    ([257, 1500, 31], 64, 8, 128, 8),        # G = 8
    ([900, 64, 1], 16, 1, 128, 5),           # G = 16
    ([300, 45], 8, 2, 64, 4),                # D = 64
    ([4096, 333], 8, 1, 64, 0),              # automatic split count
    ([2000, 900, 33], 8, 2, 128, 9),         # merge: one wave per row, a clamped block of 16
    ([2000, 700], 8, 2, 128, 24),            # two waves per row
    ([3000, 1200, 5], 8, 2, 128, 40),        # four waves per row, a clamped block
    ([2500, 64], 16, 4, 64, 12),             # D = 64, one wave per row
    ([4000, 300, 17], 8, 2, 128, 200),       # merge weights past the first 64 splits, empty chunks
    ([3000, 70], 8, 2, 64, 130),             # D = 64, 130 splits
    ([5000, 4100], 8, 2, 128, 256),          # the largest split count
])
def test_decode_small(afa, ctx, Hq, Hkv, D, splits):
    say(f"case decode ctx{ctx} Hq{Hq} Hkv{Hkv} D{D} splits{splits}")
    inp = gen_decode(ctx, Hq, Hkv, D, seed=len(ctx) * 10 + Hq)
    scale = 1 / math.sqrt(D)
    o, lse = run_decode(afa, inp, splits)
    o_ref, l_ref = decode_oracle(inp, scale)
    check_o(to_np(o), o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    check_lse(to_np(lse), l_ref, BF16_LSE_ABS)


def test_decode_zero_context(afa):
    say("case decode ctx 0")
    inp = gen_decode([0, 20, 0], 8, 2, 128, seed=3)
    o, lse = run_decode(afa, inp, 4)
    assert torch.all(o[0] == 0) and torch.all(o[2] == 0)
    assert torch.all(torch.isneginf(lse[0])) and torch.all(torch.isneginf(lse[2]))
    o_ref, l_ref = decode_oracle(inp, 1 / math.sqrt(128), seqs=[1])
    check_o(to_np(o[1:2]), o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)


def test_decode_split_invariance_and_permutation(afa):
    say("case decode split invariance / block permutation")
    inp = gen_decode([1000, 37, 4097], 32, 8, 128, seed=5)
    outs = [run_decode(afa, inp, s) for s in (1, 3, 16, 64)]
    for o, l in outs[1:]:
        assert (o.float() - outs[0][0].float()).abs().max().item() <= 1e-2
        assert (l - outs[0][1]).abs().max().item() <= 1e-5
    # Same logical cache under another physical placement -> bit-identical output.
    nb = inp.k_cache.shape[0]
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(1)).cuda()
    k2 = torch.empty_like(inp.k_cache)
    v2 = torch.empty_like(inp.v_cache)
    k2[perm] = inp.k_cache
    v2[perm] = inp.v_cache
    tbl = inp.block_table.long()
    tbl2 = torch.where(tbl >= 0, perm[tbl.clamp(min=0)], tbl).to(torch.int32).contiguous()
    o_a, l_a = run_decode(afa, inp, 16)
    o_b, l_b = afa.decode_paged(inp.q, k2, v2, tbl2, inp.ctx_lens, num_splits=16)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(l_a, l_b)
    o_c, l_c = run_decode(afa, inp, 16)
    assert torch.equal(o_a, o_c) and torch.equal(l_a, l_c), "repeat run differs"


@pytest.mark.parametrize("T", [1, 4])
def test_decode_workspace_contents_do_not_matter(afa, T):
    # The workspace ends with the split kernel's work counter; whatever it
    # holds on entry (huge, small or zero), every item is computed and the
    # result is bit-identical to a call on a zeroed workspace.  T = 4 with
    # G = 8 gives two column tiles, the other case scheduled by the counter.
    from attention_flash_fwd_amd import inputs
    say(f"case decode workspace garbage T{T}")
    # 5 sequences x 8 KV heads x 16 chunks = 640 items, more than the GPU
    # holds at once, so that some items come from the counter.
    inp = gen_decode([3000, 17, 900, 4096, 1], 64, 8, 128, seed=12)
    q = inputs.chunk_queries(inp.batch, T, 64, 128, seed=13, device="cuda")
    ws = afa.decode_workspace(q, inp.k_cache, inp.block_table, 16)
    ws.zero_()
    ref = afa.decode_paged_multi(q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                                 num_splits=16, workspace=ws)
    torch.cuda.synchronize()
    tail = ws[-256:].view(torch.int32)
    for fill in (-1, 1, 0x7fffffff, 5):
        tail.fill_(fill)
        o, l = afa.decode_paged_multi(q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                                      num_splits=16, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o, ref[0]) and torch.equal(l, ref[1]), f"counter fill {fill}"
    # Calls in a row reuse the counter as the previous call left it.
    for _ in range(3):
        o, l = afa.decode_paged_multi(q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                                      num_splits=16, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o, ref[0]) and torch.equal(l, ref[1])


@pytest.mark.parametrize("fp8,D,T", [(False, 128, 1), (False, 64, 3), (True, 128, 1), (True, 128, 3)])
def test_decode_single_split_writes_result_directly(afa, fp8, D, T):
    # With one chunk the split kernel writes bf16 O and lse itself (no merge
    # kernel).  Contexts of at most 16 tokens make a second chunk empty, so
    # two chunks go through the merge with weights exactly 1 and 0: the
    # results must be bit-identical, empty sequences included.
    from attention_flash_fwd_amd import inputs
    say(f"case decode single split fp8={fp8} D{D} T{T}")
    ctx = [16, 1, 0, 9, 16, 5, 12]
    inp = inputs.decode_inputs(ctx, 32, 8, D, seed=21, device="cuda", spare_blocks=2,
                               kv_format="fp8" if fp8 else "bf16", k_scale=0.03, v_scale=0.05)
    q = inputs.chunk_queries(len(ctx), T, 32, D, seed=22, device="cuda")
    if fp8:
        run = lambda s, lse=True: afa.decode_paged_fp8(q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                                                       0.03, 0.05, num_splits=s, return_lse=lse)
    else:
        run = lambda s, lse=True: afa.decode_paged_multi(q, inp.k_cache, inp.v_cache, inp.block_table,
                                                         inp.ctx_lens, num_splits=s, return_lse=lse)
    o1, l1 = run(1)
    o2, l2 = run(2)
    o3, l3 = run(1, lse=False)
    torch.cuda.synchronize()
    assert l3 is None
    assert torch.equal(o1, o2) and torch.equal(o1, o3)
    assert torch.equal(torch.isneginf(l1), torch.isneginf(l2))
    fin = torch.isfinite(l1)
    assert torch.equal(l1[fin], l2[fin])
    assert torch.all(o1[2] == 0) and torch.all(torch.isneginf(l1[2]))


def test_decode_contract_violations_give_nan(afa):
    say("case decode bad block ids / oversize ctx")
    inp = gen_decode([40, 40, 40], 8, 2, 128, seed=8, table_pad=0)
    tbl = inp.block_table.clone()
    tbl[0, 1] = inp.k_cache.shape[0] + 5          # block id past the pool
    tbl[1, 2] = -7                                 # negative block id
    ctx = inp.ctx_lens.clone()
    o, lse = afa.decode_paged(inp.q, inp.k_cache, inp.v_cache, tbl, ctx, num_splits=2)
    torch.cuda.synchronize()
    assert torch.isnan(o[0]).all() and torch.isnan(lse[0]).all()
    assert torch.isnan(o[1]).all() and torch.isnan(lse[1]).all()
    assert torch.isfinite(o[2]).all() and torch.isfinite(lse[2]).all()
    ctx2 = inp.ctx_lens.clone()
    ctx2[2] = inp.block_table.shape[1] * 16 + 1  # more tokens than the table can hold
    o, lse = afa.decode_paged(inp.q, inp.k_cache, inp.v_cache, inp.block_table, ctx2, num_splits=2)
    torch.cuda.synchronize()
    assert torch.isnan(o[2]).all() and torch.isfinite(o[0]).all()


def test_decode_matches_last_row_of_causal_prefill(afa):
    say("case decode == last causal prefill row")
    L, Hq, Hkv, D = 777, 32, 8, 128
    inp = gen_decode([L], Hq, Hkv, D, seed=12)
    kb, vb = inp.logical_kv(0)
    qp = torch.randn(1, L, Hq, D, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16).cuda()
    qp[0, L - 1] = inp.q[0]
    op, lp = afa.prefill(qp, kb[None].contiguous(), vb[None].contiguous(), causal=True)
    od, ld = run_decode(afa, inp, 5)
    assert (op[0, L - 1].float() - od[0].float()).abs().max().item() <= 2e-2
    assert (lp[0, :, L - 1] - ld[0]).abs().max().item() <= 1e-4


def sample_sequences(ctx, nseq, seed):
    """nseq sequence ids (at most all of them): always the longest and the
    shortest, then seeded random others; sorted only after the choice."""
    ctx = np.asarray(ctx)
    must = [int(np.argmax(ctx)), int(np.argmin(ctx))]
    rng = np.random.default_rng(seed)
    others = [int(x) for x in rng.permutation(len(ctx)) if int(x) not in must]
    chosen = list(dict.fromkeys(must)) + others
    return sorted(chosen[:max(nseq, len(set(must)))])


@pytest.mark.parametrize("cfg_name,nseq", [("paged_decode_b64_h32kv8_d128_ctx512-32768_bf16", 8),
                                           ("paged_decode_b4_h64kv8_d128_ctx131072_bf16", 2)])
def test_decode_full_size_sampled(afa, cfg_name, nseq):
    from attention_flash_fwd_amd import inputs
    cfg = inputs.CONFIGS[cfg_name]
    say(f"case {cfg.name} (sampled sequences, num_splits={cfg.num_splits})")
    inp = inputs.decode_config_inputs(cfg, device="cuda")
    o, lse = run_decode(afa, inp, cfg.num_splits)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    seqs = sample_sequences(inp.ctx, nseq, seed=77)
    o_ref, l_ref = decode_oracle(inp, cfg.scale, seqs)
    check_o(to_np(o)[seqs], o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    check_lse(to_np(lse)[seqs], l_ref, BF16_LSE_ABS)
    del inp
    torch.cuda.empty_cache()


# ------------------------------------------------------ paged (chunked) prefill ---
def gen_paged_prefill(ctx, Sq, Hq, Hkv, D, seed, **kw):
    from attention_flash_fwd_amd import inputs
    inp = inputs.decode_inputs(ctx, Hq, Hkv, D, seed=seed, device="cuda", **kw)
    q = inputs.chunk_queries(len(ctx), Sq, Hq, D, seed=seed, device="cuda")
    return inp, q


def paged_prefill_oracle(inp, q, causal, scale, seqs=None):
    qn = to_np(q)
    os_, ls_ = [], []
    for b in (range(len(inp.ctx)) if seqs is None else seqs):
        kb, vb = inp.logical_kv(b, device="cpu")
        o, l = oracle.attention(qn[b:b + 1], kb.float().numpy()[None], vb.float().numpy()[None],
                                causal, scale)
        os_.append(o[0])
        ls_.append(l[0])
    return np.stack(os_), np.stack(ls_)


@pytest.mark.parametrize("ctx,Sq,Hq,Hkv,D,causal", [
    ([300, 77, 1000, 130], 70, 8, 2, 128, True),     # ragged lengths, GQA
    ([16, 200], 70, 8, 2, 128, True),                # ctx < Sq: leading rows see no key
    ([513, 64], 64, 4, 4, 128, False),               # non-causal, MHA
    ([129, 700], 130, 32, 8, 128, True),             # several q-tiles and a ragged tail
    ([390, 45], 45, 8, 1, 64, True),                 # D = 64, G = 8, Sq = ctx for one sequence
])
def test_prefill_paged_small(afa, ctx, Sq, Hq, Hkv, D, causal):
    say(f"case prefill_paged ctx{ctx} Sq{Sq} Hq{Hq} Hkv{Hkv} D{D} causal{causal}")
    inp, q = gen_paged_prefill(ctx, Sq, Hq, Hkv, D, seed=sum(ctx) + Sq, spare_blocks=3)
    scale = 1 / math.sqrt(D)
    o, lse = afa.prefill_paged(q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                               causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = paged_prefill_oracle(inp, q, causal, scale)
    check_o(to_np(o), o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    check_lse(to_np(lse), l_ref, BF16_LSE_ABS)


def test_prefill_paged_scores_growing_along_keys(afa):
    """The paged kernel's softmax under scores that grow along the keys (key
    norms ramped 1x -> 6x), so the exponent reference moves after a row's
    first tile."""
    ctx, Sq, Hq, Hkv, D = [700, 333], 300, 8, 2, 128
    say(f"case prefill_paged growing scores ctx{ctx} Sq{Sq}")
    inp, q = gen_paged_prefill(ctx, Sq, Hq, Hkv, D, seed=61, spare_blocks=3)
    bs = inp.k_cache.shape[1]
    tbl = inp.block_table.cpu()
    k_cache = inp.k_cache.clone()
    ks, vs = [], []
    for b, n in enumerate(ctx):
        r = 1.0 + 5.0 * torch.arange(n, dtype=torch.float32) / (n - 1)
        kb, vb = inp.logical_kv(b, device="cpu")
        kb = (kb.float() * r[:, None, None]).to(torch.bfloat16)
        for lb in range((n + bs - 1) // bs):
            lo, hi = lb * bs, min(n, (lb + 1) * bs)
            k_cache[int(tbl[b, lb]), :hi - lo] = kb[lo:hi].to(k_cache.device)
        ks.append(kb)
        vs.append(vb)
    scale = 1 / math.sqrt(D)
    o, lse = afa.prefill_paged(q, k_cache, inp.v_cache, inp.block_table, inp.ctx_lens, causal=True, scale=scale)
    torch.cuda.synchronize()
    qn = to_np(q)
    ref = [oracle.attention(qn[b:b + 1], ks[b].float().numpy()[None], vs[b].float().numpy()[None], True, scale)
           for b in range(len(ctx))]
    check_o(to_np(o), np.concatenate([r_[0] for r_ in ref]), BF16_MAX_ABS, BF16_MEAN_ABS)
    check_lse(to_np(lse), np.concatenate([r_[1] for r_ in ref]), BF16_LSE_ABS)


def test_prefill_paged_equals_contiguous_and_permutation(afa):
    # With the whole sequence as the chunk, paged prefill is the contiguous
    # prefill on the same keys: same kernel arithmetic, bit-identical output.
    say("case prefill_paged == prefill / block permutation")
    S, Hq, Hkv, D = 333, 16, 4, 128
    inp, q = gen_paged_prefill([S, S], S, Hq, Hkv, D, seed=21, spare_blocks=5)
    k = torch.stack([inp.logical_kv(b)[0] for b in range(2)]).contiguous()
    v = torch.stack([inp.logical_kv(b)[1] for b in range(2)]).contiguous()
    o_c, l_c = afa.prefill(q, k, v, causal=True)
    o_p, l_p = afa.prefill_paged(q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens)
    torch.cuda.synchronize()
    assert torch.equal(o_c, o_p) and torch.equal(l_c, l_p)
    nb = inp.k_cache.shape[0]
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(2)).cuda()
    k2 = torch.empty_like(inp.k_cache)
    v2 = torch.empty_like(inp.v_cache)
    k2[perm] = inp.k_cache
    v2[perm] = inp.v_cache
    tbl = inp.block_table.long()
    tbl2 = torch.where(tbl >= 0, perm[tbl.clamp(min=0)], tbl).to(torch.int32).contiguous()
    o_q, l_q = afa.prefill_paged(q, k2, v2, tbl2, inp.ctx_lens)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_q) and torch.equal(l_p, l_q)


def test_prefill_paged_zero_context_and_contract_violations(afa):
    say("case prefill_paged ctx 0 / bad block ids / oversize ctx")
    inp, q = gen_paged_prefill([0, 50, 50, 50], 20, 8, 2, 128, seed=9)
    tbl = inp.block_table.clone()
    tbl[2, 1] = inp.k_cache.shape[0] + 3           # block id past the pool
    ctx = inp.ctx_lens.clone()
    ctx[3] = inp.block_table.shape[1] * 16 + 1     # more tokens than the table can hold
    o, lse = afa.prefill_paged(q, inp.k_cache, inp.v_cache, tbl, ctx)
    torch.cuda.synchronize()
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))
    assert torch.isfinite(o[1]).all() and torch.isfinite(lse[1]).all()
    assert torch.isnan(o[2]).all() and torch.isnan(lse[2]).all()
    assert torch.isnan(o[3]).all() and torch.isnan(lse[3]).all()
    o_ref, l_ref = paged_prefill_oracle(inp, q, True, 1 / math.sqrt(128), seqs=[1])
    check_o(to_np(o[1:2]), o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    check_lse(to_np(lse[1:2]), l_ref, BF16_LSE_ABS)


def test_prefill_paged_long_chunk_sampled(afa):
    # The last 2048-token chunk of two 8192-token prompts (the benchmark's
    # chunked-prefill workload), compared on sampled query rows.
    from attention_flash_fwd_amd import inputs
    cfg = inputs.CHUNKED_PREFILL
    say(f"case {cfg.name} (sampled rows)")
    inp, q = gen_paged_prefill([cfg.ctx] * cfg.batch, cfg.chunk, cfg.n_q_heads, cfg.n_kv_heads,
                               cfg.head_dim, seed=cfg.seed)
    o, lse = afa.prefill_paged(q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                               causal=True, scale=cfg.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    rng = np.random.default_rng(5)
    qn = to_np(q)
    rows = [(int(rng.integers(cfg.batch)), int(rng.integers(cfg.n_q_heads)), int(rng.integers(cfg.chunk)))
            for _ in range(48)] + [(0, 0, 0), (cfg.batch - 1, cfg.n_q_heads - 1, cfg.chunk - 1)]
    kv = [inp.logical_kv(b, device="cpu") for b in range(cfg.batch)]
    k = np.stack([x[0].float().numpy() for x in kv])
    v = np.stack([x[1].float().numpy() for x in kv])
    o_ref, l_ref = oracle.attention_rows(qn, k, v, True, cfg.scale, rows)
    got = np.stack([to_np(o[b, i, h]) for (b, h, i) in rows])
    got_l = np.array([lse[b, h, i].item() for (b, h, i) in rows])
    check_o(got, o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    check_lse(got_l, l_ref, BF16_LSE_ABS)


# ------------------------------------------------------ multi-token decode ---
@pytest.mark.parametrize("ctx,T,Hq,Hkv,D,splits", [
    ([300, 77, 1000, 5], 4, 8, 2, 128, 4),      # G*T = 16; ctx 5 > T
    ([2, 700], 3, 8, 2, 128, 3),                # ctx < T: the first token sees nothing
    ([513, 2049], 2, 64, 8, 128, 16),           # the long-context head layout, T = 2
    ([129, 4000], 8, 16, 8, 128, 0),            # G = 2, T = 8, automatic splits
    ([390, 45], 4, 8, 2, 64, 5),                # D = 64
    ([300, 1500], 4, 64, 8, 128, 8),            # G*T = 32: two column tiles
    ([77, 2049, 600], 5, 64, 8, 128, 6),        # G*T = 40: a partial third tile
    ([513, 31], 1, 64, 2, 128, 4),              # one token, G = 32
    ([300, 1200], 8, 64, 8, 128, 4),            # 4 tiles in one workgroup, Q operands in LDS
    ([1000, 45, 333], 10, 64, 8, 128, 5),       # 5 tiles: groups of 3, one empty tile
    ([64, 700], 14, 64, 8, 128, 2),             # 7 tiles: groups of 4 (Q in LDS), one empty tile
    ([513, 2000], 16, 16, 1, 128, 6),           # 256 columns: 16 tiles, 4 groups of 4
    ([257, 90], 7, 32, 4, 64, 2),               # D = 64, 4 tiles in one workgroup
    ([400, 901], 13, 32, 2, 64, 3),             # D = 64, 13 tiles: 4 groups of 4, three empty
])
def test_decode_multi_matches_oracle_and_chunked_prefill(afa, ctx, T, Hq, Hkv, D, splits):
    say(f"case decode_multi ctx{ctx} T{T} Hq{Hq} Hkv{Hkv} D{D} splits{splits}")
    inp, q = gen_paged_prefill(ctx, T, Hq, Hkv, D, seed=sum(ctx) * 3 + T, spare_blocks=2)
    scale = 1 / math.sqrt(D)
    o, lse = afa.decode_paged_multi(q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                                    num_splits=splits, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = paged_prefill_oracle(inp, q, True, scale)
    check_o(to_np(o), o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    check_lse(to_np(lse), l_ref, BF16_LSE_ABS)
    # Same computation as the chunked-prefill entry point (different kernel).
    o_p, l_p = afa.prefill_paged(q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                                 causal=True, scale=scale)
    torch.cuda.synchronize()
    assert (o.float() - o_p.float()).abs().max().item() <= 2e-2
    fin = torch.isfinite(l_p)
    assert torch.equal(fin, torch.isfinite(lse))
    assert (lse[fin] - l_p[fin]).abs().max().item() <= 1e-4


def test_decode_multi_single_token_is_decode(afa):
    say("case decode_multi T=1 == decode_paged")
    inp = gen_decode([1000, 37, 4097], 32, 8, 128, seed=5)
    o1, l1 = afa.decode_paged(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens, num_splits=8)
    o2, l2 = afa.decode_paged_multi(inp.q[:, None].contiguous(), inp.k_cache, inp.v_cache,
                                    inp.block_table, inp.ctx_lens, num_splits=8)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2[:, 0]) and torch.equal(l1, l2[:, :, 0])


# ------------------------------------------------------ fp8 (e4m3) KV decode ---
def fp8_oracle(inp, q, scale, seqs=None):
    """Oracle on the cache's e4m3 codes: q [B,Hq,D] (one token) or [B,T,Hq,D]."""
    seqs = list(range(len(inp.ctx))) if seqs is None else seqs
    kv = [inp.logical_kv(b, device="cpu") for b in seqs]
    qn = to_np(q)
    if q.dim() == 3:
        return oracle.decode_fp8(qn[seqs], [x[0].numpy() for x in kv], [x[1].numpy() for x in kv],
                                 scale, inp.k_scale, inp.v_scale)
    os_, ls_ = [], []
    for i, b in enumerate(seqs):
        k = oracle.e4m3_decode(kv[i][0].numpy()).astype(np.float32)[None]
        v = oracle.e4m3_decode(kv[i][1].numpy()).astype(np.float32)[None]
        o, l = oracle.attention(qn[b:b + 1], k, v, True, scale * inp.k_scale)
        os_.append(o[0] * inp.v_scale)
        ls_.append(l[0])
    return np.stack(os_), np.stack(ls_)


@pytest.mark.parametrize("ctx,T,Hq,Hkv,D,splits,ks,vs", [
    ([1, 15, 16, 17, 513], 1, 8, 2, 128, 4, 2.0 ** -5, 2.0 ** -5),
    ([100, 2000], 1, 32, 8, 128, 16, 0.0371, 0.0219),      # scales that are not powers of two
    ([257, 1500, 31], 1, 64, 8, 128, 8, 0.03, 0.05),       # G = 8
    ([300, 45], 1, 8, 2, 64, 3, 0.04, 0.04),                # D = 64
    ([300, 77, 1000], 4, 8, 2, 128, 4, 0.03, 0.03),        # 4 new tokens per sequence
    ([700, 90], 4, 64, 8, 128, 8, 0.03, 0.05),             # G*T = 32: two column tiles
    ([700, 90], 6, 64, 8, 128, 8, 0.03, 0.05),             # three column tiles in one workgroup
    ([700, 90], 8, 64, 8, 128, 8, 0.04, 0.03),             # four tiles, Q operands in LDS
    ([300, 45], 8, 32, 4, 64, 3, 0.04, 0.02),              # D = 64, four column tiles
])
def test_decode_fp8_matches_oracle(afa, ctx, T, Hq, Hkv, D, splits, ks, vs):
    from attention_flash_fwd_amd import inputs
    say(f"case decode_fp8 ctx{ctx} T{T} Hq{Hq} Hkv{Hkv} D{D} splits{splits} ks{ks} vs{vs}")
    inp = inputs.decode_inputs(ctx, Hq, Hkv, D, seed=len(ctx) * 7 + Hq + T, device="cuda", spare_blocks=2,
                               kv_format="fp8", k_scale=ks, v_scale=vs)
    q = inp.q if T == 1 else inputs.chunk_queries(len(ctx), T, Hq, D, seed=5, device="cuda")
    scale = 1 / math.sqrt(D)
    o, lse = afa.decode_paged_fp8(q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens, ks, vs,
                                  num_splits=splits, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = fp8_oracle(inp, q, scale)
    check_o(to_np(o), o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    check_lse(to_np(lse), l_ref, BF16_LSE_ABS)


def test_decode_fp8_permutation_and_nan_contract(afa):
    from attention_flash_fwd_amd import inputs
    say("case decode_fp8 block permutation / bad block id")
    inp = inputs.decode_inputs([1000, 37, 4097], 32, 8, 128, seed=6, device="cuda", kv_format="fp8",
                               k_scale=0.03, v_scale=0.04)
    o_a, l_a = afa.decode_paged_fp8(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                                    0.03, 0.04, num_splits=16)
    nb = inp.k_cache.shape[0]
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(3)).cuda()
    k2 = torch.empty_like(inp.k_cache)
    v2 = torch.empty_like(inp.v_cache)
    k2[perm] = inp.k_cache
    v2[perm] = inp.v_cache
    tbl = inp.block_table.long()
    tbl2 = torch.where(tbl >= 0, perm[tbl.clamp(min=0)], tbl).to(torch.int32).contiguous()
    o_b, l_b = afa.decode_paged_fp8(inp.q, k2, v2, tbl2, inp.ctx_lens, 0.03, 0.04, num_splits=16)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(l_a, l_b)
    tbl3 = inp.block_table.clone()
    tbl3[1, 0] = -3
    o_c, l_c = afa.decode_paged_fp8(inp.q, inp.k_cache, inp.v_cache, tbl3, inp.ctx_lens, 0.03, 0.04,
                                    num_splits=16)
    torch.cuda.synchronize()
    assert torch.isnan(o_c[1]).all() and torch.isnan(l_c[1]).all()
    assert torch.equal(o_c[0], o_a[0]) and torch.equal(o_c[2], o_a[2])


# --------------------------------------- benchmark workloads beyond the step ---
# The benchmark times two more decode workloads on the batch-64 cache shape:
# an e4m3 copy of the cache (scale 1/32, 16 chunks) and four new tokens per
# sequence (the library's split count).  Both are checked here at that size,
# in the same launch configuration, on sampled sequences.
BENCH_FP8_SCALE = 1.0 / 32
BENCH_MULTI_T = 4


def test_decode_fp8_benchmark_workload_sampled(afa):
    from attention_flash_fwd_amd import inputs
    cfg = inputs.DECODE_B64
    say(f"case {cfg.name} fp8 e4m3 cache, scale 1/32, {cfg.num_splits} splits (sampled sequences)")
    ctx = inputs.decode_context_lengths(cfg.batch, cfg.ctx_min, cfg.ctx_max, cfg.seed)
    inp = inputs.decode_inputs(ctx, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.seed, "cuda",
                               kv_format="fp8", k_scale=BENCH_FP8_SCALE, v_scale=BENCH_FP8_SCALE)
    o, lse = afa.decode_paged_fp8(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                                  BENCH_FP8_SCALE, BENCH_FP8_SCALE, num_splits=cfg.num_splits,
                                  scale=cfg.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    seqs = sample_sequences(ctx, 8, seed=78)
    assert int(np.argmax(ctx)) in seqs and int(np.argmin(ctx)) in seqs
    o_ref, l_ref = fp8_oracle(inp, inp.q, cfg.scale, seqs)
    check_o(to_np(o)[seqs], o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    check_lse(to_np(lse)[seqs], l_ref, BF16_LSE_ABS)
    del inp
    torch.cuda.empty_cache()


def test_decode_multi_benchmark_workload_sampled(afa):
    from attention_flash_fwd_amd import inputs
    cfg = inputs.DECODE_B64
    say(f"case {cfg.name} T={BENCH_MULTI_T}, library split count (sampled sequences)")
    inp = inputs.decode_config_inputs(cfg, device="cuda")
    q = inputs.chunk_queries(cfg.batch, BENCH_MULTI_T, cfg.n_q_heads, cfg.head_dim, seed=cfg.seed,
                             device="cuda")
    ws = afa.decode_workspace(q, inp.k_cache, inp.block_table, 0)
    o, lse = afa.decode_paged_multi(q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                                    num_splits=0, scale=cfg.scale, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    seqs = sample_sequences(inp.ctx, 8, seed=79)
    o_ref, l_ref = paged_prefill_oracle(inp, q, True, cfg.scale, seqs=seqs)
    check_o(to_np(o)[seqs], o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    check_lse(to_np(lse)[seqs], l_ref, BF16_LSE_ABS)
    del inp
    torch.cuda.empty_cache()


def test_decode_fp8_every_finite_code(afa):
    # Every finite e4m3 code (254 of 256; 0x7F and 0xFF are NaN) sits in the
    # cache of a one-token sequence, as a K element and as a V element.  With
    # one visible key P = 1 exactly, so O is that V row widened to bf16
    # (exact: every e4m3 value is a bf16 value) and must equal the oracle's
    # decoding bit for bit.  Query head h is the unit vector e_h and the score
    # scale is 1, so lse of head h is the widened K element h times k_scale.
    from attention_flash_fwd_amd import inputs
    say("case decode_fp8 every finite e4m3 code (V exact, K through lse)")
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    D, Hq, Hkv, B = 128, 128, 1, 2
    codes = np.stack([finite[(b * D + np.arange(D)) % finite.size] for b in range(B)])    # [B, D]
    assert set(codes.ravel().tolist()) == set(finite.tolist())
    inp = inputs.decode_inputs([1] * B, Hq, Hkv, D, seed=3, device="cuda", spare_blocks=1,
                               kv_format="fp8", k_scale=1.0, v_scale=1.0)
    for b in range(B):
        blk = int(inp.block_table[b, 0])
        row = torch.from_numpy(codes[b]).cuda()
        inp.k_cache[blk, 0, 0] = row
        inp.v_cache[blk, 0, 0] = row
    q = torch.eye(D, dtype=torch.bfloat16, device="cuda")[None].expand(B, Hq, D).contiguous()
    for ks in (1.0, 0.5):
        o, lse = afa.decode_paged_fp8(q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                                      ks, 1.0, num_splits=1, scale=1.0)
        torch.cuda.synchronize()
        want_v = oracle.e4m3_decode(codes)                                   # [B, D] float64
        got = to_np(o).astype(np.float64)                                    # [B, Hq, D]
        assert np.array_equal(got, np.broadcast_to(want_v[:, None, :], got.shape)), \
            report_mismatch(got[:, 0], want_v)
        want_l = want_v * ks                                                 # head h sees K element h
        np.testing.assert_allclose(to_np(lse).astype(np.float64), want_l, rtol=2e-6, atol=1e-30)
        # the same against the fp8 oracle entry point
        kv = [(codes[b][None, None, :], codes[b][None, None, :]) for b in range(B)]
        o_ref, l_ref = oracle.decode_fp8(to_np(q), [x[0] for x in kv], [x[1] for x in kv], 1.0, ks, 1.0)
        assert np.array_equal(got, o_ref)
        np.testing.assert_allclose(to_np(lse), l_ref, rtol=2e-6)


def report_mismatch(got, want):
    bad = np.argwhere(got != want)
    return f"{len(bad)} mismatches, first at {bad[:4].tolist()}"


def test_prefill_batch_and_head_permutation(afa):
    # Batch entries and KV-head groups are independent: permuting them in the
    # input permutes the output, bit for bit (same kernel arithmetic per row).
    say("case prefill batch / head-group permutation")
    B, S, Hq, Hkv, D = 3, 300, 8, 4, 128
    G = Hq // Hkv
    q, k, v = gen_prefill(B, S, S, Hq, Hkv, D, torch.bfloat16, 404)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    o, lse = afa.prefill(q, k, v, causal=True)
    bp = torch.tensor([2, 0, 1], device="cuda")
    kp = torch.tensor([3, 1, 0, 2], device="cuda")
    qp = torch.stack([torch.arange(G, device="cuda") + G * int(h) for h in kp]).reshape(-1)
    o2, lse2 = afa.prefill(q[bp][:, :, qp].contiguous(), k[bp][:, :, kp].contiguous(),
                           v[bp][:, :, kp].contiguous(), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o2, o[bp][:, :, qp]) and torch.equal(lse2, lse[bp][:, qp])


def test_decode_batch_and_head_permutation(afa):
    # Same for paged decode: permuting the sequences (with their table rows
    # and lengths) and the KV-head groups permutes the output bit for bit.
    say("case decode batch / head-group permutation")
    Hq, Hkv, D = 16, 4, 128
    G = Hq // Hkv
    inp = gen_decode([700, 33, 2100, 16], Hq, Hkv, D, seed=405)
    o, lse = run_decode(afa, inp, 4)
    bp = torch.tensor([3, 0, 2, 1], device="cuda")
    kp = torch.tensor([2, 0, 3, 1], device="cuda")
    qp = torch.stack([torch.arange(G, device="cuda") + G * int(h) for h in kp]).reshape(-1)
    o2, lse2 = afa.decode_paged(inp.q[bp][:, qp].contiguous(), inp.k_cache[:, :, kp].contiguous(),
                                inp.v_cache[:, :, kp].contiguous(), inp.block_table[bp].contiguous(),
                                inp.ctx_lens[bp].contiguous(), num_splits=4)
    torch.cuda.synchronize()
    assert torch.equal(o2, o[bp][:, qp]) and torch.equal(lse2, lse[bp][:, qp])


# ------------------------------------- decode with more than 32 columns ---
# More than 32 (token, head) columns over a bf16 cache take the wide split
# kernel: 32 columns per wave, two or four waves per workgroup, 32-token
# steps shared through LDS.  Cases: both workgroup widths, more than one
# column group, D = 64, sign and size of the scale, the NaN contract, the
# single-chunk direct write, and the 128K cache at the benchmark's size.
@pytest.mark.parametrize("ctx,T,Hq,Hkv,D,splits,scale_mul,q_mul", [
    ([700, 33, 1], 8, 64, 8, 128, 3, -1.0, 1.0),    # 64 columns, negative scale
    ([700, 95], 16, 64, 8, 128, 2, 1.0, 16.0),      # 128 columns, large logits
    ([400, 60], 8, 32, 4, 64, 2, 0.0, 1.0),         # D = 64, zero scale: uniform weights
    ([250, 81], 20, 64, 8, 128, 4, 1.0, 1.0),       # 160 columns: two groups, the second one-quarter full
])
def test_decode_wide_scale_and_groups(afa, ctx, T, Hq, Hkv, D, splits, scale_mul, q_mul):
    say(f"case decode wide ctx{ctx} T{T} Hq{Hq} Hkv{Hkv} D{D} splits{splits} scale x{scale_mul} q x{q_mul}")
    inp, q = gen_paged_prefill(ctx, T, Hq, Hkv, D, seed=sum(ctx) + 7 * T, spare_blocks=2)
    q = (q * q_mul).contiguous()
    scale = scale_mul / math.sqrt(D)
    o, lse = afa.decode_paged_multi(q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                                    num_splits=splits, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = paged_prefill_oracle(inp, q, True, scale)
    check_o(to_np(o), o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    check_lse(to_np(lse), l_ref, BF16_LSE_ABS)


@pytest.mark.parametrize("T", [8, 20])
def test_decode_wide_contract_violations_give_nan(afa, T):
    say(f"case decode wide bad block ids / oversize ctx T{T}")
    inp, q = gen_paged_prefill([300, 300, 300, 300], T, 64, 8, 128, seed=44, spare_blocks=2, table_pad=0)
    tbl = inp.block_table.clone()
    # Each wave fetches one of the two cache blocks of a 32-token step, so
    # bad ids go in both the second (odd) and the first (even) block of a
    # step: every column of the sequence must still come out NaN.
    tbl[0, 3] = inp.k_cache.shape[0] + 5          # block id past the pool (odd block of step 1)
    tbl[1, 17] = -7                                # negative block id (second chunk, odd block)
    tbl[3, 4] = inp.k_cache.shape[0]               # first id past the pool (even block of step 2)
    o, lse = afa.decode_paged_multi(q, inp.k_cache, inp.v_cache, tbl, inp.ctx_lens, num_splits=2)
    torch.cuda.synchronize()
    for b in (0, 1, 3):
        assert torch.isnan(o[b]).all() and torch.isnan(lse[b]).all(), b
    assert torch.isfinite(o[2]).all() and torch.isfinite(lse[2]).all()
    ctx2 = inp.ctx_lens.clone()
    ctx2[2] = inp.block_table.shape[1] * 16 + 1  # more tokens than the table can hold
    o, lse = afa.decode_paged_multi(q, inp.k_cache, inp.v_cache, inp.block_table, ctx2, num_splits=1)
    torch.cuda.synchronize()
    assert torch.isnan(o[2]).all() and torch.isnan(lse[2]).all()
    for b in (0, 1, 3):
        assert torch.isfinite(o[b]).all(), b


@pytest.mark.parametrize("T,Hq,Hkv,D", [(8, 64, 8, 128), (16, 64, 8, 128), (12, 32, 4, 64)])
def test_decode_wide_single_split_writes_result_directly(afa, T, Hq, Hkv, D):
    # As for the narrow kernel: one chunk writes bf16 O and lse directly, two
    # chunks of which the second is empty go through the merge with weights
    # 1 and 0, and the results are bit-identical, empty sequences included.
    from attention_flash_fwd_amd import inputs
    say(f"case decode wide single split T{T} Hq{Hq} Hkv{Hkv} D{D}")
    ctx = [16, 1, 0, 9, 16, 5, 12]
    inp = inputs.decode_inputs(ctx, Hq, Hkv, D, seed=23, device="cuda", spare_blocks=2)
    q = inputs.chunk_queries(len(ctx), T, Hq, D, seed=24, device="cuda")
    run = lambda s: afa.decode_paged_multi(q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                                           num_splits=s)
    o1, l1 = run(1)
    o2, l2 = run(2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(torch.isneginf(l1), torch.isneginf(l2))
    fin = torch.isfinite(l1)
    assert torch.equal(l1[fin], l2[fin])
    assert torch.all(o1[2] == 0) and torch.all(torch.isneginf(l1[2]))
    o_ref, l_ref = paged_prefill_oracle(inp, q, True, 1 / math.sqrt(D))
    check_o(to_np(o1), o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    fin_ref = np.isfinite(l_ref)
    assert np.array_equal(fin_ref, to_np(fin))
    check_lse(to_np(l1)[fin_ref], l_ref[fin_ref], BF16_LSE_ABS)


@pytest.mark.parametrize("T", [8, 16])
def test_decode_wide_128k_sampled(afa, T):
    # The 128K-context cache (4 sequences, 64 query / 8 KV heads) with T new
    # tokens at the library's split count; sampled (sequence, head, token)
    # rows of two sequences against the oracle, every token of one head.
    from attention_flash_fwd_amd import inputs
    cfg = inputs.DECODE_128K
    say(f"case {cfg.name} T={T}, library split count (sampled rows)")
    inp = inputs.decode_config_inputs(cfg, device="cuda")
    q = inputs.chunk_queries(cfg.batch, T, cfg.n_q_heads, cfg.head_dim, seed=cfg.seed + T, device="cuda")
    o, lse = afa.decode_paged_multi(q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                                    num_splits=0, scale=cfg.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    seqs = [0, cfg.batch - 1]
    rng = np.random.default_rng(90 + T)
    rows = [(int(rng.integers(len(seqs))), int(rng.integers(cfg.n_q_heads)), int(rng.integers(T)))
            for _ in range(24)] + [(1, cfg.n_q_heads - 1, t) for t in range(T)]
    kv = [inp.logical_kv(b, device="cpu") for b in seqs]
    k = np.stack([x[0].float().numpy() for x in kv])
    v = np.stack([x[1].float().numpy() for x in kv])
    del kv
    qn = to_np(q)[seqs]
    o_ref, l_ref = oracle.attention_rows(qn, k, v, True, cfg.scale, rows)
    got = np.stack([to_np(o[seqs[bi], t, h]) for (bi, h, t) in rows])
    got_l = np.array([lse[seqs[bi], h, t].item() for (bi, h, t) in rows])
    check_o(got, o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    check_lse(got_l, l_ref, BF16_LSE_ABS)
    del inp, k, v
    torch.cuda.empty_cache()


# ------------------------------------ single-token decode, four-head items ---
# With one new token over a bf16 cache, KV heads in multiples of four, at
# least one item per compute unit and chunks of at most 2048 tokens, the
# split kernel's items are (chunk, four KV heads, sequence), one head per
# wave.  Many short sequences reach that regime at small sizes: the cases
# check every sequence, empty and one-token ones included, at one chunk (the
# direct write), two and three chunks, and the NaN contract.
def head_group_regime(B, Hkv, splits, max_tokens):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return Hkv % 4 == 0 and B * (Hkv // 4) * splits >= cus and -(-max_tokens // splits) <= 2048


@pytest.mark.parametrize("D,splits", [(128, 1), (128, 2), (128, 3), (64, 2)])
def test_decode_head_group_items(afa, D, splits):
    say(f"case decode four-head items D{D} splits{splits}")
    rng = np.random.default_rng(31 + D + splits)
    B, Hq, Hkv = 160, 32, 8
    ctx = [int(x) for x in rng.integers(0, 1500, B)]
    ctx[:4] = [0, 1, 16, 17]
    inp = gen_decode(ctx, Hq, Hkv, D, seed=33 + splits)
    assert head_group_regime(B, Hkv, splits, inp.block_table.shape[1] * 16)
    o, lse = run_decode(afa, inp, splits)
    o_ref, l_ref = decode_oracle(inp, 1 / math.sqrt(D))
    check_o(to_np(o), o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    fin = np.isfinite(l_ref)
    assert np.array_equal(fin, np.isfinite(to_np(lse)))
    check_lse(to_np(lse)[fin], l_ref[fin], BF16_LSE_ABS)
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))


def test_decode_head_group_items_nan_contract(afa):
    say("case decode four-head items: bad block ids / oversize ctx")
    B, Hq, Hkv, D = 160, 32, 8, 128
    inp = gen_decode([200] * B, Hq, Hkv, D, seed=35, table_pad=0)
    assert head_group_regime(B, Hkv, 2, inp.block_table.shape[1] * 16)
    tbl = inp.block_table.clone()
    tbl[3, 2] = inp.k_cache.shape[0] + 9          # block id past the pool
    tbl[70, 12] = -1                               # negative block id, second chunk
    o, lse = afa.decode_paged(inp.q, inp.k_cache, inp.v_cache, tbl, inp.ctx_lens, num_splits=2)
    torch.cuda.synchronize()
    bad = torch.zeros(B, dtype=torch.bool)
    bad[3] = bad[70] = True
    assert torch.isnan(o[bad]).all() and torch.isnan(lse[bad]).all()
    assert torch.isfinite(o[~bad]).all() and torch.isfinite(lse[~bad]).all()
    ctx2 = inp.ctx_lens.clone()
    ctx2[5] = inp.block_table.shape[1] * 16 + 1   # more tokens than the table can hold
    o, lse = afa.decode_paged(inp.q, inp.k_cache, inp.v_cache, inp.block_table, ctx2, num_splits=1)
    torch.cuda.synchronize()
    assert torch.isnan(o[5]).all() and torch.isnan(lse[5]).all()
    keep = torch.ones(B, dtype=torch.bool)
    keep[5] = False
    assert torch.isfinite(o[keep]).all()


@pytest.mark.parametrize("splits", [1, 2])
def test_decode_fp8_head_group_items(afa, splits):
    # The e4m3 cache in the four-head regime, sequences of mixed lengths
    # (handed out longest first), against the fp8 oracle.
    from attention_flash_fwd_amd import inputs
    say(f"case decode_fp8 four-head items splits{splits}")
    rng = np.random.default_rng(41 + splits)
    B, Hq, Hkv, D = 160, 32, 8, 128
    ctx = [int(x) for x in rng.integers(0, 1500, B)]
    ctx[:3] = [0, 1, 1499]
    inp = inputs.decode_inputs(ctx, Hq, Hkv, D, seed=43 + splits, device="cuda", spare_blocks=2, table_pad=2,
                               kv_format="fp8", k_scale=0.04, v_scale=0.07)
    assert head_group_regime(B, Hkv, splits, inp.block_table.shape[1] * 16)
    o, lse = afa.decode_paged_fp8(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                                  0.04, 0.07, num_splits=splits, scale=1 / math.sqrt(D))
    torch.cuda.synchronize()
    o_ref, l_ref = fp8_oracle(inp, inp.q, 1 / math.sqrt(D))
    check_o(to_np(o), o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    fin = np.isfinite(l_ref)
    assert np.array_equal(fin, np.isfinite(to_np(lse)))
    check_lse(to_np(lse)[fin], l_ref[fin], BF16_LSE_ABS)


@pytest.mark.parametrize("ctx,T,Hq,Hkv,D,splits", [
    ([700, 33, 1], 8, 64, 8, 128, 3),          # 64 columns: still the 16-column tiles on e4m3
    ([700, 95], 16, 64, 8, 128, 2),            # 128 columns: four waves of 32
    ([250, 81, 0], 20, 64, 8, 128, 4),         # 160 columns: two column groups, an empty sequence
    ([300, 77], 8, 64, 8, 64, 3),              # D = 64: stays on the 16-column tiles
])
def test_decode_fp8_wide_columns(afa, ctx, T, Hq, Hkv, D, splits):
    # More than 64 (token, head) columns over an e4m3 cache at head_dim 128:
    # the wide split kernel widens each step's V rows to bf16 in LDS once for
    # all waves (64 columns and D = 64 stay on the 16-column tiles).
    from attention_flash_fwd_amd import inputs
    say(f"case decode_fp8 wide ctx{ctx} T{T} Hq{Hq} Hkv{Hkv} D{D} splits{splits}")
    inp = inputs.decode_inputs(ctx, Hq, Hkv, D, seed=sum(ctx) + T, device="cuda", spare_blocks=2,
                               kv_format="fp8", k_scale=0.035, v_scale=0.06)
    q = inputs.chunk_queries(len(ctx), T, Hq, D, seed=7 + T, device="cuda")
    scale = 1 / math.sqrt(D)
    o, lse = afa.decode_paged_fp8(q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens, 0.035, 0.06,
                                  num_splits=splits, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = fp8_oracle(inp, q, scale)
    check_o(to_np(o), o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    fin = np.isfinite(l_ref)
    assert np.array_equal(fin, np.isfinite(to_np(lse)))
    check_lse(to_np(lse)[fin], l_ref[fin], BF16_LSE_ABS)
