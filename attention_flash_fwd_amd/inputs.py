"""Seeded synthetic inputs for attention prefill and paged decode.

This module holds no attention arithmetic: it only draws iid N(0, 1) values,
rounds them to the storage dtype and lays them out.  The HIP path, the oracle
and the benchmark all take their inputs from here.

Recipe
------
* Values: fp32 N(0, 1) drawn with a ``torch.Generator`` on the requested device
  (CPU: Mersenne Twister; GPU: Philox), then rounded to bf16 with
  round-to-nearest-even (``Tensor.to(torch.bfloat16)``); the fp32 workload keeps
  them as drawn.  Each tensor (and, for the KV cache, each sequence's K and V)
  has its own seed derived from the config seed, so any part can be
  regenerated on its own.
* Structure (context lengths, block-table permutation): numpy PCG64 on the
  host, identical whatever device holds the values.
* Paged KV cache: 16-token blocks, pool layout [num_blocks, 16, Hkv, D]; the
  block table maps each sequence's logical blocks to a random permutation of
  the pool; every slot that no token occupies (the tail of a sequence's last
  block, spare blocks) holds NaN so that a kernel touching one shows it.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

BLOCK_SIZE = 16

_TAG = {"q": 1, "k": 2, "v": 3}


def _seed_for(seed: int, tag: str, index: int = 0) -> int:
    return (int(seed) * 1_000_003 + _TAG[tag] * 100_019 + int(index) * 7_919) % (2**63 - 1)


def _normal(shape, seed: int, tag: str, index: int, device, dtype) -> torch.Tensor:
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(_seed_for(seed, tag, index))
    x = torch.randn(*shape, generator=g, device=dev, dtype=torch.float32)
    return x if dtype == torch.float32 else x.to(dtype)


# --------------------------------------------------------------------------
# Named workloads (shapes and distributions as the pages' scenarios describe:
# an 8K-token prompt prefill, 32K-class decode contexts, 100K-class contexts).
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class PrefillConfig:
    name: str
    batch: int
    seqlen: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    causal: bool
    dtype: torch.dtype
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def flops(self) -> float:
        """Algorithmic FLOPs: 2 per multiply-add of QK^T and of PV over the
        visible (query, key) pairs only."""
        n = self.seqlen
        pairs = n * (n + 1) // 2 if self.causal else n * n
        return 4.0 * self.head_dim * self.batch * self.n_q_heads * pairs


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ctx_min: int
    ctx_max: int
    num_splits: int
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


TINY_F32 = PrefillConfig("tiny_noncausal_f32_s128_d64", 1, 128, 1, 1, 64, False,
                         torch.float32, 1)
PREFILL_2K = PrefillConfig("causal_gqa_prefill_b4_h32kv8_s2048_d128_bf16", 4, 2048, 32, 8,
                           128, True, torch.bfloat16, 2)
PREFILL_8K = PrefillConfig("causal_gqa_prefill_b2_h32kv8_s8192_d128_bf16", 2, 8192, 32, 8,
                           128, True, torch.bfloat16, 3)
DECODE_B64 = DecodeConfig("paged_decode_b64_h32kv8_d128_ctx512-32768_bf16", 64, 32, 8, 128,
                          512, 32768, 16, 4)
DECODE_128K = DecodeConfig("paged_decode_b4_h64kv8_d128_ctx131072_bf16", 4, 64, 8, 128,
                           131072, 131072, 64, 5)



@dataclass(frozen=True)
class ChunkedPrefillConfig:
    """The last ``chunk`` tokens of ``batch`` prompts of ``ctx`` tokens whose
    keys and values sit in a shuffled paged cache (chunked prefill)."""
    name: str
    batch: int
    ctx: int
    chunk: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def flops(self) -> float:
        """Algorithmic FLOPs over the visible (query, key) pairs: query i of
        the chunk sees ctx - chunk + i + 1 keys."""
        pairs = self.chunk * (self.ctx - self.chunk) + self.chunk * (self.chunk + 1) // 2
        return 4.0 * self.head_dim * self.batch * self.n_q_heads * pairs


CHUNKED_PREFILL = ChunkedPrefillConfig("chunked_prefill_b2_ctx8192_chunk2048_h32kv8_d128_bf16",
                                       2, 8192, 2048, 32, 8, 128, 6)

CONFIGS = {c.name: c for c in (TINY_F32, PREFILL_2K, PREFILL_8K, DECODE_B64, DECODE_128K,
                               CHUNKED_PREFILL)}


# --------------------------------------------------------------------------
# Prefill
# --------------------------------------------------------------------------
def prefill_inputs(batch, seqlen_q, seqlen_k, n_q_heads, n_kv_heads, head_dim,
                   dtype=torch.bfloat16, seed=0, device="cpu"):
    """q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D], contiguous, iid N(0,1) in ``dtype``."""
    q = _normal((batch, seqlen_q, n_q_heads, head_dim), seed, "q", 0, device, dtype)
    k = _normal((batch, seqlen_k, n_kv_heads, head_dim), seed, "k", 0, device, dtype)
    v = _normal((batch, seqlen_k, n_kv_heads, head_dim), seed, "v", 0, device, dtype)
    return q, k, v


def prefill_config_inputs(cfg: PrefillConfig, device="cpu"):
    return prefill_inputs(cfg.batch, cfg.seqlen, cfg.seqlen, cfg.n_q_heads, cfg.n_kv_heads,
                          cfg.head_dim, cfg.dtype, cfg.seed, device)


# --------------------------------------------------------------------------
# Paged decode
# --------------------------------------------------------------------------
@dataclass
class DecodeInputs:
    q: torch.Tensor            # [B, Hq, D] bf16
    k_cache: torch.Tensor      # [num_blocks, 16, Hkv, D] bf16, NaN where unused
    v_cache: torch.Tensor
    block_table: torch.Tensor  # [B, max_blocks] int32, -1 past each sequence
    ctx_lens: torch.Tensor     # [B] int32
    seed: int
    device: str
    block_size: int = BLOCK_SIZE
    ctx: list = field(default_factory=list)
    kv_format: str = "bf16"    # "bf16", or "fp8": uint8 e4m3 codes of value / scale
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def batch(self):
        return self.q.shape[0]

    @property
    def n_kv_heads(self):
        return self.k_cache.shape[2]

    @property
    def head_dim(self):
        return self.q.shape[2]

    def logical_kv(self, b: int, device=None):
        """The unpaged K/V of sequence b, [ctx_b, Hkv, D], regenerated from
        its seed (never read back from the paged pool)."""
        dev = self.device if device is None else device
        n = self.ctx[b]
        shape = (n, self.n_kv_heads, self.head_dim)
        k = _kv_values(shape, self.seed, "k", b + 1, self.device, self.kv_format, self.k_scale)
        v = _kv_values(shape, self.seed, "v", b + 1, self.device, self.kv_format, self.v_scale)
        return k.to(dev), v.to(dev)


E4M3_NAN_CODE = 0x7F          # an e4m3 NaN: fills unused fp8 cache slots


def _kv_values(shape, seed, tag, index, device, kv_format, kv_scale):
    """Cached K or V values: bf16, or the e4m3 codes (uint8) of value / scale
    with torch's float8_e4m3fn conversion (N(0, 1) / scale stays far below
    the e4m3 maximum of 448 for the scales used here)."""
    if kv_format == "bf16":
        return _normal(shape, seed, tag, index, device, torch.bfloat16)
    if kv_format != "fp8":
        raise ValueError(kv_format)
    x = _normal(shape, seed, tag, index, device, torch.float32)
    return (x / kv_scale).to(torch.float8_e4m3fn).view(torch.uint8)


def decode_context_lengths(batch, ctx_min, ctx_max, seed):
    """Per-sequence context lengths, uniform integers in [ctx_min, ctx_max]."""
    rng = np.random.default_rng(seed)
    if ctx_min == ctx_max:
        return [int(ctx_min)] * batch
    return [int(x) for x in rng.integers(ctx_min, ctx_max, size=batch, endpoint=True)]


def decode_inputs(ctx, n_q_heads, n_kv_heads, head_dim, seed=0, device="cpu",
                  spare_blocks=0, block_size=BLOCK_SIZE, table_pad=0, kv_format="bf16",
                  k_scale=1.0, v_scale=1.0):
    """Paged decode inputs for per-sequence context lengths ``ctx``.

    The pool holds exactly the blocks the sequences need plus ``spare_blocks``
    unused ones; a seeded permutation assigns pool blocks to (sequence,
    logical block).  ``table_pad`` widens the table past the longest sequence.
    """
    ctx = [int(c) for c in ctx]
    B = len(ctx)
    nblk = [(c + block_size - 1) // block_size for c in ctx]
    total = sum(nblk) + int(spare_blocks)
    max_blocks = max(1, max(nblk) if nblk else 1) + int(table_pad)
    rng = np.random.default_rng(np.random.SeedSequence([int(seed), 0xB10C]))
    perm = rng.permutation(total).astype(np.int32)

    table = np.full((B, max_blocks), -1, np.int32)
    off = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += nblk[b]

    dev = torch.device(device)
    q = _normal((B, n_q_heads, head_dim), seed, "q", 0, device, torch.bfloat16)
    pool_shape = (max(total, 1), block_size, n_kv_heads, head_dim)
    if kv_format == "fp8":
        k_cache = torch.full(pool_shape, E4M3_NAN_CODE, dtype=torch.uint8, device=dev)
        v_cache = torch.full_like(k_cache, E4M3_NAN_CODE)
    else:
        k_cache = torch.full(pool_shape, float("nan"), dtype=torch.bfloat16, device=dev)
        v_cache = torch.full_like(k_cache, float("nan"))
    kf = k_cache.view(-1, n_kv_heads, head_dim)
    vf = v_cache.view(-1, n_kv_heads, head_dim)
    tbl_dev = torch.from_numpy(table).to(dev)
    for b in range(B):
        if ctx[b] == 0:
            continue
        shape = (ctx[b], n_kv_heads, head_dim)
        kb = _kv_values(shape, seed, "k", b + 1, device, kv_format, k_scale)
        vb = _kv_values(shape, seed, "v", b + 1, device, kv_format, v_scale)
        t = torch.arange(ctx[b], device=dev)
        slots = tbl_dev[b, t // block_size].long() * block_size + (t % block_size)
        kf[slots] = kb
        vf[slots] = vb
        del kb, vb, t, slots
    inp = DecodeInputs(q=q, k_cache=k_cache, v_cache=v_cache, block_table=tbl_dev,
                       ctx_lens=torch.tensor(ctx, dtype=torch.int32, device=dev),
                       seed=int(seed), device=str(dev), block_size=block_size, ctx=ctx,
                       kv_format=kv_format, k_scale=float(k_scale), v_scale=float(v_scale))
    return inp


def chunk_queries(batch, seqlen_q, n_q_heads, head_dim, seed=0, device="cpu"):
    """Queries of a prefill chunk, [B, Sq, Hq, D] bf16: the last Sq tokens of
    each sequence whose keys and values ``decode_inputs`` placed in the cache
    (drawn from their own seed stream, independent of the cache values)."""
    return _normal((batch, seqlen_q, n_q_heads, head_dim), seed, "q", 1, device, torch.bfloat16)


def decode_config_inputs(cfg: DecodeConfig, device="cpu"):
    ctx = decode_context_lengths(cfg.batch, cfg.ctx_min, cfg.ctx_max, cfg.seed)
    return decode_inputs(ctx, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.seed, device)


def decode_kv_bytes(ctx, n_kv_heads, head_dim, elem_bytes=2):
    """K and V bytes of the cached tokens, read once per KV head."""
    return 2 * sum(int(c) for c in ctx) * n_kv_heads * head_dim * elem_bytes
