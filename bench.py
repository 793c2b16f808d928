"""Benchmark of the attention hot path on one MI355X.

One step = one pass over the whole path on one synthetic batch:
  * causal GQA prefill, bf16: batch 2, 32 query / 8 KV heads, seqlen 8192,
    head_dim 128 (attn_prefill);
  * paged split-KV decode, bf16: batch 64, 32 / 8 heads, head_dim 128,
    context lengths uniform in [512, 32768], 16-token blocks, shuffled table,
    16 splits (attn_decode_paged);
  * long-context paged decode, bf16: batch 4, 64 / 8 heads, context 131072,
    64 splits (attn_decode_paged).
Inputs are resident in HBM before timing; outputs and workspaces are
preallocated.  `value` is the whole step's speed-of-light time (prefill FLOPs
at the bf16 MFMA peak plus decode KV bytes at the HBM peak) over its measured
time, in percent; the per-part absolute rates are in `parts`.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --split-sweep      (Flash-Decoding split threshold sweep, one JSON line)
       python bench.py --compare-sdpa     (PyTorch's fused attention beside attn_prefill)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_FLOPS = 2.5e15      # MI355X dense bf16 MFMA
PEAK_HBM_BPS = 8.0e12         # MI355X HBM3E
COPY_BYTES = 1 << 30          # calibration copy (profiling runs only)
# Workloads beyond the hot path's step, timed on their own after it (never
# part of `value` or `ms_per_step`).
EXTRAS = ("prefill_2k", "chunked_prefill", "decode_multi", "decode_multi_128k", "decode_b64_fp8")
FP8_SCALE = 1.0 / 32          # per-tensor K and V scale of the fp8 extra
MULTI_T = 4                   # new tokens per sequence in the multi-token decode extra
MULTI_128K_T = 16             # new tokens per sequence over the 128K-context cache (128 columns)
METRIC = "prefill attn TFLOP/s + decode KV GB/s, % of MI355X bf16/HBM peak"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--parts", default="prefill,decode_b64,decode_128k," + ",".join(EXTRAS),
                   help="comma-separated subset (for profiling runs); 'copy' adds a plain "
                        "1 GiB device-to-device copy that calibrates the HBM byte counters")
    p.add_argument("--multi-t", type=int, default=MULTI_T,
                   help="new tokens per sequence of the decode_multi extra (profiling runs)")
    p.add_argument("--multi-workload", choices=("b64", "128k"), default="b64",
                   help="cache of the decode_multi extra: the batch-64 or the 128K-context decode "
                        "workload (profiling runs)")
    p.add_argument("--split-sweep", action="store_true",
                   help="instead of the benchmark, sweep paged decode over context lengths and "
                        "batch sizes with one chunk (Flash-Decoding off), the library's automatic "
                        "count and every explicit count; one JSON line")
    p.add_argument("--multi-split-sweep", action="store_true",
                   help="instead of the benchmark, sweep multi-token paged decode (2-32 new tokens "
                        "per sequence) over equal and mixed context lengths with the library's "
                        "automatic chunk count and every explicit count; one JSON line")
    p.add_argument("--compare-sdpa", action="store_true",
                   help="instead of the benchmark, time PyTorch's fused attention (SDPA, flash "
                        "backend) beside attn_prefill on the prefill workload; one JSON line")
    return p.parse_args()


def compare_sdpa(steps, warmup):
    """Context, not the benchmark: PyTorch's fused attention on the same
    causal GQA prefill input as attn_prefill.  Only the flash backend is
    allowed, so an unsupported case raises instead of falling back to the
    bf16 math path.  K and V are expanded to the query heads beforehand
    (untimed), since the call is made without a GQA layout."""
    import torch
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel

    import attention_flash_fwd_amd as afa
    from attention_flash_fwd_amd import _lib, inputs

    _lib.load()
    cfg = inputs.PREFILL_8K
    q, k, v = inputs.prefill_config_inputs(cfg, device=torch.device("cuda:0"))     # [B, S, H, D]
    rep_ = q.shape[2] // k.shape[2]
    qt = q.transpose(1, 2).contiguous()
    kt = k.repeat_interleave(rep_, dim=2).transpose(1, 2).contiguous()
    vt = v.repeat_interleave(rep_, dim=2).transpose(1, 2).contiguous()

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    def sdpa():
        return F.scaled_dot_product_attention(qt, kt, vt, is_causal=True)

    # Three interleaved rounds, the best of each, so that neither side is
    # timed alone on a cold or a hot chip.
    ours_ms = sdpa_ms = float("inf")
    with sdpa_kernel(SDPBackend.FLASH_ATTENTION):
        for _ in range(3):
            ours_ms = min(ours_ms, timed(lambda: afa.prefill(q, k, v, causal=True, return_lse=False)))
            sdpa_ms = min(sdpa_ms, timed(sdpa))
        o_sdpa = sdpa().transpose(1, 2)
    o_ours, _ = afa.prefill(q, k, v, causal=True, return_lse=False)
    torch.cuda.synchronize()
    flops = cfg.flops()
    print(json.dumps({"compare": "torch_sdpa_flash", "workload": cfg.name, "torch": torch.__version__,
                      "attn_prefill_ms": ours_ms, "attn_prefill_tflops": flops / ours_ms / 1e9,
                      "sdpa_ms": sdpa_ms, "sdpa_tflops": flops / sdpa_ms / 1e9,
                      "speedup": sdpa_ms / ours_ms,
                      "max_abs_diff": (o_sdpa.float() - o_ours.float()).abs().max().item()}))


def stats(ms_list):
    """Mean, median and minimum of per-call event times (ms)."""
    xs = sorted(ms_list)
    n = len(xs)
    med = xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])
    return {"ms": sum(xs) / n, "ms_median": med, "ms_min": xs[0]}


SWEEP_CTX = (256, 512, 1024, 2048, 4096, 8192, 16384, 32768, 131072)
SWEEP_BATCH = (1, 4, 16, 64)
SWEEP_THRESHOLDS = (256, 512, 1024, 2048, 4096)


def split_sweep(reps):
    """Flash-Decoding threshold sweep ("GPU Kernel 调度：大模型推理的拐点 2026",
    checklist item 2 and advice 2: measure decode latency with the split
    enabled and disabled over sequence lengths, find the knee, and check that
    where splitting applies it is at least 30% faster).

    Workload: bf16 paged decode, 32 query / 8 KV heads, head_dim 128,
    shuffled 16-token blocks; each (context L, batch) with equal lengths, and
    (from 1024 tokens and 4 sequences on) again with lengths drawn uniformly
    from 512 to L (seeded).  For each: one chunk (splitting off), the
    library's automatic count, and every power-of-two count up to 256
    (chunks of at least 16 tokens); the
    median of `reps` event-timed calls each, interleaved over three rounds
    (best round kept).  Batch 64 at 131072 tokens (34 GB of cache) is left
    out; the other shapes fit with room to spare."""
    import torch

    import attention_flash_fwd_amd as afa
    from attention_flash_fwd_amd import _lib, inputs

    _lib.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    Hq, Hkv, D = 32, 8, 128
    rows = []
    shapes = [(L, B, False) for L in SWEEP_CTX for B in SWEEP_BATCH if L * B <= 32768 * 64]
    shapes += [(L, B, True) for L in SWEEP_CTX for B in SWEEP_BATCH if L * B <= 32768 * 64 and L > 512 and B > 1]
    for L, B, mix in shapes:
        ctx = inputs.decode_context_lengths(B, 512, L, seed=L + B) if mix else [L] * B
        inp = inputs.decode_inputs(ctx, Hq, Hkv, D, seed=L + B, device=dev)
        counts = [1] + [c for c in (2, 4, 8, 16, 32, 64, 128, 256) if (L + c - 1) // c >= 16]
        auto = afa.decode_num_splits(B, Hkv, inp.block_table.shape[1], 16, 0)
        o = torch.empty_like(inp.q)
        lse = torch.empty(inp.q.shape[:2], dtype=torch.float32, device=dev)
        wss = {c: afa.decode_workspace(inp.q, inp.k_cache, inp.block_table, c)
               for c in set(counts + [auto])}

        def call(c):
            afa.decode_paged(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                             num_splits=c, out=o, lse_out=lse, workspace=wss[c])

        best = {c: float("inf") for c in wss}
        for _ in range(3):
            for c in wss:
                for _ in range(3):
                    call(c)
                evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(reps)]
                for a_ev, b_ev in evs:
                    a_ev.record(stream)
                    call(c)
                    b_ev.record(stream)
                torch.cuda.synchronize()
                best[c] = min(best[c], stats([a_ev.elapsed_time(b_ev) for a_ev, b_ev in evs])["ms_median"])
        c_best = min(best, key=best.get)
        row = {"ctx": L, "batch": B, "lengths": "mixed" if mix else "equal",
               "off_us": best[1] * 1e3, "auto_splits": auto,
               "auto_us": best[auto] * 1e3, "best_splits": c_best, "best_us": best[c_best] * 1e3,
               "auto_vs_best": best[auto] / best[c_best], "auto_speedup_vs_off": best[1] / best[auto],
               "by_splits_us": {str(c): best[c] * 1e3 for c in sorted(best)}}
        rows.append(row)
        print(f"sweep ctx {L} batch {B} {row['lengths']}: off {row['off_us']:.1f} us, auto({auto}) {row['auto_us']:.1f} us, "
              f"best({c_best}) {row['best_us']:.1f} us", file=sys.stderr, flush=True)
        del inp, wss, o, lse
        torch.cuda.empty_cache()
    # The page's threshold policy: split (at the library's count) only when
    # the context reaches the threshold, else one chunk (equal lengths).
    eq = [r for r in rows if r["lengths"] == "equal"]
    mixed = [r for r in rows if r["lengths"] == "mixed"]
    policy = {}
    for t in SWEEP_THRESHOLDS:
        tot = sum((r["auto_us"] if r["ctx"] >= t else r["off_us"]) for r in eq)
        policy[str(t)] = {"sum_us_over_shapes": tot}
    tot_auto = sum(r["auto_us"] for r in eq)
    # Where splitting applies (the library picks more than one chunk), how
    # much faster than one chunk is it?
    split_rows = [r for r in eq if r["auto_splits"] > 1]
    print(json.dumps({
        "sweep": "flash_decoding_split_threshold",
        "workload": "paged_decode_h32kv8_d128_bf16, equal contexts per batch, and contexts drawn from 512..L",
        "reps": reps, "rows": rows, "threshold_policy": policy,
        "library_policy_sum_us": tot_auto,
        "auto_within_5pct_of_best": sum(1 for r in eq if r["auto_vs_best"] <= 1.05),
        "shapes": len(eq),
        "split_shapes_30pct_faster_than_off": sum(1 for r in split_rows if r["auto_speedup_vs_off"] >= 1 / 0.7),
        "split_shapes": len(split_rows),
        "mixed": {"shapes": len(mixed),
                  "auto_within_5pct_of_best": sum(1 for r in mixed if r["auto_vs_best"] <= 1.05),
                  "mean_auto_vs_best": sum(r["auto_vs_best"] for r in mixed) / max(1, len(mixed)),
                  "max_auto_vs_best": max((r["auto_vs_best"] for r in mixed), default=1.0)},
    }), flush=True)


MSWEEP_T = (2, 4, 8, 16, 32)
MSWEEP_CTX = (8192, 32768)
MSWEEP_BATCH = (4, 16, 32, 64)


def multi_split_sweep(reps):
    """Chunk counts of attn_decode_paged_multi against every explicit count.

    Workload: bf16 paged decode, 32 query / 8 KV heads, head_dim 128, T new
    tokens per sequence (4 T columns per KV head: up to 32 in the narrow
    split kernel, more in the wide one).  Each (T, L, batch) twice: every
    sequence L tokens long, and lengths drawn uniformly from 512 to L (seeded;
    the decode workloads' mix).  For each, the automatic count and every
    power-of-two count up to 64 with chunks of at least 64 tokens; the median
    of `reps` event-timed calls each, interleaved over three rounds (best
    round kept)."""
    import torch

    import attention_flash_fwd_amd as afa
    from attention_flash_fwd_amd import _lib, inputs

    lib = _lib.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    Hq, Hkv, D = 32, 8, 128
    rows = []
    for T in MSWEEP_T:
        for L in MSWEEP_CTX:
            for B in MSWEEP_BATCH:
                for mix in (False, True):
                    ctx = inputs.decode_context_lengths(B, 512, L, seed=L + B) if mix else [L] * B
                    inp = inputs.decode_inputs(ctx, Hq, Hkv, D, seed=L + B + T, device=dev)
                    q = inputs.chunk_queries(B, T, Hq, D, seed=7, device=dev)
                    o = torch.empty_like(q)
                    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
                    mb = inp.block_table.shape[1]
                    per_split = B * T * Hq * (D + 1) * 4
                    auto = int(lib.attn_decode_multi_workspace_bytes(B, T, Hq, Hkv, D, mb, 16, 0) // per_split)
                    counts = sorted(set([1] + [c for c in (2, 4, 8, 16, 32, 64) if (L + c - 1) // c >= 64] + [auto]))
                    wss = {c: torch.empty(int(lib.attn_decode_multi_workspace_bytes(B, T, Hq, Hkv, D, mb, 16, c)),
                                          dtype=torch.uint8, device=dev) for c in counts}

                    def call(c):
                        afa.decode_paged_multi(q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                                               num_splits=c, out=o, lse_out=lse, workspace=wss[c])

                    best = {c: float("inf") for c in counts}
                    for _ in range(3):
                        for c in counts:
                            for _ in range(3):
                                call(c)
                            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                                   for _ in range(reps)]
                            for a_ev, b_ev in evs:
                                a_ev.record(stream)
                                call(c)
                                b_ev.record(stream)
                            torch.cuda.synchronize()
                            best[c] = min(best[c], stats([a_ev.elapsed_time(b_ev) for a_ev, b_ev in evs])["ms_median"])
                    c_best = min(best, key=best.get)
                    row = {"tokens": T, "ctx": L, "batch": B, "lengths": "mixed" if mix else "equal",
                           "auto_splits": auto, "auto_us": best[auto] * 1e3, "best_splits": c_best,
                           "best_us": best[c_best] * 1e3, "auto_vs_best": best[auto] / best[c_best],
                           "by_splits_us": {str(c): best[c] * 1e3 for c in counts}}
                    rows.append(row)
                    print(f"multi sweep T {T} ctx {L} batch {B} {row['lengths']}: auto({auto}) {row['auto_us']:.1f} us, "
                          f"best({c_best}) {row['best_us']:.1f} us", file=sys.stderr, flush=True)
                    del inp, wss, o, lse, q
                    torch.cuda.empty_cache()
    summary = {}
    for kind in ("equal", "mixed"):
        r = [x["auto_vs_best"] for x in rows if x["lengths"] == kind]
        summary[kind] = {"shapes": len(r), "mean_auto_vs_best": sum(r) / len(r), "max_auto_vs_best": max(r),
                         "within_5pct": sum(1 for x in r if x <= 1.05)}
    print(json.dumps({"sweep": "multi_token_split_count",
                      "workload": "paged_decode_multi_h32kv8_d128_bf16, equal and mixed (512..L) contexts",
                      "reps": reps, "rows": rows, "summary": summary}), flush=True)


def decode_bytes(inp, n_q_heads):
    """Algorithmic bytes of one paged decode call: K and V of every cached
    token once per KV head, Q and O once, the used block-table entries and
    the context lengths."""
    from attention_flash_fwd_amd import inputs
    B, Hq, D = inp.q.shape
    kv = inputs.decode_kv_bytes(inp.ctx, inp.n_kv_heads, D)
    used_blocks = sum((c + 15) // 16 for c in inp.ctx)
    return kv + 2 * B * Hq * D * 2 + used_blocks * 4 + B * 4


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "prefill": ["attention_flash_fwd_amd/csrc/prefill_bf16.hip", "attention_flash_fwd_amd/csrc/gfx950.hpp",
                "attention_flash_fwd_amd/csrc/kernels.hpp"],
    "decode": ["attention_flash_fwd_amd/csrc/decode.hip", "attention_flash_fwd_amd/csrc/decode_wide.hip",
               "attention_flash_fwd_amd/csrc/gfx950.hpp",
               "attention_flash_fwd_amd/csrc/kernels.hpp"],
}
def sources_of(part):
    return KERNEL_SOURCES["prefill" if "prefill" in part else "decode"]


def load_traffic(part, kernel_digest=None):
    """HBM bytes (read + write) per call of `part` from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE runs, if they were taken on the current
    kernel source; else None."""
    if kernel_digest is None:
        kernel_digest = source_digest(sources_of(part))
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(part)
    if rec is None or rec.get("source_digest") != kernel_digest:
        return None
    return rec.get("hbm_bytes")


def cpu_baseline(parts, pf_cfg, pf_in, dec_parts):
    """Time the fp64 oracle on a bounded sample of each part and scale to the
    whole step.  Returns the same %-of-peak figure as `value` (and rates)."""
    import numpy as np
    import torch

    import oracle

    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    threads = max(1, min(threads, 64))
    detail = {}
    cpu_step_s = 0.0
    sol_s = 0.0
    if "prefill" in parts:
        q, k, v = pf_in
        rng = np.random.default_rng(0)
        B, S, Hq, D = q.shape
        n_rows = 131072
        rows = [(int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(S))) for _ in range(n_rows)]
        qn = q.float().cpu().numpy()
        kn = k.float().cpu().numpy()
        vn = v.float().cpu().numpy()
        print(f"cpu baseline: prefill, {n_rows} rows on {threads} threads", file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        oracle.attention_rows(qn, kn, vn, True, pf_cfg.scale, rows, nthreads=threads)
        dt = time.perf_counter() - t0
        flops_sample = sum(4.0 * D * (i + 1) for (_, _, i) in rows)
        rate = flops_sample / dt
        cpu_step_s += pf_cfg.flops() / rate
        sol_s += pf_cfg.flops() / PEAK_BF16_FLOPS
        detail["prefill_gflops"] = rate / 1e9
        detail["prefill_sample"] = f"{n_rows} random query rows of all {B * Hq} heads"
    for name, (inp, Hq, scale, nbytes) in dec_parts.items():
        n_seq = 16
        seqs = list(range(min(n_seq, inp.batch)))
        qn = inp.q.float().cpu().numpy()
        ks, vs, byts = [], [], 0
        for b in seqs:
            kb, vb = inp.logical_kv(b, device="cpu")
            ks.append(kb.float().numpy())
            vs.append(vb.float().numpy())
            byts += 2 * kb.numel() * 2
        print(f"cpu baseline: {name}, {len(seqs)} sequences", file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        oracle.decode(qn[seqs], ks, vs, scale, nthreads=threads)
        dt = time.perf_counter() - t0
        rate = byts / dt
        cpu_step_s += nbytes / rate
        sol_s += nbytes / PEAK_HBM_BPS
        detail[f"{name}_gbps"] = rate / 1e9
        detail[f"{name}_sample"] = f"sequences {seqs}"
    value = 100.0 * sol_s / cpu_step_s if cpu_step_s > 0 else None
    return {"value": value, "unit": "% of MI355X peak (same step, oracle on host)",
            "cores": threads, "kind": "oracle",
            "sample": "; ".join(f"{k}: {v}" for k, v in detail.items() if k.endswith("sample")),
            "step_seconds_extrapolated": cpu_step_s,
            **{k: v for k, v in detail.items() if not k.endswith("sample")}}


def main():
    args = parse()
    if args.compare_sdpa:
        compare_sdpa(args.steps, args.warmup)
        return
    if args.split_sweep:
        split_sweep(reps=max(5, min(args.steps, 50)))
        return
    if args.multi_split_sweep:
        multi_split_sweep(reps=max(5, min(args.steps, 50)))
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    import torch

    import attention_flash_fwd_amd as afa
    from attention_flash_fwd_amd import _lib, inputs

    _lib.load()
    dev = torch.device("cuda:0")
    parts = [p for p in args.parts.split(",") if p]

    # ---- inputs, resident in HBM ---------------------------------------
    pf_cfg = inputs.PREFILL_8K
    pf_in = inputs.prefill_config_inputs(pf_cfg, device=dev) if "prefill" in parts else None
    dec_cfgs = {"decode_b64": inputs.DECODE_B64, "decode_128k": inputs.DECODE_128K}
    dec = {}
    for name, cfg in dec_cfgs.items():
        if name not in parts:
            continue
        inp = inputs.decode_config_inputs(cfg, device=dev)
        ws = afa.decode_workspace(inp.q, inp.k_cache, inp.block_table, cfg.num_splits)
        o = torch.empty_like(inp.q)
        lse = torch.empty(inp.q.shape[:2], dtype=torch.float32, device=dev)
        dec[name] = (cfg, inp, ws, o, lse)
    extra_in = {}
    if "prefill_2k" in parts:
        p2 = inputs.PREFILL_2K
        q2, k2, v2 = inputs.prefill_config_inputs(p2, device=dev)
        o2 = torch.empty_like(q2)
        l2 = torch.empty((p2.batch, p2.n_q_heads, p2.seqlen), dtype=torch.float32, device=dev)
        extra_in["prefill_2k"] = (p2, q2, k2, v2, o2, l2)
    if "chunked_prefill" in parts:
        cp = inputs.CHUNKED_PREFILL
        cinp = inputs.decode_inputs([cp.ctx] * cp.batch, cp.n_q_heads, cp.n_kv_heads, cp.head_dim,
                                    seed=cp.seed, device=dev)
        cq = inputs.chunk_queries(cp.batch, cp.chunk, cp.n_q_heads, cp.head_dim, seed=cp.seed, device=dev)
        co = torch.empty_like(cq)
        clse = torch.empty((cp.batch, cp.n_q_heads, cp.chunk), dtype=torch.float32, device=dev)
        extra_in["chunked_prefill"] = (cp, cinp, cq, co, clse)
    multi_t = args.multi_t
    if "decode_multi" in parts:
        mcfg = inputs.DECODE_B64 if args.multi_workload == "b64" else inputs.DECODE_128K
        minp = inputs.decode_config_inputs(mcfg, device=dev)
        mq = inputs.chunk_queries(mcfg.batch, multi_t, mcfg.n_q_heads, mcfg.head_dim, seed=mcfg.seed, device=dev)
        mws = afa.decode_workspace(mq, minp.k_cache, minp.block_table, 0)     # the library's split count
        mo = torch.empty_like(mq)
        mlse = torch.empty((mcfg.batch, mcfg.n_q_heads, multi_t), dtype=torch.float32, device=dev)
        extra_in["decode_multi"] = (mcfg, minp, mq, mws, mo, mlse)
    if "decode_multi_128k" in parts:
        kcfg = inputs.DECODE_128K
        kinp = dec["decode_128k"][1] if "decode_128k" in dec else inputs.decode_config_inputs(kcfg, device=dev)
        kq = inputs.chunk_queries(kcfg.batch, MULTI_128K_T, kcfg.n_q_heads, kcfg.head_dim, seed=kcfg.seed + 1,
                                  device=dev)
        kws = afa.decode_workspace(kq, kinp.k_cache, kinp.block_table, 0)     # the library's split count
        ko = torch.empty_like(kq)
        klse = torch.empty((kcfg.batch, kcfg.n_q_heads, MULTI_128K_T), dtype=torch.float32, device=dev)
        extra_in["decode_multi_128k"] = (kcfg, kinp, kq, kws, ko, klse)
    if "decode_b64_fp8" in parts:
        fcfg = inputs.DECODE_B64
        fctx = inputs.decode_context_lengths(fcfg.batch, fcfg.ctx_min, fcfg.ctx_max, fcfg.seed)
        finp = inputs.decode_inputs(fctx, fcfg.n_q_heads, fcfg.n_kv_heads, fcfg.head_dim, fcfg.seed, dev,
                                    kv_format="fp8", k_scale=FP8_SCALE, v_scale=FP8_SCALE)
        fws = afa.decode_workspace(finp.q, finp.k_cache, finp.block_table, fcfg.num_splits)
        fo = torch.empty_like(finp.q)
        flse = torch.empty(finp.q.shape[:2], dtype=torch.float32, device=dev)
        extra_in["decode_b64_fp8"] = (fcfg, finp, fws, fo, flse)
    if pf_in is not None:
        q, k, v = pf_in
        pf_o = torch.empty_like(q)
        pf_lse = torch.empty((pf_cfg.batch, pf_cfg.n_q_heads, pf_cfg.seqlen), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def run_prefill():
        afa.prefill(q, k, v, causal=True, scale=pf_cfg.scale, out=pf_o, lse_out=pf_lse)

    def run_decode(name):
        cfg, inp, ws, o, lse = dec[name]
        afa.decode_paged(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.ctx_lens,
                         num_splits=cfg.num_splits, scale=cfg.scale, out=o, lse_out=lse, workspace=ws)

    runners = []
    if "copy" in parts:
        copy_src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
        copy_dst = torch.empty_like(copy_src)
        runners.append(("copy", lambda: copy_dst.copy_(copy_src)))
    if pf_in is not None:
        runners.append(("prefill", run_prefill))
    for name in dec:
        runners.append((name, lambda n=name: run_decode(n)))

    def run_chunked():
        cp, cinp, cq, co, clse = extra_in["chunked_prefill"]
        afa.prefill_paged(cq, cinp.k_cache, cinp.v_cache, cinp.block_table, cinp.ctx_lens, causal=True,
                          scale=cp.scale, out=co, lse_out=clse)

    def run_multi(name="decode_multi"):
        mcfg, minp, mq, mws, mo, mlse = extra_in[name]
        afa.decode_paged_multi(mq, minp.k_cache, minp.v_cache, minp.block_table, minp.ctx_lens,
                               num_splits=0, scale=mcfg.scale, out=mo, lse_out=mlse,
                               workspace=mws)

    def run_fp8():
        fcfg, finp, fws, fo, flse = extra_in["decode_b64_fp8"]
        afa.decode_paged_fp8(finp.q, finp.k_cache, finp.v_cache, finp.block_table, finp.ctx_lens,
                             FP8_SCALE, FP8_SCALE, num_splits=fcfg.num_splits, scale=fcfg.scale, out=fo,
                             lse_out=flse, workspace=fws)

    def run_prefill_2k():
        p2, q2, k2, v2, o2, l2 = extra_in["prefill_2k"]
        afa.prefill(q2, k2, v2, causal=True, scale=p2.scale, out=o2, lse_out=l2)

    extra_runners = []
    if "prefill_2k" in extra_in:
        extra_runners.append(("prefill_2k", run_prefill_2k))
    if "decode_b64_fp8" in extra_in:
        extra_runners.append(("decode_b64_fp8", run_fp8))
    if "chunked_prefill" in extra_in:
        extra_runners.append(("chunked_prefill", run_chunked))
    if "decode_multi" in extra_in:
        extra_runners.append(("decode_multi", run_multi))
    if "decode_multi_128k" in extra_in:
        extra_runners.append(("decode_multi_128k", lambda: run_multi("decode_multi_128k")))

    for _ in range(args.warmup):
        for _, fn in runners + extra_runners:
            fn()
    torch.cuda.synchronize()

    # ---- timed region: events around every part of every step ----------
    stream = torch.cuda.current_stream(dev)
    ev = {name: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(args.steps)] for name, _ in runners}
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for s in range(args.steps):
        for name, fn in runners:
            a, b = ev[name][s]
            a.record(stream)
            fn()
            b.record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps

    part_stats = {name: stats([a.elapsed_time(b) for a, b in ev[name]]) for name, _ in runners}
    part_ms = {name: st["ms"] for name, st in part_stats.items()}

    # ---- extras: timed on their own, after the step ----------------------
    extras = {}
    for name, fn in extra_runners:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for a_ev, b_ev in evs:
            a_ev.record(stream)
            fn()
            b_ev.record(stream)
        torch.cuda.synchronize()
        st = stats([a_ev.elapsed_time(b_ev) for a_ev, b_ev in evs])
        ms = st["ms"]
        if name == "prefill_2k":
            p2 = extra_in[name][0]
            tf = p2.flops() / (ms * 1e-3) / 1e12
            extras[name] = {"workload": p2.name, **st, "tflops": tf,
                            "frac_of_peak": tf * 1e12 / PEAK_BF16_FLOPS, "flops": p2.flops(),
                            "tflops_at_median": p2.flops() / (st["ms_median"] * 1e-3) / 1e12}
        elif name == "chunked_prefill":
            cp = extra_in[name][0]
            tf = cp.flops() / (ms * 1e-3) / 1e12
            extras[name] = {"workload": cp.name, **st, "tflops": tf,
                            "frac_of_peak": tf * 1e12 / PEAK_BF16_FLOPS, "flops": cp.flops()}
        elif name == "decode_b64_fp8":
            fcfg, finp = extra_in[name][:2]
            B, Hq, D = finp.q.shape
            used_blocks = sum((c + 15) // 16 for c in finp.ctx)
            nb = (inputs.decode_kv_bytes(finp.ctx, finp.n_kv_heads, D, elem_bytes=1) + 2 * B * Hq * D * 2
                  + used_blocks * 4 + B * 4)
            gbps = nb / (ms * 1e-3) / 1e9
            extras[name] = {"workload": fcfg.name.replace("bf16", "fp8kv"), **st, "gbps": gbps,
                            "frac_of_peak": gbps * 1e9 / PEAK_HBM_BPS, "bytes": nb,
                            "num_splits": fcfg.num_splits, "kv_format": "e4m3, per-tensor scale"}
        elif name in ("decode_multi", "decode_multi_128k"):
            mcfg, minp, mq, mws = extra_in[name][:4]
            tq = mq.shape[1]
            nb = decode_bytes(minp, mcfg.n_q_heads) + 2 * (tq - 1) * mq[:, 0].numel() * 2
            gbps = nb / (ms * 1e-3) / 1e9
            # the library's split count, read back from its workspace size (fp32 partial
            # outputs and log-sum-exps per (sequence, token, query head, split), 256-byte aligned)
            splits = mws.numel() // (mq.shape[0] * mq.shape[1] * mq.shape[2] * (mq.shape[3] + 1) * 4)
            extras[name] = {"workload": f"{mcfg.name}_T{tq}", **st, "gbps": gbps,
                            "frac_of_peak": gbps * 1e9 / PEAK_HBM_BPS, "bytes": nb,
                            "num_splits": int(splits)}
    out_parts = {}
    sol_ms = 0.0
    if pf_in is not None:
        fl = pf_cfg.flops()
        tf = fl / (part_ms["prefill"] * 1e-3) / 1e12
        sol_ms += fl / PEAK_BF16_FLOPS * 1e3
        out_parts["prefill"] = {"workload": pf_cfg.name, **part_stats["prefill"], "tflops": tf,
                                "frac_of_peak": tf * 1e12 / PEAK_BF16_FLOPS, "flops": fl,
                                "tflops_at_median": fl / (part_stats["prefill"]["ms_median"] * 1e-3) / 1e12}
    for name, (cfg, inp, ws, o, lse) in dec.items():
        nb = decode_bytes(inp, cfg.n_q_heads)
        gbps = nb / (part_ms[name] * 1e-3) / 1e9
        sol_ms += nb / PEAK_HBM_BPS * 1e3
        out_parts[name] = {"workload": cfg.name, **part_stats[name], "gbps": gbps,
                           "frac_of_peak": gbps * 1e9 / PEAK_HBM_BPS, "bytes": nb,
                           "num_splits": cfg.num_splits, "sum_ctx": sum(inp.ctx)}
    if "copy" in part_ms:
        out_parts["copy"] = {"workload": f"device copy of {COPY_BYTES} B", "ms": part_ms["copy"],
                             "gbps": 2 * COPY_BYTES / (part_ms["copy"] * 1e-3) / 1e9}
    path_ms = ms_per_step - part_ms.get("copy", 0.0)
    value = 100.0 * sol_ms / path_ms if sol_ms > 0 and path_ms > 0 else None

    roofline = None
    if pf_in is not None:
        digest = source_digest(KERNEL_SOURCES["prefill"])
        achieved = out_parts["prefill"]["tflops"]
        roofline = {"bound": "mfma", "kernel": "prefill_bf16_kernel<128, true, false, 4>",
                    "achieved": achieved, "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                    "frac": achieved * 1e12 / PEAK_BF16_FLOPS, "traffic": load_traffic("prefill", digest),
                    "per_launch_flops": pf_cfg.flops(), "avg_launch_ms": part_ms["prefill"],
                    "kernel_digest": digest}
    decode_roofline = {
        name: {"bound": "hbm", "achieved": p["gbps"], "peak": PEAK_HBM_BPS / 1e9, "unit": "GB/s",
               "frac": p["frac_of_peak"], "per_launch_bytes": p["bytes"], "avg_launch_ms": p["ms"],
               "traffic": load_traffic(name),
               "note": "split + combine kernels of one attn_decode_paged call"}
        for name, p in out_parts.items() if name.startswith("decode")}

    cpu = None
    if not args.no_cpu_baseline:
        dec_parts = {name: (inp, cfg.n_q_heads, cfg.scale, out_parts[name]["bytes"])
                     for name, (cfg, inp, ws, o, lse) in dec.items()}
        cpu = cpu_baseline(parts, pf_cfg, pf_in, dec_parts)

    for name, rec in extras.items():
        rec["traffic"] = load_traffic(name)
    workload = " + ".join(out_parts[p]["workload"] for p in out_parts if p != "copy")
    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "% of peak (step speed-of-light time / measured step time)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded iid N(0,1), bf16; shuffled paged KV cache)",
        "config": {"workload": workload, "parts": list(out_parts)},
        "parts": out_parts,
        "roofline": roofline,
        "roofline_decode": decode_roofline,
        "extras": extras,
        "cpu_baseline": cpu,
        "wall_s_timed_region": wall,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
