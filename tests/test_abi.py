"""The C-ABI library on the host (no GPU, no compute calls).

Checks that libattn.so loads, exports every function include/attn.h declares,
and rejects bad arguments with the documented status codes.  Rejected calls
return before any HIP call, so the device pointers here are fake values that
are never dereferenced.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

from attention_flash_fwd_amd import _lib  # noqa: E402

OK, NULL, ALIGN, SHAPE, DTYPE, UNSUP, WORKSPACE = 0, 1, 2, 3, 4, 5, 6
FAKE = 0x10000          # 64 KiB: 16-byte aligned, never dereferenced
FAKE_MIS = 0x10008      # 8-byte aligned only
BF16, F32 = 0, 1


def header_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libattn.so is not built (run __graft_entry__.build())")
    return _lib.load()


def test_header_declares_the_boundary():
    fns = header_functions()
    for name in ("attn_prefill", "attn_prefill_paged", "attn_decode_paged", "attn_decode_workspace_bytes",
                 "attn_decode_num_splits", "attn_status_string", "attn_abi_version"):
        assert name in fns
    assert set(fns) == set(_lib.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_exports_are_c_symbols():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in header_functions():
        assert name in syms, f"{name} not exported with C linkage"


def test_abi_version_and_status_strings(lib):
    assert lib.attn_abi_version() == (1 << 16) | 5
    for code in range(8):
        s = lib.attn_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.attn_status_string(99).decode() == "unknown status"


def prefill(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, Sq=8, Sk=8, Hq=4, Hkv=2, D=128,
            causal=1, scale=0.1, dtype=BF16):
    P = ctypes.c_void_p
    return lib.attn_prefill(P(q), P(k), P(v), P(o), P(lse), B, Sq, Sk, Hq, Hkv, D, causal,
                            scale, dtype, P(0))


def test_prefill_validation(lib):
    assert prefill(lib, dtype=7) == DTYPE
    assert prefill(lib, D=96) == UNSUP
    assert prefill(lib, D=256) == UNSUP
    assert prefill(lib, Hq=6, Hkv=4) == SHAPE
    assert prefill(lib, Hkv=0) == SHAPE
    assert prefill(lib, B=-1) == SHAPE
    assert prefill(lib, Sq=-3) == SHAPE
    assert prefill(lib, Sk=-1) == SHAPE
    assert prefill(lib, B=1 << 10, Sq=1 << 14, Hq=1 << 4) == SHAPE    # 2^31 elements
    assert prefill(lib, q=0) == NULL
    assert prefill(lib, o=0) == NULL
    assert prefill(lib, k=0) == NULL
    assert prefill(lib, v=0) == NULL
    assert prefill(lib, q=FAKE_MIS) == ALIGN
    assert prefill(lib, o=FAKE_MIS) == ALIGN
    assert prefill(lib, v=FAKE_MIS) == ALIGN
    assert prefill(lib, lse=FAKE + 2) == ALIGN
    # Empty problems are no-ops that need no pointers at all.
    assert prefill(lib, q=0, k=0, v=0, o=0, lse=0, B=0) == OK
    assert prefill(lib, q=0, k=0, v=0, o=0, lse=0, Sq=0) == OK


def decode(lib, q=FAKE, kc=FAKE, vc=FAKE, tbl=FAKE, ctx=FAKE, o=FAKE, lse=FAKE, B=2, Hq=8, Hkv=2,
           D=128, nblocks=10, bs=16, max_blocks=5, splits=4, scale=0.1, ws=FAKE, ws_bytes=None):
    P = ctypes.c_void_p
    if ws_bytes is None:
        ws_bytes = lib.attn_decode_workspace_bytes(B, Hq, Hkv, D, max_blocks, bs, splits)
    return lib.attn_decode_paged(P(q), P(kc), P(vc), P(tbl), P(ctx), P(o), P(lse), B, Hq, Hkv, D,
                                 nblocks, bs, max_blocks, splits, scale, P(ws), ws_bytes, P(0))


def test_decode_validation(lib):
    assert decode(lib, D=80) == UNSUP
    assert decode(lib, bs=32) == UNSUP
    assert decode(lib, Hq=514, Hkv=2) == UNSUP       # 257 query heads per KV head (> 256 columns)
    assert decode(lib, splits=257) == UNSUP
    assert decode(lib, Hq=6, Hkv=4) == SHAPE
    assert decode(lib, B=-1) == SHAPE
    assert decode(lib, nblocks=-1) == SHAPE
    assert decode(lib, q=0) == NULL
    assert decode(lib, tbl=0) == NULL
    assert decode(lib, ctx=0) == NULL
    assert decode(lib, kc=0) == NULL
    assert decode(lib, o=0) == NULL
    assert decode(lib, q=FAKE_MIS) == ALIGN
    assert decode(lib, kc=FAKE_MIS) == ALIGN
    assert decode(lib, tbl=FAKE + 2) == ALIGN
    assert decode(lib, ws=0) == WORKSPACE
    need = lib.attn_decode_workspace_bytes(2, 8, 2, 128, 5, 16, 4)
    assert decode(lib, ws_bytes=need - 1) == WORKSPACE
    assert decode(lib, B=0, q=0, o=0, tbl=0, ctx=0) == OK


def prefill_paged(lib, q=FAKE, kc=FAKE, vc=FAKE, tbl=FAKE, ctx=FAKE, o=FAKE, lse=FAKE, B=2, Sq=8,
                  Hq=8, Hkv=2, D=128, nblocks=10, bs=16, max_blocks=5, causal=1, scale=0.1):
    P = ctypes.c_void_p
    return lib.attn_prefill_paged(P(q), P(kc), P(vc), P(tbl), P(ctx), P(o), P(lse), B, Sq, Hq, Hkv, D,
                                  nblocks, bs, max_blocks, causal, scale, P(0))


def test_prefill_paged_validation(lib):
    assert prefill_paged(lib, D=96) == UNSUP
    assert prefill_paged(lib, bs=32) == UNSUP
    assert prefill_paged(lib, Hq=6, Hkv=4) == SHAPE
    assert prefill_paged(lib, B=-1) == SHAPE
    assert prefill_paged(lib, Sq=-1) == SHAPE
    assert prefill_paged(lib, nblocks=-1) == SHAPE
    assert prefill_paged(lib, Hkv=1 << 20, Hq=1 << 20) == SHAPE     # a block past 2^31 bytes
    assert prefill_paged(lib, q=0) == NULL
    assert prefill_paged(lib, tbl=0) == NULL
    assert prefill_paged(lib, ctx=0) == NULL
    assert prefill_paged(lib, vc=0) == NULL
    assert prefill_paged(lib, o=0) == NULL
    assert prefill_paged(lib, q=FAKE_MIS) == ALIGN
    assert prefill_paged(lib, vc=FAKE_MIS) == ALIGN
    assert prefill_paged(lib, ctx=FAKE + 2) == ALIGN
    assert prefill_paged(lib, lse=FAKE + 2) == ALIGN
    assert prefill_paged(lib, B=0, q=0, o=0, tbl=0, ctx=0) == OK
    assert prefill_paged(lib, Sq=0, q=0, o=0, tbl=0, ctx=0) == OK


def decode_multi(lib, T=2, q=FAKE, ws=FAKE, B=2, Hq=8, Hkv=2, D=128, max_blocks=5, splits=4, ws_bytes=None,
                 **kw):
    P = ctypes.c_void_p
    if ws_bytes is None:
        ws_bytes = lib.attn_decode_multi_workspace_bytes(B, T, Hq, Hkv, D, max_blocks, 16, splits)
    return lib.attn_decode_paged_multi(P(q), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), B, T,
                                       Hq, Hkv, D, 10, 16, max_blocks, splits, 0.1, P(ws), ws_bytes, P(0))


def test_decode_multi_validation(lib):
    assert decode_multi(lib, T=0) == SHAPE
    assert decode_multi(lib, T=65, Hq=8, Hkv=2) == UNSUP    # 4 heads x 65 tokens > 256 columns
    assert decode_multi(lib, T=17, Hq=16, Hkv=1) == UNSUP
    assert decode_multi(lib, T=4, q=FAKE_MIS) == ALIGN
    assert decode_multi(lib, T=4, ws=0) == WORKSPACE
    need = lib.attn_decode_multi_workspace_bytes(2, 4, 8, 2, 128, 5, 16, 4)
    assert decode_multi(lib, T=4, ws_bytes=need - 1) == WORKSPACE
    # The workspace holds one partial per (sequence, token, head, split).
    assert need >= 2 * 4 * 8 * 4 * 129 * 4
    assert lib.attn_decode_multi_workspace_bytes(2, 1, 8, 2, 128, 5, 16, 4) == \
        lib.attn_decode_workspace_bytes(2, 8, 2, 128, 5, 16, 4)
    assert lib.attn_decode_multi_workspace_bytes(2, 0, 8, 2, 128, 5, 16, 4) == 0


def decode_fp8(lib, ks=0.05, vs=0.05, T=1, q=FAKE, ws=FAKE, B=2, Hq=8, Hkv=2, D=128, max_blocks=5, splits=4):
    P = ctypes.c_void_p
    ws_bytes = lib.attn_decode_multi_workspace_bytes(B, T, Hq, Hkv, D, max_blocks, 16, splits)
    return lib.attn_decode_paged_fp8(P(q), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), B, T, Hq,
                                     Hkv, D, 10, 16, max_blocks, splits, 0.1, ks, vs, P(ws), ws_bytes, P(0))


def test_decode_fp8_validation(lib):
    assert decode_fp8(lib, ks=float("nan")) == SHAPE
    assert decode_fp8(lib, vs=float("inf")) == SHAPE
    assert decode_fp8(lib, D=96) == UNSUP
    assert decode_fp8(lib, T=65) == UNSUP
    assert decode_fp8(lib, q=FAKE_MIS) == ALIGN
    assert decode_fp8(lib, ws=0) == WORKSPACE
    assert decode_fp8(lib, B=0, q=0) == OK


def test_decode_item_count_limit(lib):
    # 2^20 sequences x 8 KV heads x 256 chunks = 2^31 split-kernel items:
    # rejected before any launch (the element counts alone are in range).
    assert decode_multi(lib, T=1, B=1 << 20, Hq=8, Hkv=8, D=64, max_blocks=1, splits=256) == SHAPE
    assert decode_multi(lib, T=1, B=(1 << 20) - 1, Hq=8, Hkv=8, D=64, max_blocks=1, splits=256,
                        ws=0) == WORKSPACE


def test_workspace_and_split_rules(lib):
    # Explicit split counts pass through; the workspace holds fp32 partial
    # outputs and log-sum-exps for every (sequence, query head, split), then
    # 256 bytes for the split kernel's work counter.
    for B, Hq, Hkv, D, mb, S in [(64, 32, 8, 128, 2048, 16), (4, 64, 8, 128, 8192, 64),
                                 (1, 1, 1, 64, 1, 1)]:
        assert lib.attn_decode_num_splits(B, Hkv, mb, 16, S) == S
        nbytes = lib.attn_decode_workspace_bytes(B, Hq, Hkv, D, mb, 16, S)
        assert nbytes >= B * Hq * S * (D + 1) * 4 + 256
        assert nbytes < B * Hq * S * (D + 1) * 4 + 1024
    # Automatic choice: in [1, 256], never chunks shorter than 256 tokens,
    # and enough workgroups to cover the GPU when the context allows it.
    for B, Hkv, mb in [(1, 1, 1), (4, 8, 8192), (64, 8, 2048), (1, 8, 64), (256, 8, 4)]:
        s = lib.attn_decode_num_splits(B, Hkv, mb, 16, 0)
        assert 1 <= s <= 256
        assert s <= max(1, (mb * 16 + 255) // 256)
        if (mb * 16) // 256 >= 256:
            assert B * Hkv * s >= 256
    # The library's choice on the two decode workloads and on shapes where
    # one chunk per sequence already gives one item per compute unit.
    for (B, Hkv, mb), want in [((64, 8, 2048), 16), ((4, 8, 8192), 64), ((32, 8, 64), 1),
                               ((128, 8, 32), 1), ((8, 8, 256), 4), ((1, 8, 1024), 32),
                               # up to 2048 tokens, two chunks only to fill the GPU: one
                               # chunk (no merge) instead; not at 4096 tokens
                               ((16, 8, 128), 1), ((16, 8, 64), 1), ((16, 8, 256), 2),
                               # under 1024 tokens: one chunk, however few the sequences
                               ((1, 8, 32), 1), ((16, 8, 63), 1), ((1, 8, 64), 4),
                               # splitting calls whose count at most doubles into two
                               # four-KV-head items per CU of 256 (chunks <= 2048)
                               ((64, 8, 256), 4), ((32, 8, 512), 8),
                               # ... but not by more than doubling, nor from one chunk,
                               # nor with KV heads that are not a multiple of four
                               ((16, 8, 512), 4), ((4, 8, 2048), 16), ((1, 8, 8192), 64),
                               ((8, 8, 256), 4), ((64, 8, 64), 1), ((16, 6, 512), 4)]:
        assert lib.attn_decode_num_splits(B, Hkv, mb, 16, 0) == want, (B, Hkv, mb)
    assert lib.attn_decode_num_splits(-1, 8, 4, 16, 0) == 0
    assert lib.attn_decode_workspace_bytes(1, 0, 1, 128, 4, 16, 1) == 0


def multi_splits(lib, B, T, Hq, Hkv, D, mb, S):
    """Split count of attn_decode_paged_multi, read back from its workspace size."""
    nbytes = lib.attn_decode_multi_workspace_bytes(B, T, Hq, Hkv, D, mb, 16, S)
    per_split = B * T * Hq * (D + 1) * 4
    s = nbytes // per_split
    assert s * per_split <= nbytes < (s + 1) * per_split   # only the 256-byte alignment on top
    return s


def test_multi_token_split_rule(lib):
    # One token: the single-token rule; explicit counts pass through.
    for B, Hq, Hkv, mb in [(64, 32, 8, 2048), (4, 64, 8, 8192)]:
        assert multi_splits(lib, B, 1, Hq, Hkv, 128, mb, 0) == lib.attn_decode_num_splits(B, Hkv, mb, 16, 0)
        assert multi_splits(lib, B, 4, Hq, Hkv, 128, mb, 7) == 7
    # Several tokens: chunks of 2048 * min(4, max(1, C / 4)) tokens of the
    # longest sequence, C = G * T columns, or more chunks up to about 256
    # items (column-tile groups of 4 x 16 columns each count).
    assert multi_splits(lib, 64, 2, 32, 8, 128, 2048, 0) == 8      # C = 8:  chunks of 4096 tokens
    assert multi_splits(lib, 64, 4, 32, 8, 128, 2048, 0) == 4      # C = 16: chunks of 8192 tokens
    assert multi_splits(lib, 64, 8, 32, 8, 128, 2048, 0) == 4      # C = 32: capped at 4 x 2048
    assert multi_splits(lib, 4, 8, 64, 8, 128, 8192, 0) == 16      # C = 64: 131072 / 8192
    assert multi_splits(lib, 32, 4, 32, 8, 128, 64, 0) == 1        # 256 (seq, KV head) pairs already
    assert multi_splits(lib, 8, 4, 32, 8, 128, 256, 0) == 4        # 64 pairs: 256 / 64
    assert multi_splits(lib, 1, 2, 32, 8, 128, 1024, 0) == 32      # 8 pairs: 256 / 8
    assert multi_splits(lib, 1, 2, 8, 8, 64, 4, 0) == 1            # 64 tokens: one chunk of at least 256
    assert multi_splits(lib, 16, 4, 32, 8, 128, 64, 0) == 1        # 1024 tokens: one chunk, not two for fill
    # Past 4096 tokens, from half as many workgroups as compute units on:
    # about four items per compute unit.
    assert multi_splits(lib, 24, 8, 32, 8, 128, 512, 0) == 5       # 192 workgroups: 1024 // 192
    assert multi_splits(lib, 16, 8, 32, 8, 128, 1024, 0) == 8      # 128 workgroups: 1024 / 128
    assert multi_splits(lib, 16, 8, 32, 8, 128, 256, 0) == 1       # 4096 tokens: one chunk, not two
    # More than 32 columns (wide workgroups of 64 or 128 columns): chunks
    # until about two items per compute unit (four from 128 workgroups on),
    # none shorter than 256 tokens or (batch x query heads x tokens) / 16.
    assert multi_splits(lib, 1, 32, 32, 8, 128, 8192, 0) == 64     # 8 workgroups: 512 / 8
    assert multi_splits(lib, 1, 16, 32, 8, 128, 256, 0) == 16      # 4096 tokens in chunks of 256
    assert multi_splits(lib, 4, 32, 32, 8, 128, 256, 0) == 16      # 32 workgroups: 512 / 32
    assert multi_splits(lib, 16, 32, 32, 8, 128, 256, 0) == 4      # chunks of at least 16 * 32 * 32 / 16 = 1024
    assert multi_splits(lib, 32, 32, 32, 8, 128, 256, 0) == 2      # chunks of at least 2048
    assert multi_splits(lib, 16, 16, 32, 8, 128, 1024, 0) == 8     # 128 workgroups: 1024 / 128
    assert multi_splits(lib, 24, 16, 32, 8, 128, 1024, 0) == 5     # 192 workgroups: 1024 // 192
    assert multi_splits(lib, 64, 16, 32, 8, 128, 1024, 0) == 2     # 512 workgroups: two rounds
    assert multi_splits(lib, 64, 64, 32, 8, 128, 1024, 0) == 1     # C = 256: two workgroups per pair
    for B, T, Hq, Hkv, mb in [(1, 3, 4, 1, 1), (2, 16, 16, 1, 300), (8, 5, 64, 8, 9000)]:
        s = multi_splits(lib, B, T, Hq, Hkv, 64, mb, 0)
        assert 1 <= s <= 256
        assert s <= max(1, (mb * 16 + 255) // 256)


def test_binding_rejects_cpu_tensors():
    import torch
    import attention_flash_fwd_amd as afa
    q = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        afa.prefill(q, q[:, :, :1].contiguous(), q[:, :, :1].contiguous())


def test_binding_rejects_wrong_outputs_before_any_launch():
    # A caller-supplied out / lse_out of the wrong shape or dtype would let
    # the kernels write past it (the C ABI only sees a pointer).  The binding
    # refuses it before any device check or library call, so CPU tensors
    # reach these checks here.
    import torch
    import attention_flash_fwd_amd as afa
    bf, f32 = torch.bfloat16, torch.float32
    q = torch.zeros(2, 8, 4, 64, dtype=bf)
    k = torch.zeros(2, 8, 2, 64, dtype=bf)
    bad_prefill = [
        dict(out=torch.zeros(2, 8, 4, 32, dtype=bf)),            # too small
        dict(out=torch.zeros(2, 8, 4, 64, dtype=f32)),           # fp32 out for bf16 q
        dict(lse_out=torch.zeros(2, 8, 4, dtype=f32)),           # [B,Sq,Hq] instead of [B,Hq,Sq]
        dict(lse_out=torch.zeros(2, 4, 8, dtype=bf)),            # lse must be fp32
        dict(out=torch.zeros(2, 4, 8, 64, dtype=bf).transpose(1, 2)),   # not contiguous
    ]
    for kw in bad_prefill:
        with pytest.raises(ValueError, match="out"):
            afa.prefill(q, k, k.clone(), **kw)
    # Paged entry points: q of one token [B,Hq,D] / several [B,T,Hq,D].
    kc = torch.zeros(4, 16, 2, 64, dtype=bf)
    tbl = torch.zeros(2, 2, dtype=torch.int32)
    ctx = torch.zeros(2, dtype=torch.int32)
    q1 = torch.zeros(2, 4, 64, dtype=bf)
    q3 = torch.zeros(2, 3, 4, 64, dtype=bf)
    with pytest.raises(ValueError, match="out"):
        afa.decode_paged(q1, kc, kc.clone(), tbl, ctx, out=torch.zeros(2, 4, 32, dtype=bf))
    with pytest.raises(ValueError, match="lse_out"):
        afa.decode_paged(q1, kc, kc.clone(), tbl, ctx, lse_out=torch.zeros(2, 4, 1, dtype=f32))
    with pytest.raises(ValueError, match="lse_out"):
        afa.decode_paged_multi(q3, kc, kc.clone(), tbl, ctx, lse_out=torch.zeros(2, 3, 4, dtype=f32))
    with pytest.raises(ValueError, match="out"):
        afa.decode_paged_multi(q3, kc, kc.clone(), tbl, ctx, out=torch.zeros(2, 3, 4, 64, dtype=f32))
    with pytest.raises(ValueError, match="out"):
        afa.prefill_paged(q3, kc, kc.clone(), tbl, ctx, out=torch.zeros(2, 3, 4, 63, dtype=bf))
    k8 = torch.zeros(4, 16, 2, 64, dtype=torch.uint8)
    with pytest.raises(ValueError, match="lse_out"):
        afa.decode_paged_fp8(q1, k8, k8.clone(), tbl, ctx, 1.0, 1.0, lse_out=torch.zeros(2, 4, 1, dtype=f32))
    with pytest.raises(ValueError, match="workspace"):
        afa.decode_paged(q1, kc, kc.clone(), tbl, ctx, workspace=torch.zeros(64, dtype=torch.float32))
    # Correct outputs pass these checks and reach the device check.
    with pytest.raises(ValueError, match="GPU only"):
        afa.prefill(q, k, k.clone(), out=torch.empty_like(q), lse_out=torch.zeros(2, 4, 8, dtype=f32))


def test_every_kernel_launch_stub_is_defined():
    # A kernel whose body the host pass cannot compile (for example a device
    # builtin called directly from a lambda) silently loses its launch stub;
    # the library then fails to load with an undefined symbol.
    import subprocess
    out = subprocess.run(["nm", "-u", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    missing = [line for line in out.splitlines() if "__device_stub__" in line]
    assert not missing, missing


def test_bench_refuses_more_than_one_gpu():
    # The benchmark measures one GPU; asking for more exits with a message
    # before anything touches a device.
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=root)
    assert r.returncode != 0
    assert "exactly one GPU" in r.stderr
    assert r.stdout.strip() == ""
