"""fp64 CPU oracle for exact attention forward -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never loads it, and
it shares no code with the HIP path: it is the naive definition of attention
written out in C (``oracle.c``), materialising S = scale * QK^T and P = softmax(S)
before forming O = PV, in double precision.  See ``oracle.h`` for layouts.

Parity status of each function (what pins it, see tests/test_oracle.py):
  attention / attention_rows / scores_probs -- pinned by closed forms
      (constant V, single key, causal row 0, scale 0), by hand-derived golden
      fixtures, by an mpmath brute force at 50 digits and by invariants
      (GQA = repeated-KV MHA, batch permutation, large logits);
  decode -- pinned against the last row of causal prefill and the closed forms;
  lse_combine -- pinned by the split-merge identity against unsplit attention.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (portable -O2, OpenMP, no fast-math)."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def load_library(path: str):
    """Open an oracle shared library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    L = ctypes.c_long
    I = ctypes.c_int
    Dd = ctypes.c_double
    lib.oracle_attention.argtypes = [P, P, P, P, P, L, L, L, L, L, L, I, Dd, I]
    lib.oracle_attention_rows.argtypes = [P, P, P, L, L, L, L, L, L, I, Dd,
                                          P, P, P, L, P, P, I]
    lib.oracle_scores_probs.argtypes = [P, P, L, L, L, L, L, L, I, Dd, L, L, P, P]
    lib.oracle_decode.argtypes = [P, P, P, P, P, L, L, L, L, Dd, P, P, I]
    lib.oracle_lse_combine.argtypes = [P, P, L, L, P, P]
    for fn in (lib.oracle_attention, lib.oracle_attention_rows,
               lib.oracle_scores_probs, lib.oracle_decode, lib.oracle_lse_combine):
        fn.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    _lib = load_library(LIB_PATH)
    return _lib


def _f32(x) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return a


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"{what} failed with code {rc}")


def attention(q, k, v, causal: bool, scale: float, nthreads: int = 0):
    """q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D] -> (o [B,Sq,Hq,D] f64, lse [B,Hq,Sq] f64)."""
    lib = _load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    assert k.shape == (B, Sk, Hkv, D) and v.shape == k.shape
    o = np.zeros((B, Sq, Hq, D), np.float64)
    lse = np.zeros((B, Hq, Sq), np.float64)
    rc = lib.oracle_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                              B, Sq, Sk, Hq, Hkv, D, int(bool(causal)), float(scale),
                              int(nthreads))
    _check(rc, "oracle_attention")
    return o, lse


def attention_rows(q, k, v, causal: bool, scale: float, rows, nthreads: int = 0):
    """Selected rows only.  rows: iterable of (b, hq, i) -> (o [n,D], lse [n])."""
    lib = _load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    rows = np.asarray(list(rows), dtype=np.int64).reshape(-1, 3)
    rb = np.ascontiguousarray(rows[:, 0])
    rh = np.ascontiguousarray(rows[:, 1])
    ri = np.ascontiguousarray(rows[:, 2])
    n = rows.shape[0]
    o = np.zeros((n, D), np.float64)
    lse = np.zeros((n,), np.float64)
    rc = lib.oracle_attention_rows(_ptr(q), _ptr(k), _ptr(v), B, Sq, Sk, Hq, Hkv, D,
                                   int(bool(causal)), float(scale),
                                   _ptr(rb), _ptr(rh), _ptr(ri), n,
                                   _ptr(o), _ptr(lse), int(nthreads))
    _check(rc, "oracle_attention_rows")
    return o, lse


def scores_probs(q, k, causal: bool, scale: float, b: int, hq: int):
    """Materialised S and P ([Sq, Sk] f64) of one (batch, query head)."""
    lib = _load()
    q, k = _f32(q), _f32(k)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    S = np.zeros((Sq, Sk), np.float64)
    P = np.zeros((Sq, Sk), np.float64)
    rc = lib.oracle_scores_probs(_ptr(q), _ptr(k), B, Sq, Sk, Hq, Hkv, D,
                                 int(bool(causal)), float(scale), int(b), int(hq),
                                 _ptr(S), _ptr(P))
    _check(rc, "oracle_scores_probs")
    return S, P


def decode(q, k_seqs, v_seqs, scale: float, nthreads: int = 0):
    """One-token decode on logical per-sequence caches.

    q [B,Hq,D]; k_seqs / v_seqs: list of B arrays [ctx_b, Hkv, D] (or one
    concatenated array plus a ``ctx`` list via decode_concat).
    Returns (o [B,Hq,D] f64, lse [B,Hq] f64)."""
    ctx = [int(np.asarray(kk).shape[0]) for kk in k_seqs]
    Hkv, D = np.asarray(k_seqs[0]).shape[1:]
    k_log = np.concatenate([np.asarray(kk, np.float32).reshape(-1, Hkv, D) for kk in k_seqs], 0)
    v_log = np.concatenate([np.asarray(vv, np.float32).reshape(-1, Hkv, D) for vv in v_seqs], 0)
    return decode_concat(q, k_log, v_log, ctx, scale, nthreads)


def decode_concat(q, k_log, v_log, ctx, scale: float, nthreads: int = 0):
    lib = _load()
    q, k_log, v_log = _f32(q), _f32(k_log), _f32(v_log)
    B, Hq, D = q.shape
    Hkv = k_log.shape[1]
    ctx = np.ascontiguousarray(np.asarray(ctx, dtype=np.int64))
    off = np.zeros(B, np.int64)
    if B > 1:
        off[1:] = np.cumsum(ctx)[:-1]
    assert k_log.shape[0] >= int(ctx.sum()) and v_log.shape == k_log.shape
    o = np.zeros((B, Hq, D), np.float64)
    lse = np.zeros((B, Hq), np.float64)
    rc = lib.oracle_decode(_ptr(q), _ptr(k_log), _ptr(v_log), _ptr(off), _ptr(ctx),
                           B, Hq, Hkv, D, float(scale), _ptr(o), _ptr(lse), int(nthreads))
    _check(rc, "oracle_decode")
    return o, lse


def lse_combine(o_parts, lse_parts):
    """Merge partials o_parts [n, D], lse_parts [n] -> (o [D], lse scalar)."""
    lib = _load()
    op = np.ascontiguousarray(np.asarray(o_parts, np.float64))
    lp = np.ascontiguousarray(np.asarray(lse_parts, np.float64))
    n, D = op.shape
    o = np.zeros((D,), np.float64)
    lse = np.zeros((1,), np.float64)
    rc = lib.oracle_lse_combine(_ptr(op), _ptr(lp), n, D, _ptr(o), _ptr(lse))
    _check(rc, "oracle_lse_combine")
    return o, float(lse[0])


def e4m3_decode(codes):
    """OCP FP8 E4M3 codes (uint8) -> exact float64 values, written from the
    format's definition: sign bit, 4 exponent bits with bias 7, 3 mantissa
    bits; exponent 0 encodes subnormals (m / 8) * 2^-6; exponent 15 with
    mantissa 7 is NaN; there are no infinities.  (The pages fix no 8-bit
    format; this is the reading the library documents for its FP8 KV cache,
    "5.2 推理加速的未来趋势" co-design layer on low-precision KV caches.)"""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    val = sign * val
    return np.where((e == 15) & ((c & 7) == 7), np.nan, val)


def decode_fp8(q, k_codes, v_codes, scale: float, k_scale: float, v_scale: float, nthreads: int = 0):
    """Decode over an e4m3 KV cache with per-tensor scales:
    K = e4m3(k) * k_scale, V = e4m3(v) * v_scale.  The codes decode exactly
    to fp32, k_scale joins the score scale (scale * q . (k * k_scale) =
    (scale * k_scale) * q . k) and v_scale multiplies the output (O is linear
    in V), so no value is rounded before the fp64 arithmetic of `decode`."""
    ks = [e4m3_decode(k).astype(np.float32) for k in k_codes]
    vs = [e4m3_decode(v).astype(np.float32) for v in v_codes]
    o, lse = decode(q, ks, vs, float(scale) * float(k_scale), nthreads)
    return o * float(v_scale), lse
