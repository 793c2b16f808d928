"""Pins for the fp64 CPU oracle (no GPU).

The oracle is the naive definition of attention (S = scale QK^T, P =
softmax(S), O = PV; chenyy20.com "抱infra脚", Flash Attention 基本原理 /
核心技术), which FlashAttention must reproduce exactly ("推理加速" interview
notes, FlashAttention section).  Before the oracle judges anything it is held
to facts that do not come from itself: hand-derived golden fixtures, closed
forms of special cases, a 50-digit brute force on tiny shapes, and invariants
(GQA = repeated-KV MHA, batch permutation, split/merge, decode = last causal
row).  test_oracle_mutations.py shows that these pins catch planted mistakes.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand(shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape) * scale).astype(np.float32)


# ---------------------------------------------------------------- golden ----
def _parse_value(tok: str) -> float:
    if tok == "-inf":
        return -math.inf
    if tok.startswith("ln(") and tok.endswith(")"):
        return math.log(Fraction(tok[3:-1]))
    return float(Fraction(tok))


def load_golden(path):
    items = {}
    with open(path, encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            items[key] = vals
    B, Sq, Sk, Hq, Hkv, D = (int(x) for x in items["shape"])
    g = dict(B=B, Sq=Sq, Sk=Sk, Hq=Hq, Hkv=Hkv, D=D,
             causal=bool(int(items["causal"][0])),
             scale=_parse_value(items["scale"][0]))
    g["q"] = np.array([_parse_value(t) for t in items["q"]], np.float32).reshape(B, Sq, Hq, D)
    g["k"] = np.array([_parse_value(t) for t in items["k"]], np.float32).reshape(B, Sk, Hkv, D)
    g["v"] = np.array([_parse_value(t) for t in items["v"]], np.float32).reshape(B, Sk, Hkv, D)
    g["o"] = np.array([_parse_value(t) for t in items["o"]], np.float64).reshape(B, Sq, Hq, D)
    g["lse"] = np.array([_parse_value(t) for t in items["lse"]], np.float64).reshape(B, Hq, Sq)
    return g


GOLDEN_FILES = sorted(f for f in os.listdir(GOLDEN) if f.endswith(".txt") and f != "README.txt")


@pytest.mark.parametrize("name", GOLDEN_FILES)
def test_golden_fixture(name):
    g = load_golden(os.path.join(GOLDEN, name))
    o, lse = oracle.attention(g["q"], g["k"], g["v"], g["causal"], g["scale"])
    np.testing.assert_allclose(o, g["o"], rtol=0, atol=1e-14)
    fin = np.isfinite(g["lse"])
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.all(lse[~fin] == -np.inf)
    np.testing.assert_allclose(lse[fin], g["lse"][fin], rtol=0, atol=1e-14)


def test_golden_fixtures_present():
    assert len(GOLDEN_FILES) >= 5


# ------------------------------------------------------------ P matrix -----
@pytest.mark.parametrize("causal,Sq,Sk", [(False, 9, 13), (True, 13, 13), (True, 5, 11), (True, 11, 5)])
def test_probs_rows_sum_to_one(causal, Sq, Sk):
    q = rand((2, Sq, 4, 8), 1)
    k = rand((2, Sk, 2, 8), 2)
    S, P = oracle.scores_probs(q, k, causal, 0.35, b=1, hq=3)
    assert np.all(P >= 0)
    for i in range(Sq):
        vis = [j for j in range(Sk) if (not causal) or j <= i + (Sk - Sq)]
        hid = [j for j in range(Sk) if j not in vis]
        assert np.all(P[i, hid] == 0.0)
        assert np.all(np.isneginf(S[i, hid]))
        if vis:
            assert abs(P[i].sum() - 1.0) <= 1e-12
            # P is monotone in S within a row (softmax preserves order).
            order = np.argsort(S[i, vis])
            assert np.all(np.diff(P[i, vis][order]) >= -1e-15)
        else:
            assert P[i].sum() == 0.0


def test_scores_are_scaled_dot_products():
    # S[i, j] for one hand-picked pair, computed term by term in Python.
    q = rand((1, 3, 2, 5), 3)
    k = rand((1, 4, 1, 5), 4)
    S, _ = oracle.scores_probs(q, k, False, 0.7, b=0, hq=1)
    want = 0.7 * math.fsum(float(q[0, 2, 1, d]) * float(k[0, 3, 0, d]) for d in range(5))
    assert abs(S[2, 3] - want) < 1e-15


# ------------------------------------------------------- closed forms ------
@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_gives_constant_output(causal):
    B, S, Hq, Hkv, D = 2, 23, 6, 3, 16
    q = rand((B, S, Hq, D), 5, 3.0)
    k = rand((B, S, Hkv, D), 6, 3.0)
    c = rand((B, 1, Hkv, D), 7)
    v = np.broadcast_to(c, (B, S, Hkv, D)).copy()
    o, _ = oracle.attention(q, k, v, causal, 0.9)
    for h in range(Hq):
        want = np.broadcast_to(c[:, :, h // (Hq // Hkv), :], (B, S, D))
        np.testing.assert_allclose(o[:, :, h, :], want, rtol=0, atol=1e-12)


def test_single_key_returns_its_value():
    q = rand((3, 4, 2, 8), 8)
    k = rand((3, 1, 1, 8), 9)
    v = rand((3, 1, 1, 8), 10)
    o, lse = oracle.attention(q, k, v, False, 0.25)
    for b in range(3):
        for i in range(4):
            for h in range(2):
                np.testing.assert_array_equal(o[b, i, h], v[b, 0, 0].astype(np.float64))
                want = 0.25 * math.fsum(float(x) * float(y) for x, y in zip(q[b, i, h], k[b, 0, 0]))
                assert abs(lse[b, h, i] - want) < 1e-13


def test_causal_row0_is_v0():
    q = rand((2, 17, 4, 32), 11, 4.0)
    k = rand((2, 17, 2, 32), 12, 4.0)
    v = rand((2, 17, 2, 32), 13)
    o, lse = oracle.attention(q, k, v, True, 1 / math.sqrt(32))
    for b in range(2):
        for h in range(4):
            np.testing.assert_array_equal(o[b, 0, h], v[b, 0, h // 2].astype(np.float64))
            want = math.fsum(float(x) * float(y) for x, y in zip(q[b, 0, h], k[b, 0, h // 2]))
            assert abs(lse[b, h, 0] - want / math.sqrt(32)) < 1e-12


@pytest.mark.parametrize("Sq,Sk", [(12, 12), (5, 12), (12, 5)])
def test_scale_zero_is_mean_of_visible_values(Sq, Sk):
    q = rand((1, Sq, 2, 8), 14)
    k = rand((1, Sk, 1, 8), 15)
    v = rand((1, Sk, 1, 8), 16)
    o, lse = oracle.attention(q, k, v, True, 0.0)
    for i in range(Sq):
        n = min(Sk, max(0, i + (Sk - Sq) + 1))   # keys 0 .. i + Sk - Sq
        for h in range(2):
            if n == 0:
                assert np.all(o[0, i, h] == 0) and lse[0, h, i] == -np.inf
                continue
            want = v[0, :n, 0].astype(np.float64).mean(axis=0)
            np.testing.assert_allclose(o[0, i, h], want, rtol=0, atol=1e-14)
            assert abs(lse[0, h, i] - math.log(n)) < 1e-14


# ------------------------------------------------ brute force (mpmath) -----
def _brute_force(q, k, v, causal, scale, digits=50):
    import mpmath
    mpmath.mp.dps = digits
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    o = np.zeros((B, Sq, Hq, D))
    lse = np.zeros((B, Hq, Sq))
    sc = mpmath.mpf(scale)
    for b in range(B):
        for h in range(Hq):
            for i in range(Sq):
                w = []
                for j in range(Sk):
                    if causal and j > i + (Sk - Sq):
                        continue
                    s = sc * mpmath.fsum(mpmath.mpf(float(q[b, i, h, d])) * mpmath.mpf(float(k[b, j, h // G, d]))
                                         for d in range(D))
                    w.append((j, mpmath.exp(s)))       # no max shift: exact arithmetic
                if not w:
                    lse[b, h, i] = -np.inf
                    continue
                tot = mpmath.fsum(e for _, e in w)
                lse[b, h, i] = float(mpmath.log(tot))
                for d in range(D):
                    o[b, i, h, d] = float(mpmath.fsum(e * mpmath.mpf(float(v[b, j, h // G, d])) for j, e in w) / tot)
    return o, lse


@pytest.mark.parametrize("Hq,S,D,causal", [(1, 1, 1, False), (1, 2, 4, True), (2, 3, 8, True),
                                           (2, 5, 4, False), (1, 8, 8, True), (2, 8, 1, False)])
def test_brute_force_mpmath(Hq, S, D, causal):
    q = rand((1, S, Hq, D), 100 + S, 2.0)
    k = rand((1, S, 1, D), 200 + S, 2.0)
    v = rand((1, S, 1, D), 300 + S)
    scale = 1 / math.sqrt(D)
    o, lse = oracle.attention(q, k, v, causal, scale)
    ob, lb = _brute_force(q, k, v, causal, scale)
    np.testing.assert_allclose(o, ob, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, lb, rtol=1e-13, atol=1e-14)


# ------------------------------------------------------- invariants --------
def test_gqa_equals_mha_with_repeated_kv():
    B, S, Hq, Hkv, D = 2, 19, 8, 2, 16
    q = rand((B, S, Hq, D), 20)
    k = rand((B, S, Hkv, D), 21)
    v = rand((B, S, Hkv, D), 22)
    o_gqa, l_gqa = oracle.attention(q, k, v, True, 0.3)
    k_rep = np.repeat(k, Hq // Hkv, axis=2)   # consecutive query heads share a KV head
    v_rep = np.repeat(v, Hq // Hkv, axis=2)
    o_mha, l_mha = oracle.attention(q, k_rep, v_rep, True, 0.3)
    np.testing.assert_array_equal(o_gqa, o_mha)
    np.testing.assert_array_equal(l_gqa, l_mha)


def test_batch_permutation_equivariance():
    B, S, Hq, Hkv, D = 4, 11, 4, 4, 8
    q, k, v = rand((B, S, Hq, D), 23), rand((B, S, Hkv, D), 24), rand((B, S, Hkv, D), 25)
    perm = [2, 0, 3, 1]
    o, l = oracle.attention(q, k, v, True, 0.5)
    op, lp = oracle.attention(q[perm], k[perm], v[perm], True, 0.5)
    np.testing.assert_array_equal(op, o[perm])
    np.testing.assert_array_equal(lp, l[perm])


def test_head_permutation_within_group_equivariance():
    # Query heads of one group see the same K/V: swapping two of them swaps outputs.
    B, S, Hq, Hkv, D = 1, 9, 4, 2, 8
    q, k, v = rand((B, S, Hq, D), 26), rand((B, S, Hkv, D), 27), rand((B, S, Hkv, D), 28)
    o, _ = oracle.attention(q, k, v, True, 0.5)
    q2 = q[:, :, [1, 0, 3, 2]]
    o2, _ = oracle.attention(q2, k, v, True, 0.5)
    np.testing.assert_array_equal(o2, o[:, :, [1, 0, 3, 2]])


def test_key_order_invariance_noncausal():
    # Without a mask attention is a set function of the (key, value) pairs.
    q, k, v = rand((1, 7, 2, 8), 29), rand((1, 13, 1, 8), 30), rand((1, 13, 1, 8), 31)
    perm = np.random.default_rng(0).permutation(13)
    o, l = oracle.attention(q, k, v, False, 0.4)
    o2, l2 = oracle.attention(q, k[:, perm], v[:, perm], False, 0.4)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l2, l, rtol=0, atol=1e-14)


@pytest.mark.parametrize("mult", [16.0, 1000.0])
def test_large_logits_stay_finite(mult):
    q = rand((1, 16, 1, 64), 32, mult)
    k = rand((1, 16, 1, 64), 33)
    v = rand((1, 16, 1, 64), 34)
    o, lse = oracle.attention(q, k, v, False, 1 / 8)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    if mult >= 1000:
        # O is within sum_{j != top} e^{-(S_top - S_j)} * max|v_j - v_top| of the
        # top key's value: the bound shrinks to nothing as the logits spread.
        S, _ = oracle.scores_probs(q, k, False, 1 / 8, 0, 0)
        for i in range(16):
            top = int(np.argmax(S[i]))
            gaps = S[i, top] - np.delete(S[i], top)
            spread = np.abs(np.delete(v[0, :, 0], top, axis=0) - v[0, top, 0]).max()
            bound = np.exp(-gaps).sum() * spread + 1e-12
            assert np.abs(o[0, i, 0] - v[0, top, 0]).max() <= bound
            assert lse[0, 0, i] >= S[i, top] and lse[0, 0, i] <= S[i, top] + np.log(16)


def test_rows_variant_matches_full():
    q, k, v = rand((2, 33, 4, 16), 35), rand((2, 33, 2, 16), 36), rand((2, 33, 2, 16), 37)
    o, l = oracle.attention(q, k, v, True, 0.25)
    rows = [(0, 0, 0), (1, 3, 32), (0, 2, 17), (1, 1, 5)]
    orow, lrow = oracle.attention_rows(q, k, v, True, 0.25, rows)
    for r, (b, h, i) in enumerate(rows):
        np.testing.assert_array_equal(orow[r], o[b, i, h])
        assert lrow[r] == l[b, h, i]


def test_empty_inputs():
    q = np.zeros((0, 5, 2, 8), np.float32)
    k = np.zeros((0, 5, 1, 8), np.float32)
    o, l = oracle.attention(q, k, k, True, 1.0)
    assert o.shape == (0, 5, 2, 8) and l.shape == (0, 2, 5)
    q = rand((1, 3, 1, 4), 38)
    k = np.zeros((1, 0, 1, 4), np.float32)
    o, l = oracle.attention(q, k, k, False, 1.0)
    assert np.all(o == 0) and np.all(l == -np.inf)


# --------------------------------------------------- split / merge ---------
@pytest.mark.parametrize("nsplit", [1, 2, 3, 7, 64])
def test_split_merge_identity(nsplit):
    # Attention over all keys equals the LSE merge of attention over disjoint
    # key chunks; chunks may be empty (the page's Flash-Decoding partials).
    Sk, D = 50, 16
    q = rand((1, 1, 1, D), 40, 2.0)
    k = rand((1, Sk, 1, D), 41, 2.0)
    v = rand((1, Sk, 1, D), 42)
    o_full, l_full = oracle.attention(q, k, v, False, 0.3)
    edges = np.linspace(0, Sk, nsplit + 1).round().astype(int)
    if nsplit == 64:
        edges = np.minimum(np.arange(nsplit + 1), Sk)   # many empty chunks at the end
    parts_o, parts_l = [], []
    for s in range(nsplit):
        a, b = edges[s], edges[s + 1]
        op, lp = oracle.attention(q, k[:, a:b], v[:, a:b], False, 0.3)
        parts_o.append(op[0, 0, 0])
        parts_l.append(lp[0, 0, 0])
    o, l = oracle.lse_combine(np.array(parts_o), np.array(parts_l))
    np.testing.assert_allclose(o, o_full[0, 0, 0], rtol=0, atol=1e-12)
    assert abs(l - l_full[0, 0, 0]) < 1e-12


def test_combine_all_empty():
    o, l = oracle.lse_combine(np.zeros((3, 4)), np.full(3, -np.inf))
    assert np.all(o == 0) and l == -np.inf


# ----------------------------------------------------------- decode --------
def test_decode_is_last_row_of_causal_prefill():
    Hq, Hkv, D = 8, 2, 16
    ctx = [1, 7, 30]
    q_dec = rand((3, Hq, D), 50)
    ks = [rand((n, Hkv, D), 60 + n) for n in ctx]
    vs = [rand((n, Hkv, D), 70 + n) for n in ctx]
    o, lse = oracle.decode(q_dec, ks, vs, 0.2)
    for b, n in enumerate(ctx):
        qp = rand((1, n, Hq, D), 80 + n)
        qp[0, n - 1] = q_dec[b]
        op, lp = oracle.attention(qp, ks[b][None], vs[b][None], True, 0.2)
        np.testing.assert_array_equal(o[b], op[0, n - 1])
        np.testing.assert_array_equal(lse[b], lp[0, :, n - 1])


def test_decode_zero_context():
    q = rand((2, 4, 8), 51)
    ks = [np.zeros((0, 2, 8), np.float32), rand((3, 2, 8), 52)]
    vs = [np.zeros((0, 2, 8), np.float32), rand((3, 2, 8), 53)]
    o, lse = oracle.decode(q, ks, vs, 0.5)
    assert np.all(o[0] == 0) and np.all(lse[0] == -np.inf)
    assert np.all(np.isfinite(lse[1]))


# ------------------------------------------------------------ fp8 (e4m3) ---
def test_e4m3_decode_matches_library_conversion():
    # All 256 codes against torch's float8_e4m3fn -> float32 conversion.
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = oracle.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_e4m3_decode_hand_values():
    vals = {0x38: 1.0, 0xB8: -1.0, 0x3C: 1.5, 0x7E: 448.0, 0xFE: -448.0, 0x01: 2.0 ** -9,
            0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x00: 0.0, 0x40: 2.0, 0x30: 0.5, 0x28: 0.25}
    got = oracle.e4m3_decode(np.array(list(vals), np.uint8))
    assert list(got) == list(vals.values())
    assert np.isnan(oracle.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()
    assert np.signbit(oracle.e4m3_decode(np.array([0x80], np.uint8))[0])


def _fp8_case(seed, ctx=(37, 5), Hq=4, Hkv=2, D=8):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((len(ctx), Hq, D)).astype(np.float32)
    # finite codes only (exclude the NaN codes 0x7F / 0xFF)
    kc = [rng.integers(0, 0x7F, size=(c, Hkv, D), dtype=np.uint8) | (rng.integers(0, 2, size=(c, Hkv, D), dtype=np.uint8) << 7)
          for c in ctx]
    vc = [rng.integers(0, 0x7F, size=(c, Hkv, D), dtype=np.uint8) for c in ctx]
    return q, kc, vc


def test_decode_fp8_equals_decode_of_dequantised_cache():
    # With power-of-two scales, code * scale is exact in fp32, so dequantising
    # first and running the plain decode must give the same numbers.
    q, kc, vc = _fp8_case(1)
    ks, vs, scale = 2.0 ** -5, 2.0 ** -3, 0.3
    o, l = oracle.decode_fp8(q, kc, vc, scale, ks, vs)
    kd = [(oracle.e4m3_decode(k) * ks).astype(np.float32) for k in kc]
    vd = [(oracle.e4m3_decode(v) * vs).astype(np.float32) for v in vc]
    o2, l2 = oracle.decode(q, kd, vd, scale)
    assert np.allclose(o, o2, rtol=1e-12, atol=1e-14) and np.allclose(l, l2, rtol=1e-12, atol=1e-12)


def test_decode_fp8_scale_roles():
    q, kc, vc = _fp8_case(2)
    o, l = oracle.decode_fp8(q, kc, vc, 0.25, 0.5, 1.0)
    o2, l2 = oracle.decode_fp8(q, kc, vc, 0.5, 0.25, 3.0)     # same score scale, V scaled by 3
    assert np.allclose(o2, 3.0 * o, rtol=1e-12) and np.allclose(l2, l, rtol=1e-12)
    o3, _ = oracle.decode_fp8(q, kc, vc, 0.25, 1.0, 1.0)      # different score scale
    assert not np.allclose(o3, o)
