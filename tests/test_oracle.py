"""Pins of the fp64 oracle against things other than itself: a decimal brute
force of the definition, hand-derived closed forms (tests/golden), invariants
that follow from the definition, the block-merge identity, and the decoders
against torch's own dtypes."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests.brute_decimal import attention_decimal

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def _num(x):
    return -math.inf if x == "-inf" else float(x)


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("Nq,Nk,d,causal", [
    (1, 1, 1, False), (3, 5, 2, False), (5, 5, 3, True), (4, 7, 4, True),
    (7, 3, 2, True), (8, 8, 4, False), (6, 2, 3, False), (2, 8, 1, True),
])
def test_oracle_matches_decimal_brute_force(Nq, Nk, d, causal):
    rng = np.random.default_rng(Nq * 100 + Nk * 10 + d)
    q = rng.standard_normal((1, 1, Nq, d)) * 2
    k = rng.standard_normal((1, 1, Nk, d)) * 2
    v = rng.standard_normal((1, 1, Nk, d))
    scale = 0.8
    o, lse = oracle.attention(q, k, v, causal, scale)
    ob, lb = attention_decimal(q[0, 0], k[0, 0], v[0, 0], causal, scale)
    np.testing.assert_allclose(o[0, 0], ob, rtol=0, atol=1e-12)
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[0, 0][fin], lb[fin], rtol=0, atol=1e-12)
    assert np.all(np.isneginf(lse[0, 0][~fin]))


# -------------------------------------------------------------- closed forms
def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden()["attention"], ids=lambda c: c["name"])
def test_oracle_closed_forms(case):
    q = np.array(case["q"], dtype=np.float64)[None, None]
    k = np.array(case["k"], dtype=np.float64)[None, None]
    v = np.array(case["v"], dtype=np.float64)[None, None]
    o, lse = oracle.attention(q, k, v, case["causal"], case["scale"])
    np.testing.assert_allclose(o[0, 0], np.array(case["o"]), rtol=0, atol=1e-12)
    want = np.array([_num(x) for x in case["lse"]])
    fin = np.isfinite(want)
    np.testing.assert_allclose(lse[0, 0][fin], want[fin], rtol=0, atol=1e-12)
    assert np.all(np.isneginf(lse[0, 0][~fin]))


@pytest.mark.parametrize("case", _golden()["merge"], ids=lambda c: c["name"])
def test_merge_closed_forms(case):
    def st(s):
        return (np.array(s["o"], dtype=np.float64), np.array([_num(x) for x in s["m"]]),
                np.array(s["l"], dtype=np.float64))
    o, m, l = oracle.merge(st(case["a"]), st(case["b"]))
    np.testing.assert_allclose(o, np.array(case["o"]), atol=1e-12)
    np.testing.assert_allclose(m, [_num(x) for x in case["m"]], atol=1e-12)
    np.testing.assert_allclose(l, case["l"], atol=1e-12)
    np.testing.assert_allclose(oracle.state_lse(m, l), [_num(x) for x in case["lse"]], atol=1e-12)


# ---------------------------------------------------------------- invariants
def test_closed_form_two_keys_general():
    # d = 1, two keys: O = sigma(s1 - s2) v1 + sigma(s2 - s1) v2.
    rng = np.random.default_rng(3)
    for _ in range(20):
        qv, k1, k2, v1, v2 = rng.standard_normal(5) * 3
        scale = rng.uniform(0.1, 2.0)
        s1, s2 = scale * qv * k1, scale * qv * k2
        sig = lambda x: 1.0 / (1.0 + math.exp(-x))
        want = sig(s1 - s2) * v1 + sig(s2 - s1) * v2
        o, lse = oracle.attention(np.array([[[[qv]]]]), np.array([[[[k1], [k2]]]]),
                                  np.array([[[[v1], [v2]]]]), False, scale)
        assert abs(o[0, 0, 0, 0] - want) < 1e-12
        assert abs(lse[0, 0, 0] - (max(s1, s2) + math.log1p(math.exp(-abs(s1 - s2))))) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows(causal):
    B, H, Nq, Nk, d = 2, 3, 37, 41, 16
    q, k, v = _rand((B, H, Nq, d), 1), _rand((B, H, Nk, d), 2), _rand((B, H, Nk, d), 3)
    scale = 0.3
    o, lse, p = oracle.attention(q, k, v, causal, scale, want_p=True)
    # rows of P sum to one, P_ij = exp(s_ij - LSE_i) on the allowed keys, 0 elsewhere
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-12)
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    allowed = np.ones((Nq, Nk), dtype=bool)
    if causal:
        allowed = np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + Nk - Nq
    want_p = np.where(allowed, np.exp(s - lse[..., None]), 0.0)
    np.testing.assert_allclose(p, want_p, atol=1e-12)
    np.testing.assert_allclose(o, p @ v, atol=1e-12)


def test_single_key_returns_value():
    q, k, v = _rand((2, 2, 9, 8), 4), _rand((2, 2, 1, 8), 5), _rand((2, 2, 1, 8), 6)
    o, lse = oracle.attention(q, k, v, False, 0.5)
    np.testing.assert_allclose(o, np.broadcast_to(v, o.shape), atol=0)
    np.testing.assert_allclose(lse, 0.5 * np.einsum("bhid,bhjd->bhi", q, k), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_mean(causal):
    Nq, Nk = 6, 10
    q, k, v = np.zeros((1, 2, Nq, 4)), _rand((1, 2, Nk, 4), 7), _rand((1, 2, Nk, 4), 8)
    o, lse = oracle.attention(q, k, v, causal, 1.3)
    for i in range(Nq):
        n = (i + Nk - Nq + 1) if causal else Nk
        np.testing.assert_allclose(o[:, :, i], v[:, :, :n].mean(axis=2), atol=1e-12)
        np.testing.assert_allclose(lse[:, :, i], math.log(n), atol=1e-12)


def test_constant_values_and_linearity_and_shift():
    q, k = _rand((1, 2, 12, 8), 9), _rand((1, 2, 15, 8), 10)
    v1, v2 = _rand((1, 2, 15, 8), 11), _rand((1, 2, 15, 8), 12)
    const = np.broadcast_to(np.arange(8.0), (1, 2, 15, 8))
    o, _ = oracle.attention(q, k, const, True, 0.7)
    np.testing.assert_allclose(o, np.broadcast_to(np.arange(8.0), o.shape), atol=1e-12)
    o1, _ = oracle.attention(q, k, v1, False, 0.7)
    o2, _ = oracle.attention(q, k, v2, False, 0.7)
    o12, _ = oracle.attention(q, k, 2.0 * v1 - 3.0 * v2, False, 0.7)
    np.testing.assert_allclose(o12, 2.0 * o1 - 3.0 * o2, atol=1e-12)
    # adding w to every key shifts row i's scores by scale*q_i.w: O unchanged, LSE shifted
    w = _rand((8,), 13)
    o_s, lse_s = oracle.attention(q, k + w, v1, False, 0.7)
    _, lse_1 = oracle.attention(q, k, v1, False, 0.7)
    np.testing.assert_allclose(o_s, o1, atol=1e-12)
    np.testing.assert_allclose(lse_s, lse_1 + 0.7 * q @ w, atol=1e-12)


def test_joint_key_value_permutation():
    q, k, v = _rand((1, 1, 10, 6), 14), _rand((1, 1, 13, 6), 15), _rand((1, 1, 13, 6), 16)
    perm = np.random.default_rng(17).permutation(13)
    o, lse = oracle.attention(q, k, v, False, 0.9)
    op, lsep = oracle.attention(q, k[:, :, perm], v[:, :, perm], False, 0.9)
    np.testing.assert_allclose(op, o, atol=1e-12)
    np.testing.assert_allclose(lsep, lse, atol=1e-12)


def test_causal_first_row_sees_only_first_key():
    q, k, v = _rand((1, 2, 8, 4), 18), _rand((1, 2, 8, 4), 19), _rand((1, 2, 8, 4), 20)
    o, lse = oracle.attention(q, k, v, True, 0.6)
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], atol=0)
    np.testing.assert_allclose(lse[:, :, 0], 0.6 * np.sum(q[:, :, 0] * k[:, :, 0], -1), atol=1e-12)
    # the last row of a square causal problem sees every key
    o_full, lse_full = oracle.attention(q, k, v, False, 0.6)
    np.testing.assert_allclose(o[:, :, -1], o_full[:, :, -1], atol=1e-12)


def test_row_subset_matches_full():
    q, k, v = _rand((2, 2, 30, 8), 21), _rand((2, 2, 30, 8), 22), _rand((2, 2, 30, 8), 23)
    rows = np.array([0, 3, 17, 29])
    o, lse = oracle.attention(q, k, v, True, 0.5)
    os_, lses = oracle.attention(q, k, v, True, 0.5, rows=rows)
    np.testing.assert_array_equal(os_, o[:, :, rows])
    np.testing.assert_array_equal(lses, lse[:, :, rows])


# ------------------------------------------------------------ merge identity
@pytest.mark.parametrize("splits", [[1, 20], [7, 3, 11], [3] * 7, [8] * 8, [1] * 9])
def test_block_states_merge_to_one_pass(splits):
    Nk = sum(splits)
    q, k, v = _rand((1, 2, 9, 8), 24, 2.0), _rand((1, 2, Nk, 8), 25, 2.0), _rand((1, 2, Nk, 8), 26)
    o, lse = oracle.attention(q, k, v, False, 0.6)
    acc = oracle.empty_state(o.shape)
    start = 0
    for n in splits:
        st = oracle.block_state(q, k[:, :, start:start + n], v[:, :, start:start + n], False, 0, start, 0.6)
        acc = oracle.merge(acc, st)
        start += n
    np.testing.assert_allclose(acc[0], o, atol=1e-12)
    np.testing.assert_allclose(oracle.state_lse(acc[1], acc[2]), lse, atol=1e-12)


def test_causal_block_states_merge_to_one_pass():
    # global positions: the local query shard sits at the end of the sequence
    Nq, Nk, blk = 12, 40, 8
    q, k, v = _rand((1, 1, Nq, 4), 27), _rand((1, 1, Nk, 4), 28), _rand((1, 1, Nk, 4), 29)
    o, lse = oracle.attention(q, k, v, True, 0.9)  # bottom-right: q_pos0 = Nk - Nq
    acc = oracle.empty_state(o.shape)
    for s0 in range(0, Nk, blk):
        st = oracle.block_state(q, k[:, :, s0:s0 + blk], v[:, :, s0:s0 + blk], True, Nk - Nq, s0, 0.9)
        acc = oracle.merge(acc, st)
    np.testing.assert_allclose(acc[0], o, atol=1e-12)
    np.testing.assert_allclose(oracle.state_lse(acc[1], acc[2]), lse, atol=1e-12)


def test_merge_commutative_associative_identity():
    q = _rand((1, 1, 5, 4), 30)
    ks = [_rand((1, 1, 6, 4), 31 + i, 2.0) for i in range(3)]
    vs = [_rand((1, 1, 6, 4), 41 + i) for i in range(3)]
    a, b, c = (oracle.block_state(q, ks[i], vs[i], False, 0, 6 * i, 1.1) for i in range(3))
    ab, ba = oracle.merge(a, b), oracle.merge(b, a)
    for x, y in zip(ab, ba):
        np.testing.assert_allclose(x, y, atol=1e-12)
    left, right = oracle.merge(oracle.merge(a, b), c), oracle.merge(a, oracle.merge(b, c))
    for x, y in zip(left, right):
        np.testing.assert_allclose(x, y, atol=1e-12)
    e = oracle.empty_state(a[0].shape)
    for x, y in zip(oracle.merge(a, e), a):
        np.testing.assert_allclose(x, y, atol=1e-15)
    for x, y in zip(oracle.merge(e, a), a):
        np.testing.assert_allclose(x, y, atol=1e-15)


def test_fully_masked_block_is_empty_state():
    q, k, v = _rand((1, 1, 4, 4), 50), _rand((1, 1, 4, 4), 51), _rand((1, 1, 4, 4), 52)
    o, m, l = oracle.block_state(q, k, v, True, 0, 10, 1.0)  # keys at 10..13, queries at 0..3
    assert np.all(o == 0) and np.all(np.isneginf(m)) and np.all(l == 0)


# ------------------------------------------------------------------ decoders
def test_bf16_decode_matches_torch_for_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode_bf16(bits.reshape(1, 1, -1, 1)).ravel()
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], want[~nan])


def test_e4m3_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    got = np.array([oracle.e4m3_value(int(c)) for c in codes])
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], want[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_e4m3_decode_applies_tile_scales():
    codes = np.full((1, 2, 300, 4), 0x38, dtype=np.uint8)  # 1.0
    scales = np.array([[[0.5, 2.0, 3.0], [1.0, 4.0, 0.25]]], dtype=np.float32)
    x = oracle.decode_e4m3(codes, scales, 128)
    for h in range(2):
        for n in range(300):
            assert np.all(x[0, h, n] == scales[0, h, n // 128])


# ------------------------------------------------------------------ gradients
def _loss(q, k, v, dout, causal, scale):
    o, _ = oracle.attention(q, k, v, causal, scale)
    return float((o * dout).sum())


@pytest.mark.parametrize("Nq,Nk,causal", [(5, 6, False), (5, 6, True), (6, 4, True), (3, 3, True)])
def test_bwd_matches_finite_differences_of_the_forward(Nq, Nk, causal):
    """Every gradient entry equals the central difference of sum(dO * O) computed with the
    (separately pinned) forward oracle; Nq > Nk causal includes rows with no key."""
    rng = np.random.default_rng(Nq * 10 + Nk + causal)
    q, k, v, do = (rng.standard_normal(s) for s in [(1, 2, Nq, 4), (1, 2, Nk, 4), (1, 2, Nk, 4), (1, 2, Nq, 4)])
    scale, h = 0.7, 1e-5
    grads = dict(zip("qkv", oracle.attention_bwd(q, k, v, do, causal, scale)))
    base = {"q": q, "k": k, "v": v}
    for name in "qkv":
        num = np.zeros_like(base[name])
        for idx in np.ndindex(base[name].shape):
            plus = {n: a.copy() for n, a in base.items()}
            minus = {n: a.copy() for n, a in base.items()}
            plus[name][idx] += h
            minus[name][idx] -= h
            num[idx] = (_loss(plus["q"], plus["k"], plus["v"], do, causal, scale)
                        - _loss(minus["q"], minus["k"], minus["v"], do, causal, scale)) / (2 * h)
        np.testing.assert_allclose(grads[name], num, atol=1e-8, rtol=0, err_msg=f"d{name}")


def test_bwd_single_key_closed_form():
    """One key: P = 1 for every row, so the output is v whatever q and k: dq = dk = 0, dv = sum_i dO_i."""
    rng = np.random.default_rng(3)
    q, do = rng.standard_normal((2, 1, 7, 8)), rng.standard_normal((2, 1, 7, 8))
    k, v = rng.standard_normal((2, 1, 1, 8)), rng.standard_normal((2, 1, 1, 8))
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, False, 0.3)
    assert np.all(dq == 0) and np.allclose(dk, 0, atol=1e-15)
    np.testing.assert_allclose(dv[:, :, 0], do.sum(axis=2), rtol=1e-14)


def test_bwd_identical_keys_give_zero_dq():
    """With every key equal, scores are constant along each row and the softmax does not depend
    on q: dq = 0 (the rows of dS sum to zero)."""
    rng = np.random.default_rng(4)
    q, do = rng.standard_normal((1, 2, 6, 8)), rng.standard_normal((1, 2, 6, 8))
    k = np.repeat(rng.standard_normal((1, 2, 1, 8)), 5, axis=2)
    v = rng.standard_normal((1, 2, 5, 8))
    dq, _, _ = oracle.attention_bwd(q, k, v, do, False, 0.9)
    np.testing.assert_allclose(dq, 0, atol=1e-13)


def test_bwd_row_subsets_and_empty_rows():
    """Subsets of rows give the same values as the full run; a causal row with no allowed key
    (Nq > Nk) has dq = 0 and changes no dk / dv."""
    rng = np.random.default_rng(5)
    q, k, v, do = (rng.standard_normal(s) for s in [(1, 2, 9, 8), (1, 2, 6, 8), (1, 2, 6, 8), (1, 2, 9, 8)])
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, True, 0.5)
    qr, kr = np.array([8, 0, 4]), np.array([5, 1])
    sq, sk, sv = oracle.attention_bwd(q, k, v, do, True, 0.5, q_rows=qr, k_rows=kr)
    np.testing.assert_array_equal(sq, dq[:, :, qr])
    np.testing.assert_array_equal(sk, dk[:, :, kr])
    np.testing.assert_array_equal(sv, dv[:, :, kr])
    assert np.all(dq[:, :, :3] == 0)  # rows 0..2 see keys <= i - 3 < 0
    do2 = do.copy()
    do2[:, :, :3] = rng.standard_normal((1, 2, 3, 8))
    _, dk2, dv2 = oracle.attention_bwd(q, k, v, do2, True, 0.5)
    np.testing.assert_array_equal(dk2, dk)
    np.testing.assert_array_equal(dv2, dv)


# ---------------------------------------------------------------- W4A16 layer
W4_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "w4a16_hand.json")


def _pack_rows(codes):
    """Dense codes [N, K] (0..15) -> words [N, K/8]: the even-indexed codes of
    each run of eight fill the low 16 bits, four bits apiece, and the odd ones
    the high 16 bits (the library's format)."""
    codes = np.asarray(codes, dtype=np.uint32)
    N, K = codes.shape
    c = codes.reshape(N, K // 8, 8)
    lo = c[..., 0] | (c[..., 2] << 4) | (c[..., 4] << 8) | (c[..., 6] << 12)
    hi = c[..., 1] | (c[..., 3] << 4) | (c[..., 5] << 8) | (c[..., 7] << 12)
    return (lo | (hi << 16)).astype(np.uint32)


def _h(x):
    return np.asarray(x, dtype=np.float16).view(np.uint16)


def test_w4_word_layout_matches_hand_fixture():
    g = json.load(open(W4_GOLDEN))
    for case in g["words"]:
        w = np.array([int(case["word"], 16)], dtype=np.uint32)
        assert [oracle.w4_value(w, k) for k in range(8)] == case["codes"], case["word"]


def test_w4a16_worked_example_from_hand_fixture():
    ex = json.load(open(W4_GOLDEN))["worked_example"]
    packed = np.array([[int(w, 16) for w in row] for row in ex["packed"]], dtype=np.uint32)
    y = oracle.w4a16(_h(ex["x"]), packed, np.array(ex["zeros"], dtype=np.uint8), _h(ex["scales"]), ex["group"])
    np.testing.assert_array_equal(y, np.array(ex["y"]))


def test_w4a16_pack_roundtrip_matches_dense_matmul():
    rng = np.random.default_rng(41)
    M, N, K, G = 3, 5, 256, 64
    codes = rng.integers(0, 16, size=(N, K))
    zeros = rng.integers(0, 16, size=(N, K // G)).astype(np.uint8)
    scales = rng.uniform(0.01, 0.1, size=(N, K // G)).astype(np.float16)
    x = rng.standard_normal((M, K)).astype(np.float16)
    w = (codes - np.repeat(zeros.astype(np.int64), G, axis=1)) * np.repeat(scales.astype(np.float64), G, axis=1)
    ref = x.astype(np.float64) @ w.T
    y = oracle.w4a16(x.view(np.uint16), _pack_rows(codes), zeros, scales.view(np.uint16), G)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_w4a16_one_hot_activations_read_back_every_weight():
    rng = np.random.default_rng(42)
    N, K, G = 4, 256, 128
    codes = rng.integers(0, 16, size=(N, K))
    zeros = rng.integers(0, 16, size=(N, K // G)).astype(np.uint8)
    scales = np.array(rng.choice([0.25, 0.5, 2.0, 0.125], size=(N, K // G)), dtype=np.float16)
    y = oracle.w4a16(np.eye(K, dtype=np.float16).view(np.uint16), _pack_rows(codes), zeros,
                     scales.view(np.uint16), G)
    for n in range(N):
        for k in range(K):
            g = k // G
            assert y[k, n] == (int(codes[n, k]) - int(zeros[n, g])) * float(scales[n, g]), (n, k)


def test_w4a16_codes_equal_to_zero_point_give_zero():
    N, K, G = 3, 384, 128
    zeros = np.array([[0, 7, 15], [3, 3, 9], [15, 0, 1]], dtype=np.uint8)
    codes = np.repeat(zeros.astype(np.int64), G, axis=1)
    x = np.random.default_rng(43).standard_normal((2, K)).astype(np.float16)
    y = oracle.w4a16(x.view(np.uint16), _pack_rows(codes), zeros, _h(np.ones((N, K // G))), G)
    assert np.all(y == 0.0)


def test_w4a16_quantized_layer_is_within_rounding_of_the_float_layer():
    # Asymmetric 4-bit quantization of a float matrix per group of 128: each
    # dequantized weight is within one scale step of the original, so the
    # layer output is within sum_k |x_k| * scale of the unquantized product.
    rng = np.random.default_rng(44)
    M, N, K, G = 2, 6, 512, 128
    w = rng.uniform(-0.05, 0.08, size=(N, K))
    wg = w.reshape(N, K // G, G)
    lo, hi = wg.min(axis=2), wg.max(axis=2)
    s = np.float16((hi - lo) / 15.0 * (1 + 2.0**-9)).astype(np.float64)
    z = np.clip(np.round(-lo / s), 0, 15)
    q = np.clip(np.round(wg / s[..., None]) + z[..., None], 0, 15).reshape(N, K).astype(np.int64)
    x = rng.standard_normal((M, K)).astype(np.float16)
    y = oracle.w4a16(x.view(np.uint16), _pack_rows(q), z.astype(np.uint8), _h(s), G)
    ref = x.astype(np.float64) @ w.T
    bound = np.abs(x.astype(np.float64)) @ np.repeat(s, G, axis=1).T
    assert np.all(np.abs(y - ref) <= bound)
    assert np.abs(y - ref).max() > 0  # the quantization really did round


def test_w4a16_is_linear_in_the_activations():
    rng = np.random.default_rng(45)
    N, K, G = 7, 256, 128
    packed = rng.integers(0, 2**32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    zeros = rng.integers(0, 16, size=(N, K // G)).astype(np.uint8)
    scales = _h(rng.uniform(0.01, 0.1, size=(N, K // G)))
    a = rng.integers(-8, 9, size=(1, K)).astype(np.float16)
    b = rng.integers(-8, 9, size=(1, K)).astype(np.float16)
    ya = oracle.w4a16(a.view(np.uint16), packed, zeros, scales, G)
    yb = oracle.w4a16(b.view(np.uint16), packed, zeros, scales, G)
    yab = oracle.w4a16((a + 2 * b).view(np.uint16), packed, zeros, scales, G)
    np.testing.assert_allclose(yab, ya + 2 * yb, rtol=1e-12, atol=1e-12)


def test_w4a16_rejects_bad_shapes():
    x = np.zeros((1, 12), dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.w4a16(x, np.zeros((1, 1), dtype=np.uint32), np.zeros((1, 1), dtype=np.uint8),
                     np.zeros((1, 1), dtype=np.uint16), 12)
