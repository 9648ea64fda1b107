"""GPU parity: the HIP kernels, called through the C ABI, against the fp64
oracle on the same seeded inputs.  Small ragged shapes are compared element
by element over every output; the five workloads run at full size in the
launch configuration the benchmark times, compared on sampled query rows."""
import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_15_amd as eta
import oracle
from exact_tiled_attention_15_amd import configs, inputs
from tests.gpu_util import BF16_BAR, FP8_BAR, compare_lse, compare_o, dev, dev_bf16, host, say

pytestmark = pytest.mark.gpu


def _bf16_problem(B, H, Nq, Nk, d, seed):
    q = inputs.bf16_bits(inputs.normal_f32((B, H, Nq, d), seed, 0))
    k = inputs.bf16_bits(inputs.normal_f32((B, H, Nk, d), seed, 1))
    v = inputs.bf16_bits(inputs.normal_f32((B, H, Nk, d), seed, 2))
    return q, k, v


def _run_fwd(qb, kb, vb, causal, scale):
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    B, H, Nq, d = q.shape
    o = torch.full((B, H, Nq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device="cuda")
    eta.attn_fwd(q, k, v, o, lse, causal, scale)
    torch.cuda.synchronize()
    return host(o), host(lse)


SMALL = [
    # (B, H, Nq, Nk, d, causal)
    (1, 1, 1, 1, 64, False), (1, 1, 1, 1, 128, True), (1, 2, 2, 2, 128, True), (2, 1, 3, 3, 64, False),
    (1, 1, 63, 63, 128, True), (1, 1, 64, 64, 128, True), (1, 1, 65, 65, 128, True),
    (1, 2, 127, 127, 64, True), (1, 1, 128, 128, 128, False), (1, 1, 129, 129, 128, True),
    (2, 3, 200, 200, 128, True), (1, 2, 200, 200, 64, False), (1, 1, 300, 77, 128, False),
    (1, 1, 77, 300, 128, False), (1, 1, 77, 300, 128, True), (1, 1, 300, 77, 128, True),
    (1, 1, 300, 77, 64, True), (3, 1, 129, 513, 64, True), (1, 8, 256, 256, 128, True),
    (1, 1, 1000, 1000, 128, True), (2, 2, 385, 1000, 128, False),
]


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal", SMALL)
def test_attn_fwd_small_shapes(B, H, Nq, Nk, d, causal):
    say(f"attn_fwd B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal}")
    seed = 7 + Nq * 7 + Nk * 3 + d + int(causal)
    qb, kb, vb = _bf16_problem(B, H, Nq, Nk, d, seed)
    scale = 1.0 / math.sqrt(d)
    o, lse = _run_fwd(qb, kb, vb, causal, scale)
    ro, rl = oracle.attention(oracle.decode_bf16(qb), oracle.decode_bf16(kb), oracle.decode_bf16(vb),
                              causal, scale)
    compare_o(o, ro, BF16_BAR, "O")
    compare_lse(lse, rl, "LSE")


# More 256-row blocks than a chip has compute units: each workgroup of the
# persistent forward walks two or more blocks, the next block's first K/V tile
# and Q rows loading during the previous block's last tile.  Ragged last
# blocks, blocks with no allowed key (causal, Nq - Nk >= 256: rows with no key
# get O = 0 and LSE = -inf), d = 64, and block counts that are and are not
# multiples of 8 (per-XCD and plain schedules).  The last case is causal with
# a pair of query blocks for every workgroup (the paired causal schedule).
SEVERAL_BLOCKS = [
    (1, 160, 300, 300, 128, True), (1, 100, 600, 40, 128, True), (2, 65, 257, 257, 64, False),
    (1, 264, 256, 129, 128, True), (3, 97, 512, 300, 128, False), (4, 64, 512, 512, 64, True),
]


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal", SEVERAL_BLOCKS)
def test_attn_fwd_several_blocks_per_workgroup(B, H, Nq, Nk, d, causal):
    say(f"attn_fwd several blocks B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal}")
    assert B * H * ((Nq + 255) // 256) > 256
    seed = 11 + Nq * 5 + Nk * 3 + d + int(causal) + H
    qb, kb, vb = _bf16_problem(B, H, Nq, Nk, d, seed)
    scale = 1.0 / math.sqrt(d)
    o, lse = _run_fwd(qb, kb, vb, causal, scale)
    ro, rl = oracle.attention(oracle.decode_bf16(qb), oracle.decode_bf16(kb), oracle.decode_bf16(vb),
                              causal, scale)
    compare_o(o, ro, BF16_BAR, "O")
    compare_lse(lse, rl, "LSE")


@pytest.mark.parametrize("Nq,Nk,d,causal", [(256, 256, 64, False), (200, 333, 128, True), (65, 31, 64, True)])
def test_attn_fwd_f32_small(Nq, Nk, d, causal):
    say(f"attn_fwd_f32 Nq={Nq} Nk={Nk} d={d} causal={causal}")
    rng = np.random.default_rng(Nq + Nk + d)
    q, k, v = (rng.standard_normal(s).astype(np.float32) for s in [(1, 2, Nq, d), (1, 2, Nk, d), (1, 2, Nk, d)])
    o = torch.full((1, 2, Nq, d), float("nan"), device="cuda")
    lse = torch.full((1, 2, Nq), float("nan"), device="cuda")
    scale = 1.0 / math.sqrt(d)
    eta.attn_fwd_f32(dev(q), dev(k), dev(v), o, lse, causal, scale)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q, k, v, causal, scale)
    max_abs, _ = compare_o(host(o), ro, BF16_BAR, "O f32")
    assert max_abs < 1e-4  # fp32 products and probabilities: far inside the bar
    compare_lse(host(lse), rl, "LSE f32")


# ------------------------------------------------------------------ properties
def test_deterministic_and_every_output_written():
    say("determinism B=2 H=4 N=777 d=128 causal")
    qb, kb, vb = _bf16_problem(2, 4, 777, 777, 128, 99)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    outs = []
    for _ in range(5):
        o = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full(q.shape[:3], float("nan"), device="cuda")
        eta.attn_fwd(q, k, v, o, lse, True, 0.09)
        outs.append((o.clone(), lse.clone()))
    torch.cuda.synchronize()
    assert not torch.isnan(outs[0][0]).any() and not torch.isnan(outs[0][1]).any()
    for o, lse in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(lse.view(torch.int32), outs[0][1].view(torch.int32))


@pytest.mark.parametrize("B,H,N,causal", [(2, 4, 777, True), (8, 16, 2048, True), (1, 3, 1000, False)])
def test_deterministic_under_permuted_workgroup_order(B, H, N, causal):
    """Exact and deterministic ("FlashAttention-2", "Performance and efficiency"): the same output,
    bit for bit, whichever workgroup computes which (b, h, query block) tile."""
    say(f"workgroup order B={B} H={H} N={N} causal={causal}")
    qb, kb, vb = _bf16_problem(B, H, N, N, 128, 123 + N)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    o0 = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    l0 = torch.full(q.shape[:3], float("nan"), device="cuda")
    eta.attn_fwd(q, k, v, o0, l0, causal, 0.0884)
    for order in (1, 7, 12345, 2**31 + 5):
        o = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full(q.shape[:3], float("nan"), device="cuda")
        eta.attn_fwd_block_order(q, k, v, o, lse, causal, 0.0884, order)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o0.view(torch.int16)), f"order {order}: O differs"
        assert torch.equal(lse.view(torch.int32), l0.view(torch.int32)), f"order {order}: LSE differs"
    assert not torch.isnan(o0).any() and not torch.isnan(l0).any()


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_prefix_mean(causal):
    say(f"zero query causal={causal}")
    _, kb, vb = _bf16_problem(1, 2, 300, 300, 128, 5)
    qb = np.zeros((1, 2, 300, 128), dtype=np.uint16)
    o, lse = _run_fwd(qb, kb, vb, causal, 0.5)
    v = oracle.decode_bf16(vb)
    n = np.arange(1, 301) if causal else np.full(300, 300)
    mean = np.cumsum(v, axis=2) / n[None, None, :, None] if causal else np.broadcast_to(v.mean(2, keepdims=True), v.shape)
    compare_o(o, mean, BF16_BAR, "O=mean")
    compare_lse(lse, np.broadcast_to(np.log(n), lse.shape), "LSE=ln n")


def test_single_key_returns_value_exactly():
    say("Nk=1")
    qb, kb, vb = _bf16_problem(2, 2, 130, 1, 128, 6)
    o, lse = _run_fwd(qb, kb, vb, False, 0.3)
    v = oracle.decode_bf16(vb)
    np.testing.assert_array_equal(o, np.broadcast_to(v, o.shape))
    s = 0.3 * np.einsum("bhid,bhjd->bhi", oracle.decode_bf16(qb), oracle.decode_bf16(kb))
    compare_lse(lse, s, "LSE=s")


@pytest.mark.parametrize("scale", [-0.2, 0.0, 3.0])
def test_scale_sign_and_zero(scale):
    say(f"scale={scale}")
    qb, kb, vb = _bf16_problem(1, 2, 150, 190, 64, 8)
    o, lse = _run_fwd(qb, kb, vb, True, scale)
    ro, rl = oracle.attention(oracle.decode_bf16(qb), oracle.decode_bf16(kb), oracle.decode_bf16(vb), True, scale)
    compare_o(o, ro, BF16_BAR, "O")
    compare_lse(lse, rl, "LSE")


def test_empty_causal_rows():
    say("Nq > Nk causal: leading rows see no key")
    qb, kb, vb = _bf16_problem(1, 1, 300, 40, 128, 9)
    o, lse = _run_fwd(qb, kb, vb, True, 0.1)
    assert np.all(o[0, 0, :260] == 0) and np.all(np.isneginf(lse[0, 0, :260]))
    ro, rl = oracle.attention(oracle.decode_bf16(qb), oracle.decode_bf16(kb), oracle.decode_bf16(vb), True, 0.1)
    compare_o(o, ro, BF16_BAR, "O")
    compare_lse(lse, rl, "LSE")


# --------------------------------------------------------------- block states
@pytest.mark.parametrize("Nq,Nkb,causal,q_pos0,k_pos0", [
    (200, 64, False, 0, 0), (129, 300, False, 0, 0), (256, 128, True, 512, 384), (256, 128, True, 512, 640),
    (100, 90, True, 1000, 0), (200, 77, True, 100, 150), (64, 64, True, 0, 64),
])
def test_kvblock_state(Nq, Nkb, causal, q_pos0, k_pos0):
    say(f"kvblock Nq={Nq} Nkb={Nkb} causal={causal} q_pos0={q_pos0} k_pos0={k_pos0}")
    qb, kb, vb = _bf16_problem(1, 2, Nq, Nkb, 128, Nq + Nkb)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    o = torch.full((1, 2, Nq, 128), float("nan"), device="cuda")
    m = torch.full((1, 2, Nq), float("nan"), device="cuda")
    l = torch.full((1, 2, Nq), float("nan"), device="cuda")
    eta.attn_fwd_kvblock(q, k, v, o, m, l, causal, q_pos0, k_pos0, 0.125)
    torch.cuda.synchronize()
    ro, rm, rl = oracle.block_state(oracle.decode_bf16(qb), oracle.decode_bf16(kb), oracle.decode_bf16(vb),
                                    causal, q_pos0, k_pos0, 0.125)
    compare_o(host(o), ro, BF16_BAR, "O_part")
    compare_lse(host(m), rm, "m")
    gl, rl_ = host(l), rl
    np.testing.assert_array_equal(gl == 0, rl_ == 0)
    nz = rl_ > 0
    assert np.all(np.abs(gl[nz] / rl_[nz] - 1) < 1e-4)


def test_merge_matches_oracle_including_empty_states():
    say("merge with empty rows")
    rng = np.random.default_rng(11)
    B, H, Nq, d = 1, 2, 300, 128
    oa, ob = (rng.standard_normal((B, H, Nq, d)).astype(np.float32) for _ in range(2))
    ma, mb = (rng.standard_normal((B, H, Nq)).astype(np.float32) * 3 for _ in range(2))
    la, lb = (rng.uniform(1, 50, (B, H, Nq)).astype(np.float32) for _ in range(2))
    ma[0, 0, :20] = -np.inf; la[0, 0, :20] = 0; oa[0, 0, :20] = 0
    mb[0, 0, 10:30] = -np.inf; lb[0, 0, 10:30] = 0; ob[0, 0, 10:30] = 0
    to = [dev(x) for x in (oa, ma, la, ob, mb, lb)]
    of = torch.full((B, H, Nq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lf = torch.full((B, H, Nq), float("nan"), device="cuda")
    eta.attn_merge(*to, of, lf)
    torch.cuda.synchronize()
    ro, rm, rl = oracle.merge((oa, ma, la), (ob, mb, lb))
    np.testing.assert_allclose(host(to[0]), ro, atol=1e-5)
    compare_lse(host(to[1]), rm, "m")
    np.testing.assert_allclose(host(to[2]), rl, rtol=1e-5)
    # the bf16 output is the merged fp32 accumulator rounded to nearest even
    assert torch.equal(of.view(torch.int16), to[0].to(torch.bfloat16).view(torch.int16))
    compare_lse(host(lf), oracle.state_lse(rm, rl), "LSE_final")


# --------------------------------------------------------------- fp8 path
def _fp8_problem(B, H, Nq, Nk, d, seed, outliers=True, rotate=False):
    cfg = dict(B=B, H=H, Nq=Nq, Nk=Nk, d=d, dtype="fp8", outlier_frac=0.01,
               outlier_mult=20.0 if outliers else 1.0)
    return inputs.make_inputs(cfg, seed, rotate=rotate)


def _run_fp8(x, causal, scale, mode="fp8"):
    B, H, Nq, d = x["q8"].shape
    o = torch.full((B, H, Nq, d), float("nan"), device="cuda")
    lse = torch.full((B, H, Nq), float("nan"), device="cuda")
    fn = {"fp8": eta.attn_fwd_fp8, "qk16": eta.attn_fwd_fp8_qk16, "pv8": eta.attn_fwd_fp8_pv8}[mode]
    fn(dev(x["q8"]), dev(x["k8"]), dev(x["v8"]), dev(x["q_scale"]), dev(x["k_scale"]), dev(x["v_scale"]), o, lse,
       causal, scale)
    torch.cuda.synchronize()
    return host(o), host(lse)


def _fp8_ref(x, causal, scale, rows=None):
    q = oracle.decode_e4m3(x["q8"], x["q_scale"])
    k = oracle.decode_e4m3(x["k8"], x["k_scale"])
    v = oracle.decode_e4m3(x["v8"], x["v_scale"])
    return oracle.attention(q, k, v, causal, scale, rows=rows)


FP8_SHAPES = [
    # (Nq, Nk, d, causal, rotate, outliers)
    (128, 128, 128, False, False, True), (300, 257, 128, False, False, True), (200, 200, 128, True, False, True),
    (256, 640, 128, False, True, True), (130, 70, 64, False, False, True), (70, 130, 64, True, True, True),
    (333, 200, 128, True, False, False), (129, 385, 64, False, False, False),
]


# The fp8 matrix cores sum one instruction's products with limited alignment precision
# (tests/test_gpu_mfma_fp8.py measures it): an un-rotated x20 channel shared by Q and K makes one
# product per score ~400 times the others, and the scores move by ~0.1 in log2 units.  attn_fwd_fp8
# (Q.K on fp8 MFMA) therefore misses the fp8 bar on such inputs; the rotation of the same passage
# (incoherent processing) is what brings it inside.  These cases are expected failures, strictly:
# an unexpected pass fails the run.  attn_fwd_fp8_qk16 (Q.K on fp16 MFMA) meets the bar on them.
XFAIL_FP8_UNROTATED = pytest.mark.xfail(
    strict=True, raises=AssertionError,
    reason="fp8 MFMA alignment precision on an un-rotated outlier channel: Q.K error ~0.1 in log2 units")


def _fp8_cases():
    for shape in FP8_SHAPES:
        for mode in ("qk16", "fp8"):
            _, _, _, _, rotate, outliers = shape
            marks = [XFAIL_FP8_UNROTATED] if (mode == "fp8" and outliers and not rotate) else []
            yield pytest.param(*shape, mode, marks=marks)


@pytest.mark.parametrize("Nq,Nk,d,causal,rotate,outliers,mode", list(_fp8_cases()))
def test_fp8_small_shapes(Nq, Nk, d, causal, rotate, outliers, mode):
    say(f"fp8 mode={mode} Nq={Nq} Nk={Nk} d={d} causal={causal} rotate={rotate} outliers={outliers}")
    x = _fp8_problem(1, 2, Nq, Nk, d, 1000 + Nq + Nk, outliers=outliers, rotate=rotate)
    scale = 1.0 / math.sqrt(d)
    o, lse = _run_fp8(x, causal, scale, mode)
    ro, rl = _fp8_ref(x, causal, scale)
    compare_o(o, ro, FP8_BAR, f"O fp8 ({mode})")
    compare_lse(lse, rl, f"LSE fp8 ({mode})")


def test_fp8_mfma_outliers_need_rotation():
    """The fp8 matrix cores sum one instruction's products with limited
    alignment precision, so an un-rotated x20 channel perturbs the scores; the
    rotation (incoherent processing) brings the fp8 path inside the bar."""
    say("fp8 MFMA with outlier channel, with and without rotation")
    scale = 1.0 / math.sqrt(128)
    for rotate in (False, True):
        x = _fp8_problem(1, 4, 512, 512, 128, 77, outliers=True, rotate=rotate)
        o, lse = _run_fp8(x, False, scale, "fp8")
        ro, rl = _fp8_ref(x, False, scale)
        if rotate:
            compare_o(o, ro, FP8_BAR, "O fp8 rotated")
            compare_lse(lse, rl, "LSE fp8 rotated")
        else:
            err = float(np.abs(o - ro).max())
            rel = float(np.linalg.norm(o - ro) / np.linalg.norm(ro))
            say(f"  un-rotated (reported): max_abs={err:.3e} rel_frob={rel:.3e}")
            assert rel <= FP8_BAR[1]


def test_fp8_single_key_dequantizes_exactly():
    say("fp8 Nk=1: O equals the dequantized value")
    for mode in ("fp8", "qk16"):
        x = _fp8_problem(1, 2, 64, 1, 128, 5, outliers=False)
        # every finite code across the value row: exercises the e4m3 -> fp16 widening
        codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
        x["v8"] = np.resize(codes, x["v8"].shape).astype(np.uint8)
        x["v_scale"] = np.array([[[0.75], [3.0]]], dtype=np.float32)
        o, _ = _run_fp8(x, False, 0.1, mode)
        v = oracle.decode_e4m3(x["v8"], x["v_scale"])
        # equal up to one fp32 rounding of the normaliser (a wrong widening of any
        # code would be off by at least 2^-4 relative)
        np.testing.assert_allclose(o, np.broadcast_to(v, o.shape), rtol=1e-6, atol=0)


# --------------------------------------------------------- full-size workloads
def _sample_rows(Nq, n, seed):
    r = inputs.row_subset(Nq, n, seed)
    extra = np.array([0, 1, 2, 3, Nq - 1], dtype=np.int64)
    return np.unique(np.concatenate([r, extra[extra < Nq]]))


def test_workload_f32_B1_H2_N256_d64():
    name = "f32_B1_H2_N256_d64"
    say(name)
    cfg, seed = configs.WORKLOADS[name], configs.seed_of(name)
    x = inputs.make_inputs(cfg, seed)
    o = torch.empty((1, 2, 256, 64), device="cuda")
    lse = torch.empty((1, 2, 256), device="cuda")
    eta.attn_fwd_f32(dev(x["q"]), dev(x["k"]), dev(x["v"]), o, lse, False, configs.scale_of(name))
    torch.cuda.synchronize()
    ro, rl = oracle.attention(x["q"], x["k"], x["v"], False, configs.scale_of(name))
    compare_o(host(o), ro, BF16_BAR, "O")
    compare_lse(host(lse), rl, "LSE")


@pytest.mark.parametrize("name,rows_per_head", [("bf16_causal_B8_H16_N2048_d128", "all"),
                                                ("bf16_causal_B1_H8_N32768_d128", 512)])
def test_workload_bf16_causal(name, rows_per_head):
    """Full-size causal workloads: every row of every head of the headline shape, and the
    workload's 512 sampled rows per head (plus the first four and the last) of the long one."""
    say(f"{name} rows/head={rows_per_head}")
    cfg, seed = configs.WORKLOADS[name], configs.seed_of(name)
    x = inputs.make_inputs(cfg, seed)
    o, lse = _run_fwd(x["q"], x["k"], x["v"], True, configs.scale_of(name))
    rows = np.arange(cfg["Nq"]) if rows_per_head == "all" else _sample_rows(cfg["Nq"], rows_per_head, seed)
    ro, rl = oracle.attention(oracle.decode_bf16(x["q"]), oracle.decode_bf16(x["k"]), oracle.decode_bf16(x["v"]),
                              True, configs.scale_of(name), rows=rows)
    compare_o(o[:, :, rows], ro, BF16_BAR, f"O ({len(rows)} rows/head)")
    compare_lse(lse[:, :, rows], rl, "LSE")


def test_workload_kv_blocks():
    name = "bf16_kvblocks_B1_H16_Nq8192_Nk65536x8_d128"
    say(name)
    cfg, seed = configs.WORKLOADS[name], configs.seed_of(name)
    B, H, Nq, Nk, d, nb = cfg["B"], cfg["H"], cfg["Nq"], cfg["Nk"], cfg["d"], cfg["n_blocks"]
    scale = configs.scale_of(name)
    x = inputs.make_inputs(cfg, seed)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    blk = Nk // nb
    kbs = [k[:, :, i * blk:(i + 1) * blk].contiguous() for i in range(nb)]
    vbs = [v[:, :, i * blk:(i + 1) * blk].contiguous() for i in range(nb)]
    acc = [torch.empty((B, H, Nq, d), device="cuda"), torch.empty((B, H, Nq), device="cuda"),
           torch.empty((B, H, Nq), device="cuda")]
    part = [torch.empty_like(t) for t in acc]
    o_fin = torch.full((B, H, Nq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse_fin = torch.full((B, H, Nq), float("nan"), device="cuda")
    eta.attn_fwd_kvblock(q, kbs[0], vbs[0], *acc, False, 0, 0, scale)
    for i in range(1, nb):
        eta.attn_fwd_kvblock(q, kbs[i], vbs[i], *part, False, 0, i * blk, scale)
        last = i == nb - 1
        eta.attn_merge(*acc, *part, o_fin if last else None, lse_fin if last else None)
    o1 = torch.full((B, H, Nq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    l1 = torch.full((B, H, Nq), float("nan"), device="cuda")
    eta.attn_fwd(q, k, v, o1, l1, False, scale)
    torch.cuda.synchronize()
    o_b, l_b, o_1, l_1 = host(o_fin), host(lse_fin), host(o1), host(l1)
    # block-streamed result equals one-pass attention over all 65536 keys
    compare_o(o_b, o_1, BF16_BAR, "blocks vs one-pass (all rows)")
    compare_lse(l_b, l_1, "blocks vs one-pass LSE")
    rows = _sample_rows(Nq, cfg["oracle_rows"], seed)
    say(f"  oracle on {len(rows)} rows/head")
    ro, rl = oracle.attention(oracle.decode_bf16(x["q"]), oracle.decode_bf16(x["k"]), oracle.decode_bf16(x["v"]),
                              False, scale, rows=rows)
    compare_o(o_b[:, :, rows], ro, BF16_BAR, "blocks vs oracle")
    compare_lse(l_b[:, :, rows], rl, "blocks LSE vs oracle")
    compare_o(o_1[:, :, rows], ro, BF16_BAR, "one-pass vs oracle")


# ---------------------------------------------------- fp8 probabilities (NEXT)
# e4m3 keeps 3 mantissa bits: each probability is rounded by up to 2^-4 relative.  With the
# normaliser summed from the same rounded values, a row's error is sum_j w_j d_j (v_j - O), which
# for random data is a few tenths of a percent of |O| in norm and larger on rows dominated by a few
# keys.  This mode is a speed-for-accuracy trade: the drift is reported, and gated only by
# PV8_DRIFT (relative Frobenius), a bound derived from that rounding, not by the fp8 parity bar.
PV8_DRIFT = 3e-2


@pytest.mark.parametrize("Nq,Nk,d,causal", [(256, 256, 128, False), (300, 200, 128, True), (129, 517, 64, False),
                                            (64, 1, 128, False)])
def test_fp8_pv8_drift(Nq, Nk, d, causal):
    say(f"fp8 P.V in e4m3 Nq={Nq} Nk={Nk} d={d} causal={causal}")
    x = _fp8_problem(1, 2, Nq, Nk, d, Nq + 3 * Nk, outliers=True, rotate=True)
    scale = 1.0 / math.sqrt(d)
    o, lse = _run_fp8(x, causal, scale, "pv8")
    o2, _ = _run_fp8(x, causal, scale, "pv8")
    assert np.array_equal(o, o2), "not deterministic"
    ro, rl = _fp8_ref(x, causal, scale)
    assert np.all(np.isfinite(o))
    err = float(np.abs(o - ro).max())
    rel = float(np.linalg.norm(o - ro) / np.linalg.norm(ro))
    say(f"  drift: max_abs={err:.3e} rel_frob={rel:.3e} (max|ref|={float(np.abs(ro).max()):.2f})")
    assert rel <= PV8_DRIFT, f"drift {rel:.3e} > {PV8_DRIFT}"
    # the normaliser sums rounded probabilities: a row ruled by one key is off by at most ln(1 + 2^-4)
    compare_lse(lse, rl, "LSE (the normaliser of the rounded P)", bar=math.log1p(2.0 ** -4))


def test_workload_fp8_pv8_drift():
    name = "fp8_pv8_B4_H16_N4096_d128"
    say(name)
    cfg, seed = configs.WORKLOADS[name], configs.seed_of(name)
    x = inputs.make_inputs(cfg, seed, rotate=True)
    scale = configs.scale_of(name)
    o, lse = _run_fp8(x, False, scale, "pv8")
    o16, _ = _run_fp8(x, False, scale, "fp8")
    rows = _sample_rows(cfg["Nq"], 128, seed)
    ro, rl = _fp8_ref(x, False, scale, rows=rows)
    got = o[:, :, rows]
    err = float(np.abs(got - ro).max())
    rel = float(np.linalg.norm(got - ro) / np.linalg.norm(ro))
    rel16 = float(np.linalg.norm(o16[:, :, rows] - ro) / np.linalg.norm(ro))
    say(f"  drift vs oracle: max_abs={err:.3e} rel_frob={rel:.3e}; fp16-P path rel_frob={rel16:.3e}")
    assert np.all(np.isfinite(o)) and rel <= PV8_DRIFT


# ---------------------------------------------- fp4 probabilities (NEXT, FP4 half)
# attn_fwd_fp8_pv4: P as 4-bit e2m1 codes on the f8f6f4 matrix cores, by rounding each exponential
# (direct_p=0) or by mapping the score straight to the code (Direct-P, direct_p=1).  One mantissa bit
# and nothing between 0 and 0.5: the drift is large on diffuse rows and is reported, not held to the
# fp8 bar.  What is gated: exact results where the rounding is exact (one dominant key per row, equal
# V scales), determinism, and bounds that hold for any data: O is a convex combination of V rows
# (|O - O_ref| <= 2 max|V|); no rounded probability exceeds twice the exact one (the worst case is
# 4p just above 0.25 rounding to 0.5), so LSE - LSE_ref <= ln 2; and the row's largest probability,
# quantized as 4 p s_v / max s_v >= 0.75 for these inputs' V scales, keeps at least 2/3 of its value,
# so LSE >= max score + ln(2/3).
def _pv4_run(x, causal, scale, direct):
    B, H, Nq, d = x["q8"].shape
    o = torch.full((B, H, Nq, d), float("nan"), device="cuda")
    lse = torch.full((B, H, Nq), float("nan"), device="cuda")
    eta.attn_fwd_fp8_pv4(dev(x["q8"]), dev(x["k8"]), dev(x["v8"]), dev(x["q_scale"]), dev(x["k_scale"]),
                         dev(x["v_scale"]), o, lse, causal, scale, direct)
    torch.cuda.synchronize()
    return host(o), host(lse)


@pytest.mark.parametrize("direct", [False, True])
def test_fp8_pv4_one_dominant_key_is_exact(direct):
    """Each query row equals one key row (a permutation), so that key's score dominates by ~40 and
    every other probability rounds to 0: O must be that key's V row and LSE its score.  A
    wrong key order between the P codes and the V^T tile would pick another row."""
    say(f"fp8 pv4 direct={direct}: one dominant key per row")
    rng = np.random.default_rng(21)
    B, H, N, d = 1, 2, 256, 128
    kv = rng.standard_normal((B, H, N, d)) * 2.0
    k8 = torch.from_numpy(kv).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    perm = rng.permutation(N)
    q8 = np.ascontiguousarray(k8[:, :, perm])
    v8 = torch.from_numpy(rng.standard_normal((B, H, N, d))).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ones = np.ones((B, H, (N + 127) // 128), dtype=np.float32)
    x = dict(q8=q8, k8=k8, v8=v8, q_scale=ones, k_scale=ones.copy(), v_scale=ones.copy())
    o, lse = _pv4_run(x, False, 0.1, direct)
    kd, vd = oracle.decode_e4m3(k8, ones), oracle.decode_e4m3(v8, ones)
    # equal up to the earlier tile's contributions, which the rescale by exp(-(gap ~ 37)) leaves at
    # ~1e-12 (exact attention keeps them too); a wrong key would be off by O(1)
    np.testing.assert_allclose(o, vd[:, :, perm], rtol=0, atol=1e-9)
    # LSE is the dominant score itself, up to the rounding of the fp8 Q.K instruction (scores ~50)
    s_dom = 0.1 * np.einsum("bhnd,bhnd->bhn", kd[:, :, perm], kd[:, :, perm])
    np.testing.assert_allclose(lse, s_dom, rtol=0, atol=2e-2)


@pytest.mark.parametrize("direct", [False, True])
@pytest.mark.parametrize("Nq,Nk,d,causal", [(256, 256, 128, False), (300, 200, 128, True), (129, 517, 64, False)])
def test_fp8_pv4_drift_bounds(Nq, Nk, d, causal, direct):
    say(f"fp8 pv4 direct={direct} Nq={Nq} Nk={Nk} d={d} causal={causal}")
    x = _fp8_problem(1, 2, Nq, Nk, d, Nq + 3 * Nk, outliers=True, rotate=True)
    scale = 1.0 / math.sqrt(d)
    o, lse = _pv4_run(x, causal, scale, direct)
    o2, lse2 = _pv4_run(x, causal, scale, direct)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2), "not deterministic"
    q = oracle.decode_e4m3(x["q8"], x["q_scale"])
    k = oracle.decode_e4m3(x["k8"], x["k_scale"])
    v = oracle.decode_e4m3(x["v8"], x["v_scale"])
    ro, rl, rp = oracle.attention(q, k, v, causal, scale, want_p=True)
    assert np.all(np.isfinite(o))
    err = float(np.abs(o - ro).max())
    rel = float(np.linalg.norm(o - ro) / np.linalg.norm(ro))
    say(f"  drift: max_abs={err:.3e} rel_frob={rel:.3e} (max|V|={float(np.abs(v).max()):.2f})")
    assert err <= 2.0 * float(np.abs(v).max())
    live = ~np.isneginf(rl)
    m = rl + np.log(np.where(live[..., None], rp, 1.0).max(-1))  # row maximum of the scores
    assert np.all(lse[live] >= m[live] + math.log(2.0 / 3.0) - 1e-3), "LSE below the row maximum + ln(2/3)"
    assert np.all(lse[live] - rl[live] <= math.log(2.0) + 1e-3), "LSE above ln 2 + exact"


def test_workload_fp8_pv4_drift():
    """The e4m3-P workload's inputs with P in e2m1, both forms; drift next to the e4m3-P mode."""
    name = "fp8_pv8_B4_H16_N4096_d128"
    say(name + " with P in e2m1")
    cfg, seed = configs.WORKLOADS[name], configs.seed_of(name)
    x = inputs.make_inputs(cfg, seed, rotate=True)
    scale = configs.scale_of(name)
    rows = _sample_rows(cfg["Nq"], 128, seed)
    ro, rl = _fp8_ref(x, False, scale, rows=rows)
    o8, _ = _run_fp8(x, False, scale, "pv8")
    rel8 = float(np.linalg.norm(o8[:, :, rows] - ro) / np.linalg.norm(ro))
    for direct in (False, True):
        o, lse = _pv4_run(x, False, scale, direct)
        got = o[:, :, rows]
        err = float(np.abs(got - ro).max())
        rel = float(np.linalg.norm(got - ro) / np.linalg.norm(ro))
        dl = float(np.abs(lse[:, :, rows] - rl).max())
        say(f"  direct={direct}: drift max_abs={err:.3e} rel_frob={rel:.3e} lse_max={dl:.3e} "
            f"(e4m3 P: rel_frob={rel8:.3e})")
        assert np.all(np.isfinite(o)) and err <= 2.0 * float(np.abs(oracle.decode_e4m3(x["v8"], x["v_scale"])).max())


# ------------------------------------------------------------- backward
def compare_grad(got, ref, what, rel_bar=1e-2, abs_frac=2e-2):
    """Gradients: relative Frobenius error <= 1e-2 and max-abs error <= 2 % of the largest
    reference magnitude.  The kernels round P and dS to bf16 (2^-9 relative) inside fp32
    sums and round the outputs to bf16 (2^-9): about 0.2-0.4 % is expected."""
    err = np.abs(got - ref)
    big = float(np.abs(ref).max()) if ref.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / nref) if nref > 0 else float(np.linalg.norm(got))
    m = float(err.max()) if err.size else 0.0
    say(f"  {what}: max_abs={m:.3e} (max|ref|={big:.3f}) rel_frob={rel:.3e}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    assert rel <= rel_bar, f"{what}: rel_frob {rel:.3e} > {rel_bar}"
    assert m <= abs_frac * max(big, 1e-6), f"{what}: max_abs {m:.3e} > {abs_frac} * {big:.3e}"


def _run_bwd(qb, kb, vb, ob, dob, lse, causal, scale):
    q, k, v, o, do = (dev_bf16(x) for x in (qb, kb, vb, ob, dob))
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    dq = torch.full((B, H, Nq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    dk = torch.full((B, H, Nk, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    dv = torch.full((B, H, Nk, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    work = torch.full((eta.bwd_work_floats(B, H, Nq),), float("nan"), device="cuda")
    eta.attn_bwd(q, k, v, o, do, lse if torch.is_tensor(lse) else dev(lse), dq, dk, dv, work, causal, scale)
    torch.cuda.synchronize()
    return host(dq), host(dk), host(dv)


BWD_SHAPES = [
    (1, 2, 128, 128, 128, False, 0.0884),
    (1, 2, 200, 333, 128, True, 0.0884),
    (2, 1, 300, 300, 64, True, 0.125),
    (1, 2, 65, 31, 64, True, 0.125),      # Nq > Nk: rows without keys
    (1, 2, 257, 513, 128, False, 0.0884),  # ragged tiles on both sides
    (1, 1, 1, 1, 128, False, 0.0884),
    (1, 2, 96, 160, 128, True, -0.2),
    (1, 2, 96, 160, 64, False, 0.0),
    (1, 2, 384, 384, 128, True, 0.0884),  # 3 key blocks: masked diagonal tiles, then all-live ones
]


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal,scale", BWD_SHAPES)
def test_bwd_small_shapes(B, H, Nq, Nk, d, causal, scale):
    """attn_bwd against the fp64 gradient; O and LSE are the oracle's (O rounded to bf16), so
    only the backward kernels are under test."""
    say(f"bwd B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal} scale={scale}")
    seed = 7 * Nq + Nk + d
    qb, kb, vb = _bf16_problem(B, H, Nq, Nk, d, seed)
    dob = inputs.bf16_bits(inputs.normal_f32((B, H, Nq, d), seed, 6))
    qd, kd, vd, dod = (oracle.decode_bf16(x) for x in (qb, kb, vb, dob))
    ro, rl = oracle.attention(qd, kd, vd, causal, scale)
    ob = inputs.bf16_bits(ro.astype(np.float32))
    dq, dk, dv = _run_bwd(qb, kb, vb, ob, dob, rl.astype(np.float32), causal, scale)
    rdq, rdk, rdv = oracle.attention_bwd(qd, kd, vd, dod, causal, scale)
    compare_grad(dq, rdq, "dQ")
    compare_grad(dk, rdk, "dK")
    compare_grad(dv, rdv, "dV")


def test_bwd_headline_shape_end_to_end():
    """Training step of the headline shape: attn_fwd's O and LSE feed attn_bwd; sampled dQ rows
    and dK/dV rows against the fp64 gradient."""
    name = "bf16_causal_B8_H16_N2048_d128"
    say(f"bwd {name}")
    cfg, seed = configs.WORKLOADS[name], configs.seed_of(name)
    scale = configs.scale_of(name)
    x = inputs.make_inputs(cfg, seed)
    B, H, N, d = cfg["B"], cfg["H"], cfg["Nq"], cfg["d"]
    dob = inputs.bf16_bits(inputs.normal_f32((B, H, N, d), seed, 6))
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), device="cuda")
    eta.attn_fwd(q, k, v, o, lse, True, scale)
    torch.cuda.synchronize()
    ob = o.view(torch.int16).cpu().numpy().view(np.uint16)
    dq, dk, dv = _run_bwd(x["q"], x["k"], x["v"], ob, dob, lse, True, scale)
    qr = _sample_rows(N, 64, seed)
    kr = _sample_rows(N, 64, seed + 1)
    qd, kd, vd, dod = (oracle.decode_bf16(a) for a in (x["q"], x["k"], x["v"], dob))
    rdq, rdk, rdv = oracle.attention_bwd(qd, kd, vd, dod, True, scale, q_rows=qr, k_rows=kr)
    compare_grad(dq[:, :, qr], rdq, f"dQ ({len(qr)} rows/head)")
    compare_grad(dk[:, :, kr], rdk, f"dK ({len(kr)} rows/head)")
    compare_grad(dv[:, :, kr], rdv, f"dV ({len(kr)} rows/head)")


# ------------------------------------------------------- ring-attention share
def _ring_run(q, k_full, v_full, blk, order, causal, q_pos0, scale):
    """attn_fwd_ring over the blocks of k_full / v_full (blk keys each) in the given hop order."""
    B, H, Nq, d = q.shape
    kb = [k_full[:, :, b * blk:(b + 1) * blk].contiguous() for b in order]
    vb = [v_full[:, :, b * blk:(b + 1) * blk].contiguous() for b in order]
    pos = [b * blk for b in order]
    o = torch.full((B, H, Nq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, Nq), float("nan"), device="cuda")
    work = torch.full((eta.ring_work_floats(B, H, Nq, d),), float("nan"), device="cuda")
    eta.attn_fwd_ring(q, kb, vb, pos, o, lse, work, causal, q_pos0, scale)
    torch.cuda.synchronize()
    return host(o), host(lse)


@pytest.mark.parametrize("N,blk,q_pos0,Nq,causal,order", [
    (1000, 250, 500, 250, True, [2, 1, 0, 3]),     # diagonal block, two full ones, one skipped
    (1000, 250, 0, 250, True, [0, 3, 2, 1]),       # one live block: finished against the empty state
    (924, 77, 300, 130, True, list(range(12))),    # ragged: the diagonal falls inside blocks
    (600, 200, 123, 200, False, [2, 0, 1]),        # no mask: every block, any order
])
def test_ring_share_matches_oracle(N, blk, q_pos0, Nq, causal, order):
    say(f"ring N={N} blk={blk} q_pos0={q_pos0} Nq={Nq} causal={causal} order={order}")
    qb, kb, vb = _bf16_problem(1, 2, N, N, 128, N + blk)
    q_sh = qb[:, :, q_pos0:q_pos0 + Nq]
    o, lse = _ring_run(dev_bf16(q_sh), dev_bf16(kb), dev_bf16(vb), blk, order, causal, q_pos0, 0.1)
    # global causal rule for the shard = bottom-right alignment over keys [0, q_pos0 + Nq)
    kend = q_pos0 + Nq if causal else N
    ro, rl = oracle.attention(oracle.decode_bf16(q_sh), oracle.decode_bf16(kb[:, :, :kend]),
                              oracle.decode_bf16(vb[:, :, :kend]), causal, 0.1)
    compare_o(o, ro, BF16_BAR, "ring O")
    compare_lse(lse, rl, "ring LSE")


def test_ring_share_without_allowed_keys():
    say("ring with every block masked, and with no block")
    qb, kb, vb = _bf16_problem(1, 2, 300, 300, 64, 5)
    q = dev_bf16(qb[:, :, :100])
    for order in ([1, 2], []):  # blocks at keys 100.. and 200..: after every row of the shard
        o, lse = _ring_run(q, dev_bf16(kb), dev_bf16(vb), 100, order, True, 0, 0.1)
        assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_workload_ring_share():
    name = "bf16_causal_ring_B1_H16_N65536_R8_d128"
    say(name)
    cfg, seed = configs.WORKLOADS[name], configs.seed_of(name)
    B, H, Nq, Nk, d, nb = cfg["B"], cfg["H"], cfg["Nq"], cfg["Nk"], cfg["d"], cfg["n_blocks"]
    scale, q_pos0 = configs.scale_of(name), cfg["q_pos0"]
    x = inputs.make_inputs(cfg, seed)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    order = [b for b, _ in configs.ring_hops(name)]
    o_r, l_r = _ring_run(q, k, v, Nk // nb, order, True, q_pos0, scale)
    # this shard ends at the last key, so one-pass causal attention over all keys is the same problem
    assert q_pos0 + Nq == Nk
    o_1, l_1 = _run_fwd(x["q"], x["k"], x["v"], True, scale)
    compare_o(o_r, o_1, BF16_BAR, "ring vs one-pass (all rows)")
    compare_lse(l_r, l_1, "ring vs one-pass LSE")
    rows = _sample_rows(Nq, cfg["oracle_rows"], seed)
    ro, rl = oracle.attention(oracle.decode_bf16(x["q"]), oracle.decode_bf16(x["k"]), oracle.decode_bf16(x["v"]),
                              True, scale, rows=rows)
    compare_o(o_r[:, :, rows], ro, BF16_BAR, "ring vs oracle")
    compare_lse(l_r[:, :, rows], rl, "ring LSE vs oracle")


@pytest.mark.parametrize("rotate,mode", [(False, "qk16"), (True, "fp8"), (True, "qk16"),
                                         pytest.param(False, "fp8", marks=XFAIL_FP8_UNROTATED)])
def test_workload_fp8(rotate, mode):
    """The fp8 workload at full size, every row of every head, both input variants (un-rotated and
    Hadamard-rotated) on both Q.K forms; the fp8-MFMA form on un-rotated inputs is an expected
    failure (see XFAIL_FP8_UNROTATED)."""
    name = "fp8_B4_H16_N4096_d128"
    say(f"{name} rotate={rotate} mode={mode} rows/head=all")
    cfg, seed = configs.WORKLOADS[name], configs.seed_of(name)
    x = inputs.make_inputs(cfg, seed, rotate=rotate)
    scale = configs.scale_of(name)
    o, lse = _run_fp8(x, False, scale, mode)
    ro, rl = _fp8_ref(x, False, scale)
    compare_o(o, ro, FP8_BAR, f"O fp8 ({cfg['Nq']} rows/head)")
    compare_lse(lse, rl, "LSE fp8")
