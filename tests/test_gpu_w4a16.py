"""GPU parity of the W4A16 layer (4-bit weights widened in registers, fp16
activations) against the fp64 oracle, through the C ABI.

Two bars.  With integer activations and power-of-two scales every product and
partial sum the kernel forms is exact in fp32, so y must equal the oracle
rounded once to fp16, bit for bit.  With N(0,1) activations and general fp16
scales the kernel's fp32 sums round: the bar is half an fp16 ulp of each
element (2^-11 |y|, the final rounding) plus 2^-12 max|y| for the fp32
accumulation, whose size is estimated at about 1e-4 of rms(y)."""
import numpy as np
import pytest
import torch

import exact_tiled_attention_15_amd as eta
import oracle
from exact_tiled_attention_15_amd import configs, inputs
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

G = eta.W4A16_GROUP


def _upload(d):
    x = torch.from_numpy(d["x"].view(np.int16)).view(torch.float16).cuda()
    packed = torch.from_numpy(d["packed"].view(np.int32)).cuda()
    scales = torch.from_numpy(d["scales"].view(np.int16)).view(torch.float16).cuda()
    zeros = torch.from_numpy(d["zeros"]).cuda()
    return x, packed, scales, zeros


def _run(d, canary=True):
    """Returns y (float64 [M,N]) and checks that nothing outside y was written."""
    x, packed, scales, zeros = _upload(d)
    M, N = x.shape[0], packed.shape[0]
    pad = 64
    flat = torch.full((M * N + 2 * pad,), float("nan"), dtype=torch.float16, device="cuda")
    y = flat[pad:pad + M * N].view(M, N)
    nw = eta.w4a16_work_floats(M, N, x.shape[1])
    work = torch.empty(nw, dtype=torch.float32, device="cuda") if nw else None
    eta.w4a16_gemm(x, packed, scales, zeros, y, work)
    torch.cuda.synchronize()
    if canary:
        guard = torch.cat([flat[:pad], flat[pad + M * N:]])
        assert bool(torch.isnan(guard).all()), "w4a16_gemm wrote outside y"
    return y.float().cpu().numpy().astype(np.float64)


def _ref(d, rows=None):
    if rows is None:
        return oracle.w4a16(d["x"], d["packed"], d["zeros"], d["scales"], G)
    return oracle.w4a16(d["x"], d["packed"][rows], d["zeros"][rows], d["scales"][rows], G)


def _check_realistic(got, ref, what):
    err = np.abs(got - ref)
    tol = 2.0**-11 * np.abs(ref) + 2.0**-12 * float(np.abs(ref).max())
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    worst = float((err / tol).max())
    say(f"  {what}: max_abs={float(err.max()):.3e} rel_frob={rel:.3e} max|ref|={float(np.abs(ref).max()):.3f} "
        f"worst err/tol={worst:.3f}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert np.all(err <= tol), f"{what}: error above half an fp16 ulp + 2^-12 max|y| (worst ratio {worst:.3f})"
    assert rel <= 2.0**-11, f"{what}: rel_frob {rel:.3e}"


SHAPES = [
    # (M, N, K): ragged tokens and rows, one to many groups, one to several K splits
    (1, 1, 128), (1, 16, 128), (2, 17, 256), (7, 100, 1024), (16, 33, 3072), (16, 256, 8192),
    (3, 40, 28672), (16, 1000, 4096), (5, 4096, 1152), (16, 2048, 16384),
    # more than one pass of 16 tokens
    (17, 100, 1024), (40, 300, 2048), (64, 1024, 28672),
]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_w4a16_exact_inputs_bit_exact(M, N, K):
    say(f"w4a16 exact M={M} N={N} K={K} work={eta.w4a16_work_floats(M, N, K)}")
    d = inputs.make_w4a16_inputs(M, N, K, G, seed=100 + M + N + K, exact=True)
    ref = _ref(d)
    # |x| <= 2, |q - z| <= 15, 2^-7 <= s <= 2^-4: every partial sum the kernel
    # forms over any set of groups is a multiple of 2^-7 of magnitude at most
    # K * 2 * 15 / 16 < 2^17, and every in-group MFMA sum is an integer below
    # 2^24, so all of them are exact in fp32; the only rounding is the final
    # one to fp16.
    assert K * 2 * 15 / 16 < 2**17
    got = _run(d)
    want = ref.astype(np.float16).astype(np.float64)
    bad = int((got != want).sum())
    say(f"  mismatches vs fp16(oracle): {bad} of {got.size}")
    assert bad == 0


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_w4a16_realistic_inputs(M, N, K):
    say(f"w4a16 M={M} N={N} K={K}")
    d = inputs.make_w4a16_inputs(M, N, K, G, seed=200 + M + N + K)
    _check_realistic(_run(d), _ref(d), "y")


def test_w4a16_codes_at_zero_point_give_exact_zero():
    # Exact-input recipe: the kernel removes the widening offsets in fp32, so a
    # zero result is exact only when its partial sums are (as here).
    M, N, K = 16, 64, 1024
    d = inputs.make_w4a16_inputs(M, N, K, G, seed=5, exact=True)
    z = d["zeros"]
    # every code of row n, group g equals zeros[n, g]: one word per eight codes
    words = (z.astype(np.uint32) * np.uint32(0x11111111))
    d["packed"] = np.ascontiguousarray(np.repeat(words, G // 8, axis=1))
    got = _run(d)
    assert np.all(got == 0.0)


def test_w4a16_extreme_codes_and_zero_points():
    # codes 0 and 15 against zero points 15 and 0: the largest |q - z|
    M, N, K = 4, 48, 2048
    d = inputs.make_w4a16_inputs(M, N, K, G, seed=6)
    rng = np.random.default_rng(6)
    d["packed"] = rng.choice(np.array([0x00000000, 0xFFFFFFFF], dtype=np.uint32), size=d["packed"].shape)
    d["zeros"] = rng.choice(np.array([0, 15], dtype=np.uint8), size=d["zeros"].shape)
    _check_realistic(_run(d), _ref(d), "y")


def test_w4a16_is_deterministic():
    d = inputs.make_w4a16_inputs(16, 300, 28672, G, seed=7)
    a = _run(d)
    b = _run(d)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("name", ["w4a16_decode_M16_N28672_K8192_G128", "w4a16_decode_M16_N8192_K28672_G128"])
def test_w4a16_full_size_sampled_rows(name):
    cfg = configs.WORKLOADS[name]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    say(f"{name}: work={eta.w4a16_work_floats(M, N, K)}")
    d = inputs.make_w4a16_inputs(M, N, K, G, seed=cfg.get("seed", 0))
    got = _run(d, canary=False)
    rows = inputs.row_subset(N, 512, seed=11)
    _check_realistic(got[:, rows], _ref(d, rows), f"{name} on {len(rows)} sampled rows")
