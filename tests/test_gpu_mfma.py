"""How one matrix-core instruction sums its products (attn_mfma_dot), and the throughput loop
(attn_mfma_peak) that the benchmark reports the attention kernels against.

The operands are e4m3 values that are exact in bf16 and fp16, with integer magnitudes, so every
product and every partial sum is an integer below 2^24: the exact result is representable in fp32
whatever the summation order, and any difference from it is the instruction's own rounding."""
import numpy as np
import pytest
import torch

import exact_tiled_attention_15_amd as eta
import oracle
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

# e4m3 code -> value, from the oracle's decoder (exact)
E4M3 = np.array([oracle.e4m3_value(c) for c in range(256)])


def _codes_of(values):
    """e4m3 codes of exactly representable values (positive and negative)."""
    out = np.empty(values.shape, dtype=np.uint8)
    for idx, x in np.ndenumerate(values):
        c = int(np.flatnonzero(E4M3 == x)[0])
        out[idx] = c
    return out


def _dot(kind, a_vals, b_vals):
    """C = A B^T on the GPU for A, B given as float64 values [32, 64]."""
    if kind == eta.MFMA_FP8:
        a = torch.from_numpy(_codes_of(a_vals)).cuda()
        b = torch.from_numpy(_codes_of(b_vals)).cuda()
    else:
        dt = torch.bfloat16 if kind == eta.MFMA_BF16 else torch.float16
        a = torch.from_numpy(a_vals.astype(np.float32)).to(dt).cuda()
        b = torch.from_numpy(b_vals.astype(np.float32)).to(dt).cuda()
        assert np.array_equal(a.double().cpu().numpy(), a_vals)  # the values are exact in 16 bits
    c = torch.full((32, 32), float("nan"), device="cuda")
    eta.mfma_dot(kind, a, b, c)
    torch.cuda.synchronize()
    return c.double().cpu().numpy()


def _small_integers(rng, shape):
    """Integers in +-[1, 15]: exact in e4m3, bf16 and fp16; products up to 225."""
    return rng.integers(1, 16, shape).astype(np.float64) * rng.choice([-1.0, 1.0], shape)


@pytest.mark.parametrize("kind", [eta.MFMA_FP8, eta.MFMA_BF16, eta.MFMA_F16])
def test_products_of_like_size_are_summed_exactly(kind):
    say(f"mfma_dot kind={kind}: products of like size")
    rng = np.random.default_rng(3)
    a, b = _small_integers(rng, (32, 64)), _small_integers(rng, (32, 64))
    c = _dot(kind, a, b)
    np.testing.assert_array_equal(c, a @ b.T)


def test_layout_of_rows_columns_and_k():
    """One-hot operands: C_ij = A_ik B_jk picks one product; checks the row, column and k
    placement of all three instruction forms."""
    say("mfma_dot one-hot layout")
    for kind in (eta.MFMA_FP8, eta.MFMA_BF16, eta.MFMA_F16):
        for (i, j, k) in [(0, 0, 0), (5, 17, 33), (31, 2, 63), (12, 31, 31), (20, 9, 32)]:
            a = np.zeros((32, 64))
            b = np.zeros((32, 64))
            a[i, k], b[j, k] = 3.0, 5.0
            c = _dot(kind, a, b)
            want = np.zeros((32, 32))
            want[i, j] = 15.0
            np.testing.assert_array_equal(c, want)


def test_fp8_instruction_truncates_small_products_next_to_a_large_one():
    """One 448 x 448 product next to 63 small ones.  The bf16 and fp16 instructions return the
    exact sum; the fp8 instruction loses the small products' low bits on the outputs that hold
    the large product (and only there).  This is why an un-rotated outlier channel shared by Q and
    K pushes attn_fwd_fp8's scores off (Q.K on this instruction), and why rotating Q and K before
    quantization, which spreads the channel over all d, removes the effect."""
    say("mfma_dot: one large product among small ones")
    rng = np.random.default_rng(5)
    a, b = _small_integers(rng, (32, 64)), _small_integers(rng, (32, 64))
    big_rows, big_cols, k0 = np.arange(0, 32, 2), np.arange(0, 32, 3), 21
    a[big_rows, k0] = 448.0
    b[big_cols, k0] = 448.0
    exact = a @ b.T
    has_big = np.zeros((32, 32), dtype=bool)
    has_big[np.ix_(big_rows, big_cols)] = True
    for kind in (eta.MFMA_BF16, eta.MFMA_F16):
        np.testing.assert_array_equal(_dot(kind, a, b), exact)
    c8 = _dot(eta.MFMA_FP8, a, b)
    err = c8 - exact
    say(f"  fp8: outputs without the large product: max |err| = {np.abs(err[~has_big]).max():.3g}")
    say(f"  fp8: outputs with it (exact ~2.0e5): max |err| = {np.abs(err[has_big]).max():.3g}, "
        f"mean err = {err[has_big].mean():.3g}, min |err| = {np.abs(err[has_big]).min():.3g}")
    np.testing.assert_array_equal(c8[~has_big], exact[~has_big])
    # the sum of the 63 small products is at most 63 * 225 in magnitude: whatever is lost is part of it
    assert np.abs(err[has_big]).max() <= 63 * 225


def test_peak_loop_runs_and_counts_flops():
    say("mfma_peak: short loops of every kind")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.full((cus * eta.MFMA_PEAK_THREADS,), float("nan"), device="cuda")
    for kind in (eta.MFMA_BF16, eta.MFMA_F16, eta.MFMA_FP8, eta.MFMA_F32):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        eta.mfma_peak(kind, cus, 200, out)
        e0.record()
        eta.mfma_peak(kind, cus, 2000, out)
        e1.record()
        torch.cuda.synchronize()
        tf = eta.mfma_peak_flop(kind, cus, 2000) / (e0.elapsed_time(e1) * 1e-3) / 1e12
        say(f"  kind {kind}: {tf:.0f} TFLOP/s over {cus} workgroups")
        assert torch.isfinite(out).all() and tf > 0
