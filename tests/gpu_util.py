"""Helpers shared by the GPU tests: uploads and the parity metrics."""
import sys

import numpy as np
import torch

# Bars (max-abs, relative Frobenius) for O, and max-abs for LSE.
BF16_BAR = (1e-2, 5e-3)
FP8_BAR = (3e-2, 2e-2)
LSE_BAR = 1e-3


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy().astype(np.float64)


def compare_o(got: np.ndarray, ref: np.ndarray, bar, what: str):
    err = np.abs(got - ref)
    max_abs = float(err.max()) if err.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / nref) if nref > 0 else float(np.linalg.norm(got - ref))
    say(f"  {what}: max_abs={max_abs:.3e} rel_frob={rel:.3e} max|ref|={float(np.abs(ref).max()):.3f}")
    if max_abs > bar[0]:
        idx = np.unravel_index(int(np.argmax(err)), err.shape)
        r = abs(ref[idx])
        half_ulp_bf16 = 2.0 ** (np.floor(np.log2(r)) - 8) if r > 0 else 0.0
        say(f"  worst element {idx}: got={got[idx]:.6f} ref={ref[idx]:.6f} bf16 half-ulp={half_ulp_bf16:.3e}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert max_abs <= bar[0], f"{what}: max_abs {max_abs:.3e} > {bar[0]}"
    assert rel <= bar[1], f"{what}: rel_frob {rel:.3e} > {bar[1]}"
    return max_abs, rel


def compare_lse(got: np.ndarray, ref: np.ndarray, what: str, bar: float = LSE_BAR):
    neg = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), neg), f"{what}: -inf pattern differs"
    d = np.abs(got[~neg] - ref[~neg])
    m = float(d.max()) if d.size else 0.0
    say(f"  {what}: lse max_abs={m:.3e}")
    assert m <= bar, f"{what}: lse max_abs {m:.3e} > {bar}"
    return m
