"""Seeded synthetic inputs, shared by the GPU path's tests/benchmark and the
CPU oracle's.  This module draws and encodes numbers only; it holds none of
the arithmetic of attention or of the W4A16 layer.

* Normal draws: numpy PCG64 ``default_rng([seed, stream])``.
* bfloat16: round-to-nearest-even of the float32 draw (bit patterns, uint16).
* Outlier channels: max(1, round(frac * d)) channels, one set shared by Q, K
  and V, multiplied by a constant after the draw.
* Rotation ("incoherent processing" of "Scaling FlashAttention, multi-GPU
  training and weight quantization", itimpress, section 1, FP8 bullet): the
  same random orthogonal matrix M = H_d diag(sigma) / sqrt(d) (Sylvester
  Hadamard, seeded signs) multiplies Q and K on the right, so Q K^T is
  unchanged in exact arithmetic.
* W4A16 layer inputs (same page, section 3): every 32-bit word is a valid
  packing of eight 4-bit codes, so packed weights are uniform random words;
  zero points are uniform in 0..15, scales uniform in [2e-3, 6e-3] rounded to
  float16, activations N(0, 1) rounded to float16.  The "exact" variant draws
  integer activations in -2..2 and power-of-two scales 2^-7..2^-4, so every
  product and partial sum of a layer with K below 34952 is exact in float32.
* Block quantization (same passage: a separate scale per small tile): per
  (b, h, 128-token tile) scale s = float32(amax / 448) (1 when amax = 0), code
  = OCP e4m3 round-to-nearest-even of float32(x / s) clipped to +-448.
"""
import numpy as np
import torch

E4M3_MAX = 448.0


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream])


def normal_f32(shape, seed: int, stream: int) -> np.ndarray:
    return rng(seed, stream).standard_normal(shape, dtype=np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def outlier_channels(d: int, seed: int, frac: float) -> np.ndarray:
    n = max(1, int(round(frac * d)))
    return np.sort(rng(seed, 3).choice(d, size=n, replace=False))


def sylvester_hadamard(d: int) -> np.ndarray:
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotation(d: int, seed: int) -> np.ndarray:
    """Random orthogonal d x d matrix (float64): Hadamard times random signs / sqrt(d)."""
    signs = rng(seed, 4).choice(np.array([-1.0, 1.0]), size=d)
    return sylvester_hadamard(d) * signs[None, :] / np.sqrt(d)


def quantize_e4m3_tiles(x: np.ndarray, tile: int = 128):
    """x float32 [B,H,N,d] -> (codes uint8 [B,H,N,d], scales float32 [B,H,ceil(N/tile)])."""
    B, H, N, d = x.shape
    nt = (N + tile - 1) // tile
    pad = nt * tile - N
    xp = np.pad(x, ((0, 0), (0, 0), (0, pad), (0, 0))) if pad else x
    xt = xp.reshape(B, H, nt, tile, d)
    amax = np.abs(xt).max(axis=(3, 4)).astype(np.float64)
    scales = (amax / E4M3_MAX).astype(np.float32)
    scales[amax == 0] = 1.0
    y = (xt / scales[:, :, :, None, None]).astype(np.float32)
    y = np.clip(y, -E4M3_MAX, E4M3_MAX)
    codes = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    codes = codes.reshape(B, H, nt * tile, d)[:, :, :N, :]
    return np.ascontiguousarray(codes), scales


def row_subset(Nq: int, n: int, seed: int) -> np.ndarray:
    """n distinct query rows, uniform without replacement, sorted (int64)."""
    if n >= Nq:
        return np.arange(Nq, dtype=np.int64)
    return np.sort(rng(seed, 5).choice(Nq, size=n, replace=False)).astype(np.int64)


def make_inputs(cfg: dict, seed: int, rotate: bool = False) -> dict:
    """Host inputs for one workload (see configs.WORKLOADS)."""
    B, H, Nq, Nk, d = cfg["B"], cfg["H"], cfg["Nq"], cfg["Nk"], cfg["d"]
    q = normal_f32((B, H, Nq, d), seed, 0)
    k = normal_f32((B, H, Nk, d), seed, 1)
    v = normal_f32((B, H, Nk, d), seed, 2)
    if cfg["dtype"] == "f32":
        return dict(q=q, k=k, v=v)
    if cfg["dtype"] == "bf16":
        return dict(q=bf16_bits(q), k=bf16_bits(k), v=bf16_bits(v))
    if cfg["dtype"] == "fp8":
        ch = outlier_channels(d, seed, cfg.get("outlier_frac", 0.01))
        mult = np.float32(cfg.get("outlier_mult", 20.0))
        for t in (q, k, v):
            t[..., ch] *= mult
        if rotate:
            m = rotation(d, seed)
            q = (q.astype(np.float64) @ m).astype(np.float32)
            k = (k.astype(np.float64) @ m).astype(np.float32)
        q8, qs = quantize_e4m3_tiles(q)
        k8, ks = quantize_e4m3_tiles(k)
        v8, vs = quantize_e4m3_tiles(v)
        return dict(q8=q8, k8=k8, v8=v8, q_scale=qs, k_scale=ks, v_scale=vs, channels=ch,
                    q_unquantized=q, k_unquantized=k, v_unquantized=v)
    raise ValueError(cfg["dtype"])


def fp16_bits(x: np.ndarray) -> np.ndarray:
    """float -> IEEE binary16 bit patterns, round to nearest even."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def make_w4a16_inputs(M: int, N: int, K: int, group: int, seed: int, exact: bool = False) -> dict:
    """Host inputs of one W4A16 layer call: x fp16 bits [M, K], packed uint32
    [N, K/8], zeros uint8 [N, K/group], scales fp16 bits [N, K/group]."""
    if K % 8 or K % group:
        raise ValueError("K must be a multiple of 8 and of the group size")
    ng = K // group
    g = rng(seed, 10)
    packed = g.integers(0, 2**32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    zeros = g.integers(0, 16, size=(N, ng), dtype=np.uint8)
    if exact:
        scales = np.exp2(g.integers(-7, -3, size=(N, ng))).astype(np.float32)
        x = rng(seed, 11).integers(-2, 3, size=(M, K)).astype(np.float32)
    else:
        scales = g.uniform(2e-3, 6e-3, size=(N, ng)).astype(np.float32)
        x = normal_f32((M, K), seed, 11)
    return dict(x=fp16_bits(x), packed=packed, zeros=zeros, scales=fp16_bits(scales))
