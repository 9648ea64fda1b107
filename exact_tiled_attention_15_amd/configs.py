"""The five synthetic workloads: shapes, dtypes, masks and seeds.

Inputs are seeded synthetic draws with these shapes and value distributions;
no public benchmark, evaluation suite or dataset is involved.  The seed of
workload i is 1000 + i; its sub-streams are 0/1/2 for Q/K/V, 3 for the outlier
channels, 4 for the rotation signs, 5 for the sampled query rows.
"""
import math

WORKLOADS = {
    # Tiny fp32 attention: fp32 matrix cores, full-size oracle in well under a second.
    "f32_B1_H2_N256_d64": dict(index=0, B=1, H=2, Nq=256, Nk=256, d=64, dtype="f32",
                               causal=False),
    # GPT-style training shape, causal.
    "bf16_causal_B8_H16_N2048_d128": dict(index=1, B=8, H=16, Nq=2048, Nk=2048, d=128,
                                          dtype="bf16", causal=True),
    # Long sequence, small batch: sequence-length parallelism must fill the chip.
    "bf16_causal_B1_H8_N32768_d128": dict(index=2, B=1, H=8, Nq=32768, Nk=32768, d=128,
                                          dtype="bf16", causal=True, oracle_rows=512),
    # One GPU's ring-attention share: local queries, K/V delivered in 8 blocks.
    "bf16_kvblocks_B1_H16_Nq8192_Nk65536x8_d128": dict(index=3, B=1, H=16, Nq=8192, Nk=65536,
                                                       d=128, dtype="bf16", causal=False,
                                                       n_blocks=8, oracle_rows=512),
    # Block-quantized e4m3 with 1% outlier channels (x20), optional Hadamard rotation.
    "fp8_B4_H16_N4096_d128": dict(index=4, B=4, H=16, Nq=4096, Nk=4096, d=128, dtype="fp8",
                                  causal=False, outlier_frac=0.01, outlier_mult=20.0,
                                  oracle_rows=512),
}

HEADLINE = "bf16_causal_B8_H16_N2048_d128"


def seed_of(name: str) -> int:
    return 1000 + WORKLOADS[name]["index"]


def scale_of(name: str) -> float:
    return 1.0 / math.sqrt(WORKLOADS[name]["d"])


def flops(B: int, H: int, Nq: int, Nk: int, d: int, causal: bool) -> float:
    """Metric convention: 4*B*H*Nq*Nk*d, halved for a causal mask."""
    f = 4.0 * B * H * Nq * Nk * d
    return f / 2 if causal else f
