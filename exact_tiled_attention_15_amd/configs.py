"""The synthetic workloads: shapes, dtypes, masks and seeds.

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
    # One GPU's share of causal ring attention: the last of 8 ranks over a 65536-token
    # sequence (contiguous sharding, the most loaded rank); its shard of 8192 query rows
    # sits at global positions 57344.., and the ring delivers its own K/V block first,
    # then its predecessors' (hop order 7, 6, .., 0).
    "bf16_causal_ring_B1_H16_N65536_R8_d128": dict(index=5, B=1, H=16, Nq=8192, Nk=65536, d=128,
                                                   dtype="bf16", causal=True, n_blocks=8,
                                                   q_pos0=57344, ring=True, oracle_rows=512),
    # The kvblocks share with the 8 K/V blocks arriving from page-locked host memory,
    # each block's transfer overlapped with the previous block's attention (the host link
    # stands in for the ring's peer link).
    "bf16_ring_host_B1_H16_Nq8192_Nk65536x8_d128": dict(index=10, B=1, H=16, Nq=8192, Nk=65536,
                                                        d=128, dtype="bf16", causal=False,
                                                        n_blocks=8, host_kv=True, oracle_rows=512),
    # The backward pass (dQ, dK, dV from the saved LSE) of the GPT-style causal shape; dO
    # is a seeded N(0,1) draw (sub-stream 6).
    "bwd_bf16_causal_B8_H16_N2048_d128": dict(index=6, B=8, H=16, Nq=2048, Nk=2048, d=128,
                                              dtype="bf16", causal=True, backward=True),
    # Block-quantized e4m3 with 1% outlier channels (x20), optional Hadamard rotation.
    # Timed with the rotation applied (the fp8 matrix cores need it on outlier channels).
    "fp8_B4_H16_N4096_d128": dict(index=4, B=4, H=16, Nq=4096, Nk=4096, d=128, dtype="fp8",
                                  causal=False, outlier_frac=0.01, outlier_mult=20.0,
                                  oracle_rows=512, rotate=True),
    # The same workload (same seed and draws) without the rotation, Q.K on fp16 matrix cores
    # over the widened codes (attn_fwd_fp8_qk16): the form that meets the fp8 bar on an
    # un-rotated outlier channel.
    "fp8_norot_qk16_B4_H16_N4096_d128": dict(index=4, B=4, H=16, Nq=4096, Nk=4096, d=128, dtype="fp8",
                                             causal=False, outlier_frac=0.01, outlier_mult=20.0,
                                             oracle_rows=512, rotate=False, qk16=True),
    # The same recipe with the probabilities in e4m3 too (both products on fp8 matrix cores).
    "fp8_pv8_B4_H16_N4096_d128": dict(index=7, B=4, H=16, Nq=4096, Nk=4096, d=128, dtype="fp8",
                                      causal=False, outlier_frac=0.01, outlier_mult=20.0,
                                      oracle_rows=512, rotate=True, pv8=True),
    # The same inputs with the probabilities as 4-bit e2m1 codes (P.V on the f8f6f4 matrix cores
    # with V's e4m3 codes): each exponential rounded, and Direct-P (score mapped straight to the
    # code).  Same seed as the e4m3-P workload, so the drifts compare on identical inputs.
    "fp8_pv4_B4_H16_N4096_d128": dict(index=7, B=4, H=16, Nq=4096, Nk=4096, d=128, dtype="fp8",
                                      causal=False, outlier_frac=0.01, outlier_mult=20.0,
                                      oracle_rows=512, rotate=True, pv4=True),
    "fp8_directp_B4_H16_N4096_d128": dict(index=7, B=4, H=16, Nq=4096, Nk=4096, d=128, dtype="fp8",
                                          causal=False, outlier_frac=0.01, outlier_mult=20.0,
                                          oracle_rows=512, rotate=True, pv4=True, direct_p=True),
    # W4A16 linear layers of token-by-token decoding ("Scaling FlashAttention, multi-GPU
    # training and weight quantization", section 3: a 70-billion-parameter model whose
    # weights, not its arithmetic, bound each generated token).  The two shapes of a
    # 70B-class MLP (hidden size 8192, intermediate 28672) for a batch of 16 sequences,
    # groups of 128.  Weights are seeded random words, scales and zero points seeded
    # draws (inputs.make_w4a16_inputs); the benchmark rotates through enough copies of
    # the weights that none is still in the 256 MB last-level cache when it is re-read.
    "w4a16_decode_M16_N28672_K8192_G128": dict(index=8, kind="w4a16", M=16, N=28672, K=8192,
                                               group=128, seed=1008, weight_copies=4),
    "w4a16_decode_M16_N8192_K28672_G128": dict(index=9, kind="w4a16", M=16, N=8192, K=28672,
                                               group=128, seed=1009, weight_copies=4),
    # Matrix-core throughput loops (attn_mfma_peak): one workgroup of 8 wavefronts per compute
    # unit, four independent accumulator chains per wavefront, register operands.  The measured
    # peak that the attention workloads are also reported against.
    "mfma_peak_bf16": dict(index=11, kind="mfma", mfma="bf16", iters=100000),
    "mfma_peak_fp8": dict(index=12, kind="mfma", mfma="fp8", iters=50000),
    "mfma_peak_f16": dict(index=13, kind="mfma", mfma="f16", iters=100000),
    "mfma_peak_f32": dict(index=14, kind="mfma", mfma="f32", iters=50000),
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


def ring_hops(name: str):
    """(block index, global key position) per hop of a ring workload, in hop order."""
    cfg = WORKLOADS[name]
    nb, blk = cfg["n_blocks"], cfg["Nk"] // cfg["n_blocks"]
    own = cfg["q_pos0"] // blk
    order = [(own - h) % nb for h in range(nb)]
    return [(b, b * blk) for b in order]


def workload_flops(name: str) -> float:
    """FLOPs credited to one pass of a workload: the metric convention, except that a
    causal ring share counts its allowed (query, key) pairs exactly and a backward pass
    counts 2.5 times its forward (the usual convention for attention training)."""
    cfg = WORKLOADS[name]
    B, H, Nq, Nk, d = cfg["B"], cfg["H"], cfg["Nq"], cfg["Nk"], cfg["d"]
    if cfg.get("backward"):
        # five matrix products of 2 Nq Nk d each against the forward's two
        return 2.5 * flops(B, H, Nq, Nk, d, cfg["causal"])
    if cfg.get("ring") and cfg["causal"]:
        q0 = cfg["q_pos0"]
        pairs = Nq * q0 + Nq * (Nq + 1) // 2  # row q0 + i sees keys 0 .. q0 + i
        return 4.0 * B * H * d * pairs
    return flops(B, H, Nq, Nk, d, cfg["causal"])


def w4a16_bytes(name: str) -> int:
    """Bytes one W4A16 call must move at least: packed weights (K/2 per row), fp16
    scales and byte zero points per group, fp16 activations in and fp16 outputs out."""
    cfg = WORKLOADS[name]
    M, N, K, G = cfg["M"], cfg["N"], cfg["K"], cfg["group"]
    return N * K // 2 + N * (K // G) * 3 + M * K * 2 + M * N * 2
