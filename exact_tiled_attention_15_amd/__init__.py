"""Exact, IO-aware attention forward for AMD Instinct MI355X (gfx950), and the
W4A16 linear layer (4-bit weights widened in registers).

The compute lives in libattn.so (hand-written HIP kernels behind the C ABI of
include/attn.h); this package is its thin Python binding plus the seeded
synthetic-input generators and workload table used by the tests and the
benchmark.
"""
from ._lib import (  # noqa: F401
    ATTN_ERR_HIP,
    ATTN_ERR_INVALID,
    ATTN_ERR_UNSUPPORTED,
    ATTN_OK,
    FP8_TILE,
    MFMA_BF16,
    MFMA_F16,
    MFMA_F32,
    MFMA_FP8,
    MFMA_PEAK_THREADS,
    W4A16_GROUP,
    W4A16_MAX_M,
    W4A16_NOALLOC_MAX_WORK_FLOATS,
    W4A16_TOKENS_PER_PASS,
    AttnError,
    abi_version,
    attn_bwd,
    attn_fwd_block_order,
    attn_fwd,
    attn_fwd_f32,
    attn_fwd_fp8,
    attn_fwd_fp8_pv4,
    attn_fwd_fp8_pv8,
    attn_fwd_fp8_qk16,
    attn_fwd_kvblock,
    attn_fwd_ring,
    attn_fwd_ring_host,
    attn_merge,
    bwd_work_floats,
    lib,
    mfma_dot,
    mfma_peak,
    mfma_peak_flop,
    ring_stage_bytes,
    ring_work_floats,
    status_str,
    w4a16_gemm,
    w4a16_gemm_noalloc,
    w4a16_work_floats,
)
