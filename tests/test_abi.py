"""CPU-side checks of the C ABI: the built library exports every function
include/attn.h declares, and rejects invalid arguments on the host (before
any HIP call, so these run without a GPU).  No compute call is made here."""
import ctypes
import os
import re

import pytest

import exact_tiled_attention_15_amd as eta

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(REPO, "include", h) for h in sorted(os.listdir(os.path.join(REPO, "include")))
           if h.endswith(".h")]

P16 = ctypes.c_void_p(0x10000)   # never dereferenced: every call below fails validation
P16b = ctypes.c_void_p(0x20000)
P16c = ctypes.c_void_p(0x30000)
P16d = ctypes.c_void_p(0x40000)
P4 = ctypes.c_void_p(0x50004)
MIS = ctypes.c_void_p(0x60008)   # 8-byte aligned only
NUL = None


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b((?:attn|w4a16)_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"attn_fwd", "attn_fwd_f32", "attn_fwd_kvblock", "attn_merge", "attn_fwd_fp8",
            "attn_abi_version", "attn_status_str", "w4a16_gemm", "w4a16_work_floats",
            "attn_mfma_peak", "attn_mfma_dot", "attn_mfma_peak_flop", "attn_fwd_block_order",
            "w4a16_gemm_noalloc"} <= set(names)
    L = eta.lib()
    for n in names:
        assert hasattr(L, n), f"{n} not exported by libattn.so"


def test_version_and_status_strings():
    assert eta.abi_version() == 1
    for s in range(4):
        assert eta.status_str(s).startswith("ATTN_")
    assert "unknown" in eta.status_str(99)


def fwd(*, q=P16, k=P16b, v=P16c, o=P16d, lse=NUL, B=1, H=1, Nq=8, Nk=8, d=64, causal=0, scale=0.125):
    return eta.lib().attn_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=NUL), eta.ATTN_ERR_INVALID),
    (dict(o=NUL), eta.ATTN_ERR_INVALID),
    (dict(B=0), eta.ATTN_ERR_INVALID),
    (dict(H=-1), eta.ATTN_ERR_INVALID),
    (dict(Nq=0), eta.ATTN_ERR_INVALID),
    (dict(Nk=0), eta.ATTN_ERR_INVALID),
    (dict(d=0), eta.ATTN_ERR_INVALID),
    (dict(d=96), eta.ATTN_ERR_UNSUPPORTED),
    (dict(d=256), eta.ATTN_ERR_UNSUPPORTED),
    (dict(k=MIS), eta.ATTN_ERR_INVALID),
    (dict(lse=ctypes.c_void_p(0x50002)), eta.ATTN_ERR_INVALID),
    (dict(scale=float("nan")), eta.ATTN_ERR_INVALID),
    (dict(scale=float("inf")), eta.ATTN_ERR_INVALID),
    (dict(Nq=(1 << 30) + 1), eta.ATTN_ERR_INVALID),
    (dict(B=1 << 16, H=1 << 16, Nq=1024), eta.ATTN_ERR_INVALID),  # grid > 2^31 in 64-bit math
])
def test_attn_fwd_validation(kw, want):
    assert fwd(**kw) == want


def test_f32_and_fp8_validation():
    L = eta.lib()
    assert L.attn_fwd_f32(P16, P16b, P16c, NUL, NUL, 1, 1, 8, 8, 64, 0, 0.1, None) == eta.ATTN_ERR_INVALID
    assert L.attn_fwd_f32(P16, P16b, P16c, P16d, NUL, 1, 1, 8, 8, 32, 0, 0.1, None) == eta.ATTN_ERR_UNSUPPORTED
    fp8 = lambda qs, ks, vs, d=128: L.attn_fwd_fp8(P16, P16b, P16c, qs, ks, vs, P16d, NUL, 1, 1, 8, 8, d, 0,
                                                   0.1, None)
    assert fp8(NUL, P4, P4) == eta.ATTN_ERR_INVALID
    assert fp8(P4, P4, ctypes.c_void_p(0x50001)) == eta.ATTN_ERR_INVALID
    assert fp8(P4, P4, P4, d=80) == eta.ATTN_ERR_UNSUPPORTED


def test_kvblock_and_merge_validation():
    L = eta.lib()
    kv = lambda m, l, causal=0, qp=0, kp=0: L.attn_fwd_kvblock(P16, P16b, P16c, P16d, m, l, 1, 1, 8, 8, 64,
                                                               causal, qp, kp, 0.1, None)
    assert kv(NUL, P4) == eta.ATTN_ERR_INVALID
    assert kv(P4, NUL) == eta.ATTN_ERR_INVALID
    assert kv(P4, P4, causal=1, qp=-1) == eta.ATTN_ERR_INVALID
    assert kv(P4, P4, causal=1, kp=-5) == eta.ATTN_ERR_INVALID
    mg = lambda oa, op, d=128, of=NUL, ma=P4, mp=ctypes.c_void_p(0x70004): L.attn_merge(
        oa, ma, ctypes.c_void_p(0x80004), op, mp, ctypes.c_void_p(0x90004), of, NUL, 1, 1, 8, d, None)
    assert mg(NUL, P16b) == eta.ATTN_ERR_INVALID
    assert mg(P16, P16b, d=130) == eta.ATTN_ERR_UNSUPPORTED
    assert mg(P16, P16b, d=2048) == eta.ATTN_ERR_UNSUPPORTED
    assert mg(P16, P16) == eta.ATTN_ERR_INVALID            # o_acc aliases o_part
    assert mg(P16, P16b, ma=P4, mp=P4) == eta.ATTN_ERR_INVALID  # m_acc aliases m_part
    assert mg(P16, P16b, of=ctypes.c_void_p(0x50002)) == eta.ATTN_ERR_INVALID


def test_ring_validation():
    """attn_fwd_ring rejects bad arguments before any launch (fake pointers are never touched)."""
    L = eta.lib()
    assert L.attn_ring_work_floats(1, 2, 8, 64) == 16 * 64 + 2 * 16  # accumulated O, m, l
    assert L.attn_ring_work_floats(0, 2, 8, 64) == 0
    ks = (ctypes.c_void_p * 2)(0x100000, 0x200000)
    vs = (ctypes.c_void_p * 2)(0x300000, 0x400000)
    pos = (ctypes.c_int64 * 2)(0, 8)
    bad_pos = (ctypes.c_int64 * 2)(0, -8)
    mis = (ctypes.c_void_p * 2)(0x100000, 0x200004)
    nulls = (ctypes.c_void_p * 2)(0x100000, 0)
    ring = lambda n=2, k=ks, v=vs, p=pos, q=P16, o=P16b, w=P16c, causal=1, qp=8, d=64, scale=0.1: L.attn_fwd_ring(
        q, k, v, p, n, o, NUL, w, 1, 1, 8, 8, d, causal, qp, scale, None)
    assert ring(n=-1) == eta.ATTN_ERR_INVALID
    assert ring(k=None) == eta.ATTN_ERR_INVALID           # NULL arrays with blocks
    assert ring(p=None) == eta.ATTN_ERR_INVALID
    assert ring(p=bad_pos) == eta.ATTN_ERR_INVALID         # negative position, causal
    assert ring(qp=-1) == eta.ATTN_ERR_INVALID
    assert ring(k=mis) == eta.ATTN_ERR_INVALID             # misaligned block
    assert ring(v=nulls) == eta.ATTN_ERR_INVALID           # NULL block
    assert ring(w=NUL) == eta.ATTN_ERR_INVALID             # no workspace
    assert ring(w=MIS) == eta.ATTN_ERR_INVALID             # misaligned workspace
    assert ring(d=96) == eta.ATTN_ERR_UNSUPPORTED
    assert ring(scale=float("nan")) == eta.ATTN_ERR_INVALID


def test_ring_host_validation():
    """attn_fwd_ring_host rejects bad arguments before any HIP call."""
    L = eta.lib()
    assert L.attn_ring_stage_bytes(1, 2, 8, 64) == 4 * 2 * 8 * 64 * 2  # two slots of K and V, bf16
    assert L.attn_ring_stage_bytes(1, 2, 0, 64) == 0
    ks = (ctypes.c_void_p * 2)(0x100000, 0x200001)  # host blocks need no alignment
    vs = (ctypes.c_void_p * 2)(0x300000, 0x400000)
    nulls = (ctypes.c_void_p * 2)(0x100000, 0)
    pos = (ctypes.c_int64 * 2)(0, 8)
    work_bytes = L.attn_ring_work_floats(1, 1, 8, 64) * 4
    inside_work = ctypes.c_void_p(0x30000 + (work_bytes // 2 // 16) * 16)
    ring = lambda n=2, k=ks, v=vs, w=P16c, st=P16d, causal=1, qp=8, d=64: L.attn_fwd_ring_host(
        P16, k, v, pos, n, P16b, NUL, w, st, 1, 1, 8, 8, d, causal, qp, 0.1, None)
    assert ring(n=-1) == eta.ATTN_ERR_INVALID
    assert ring(k=None) == eta.ATTN_ERR_INVALID          # NULL array with blocks
    assert ring(v=nulls) == eta.ATTN_ERR_INVALID         # NULL host block
    assert ring(st=NUL) == eta.ATTN_ERR_INVALID          # no staging buffer
    assert ring(st=MIS) == eta.ATTN_ERR_INVALID          # misaligned staging buffer
    assert ring(st=P16c) == eta.ATTN_ERR_INVALID         # staging buffer is the workspace
    assert ring(st=inside_work) == eta.ATTN_ERR_INVALID  # ... or overlaps it
    assert ring(w=NUL) == eta.ATTN_ERR_INVALID
    assert ring(qp=-1) == eta.ATTN_ERR_INVALID
    assert ring(d=96) == eta.ATTN_ERR_UNSUPPORTED


def test_bwd_validation():
    """attn_bwd rejects bad arguments before any launch."""
    L = eta.lib()
    assert L.attn_bwd_work_floats(2, 3, 5) == 30
    assert L.attn_bwd_work_floats(2, 0, 5) == 0
    P = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(8)]
    bwd = lambda lse=P4, work=ctypes.c_void_p(0x900004), d=64, scale=0.1, dq=P[5]: L.attn_bwd(
        P[0], P[1], P[2], P[3], P[4], lse, dq, P[6], P[7], work, 1, 2, 8, 8, d, 1, scale, None)
    assert bwd(lse=NUL) == eta.ATTN_ERR_INVALID
    assert bwd(work=NUL) == eta.ATTN_ERR_INVALID
    assert bwd(dq=MIS) == eta.ATTN_ERR_INVALID
    assert bwd(d=96) == eta.ATTN_ERR_UNSUPPORTED
    assert bwd(scale=float("inf")) == eta.ATTN_ERR_INVALID


# ---------------------------------------------------------------- W4A16 layer
@pytest.mark.parametrize("M,N,K,want", [
    (16, 28672, 8192, 0),                # 64 groups: one split, y written directly
    (16, 8192, 28672, 4 * 16 * 8192),    # 224 groups: four splits of 56
    (1, 16, 4096, 32 * 1 * 16),          # one tile: K cut into one split per group
    (4, 100, 1024, 8 * 4 * 100),         # seven tiles, eight groups
    (16, 4096, 128, 0),                  # one group
    (17, 16, 4096, 32 * 16 * 16),         # two passes of 16 tokens share one workspace
    (0, 16, 128, 0), (4097, 16, 128, 0), (1, 16, 100, 0),  # rejected sizes
])
def test_w4a16_work_floats(M, N, K, want):
    assert eta.w4a16_work_floats(M, N, K) == want


def test_w4a16_work_floats_rejects_other_group_sizes():
    assert eta.w4a16_work_floats(1, 16, 256, 64) == 0


def w4(*, x=P16, packed=P16b, scales=P4, zeros=P4, y=P4, work=NUL, M=4, N=32, K=256, group=128):
    return eta.lib().w4a16_gemm(x, packed, scales, zeros, y, work, M, N, K, group, None)


@pytest.mark.parametrize("kw,want", [
    (dict(x=NUL), eta.ATTN_ERR_INVALID),
    (dict(packed=NUL), eta.ATTN_ERR_INVALID),
    (dict(scales=NUL), eta.ATTN_ERR_INVALID),
    (dict(zeros=NUL), eta.ATTN_ERR_INVALID),
    (dict(y=NUL), eta.ATTN_ERR_INVALID),
    (dict(x=MIS), eta.ATTN_ERR_INVALID),
    (dict(packed=P4), eta.ATTN_ERR_INVALID),
    (dict(scales=ctypes.c_void_p(0x50001)), eta.ATTN_ERR_INVALID),
    (dict(y=ctypes.c_void_p(0x50001)), eta.ATTN_ERR_INVALID),
    (dict(M=0), eta.ATTN_ERR_INVALID),
    (dict(N=0), eta.ATTN_ERR_INVALID),
    (dict(K=0), eta.ATTN_ERR_INVALID),
    (dict(K=200), eta.ATTN_ERR_INVALID),
    (dict(N=2**30 + 1), eta.ATTN_ERR_INVALID),
    (dict(K=2**24 + 128), eta.ATTN_ERR_INVALID),
    (dict(group=64, K=256), eta.ATTN_ERR_UNSUPPORTED),
    (dict(group=0), eta.ATTN_ERR_INVALID),
    (dict(M=4097), eta.ATTN_ERR_UNSUPPORTED),
    (dict(work=NUL, M=1, N=16, K=4096), eta.ATTN_ERR_INVALID),          # needs a workspace
    (dict(work=ctypes.c_void_p(0x50002), M=1, N=16, K=4096), eta.ATTN_ERR_INVALID),
])
def test_w4a16_rejects_bad_arguments(kw, want):
    assert w4(**kw) == want


def test_mfma_probe_validation_and_flop():
    L = eta.lib()
    assert L.attn_mfma_peak(eta.MFMA_BF16, 0, 10, P4, None) == eta.ATTN_ERR_INVALID
    assert L.attn_mfma_peak(eta.MFMA_BF16, 4, 0, P4, None) == eta.ATTN_ERR_INVALID
    assert L.attn_mfma_peak(eta.MFMA_BF16, 4, 10, NUL, None) == eta.ATTN_ERR_INVALID
    assert L.attn_mfma_peak(eta.MFMA_BF16, 4, 10, ctypes.c_void_p(0x50002), None) == eta.ATTN_ERR_INVALID
    assert L.attn_mfma_peak(7, 4, 10, P4, None) == eta.ATTN_ERR_UNSUPPORTED
    assert L.attn_mfma_dot(eta.MFMA_FP8, NUL, P16b, P4, None) == eta.ATTN_ERR_INVALID
    assert L.attn_mfma_dot(eta.MFMA_FP8, MIS, P16b, P4, None) == eta.ATTN_ERR_INVALID
    assert L.attn_mfma_dot(eta.MFMA_F32, P16, P16b, P4, None) == eta.ATTN_ERR_UNSUPPORTED
    # FLOP per launch: workgroups x 8 wavefronts x iters x 4 instructions x FLOP per instruction
    assert eta.mfma_peak_flop(eta.MFMA_BF16, 256, 100) == 256 * 8 * 100 * 4 * 2 * 32 * 32 * 16
    assert eta.mfma_peak_flop(eta.MFMA_FP8, 3, 5) == 3 * 8 * 5 * 4 * 2 * 32 * 32 * 64
    assert eta.mfma_peak_flop(eta.MFMA_F32, 1, 1) == 8 * 4 * 2 * 32 * 32 * 2
    assert eta.mfma_peak_flop(9, 1, 1) == 0 and eta.mfma_peak_flop(eta.MFMA_BF16, 0, 1) == 0


# Entry points that allocate device (or pinned host) memory.  The library's
# calls work in caller-owned buffers (the pages' O(N)-memory property: no N x N
# matrix, and here no allocation at all), so its dynamic symbol table must not
# import any of them.
ALLOCATORS = ("hipMalloc", "hipExtMalloc", "hipHostMalloc", "hipHostAlloc", "hipFree", "hipMemPool",
              "hipMemCreate", "hipMemMap", "hipMallocAsync", "hipMemAllocHost")


def test_library_imports_no_allocator():
    import shutil
    import subprocess

    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    path = os.path.join(REPO, "exact_tiled_attention_15_amd", "libattn.so")
    out = subprocess.run([nm, "-D", "--undefined-only", path], capture_output=True, text=True, check=True).stdout
    imported = {line.split()[-1].split("@")[0] for line in out.splitlines() if line.strip()}
    assert "hipLaunchKernel" in imported  # the listing is the library's real import table
    bad = sorted(s for s in imported if s.startswith(ALLOCATORS))
    assert not bad, f"libattn.so imports allocating entry points: {bad}"
