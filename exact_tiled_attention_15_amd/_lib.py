"""ctypes binding of libattn.so (include/attn.h, attn_diag.h, w4a16.h, mfma_probe.h).

Argument marshalling only: every function here checks that the torch tensors
it is handed have the dtype/shape/device the C entry point documents, passes
their device pointers and sizes, and raises AttnError on a non-zero status.
All computation happens in the library's HIP kernels.  There is no fallback:
if libattn.so is missing or cannot be loaded, every call raises.
"""
import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

ATTN_OK = 0
ATTN_ERR_INVALID = 1
ATTN_ERR_UNSUPPORTED = 2
ATTN_ERR_HIP = 3
FP8_TILE = 128
W4A16_GROUP = 128
W4A16_MAX_M = 4096
W4A16_TOKENS_PER_PASS = 16
W4A16_NOALLOC_MAX_WORK_FLOATS = 1 << 21
MFMA_BF16, MFMA_F16, MFMA_FP8, MFMA_F32 = 0, 1, 2, 3
MFMA_PEAK_THREADS = 512


class AttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libattn.so once; raise loudly when it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python exact_tiled_attention_15_amd/build.py`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_int64
    L.attn_abi_version.restype = i
    L.attn_abi_version.argtypes = []
    L.attn_status_str.restype = ctypes.c_char_p
    L.attn_status_str.argtypes = [i]
    L.attn_fwd.restype = i
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    L.attn_fwd_f32.restype = i
    L.attn_fwd_f32.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    L.attn_fwd_kvblock.restype = i
    L.attn_fwd_kvblock.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i64, i64, f, vp]
    L.attn_merge.restype = i
    L.attn_merge.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, vp]
    L.attn_bwd_work_floats.restype = ctypes.c_size_t
    L.attn_bwd_work_floats.argtypes = [i, i, i]
    L.attn_bwd.restype = i
    L.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    L.attn_ring_work_floats.restype = ctypes.c_size_t
    L.attn_ring_work_floats.argtypes = [i, i, i, i]
    L.attn_fwd_ring.restype = i
    L.attn_fwd_ring.argtypes = [vp, vp, vp, vp, i, vp, vp, vp, i, i, i, i, i, i, i64, f, vp]
    L.attn_ring_stage_bytes.restype = ctypes.c_size_t
    L.attn_ring_stage_bytes.argtypes = [i, i, i, i]
    L.attn_fwd_ring_host.restype = i
    L.attn_fwd_ring_host.argtypes = [vp, vp, vp, vp, i, vp, vp, vp, vp, i, i, i, i, i, i, i64, f, vp]
    for name in ("attn_fwd_fp8", "attn_fwd_fp8_qk16", "attn_fwd_fp8_pv8"):
        fn = getattr(L, name)
        fn.restype = i
        fn.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    L.attn_fwd_fp8_pv4.restype = i
    L.attn_fwd_fp8_pv4.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    L.w4a16_work_floats.restype = ctypes.c_size_t
    L.w4a16_work_floats.argtypes = [i64, i64, i64, i64]
    L.w4a16_gemm.restype = i
    L.w4a16_gemm.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, vp]
    L.w4a16_gemm_noalloc.restype = i
    L.w4a16_gemm_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp]
    L.attn_fwd_block_order.restype = i
    L.attn_fwd_block_order.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, ctypes.c_uint32, vp]
    L.attn_mfma_peak_flop.restype = ctypes.c_double
    L.attn_mfma_peak_flop.argtypes = [i, i, i]
    L.attn_mfma_peak.restype = i
    L.attn_mfma_peak.argtypes = [i, i, i, vp, vp]
    L.attn_mfma_dot.restype = i
    L.attn_mfma_dot.argtypes = [i, vp, vp, vp, vp]
    _lib = L
    return L


def _check(status: int, what: str):
    if status != ATTN_OK:
        raise AttnError(status, f"{what}: {lib().attn_status_str(status).decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _want(t, dtype, shape, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")


def abi_version() -> int:
    return lib().attn_abi_version()


def status_str(s: int) -> str:
    return lib().attn_status_str(s).decode()


def attn_fwd(q, k, v, o, lse, causal: bool, scale: float, stream=None):
    """q [B,H,Nq,d], k/v [B,H,Nk,d], o [B,H,Nq,d] bf16; lse [B,H,Nq] fp32 or None."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    _want(q, torch.bfloat16, (B, H, Nq, d), "q")
    _want(k, torch.bfloat16, (B, H, Nk, d), "k")
    _want(v, torch.bfloat16, (B, H, Nk, d), "v")
    _want(o, torch.bfloat16, (B, H, Nq, d), "o")
    if lse is not None:
        _want(lse, torch.float32, (B, H, Nq), "lse")
    _check(lib().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d,
                          int(bool(causal)), float(scale), _stream(stream)), "attn_fwd")


def attn_fwd_f32(q, k, v, o, lse, causal: bool, scale: float, stream=None):
    """As attn_fwd with float32 q/k/v/o."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    _want(q, torch.float32, (B, H, Nq, d), "q")
    _want(k, torch.float32, (B, H, Nk, d), "k")
    _want(v, torch.float32, (B, H, Nk, d), "v")
    _want(o, torch.float32, (B, H, Nq, d), "o")
    if lse is not None:
        _want(lse, torch.float32, (B, H, Nq), "lse")
    _check(lib().attn_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d,
                              int(bool(causal)), float(scale), _stream(stream)), "attn_fwd_f32")


def attn_fwd_kvblock(q, k_blk, v_blk, o_part, m_part, l_part, causal: bool, q_pos0: int,
                     k_pos0: int, scale: float, stream=None):
    """Partial state of q against one K/V block: o_part fp32, m_part/l_part fp32 [B,H,Nq]."""
    B, H, Nq, d = q.shape
    Nkb = k_blk.shape[2]
    _want(q, torch.bfloat16, (B, H, Nq, d), "q")
    _want(k_blk, torch.bfloat16, (B, H, Nkb, d), "k_blk")
    _want(v_blk, torch.bfloat16, (B, H, Nkb, d), "v_blk")
    _want(o_part, torch.float32, (B, H, Nq, d), "o_part")
    _want(m_part, torch.float32, (B, H, Nq), "m_part")
    _want(l_part, torch.float32, (B, H, Nq), "l_part")
    _check(lib().attn_fwd_kvblock(_ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(o_part), _ptr(m_part),
                                  _ptr(l_part), B, H, Nq, Nkb, d, int(bool(causal)), int(q_pos0),
                                  int(k_pos0), float(scale), _stream(stream)), "attn_fwd_kvblock")


def attn_merge(o_acc, m_acc, l_acc, o_part, m_part, l_part, o_final=None, lse_final=None,
               stream=None):
    """Merge a block state into the accumulator (in place); optional bf16 O / LSE outputs."""
    B, H, Nq, d = o_acc.shape
    _want(o_acc, torch.float32, (B, H, Nq, d), "o_acc")
    _want(m_acc, torch.float32, (B, H, Nq), "m_acc")
    _want(l_acc, torch.float32, (B, H, Nq), "l_acc")
    _want(o_part, torch.float32, (B, H, Nq, d), "o_part")
    _want(m_part, torch.float32, (B, H, Nq), "m_part")
    _want(l_part, torch.float32, (B, H, Nq), "l_part")
    if o_final is not None:
        _want(o_final, torch.bfloat16, (B, H, Nq, d), "o_final")
    if lse_final is not None:
        _want(lse_final, torch.float32, (B, H, Nq), "lse_final")
    _check(lib().attn_merge(_ptr(o_acc), _ptr(m_acc), _ptr(l_acc), _ptr(o_part), _ptr(m_part),
                            _ptr(l_part), _ptr(o_final), _ptr(lse_final), B, H, Nq, d,
                            _stream(stream)), "attn_merge")


def bwd_work_floats(B: int, H: int, Nq: int) -> int:
    """Size (fp32 elements) of the workspace attn_bwd needs."""
    return int(lib().attn_bwd_work_floats(B, H, Nq))


def attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, work, causal: bool, scale: float, stream=None):
    """Gradients of sum(dout * O): q/o/dout/dq bf16 [B,H,Nq,d], k/v/dk/dv bf16 [B,H,Nk,d],
    lse fp32 [B,H,Nq] from attn_fwd, work fp32 of bwd_work_floats(B,H,Nq)."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    for t, n in ((q, "q"), (o, "o"), (dout, "dout"), (dq, "dq")):
        _want(t, torch.bfloat16, (B, H, Nq, d), n)
    for t, n in ((k, "k"), (v, "v"), (dk, "dk"), (dv, "dv")):
        _want(t, torch.bfloat16, (B, H, Nk, d), n)
    _want(lse, torch.float32, (B, H, Nq), "lse")
    _want(work, torch.float32, (bwd_work_floats(B, H, Nq),), "work")
    _check(lib().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                          _ptr(dv), _ptr(work), B, H, Nq, Nk, d, int(bool(causal)), float(scale),
                          _stream(stream)), "attn_bwd")


def ring_work_floats(B: int, H: int, Nq: int, d: int) -> int:
    """Size (fp32 elements) of the workspace attn_fwd_ring needs."""
    return int(lib().attn_ring_work_floats(B, H, Nq, d))


def attn_fwd_ring(q, k_blks, v_blks, k_pos, o, lse, work, causal: bool, q_pos0: int, scale: float,
                  stream=None):
    """One GPU's ring-attention share: q bf16 [B,H,Nq,d] at global rows q_pos0.. against the
    K/V blocks k_blks[b], v_blks[b] (bf16 [B,H,Nk_blk,d]) at global key positions k_pos[b]..,
    in hop order; o bf16 [B,H,Nq,d], lse fp32 [B,H,Nq] or None, work fp32 of ring_work_floats."""
    B, H, Nq, d = q.shape
    n = len(k_blks)
    if len(v_blks) != n or len(k_pos) != n:
        raise ValueError("k_blks, v_blks and k_pos must have the same length")
    Nkb = k_blks[0].shape[2] if n else 1
    _want(q, torch.bfloat16, (B, H, Nq, d), "q")
    for b in range(n):
        _want(k_blks[b], torch.bfloat16, (B, H, Nkb, d), f"k_blks[{b}]")
        _want(v_blks[b], torch.bfloat16, (B, H, Nkb, d), f"v_blks[{b}]")
    _want(o, torch.bfloat16, (B, H, Nq, d), "o")
    if lse is not None:
        _want(lse, torch.float32, (B, H, Nq), "lse")
    _want(work, torch.float32, (ring_work_floats(B, H, Nq, d),), "work")
    kp = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in k_blks])
    vp_ = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in v_blks])
    pos = (ctypes.c_int64 * max(n, 1))(*[int(x) for x in k_pos])
    _check(lib().attn_fwd_ring(_ptr(q), kp, vp_, pos, n, _ptr(o), _ptr(lse), _ptr(work), B, H, Nq, Nkb, d,
                               int(bool(causal)), int(q_pos0), float(scale), _stream(stream)), "attn_fwd_ring")


def ring_stage_bytes(B: int, H: int, Nk_blk: int, d: int) -> int:
    """Size (bytes) of the device staging buffer attn_fwd_ring_host needs (two K/V slots)."""
    return int(lib().attn_ring_stage_bytes(B, H, Nk_blk, d))


def attn_fwd_ring_host(q, k_blks, v_blks, k_pos, o, lse, work, stage, causal: bool, q_pos0: int,
                       scale: float, stream=None):
    """attn_fwd_ring with the K/V blocks in host memory: k_blks[b], v_blks[b] are contiguous CPU
    bf16 tensors [B,H,Nk_blk,d] (page-locked, e.g. pin_memory(), for the copies to overlap the
    attention); stage is a device uint8 buffer of ring_stage_bytes(B,H,Nk_blk,d) bytes."""
    B, H, Nq, d = q.shape
    n = len(k_blks)
    if len(v_blks) != n or len(k_pos) != n:
        raise ValueError("k_blks, v_blks and k_pos must have the same length")
    Nkb = k_blks[0].shape[2] if n else 1
    _want(q, torch.bfloat16, (B, H, Nq, d), "q")
    for b in range(n):
        for name, t in ((f"k_blks[{b}]", k_blks[b]), (f"v_blks[{b}]", v_blks[b])):
            if t.dtype != torch.bfloat16 or tuple(t.shape) != (B, H, Nkb, d):
                raise ValueError(f"{name} must be bf16 of shape {(B, H, Nkb, d)}")
            if t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous host tensor")
    _want(o, torch.bfloat16, (B, H, Nq, d), "o")
    if lse is not None:
        _want(lse, torch.float32, (B, H, Nq), "lse")
    _want(work, torch.float32, (ring_work_floats(B, H, Nq, d),), "work")
    # with no block the slot size is undefined: any staging buffer will do
    _want(stage, torch.uint8, (ring_stage_bytes(B, H, Nkb, d) if n else stage.numel(),), "stage")
    kp = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in k_blks])
    vp_ = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in v_blks])
    pos = (ctypes.c_int64 * max(n, 1))(*[int(x) for x in k_pos])
    _check(lib().attn_fwd_ring_host(_ptr(q), kp, vp_, pos, n, _ptr(o), _ptr(lse), _ptr(work), _ptr(stage), B, H,
                                    Nq, Nkb, d, int(bool(causal)), int(q_pos0), float(scale), _stream(stream)),
           "attn_fwd_ring_host")


def _fwd_fp8(entry, q8, k8, v8, q_scale, k_scale, v_scale, o, lse, causal, scale, stream, extra=()):
    B, H, Nq, d = q8.shape
    Nk = k8.shape[2]
    nqt = (Nq + FP8_TILE - 1) // FP8_TILE
    nkt = (Nk + FP8_TILE - 1) // FP8_TILE
    _want(q8, torch.uint8, (B, H, Nq, d), "q8")
    _want(k8, torch.uint8, (B, H, Nk, d), "k8")
    _want(v8, torch.uint8, (B, H, Nk, d), "v8")
    _want(q_scale, torch.float32, (B, H, nqt), "q_scale")
    _want(k_scale, torch.float32, (B, H, nkt), "k_scale")
    _want(v_scale, torch.float32, (B, H, nkt), "v_scale")
    _want(o, torch.float32, (B, H, Nq, d), "o")
    if lse is not None:
        _want(lse, torch.float32, (B, H, Nq), "lse")
    fn = getattr(lib(), entry)
    _check(fn(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale), _ptr(o), _ptr(lse),
              B, H, Nq, Nk, d, int(bool(causal)), float(scale), *extra, _stream(stream)), entry)


def attn_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, o, lse, causal: bool, scale: float,
                 stream=None):
    """e4m3 codes (uint8) with fp32 per-128-token-tile scales; QK^T on fp8 matrix cores."""
    _fwd_fp8("attn_fwd_fp8", q8, k8, v8, q_scale, k_scale, v_scale, o, lse, causal, scale, stream)


def attn_fwd_fp8_qk16(q8, k8, v8, q_scale, k_scale, v_scale, o, lse, causal: bool, scale: float,
                      stream=None):
    """As attn_fwd_fp8 with QK^T on fp16 matrix cores over exactly widened codes."""
    _fwd_fp8("attn_fwd_fp8_qk16", q8, k8, v8, q_scale, k_scale, v_scale, o, lse, causal, scale, stream)


def attn_fwd_fp8_pv8(q8, k8, v8, q_scale, k_scale, v_scale, o, lse, causal: bool, scale: float,
                     stream=None):
    """As attn_fwd_fp8 with P in e4m3 and P.V on fp8 matrix cores (faster, drifts by P's rounding)."""
    _fwd_fp8("attn_fwd_fp8_pv8", q8, k8, v8, q_scale, k_scale, v_scale, o, lse, causal, scale, stream)


def attn_fwd_fp8_pv4(q8, k8, v8, q_scale, k_scale, v_scale, o, lse, causal: bool, scale: float,
                     direct_p: bool = False, stream=None):
    """As attn_fwd_fp8_pv8 with P as 4-bit e2m1 codes: each exponential rounded (direct_p False) or
    the score mapped straight to the code (Direct-P)."""
    _fwd_fp8("attn_fwd_fp8_pv4", q8, k8, v8, q_scale, k_scale, v_scale, o, lse, causal, scale, stream,
             extra=(int(bool(direct_p)),))


def w4a16_work_floats(M: int, N: int, K: int, group: int = W4A16_GROUP) -> int:
    """Size (fp32 elements) of the workspace w4a16_gemm needs (0 for none)."""
    return int(lib().w4a16_work_floats(M, N, K, group))


def w4a16_gemm(x, packed, scales, zeros, y, work=None, group: int = W4A16_GROUP, stream=None):
    """y [M,N] fp16 = x [M,K] fp16 . W^T, W given as 4-bit codes: packed int32 [N,K/8] (bits as
    uint32), scales fp16 [N,K/group], zeros uint8 [N,K/group]; work fp32 of w4a16_work_floats
    elements (None when that is 0)."""
    M, K = x.shape
    N = packed.shape[0]
    if K % 8 or K % group:
        raise ValueError("K must be a multiple of 8 and of the group size")
    _want(x, torch.float16, (M, K), "x")
    _want(packed, torch.int32, (N, K // 8), "packed")
    _want(scales, torch.float16, (N, K // group), "scales")
    _want(zeros, torch.uint8, (N, K // group), "zeros")
    _want(y, torch.float16, (M, N), "y")
    nw = w4a16_work_floats(M, N, K, group)
    if nw:
        _want(work, torch.float32, (nw,), "work")
    _check(lib().w4a16_gemm(_ptr(x), _ptr(packed), _ptr(scales), _ptr(zeros), _ptr(y),
                            _ptr(work) if nw else None, M, N, K, group, _stream(stream)), "w4a16_gemm")


def w4a16_gemm_noalloc(x, packed, scales, zeros, y, group: int = W4A16_GROUP, stream=None):
    """w4a16_gemm with its split partials in the library's fixed device array (no workspace)."""
    M, K = x.shape
    N = packed.shape[0]
    if K % 8 or K % group:
        raise ValueError("K must be a multiple of 8 and of the group size")
    _want(x, torch.float16, (M, K), "x")
    _want(packed, torch.int32, (N, K // 8), "packed")
    _want(scales, torch.float16, (N, K // group), "scales")
    _want(zeros, torch.uint8, (N, K // group), "zeros")
    _want(y, torch.float16, (M, N), "y")
    _check(lib().w4a16_gemm_noalloc(_ptr(x), _ptr(packed), _ptr(scales), _ptr(zeros), _ptr(y), M, N, K, group,
                                    _stream(stream)), "w4a16_gemm_noalloc")


def attn_fwd_block_order(q, k, v, o, lse, causal: bool, scale: float, order: int, stream=None):
    """attn_fwd with the workgroup -> tile assignment permuted by `order` (diagnostic)."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    _want(q, torch.bfloat16, (B, H, Nq, d), "q")
    _want(k, torch.bfloat16, (B, H, Nk, d), "k")
    _want(v, torch.bfloat16, (B, H, Nk, d), "v")
    _want(o, torch.bfloat16, (B, H, Nq, d), "o")
    if lse is not None:
        _want(lse, torch.float32, (B, H, Nq), "lse")
    _check(lib().attn_fwd_block_order(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d,
                                      int(bool(causal)), float(scale), int(order), _stream(stream)),
           "attn_fwd_block_order")


def mfma_peak_flop(kind: int, workgroups: int, iters: int) -> float:
    """FLOP of one attn_mfma_peak launch."""
    return lib().attn_mfma_peak_flop(kind, workgroups, iters)


def mfma_peak(kind: int, workgroups: int, iters: int, out, stream=None):
    """Matrix-core throughput loop; out: fp32 device tensor of workgroups * MFMA_PEAK_THREADS."""
    _want(out, torch.float32, (workgroups * MFMA_PEAK_THREADS,), "out")
    _check(lib().attn_mfma_peak(kind, workgroups, iters, _ptr(out), _stream(stream)), "attn_mfma_peak")


def mfma_dot(kind: int, a, b, c, stream=None):
    """C[32,32] = A[32,64] B (b holds B's columns as rows) on one matrix-core tile: a, b uint8
    e4m3 codes (MFMA_FP8) or bfloat16 / float16 (MFMA_BF16 / MFMA_F16); c float32."""
    dt = {MFMA_FP8: torch.uint8, MFMA_BF16: torch.bfloat16, MFMA_F16: torch.float16}.get(kind)
    if dt is None:
        raise ValueError(f"unknown kind {kind}")
    _want(a, dt, (32, 64), "a")
    _want(b, dt, (32, 64), "b")
    _want(c, torch.float32, (32, 32), "c")
    _check(lib().attn_mfma_dot(kind, _ptr(a), _ptr(b), _ptr(c), _stream(stream)), "attn_mfma_dot")
