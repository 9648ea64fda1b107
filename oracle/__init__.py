"""fp64 CPU oracle for exact softmax attention and the W4A16 layer (ctypes over attn_oracle.c).

TEST INFRASTRUCTURE ONLY: tests/, the smoke check in __graft_entry__ and the
CPU-baseline leg of bench.py may import this package; the library's compute
path never does.  The C source states what is computed and which passage of
the pages each part follows; this wrapper only moves numpy arrays in and out.
"""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attn_oracle.c")
LIB_PATH = os.path.join(HERE, "liboracle.so")


def build() -> str:
    """Compile attn_oracle.c with gcc (fp64, OpenMP, no fast-math)."""
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", tmp, SRC, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle build failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i, d = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.oracle_bf16_value.restype = d
        L.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.oracle_e4m3_value.restype = d
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_decode.restype = i
        L.oracle_decode.argtypes = [i, vp, vp, i, i64, i64, i64, i64, vp]
        L.oracle_attention.restype = i
        L.oracle_attention.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i, d, vp, i64, vp, vp, vp]
        L.oracle_block_state.restype = i
        L.oracle_block_state.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i, i64, i64, d, vp, i64,
                                         vp, vp, vp]
        L.oracle_merge.restype = None
        L.oracle_merge.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64]
        L.oracle_state_lse.restype = None
        L.oracle_state_lse.argtypes = [vp, vp, i64, vp]
        L.oracle_num_threads.restype = i
        L.oracle_num_threads.argtypes = []
        L.oracle_w4_value.restype = i
        L.oracle_w4_value.argtypes = [vp, i64]
        L.oracle_w4a16.restype = i
        L.oracle_w4a16.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, vp]
        L.oracle_attention_bwd.restype = i
        L.oracle_attention_bwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i, d, vp, i64, vp, i64,
                                           vp, vp, vp]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def num_threads() -> int:
    return _L().oracle_num_threads()


def bf16_value(bits: int) -> float:
    return _L().oracle_bf16_value(bits)


def e4m3_value(code: int) -> float:
    return _L().oracle_e4m3_value(code)


def _decode(kind, src, scales, tile, shape):
    B, H, N, d = shape
    out = np.empty(shape, dtype=np.float64)
    src = np.ascontiguousarray(src)
    sc = None if scales is None else np.ascontiguousarray(scales, dtype=np.float32)
    rc = _L().oracle_decode(kind, _p(src), _p(sc), tile, B, H, N, d, _p(out))
    if rc != 0:
        raise ValueError("oracle_decode failed")
    return out


def decode_f32(x: np.ndarray) -> np.ndarray:
    return _decode(0, np.asarray(x, dtype=np.float32), None, 1, x.shape)


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    return _decode(1, np.asarray(bits, dtype=np.uint16), None, 1, bits.shape)


def decode_e4m3(codes: np.ndarray, scales: np.ndarray, tile: int = 128) -> np.ndarray:
    return _decode(2, np.asarray(codes, dtype=np.uint8), scales, tile, codes.shape)


def attention(q, k, v, causal: bool, scale: float, rows=None, want_p: bool = False):
    """fp64 O [B,H,R,d] and LSE [B,H,R] (and P [B,H,R,Nk] if want_p) for rows R."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    R = Nq if r is None else len(r)
    o = np.empty((B, H, R, d))
    lse = np.empty((B, H, R))
    p = np.empty((B, H, R, Nk)) if want_p else None
    rc = _L().oracle_attention(_p(q), _p(k), _p(v), B, H, Nq, Nk, d, int(bool(causal)), float(scale),
                               _p(r), R, _p(o), _p(lse), _p(p))
    if rc != 0:
        raise RuntimeError(f"oracle_attention failed ({rc})")
    return (o, lse, p) if want_p else (o, lse)


def block_state(q, kb, vb, causal: bool, q_pos0: int, k_pos0: int, scale: float, rows=None):
    """Partial state (O normalised, m, l) of the rows against one K/V block."""
    q, kb, vb = _f64(q), _f64(kb), _f64(vb)
    B, H, Nq, d = q.shape
    Nkb = kb.shape[2]
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    R = Nq if r is None else len(r)
    o = np.empty((B, H, R, d))
    m = np.empty((B, H, R))
    l = np.empty((B, H, R))
    rc = _L().oracle_block_state(_p(q), _p(kb), _p(vb), B, H, Nq, Nkb, d, int(bool(causal)),
                                 int(q_pos0), int(k_pos0), float(scale), _p(r), R, _p(o), _p(m), _p(l))
    if rc != 0:
        raise RuntimeError(f"oracle_block_state failed ({rc})")
    return o, m, l


def empty_state(shape_o):
    """The identity of merge: O = 0, m = -inf, l = 0."""
    return (np.zeros(shape_o), np.full(shape_o[:-1], -np.inf), np.zeros(shape_o[:-1]))


def merge(a, b):
    """Merged state of a and b (new arrays; inputs untouched)."""
    o, m, l = (np.array(x, dtype=np.float64, copy=True) for x in a)
    ob, mb, lb = (_f64(x) for x in b)
    n = m.size
    d = o.shape[-1]
    _L().oracle_merge(_p(o), _p(m), _p(l), _p(ob), _p(mb), _p(lb), n, d)
    return o, m, l


def state_lse(m, l):
    m, l = _f64(m), _f64(l)
    out = np.empty_like(m)
    _L().oracle_state_lse(_p(m), _p(l), m.size, _p(out))
    return out


def attention_bwd(q, k, v, dout, causal: bool, scale: float, q_rows=None, k_rows=None):
    """fp64 gradients of sum(dout * O) for standard attention: dq for the query rows q_rows
    ([B,H,n_q,d], all rows if None) and dk, dv for the key rows k_rows ([B,H,n_k,d])."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    qr = None if q_rows is None else np.ascontiguousarray(q_rows, dtype=np.int64)
    kr = None if k_rows is None else np.ascontiguousarray(k_rows, dtype=np.int64)
    RQ = Nq if qr is None else len(qr)
    RK = Nk if kr is None else len(kr)
    dq = np.empty((B, H, RQ, d))
    dk = np.empty((B, H, RK, d))
    dv = np.empty((B, H, RK, d))
    rc = _L().oracle_attention_bwd(_p(q), _p(k), _p(v), _p(dout), B, H, Nq, Nk, d, int(bool(causal)),
                                   float(scale), _p(qr), RQ, _p(kr), RK, _p(dq), _p(dk), _p(dv))
    if rc != 0:
        raise RuntimeError(f"oracle_attention_bwd failed ({rc})")
    return dq, dk, dv


def fp16_value(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns -> float64 (exact)."""
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def w4_value(row_words: np.ndarray, k: int) -> int:
    """The 4-bit value of weight k from one row's packed words."""
    w = np.ascontiguousarray(row_words, dtype=np.uint32)
    return int(_L().oracle_w4_value(_p(w), int(k)))


def w4a16(x_bits, packed, zeros, scale_bits, group: int):
    """fp64 y [M, N] of the W4A16 layer: x fp16 bits [M, K], packed uint32 [N, K/8],
    zeros uint8 [N, K/G], scale fp16 bits [N, K/G]."""
    x = fp16_value(x_bits)
    sc = fp16_value(scale_bits)
    packed = np.ascontiguousarray(packed, dtype=np.uint32)
    zeros = np.ascontiguousarray(zeros, dtype=np.uint8)
    M, K = x.shape
    N = packed.shape[0]
    group = int(group)
    if group <= 0 or K % 8 or K % group or packed.shape != (N, K // 8) \
            or zeros.shape != (N, K // group) or sc.shape != (N, K // group):
        raise ValueError("oracle_w4a16: bad shape")
    y = np.empty((M, N))
    rc = _L().oracle_w4a16(_p(x), _p(packed), _p(zeros), _p(sc), M, N, K, group, _p(y))
    if rc != 0:
        raise ValueError("oracle_w4a16: bad shape")
    return y
