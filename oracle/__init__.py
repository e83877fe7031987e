"""CPU oracle for the scaled_mm hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never calls it, and
it shares no code with the HIP kernels: the arithmetic lives in ``oracle.c``
(plain loops, int64 / fp64 sums, fp32 where the method fixes fp32), built with
gcc and loaded here through ctypes.

What it follows (no formula is printed on the pages; the readings are listed in
the design notes):
  * "Helion in vLLM: A Unified Route to Tunable Linear Kernels", section "What
    the integration changes": FP8 dynamic quantization, W8A8 INT8, Block-FP8,
    and the fact that ordinary GEMM, Split-K and Swap-AB compute one and the
    same product.
  * vLLM PR #53446, sections "Summary" and "Test Plan": the batch-invariant
    bf16 matmul, i.e. the plain bf16 product whose rows must not depend on the
    batch size.
  * The 4-bit formats named in the introduction of "Helion in vLLM", in their
    block-scaled form MXFP4, whose encodings and conversion rule come from the
    OCP Microscaling Formats (MX) v1.0 specification (the pages define none),
    and INT4 weight-only (symmetric, one scale per 128-element group).

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against something other than itself (torch's own e4m3/bf16 casts, Python
integer and Fraction brute force, numpy fp64 products, closed forms and the
hand-worked fixtures under ``tests/golden/``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64


_DIGEST_PATH = _LIB_PATH + ".sha256"


def _source_digest() -> str:
    import hashlib
    with open(_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _built_digest() -> str | None:
    try:
        with open(_DIGEST_PATH) as f:
            return f.read().strip()
    except OSError:
        return None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (OpenMP, no FMA
    contraction, SSE arithmetic); the SHA-256 of the source it was built from
    is written beside it."""
    if not force and os.path.exists(_LIB_PATH) and _built_digest() == _source_digest():
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC",
           "-shared", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    with open(_DIGEST_PATH, "w") as f:
        f.write(_source_digest() + "\n")
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # rebuilt only when the source's content differs from what the library
    # was built from (file times are not trusted: copies of the tree may
    # reorder them)
    build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_e4m3_decode.restype = ctypes.c_double
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_encode_rne.restype = ctypes.c_uint8
    lib.oracle_e4m3_encode_rne.argtypes = [ctypes.c_float]
    lib.oracle_bf16_encode_rne.restype = ctypes.c_uint16
    lib.oracle_bf16_encode_rne.argtypes = [ctypes.c_float]
    lib.oracle_bf16_decode.restype = ctypes.c_float
    lib.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
    lib.oracle_quantize_fp8.restype = ctypes.c_int
    lib.oracle_quantize_fp8.argtypes = [_P, _I64, _I64, _I64, _P, _P]
    lib.oracle_quantize_fp8_block.restype = ctypes.c_int
    lib.oracle_quantize_fp8_block.argtypes = [_P, _I64, _I64, _I64, _I64, _P, _P]
    lib.oracle_gemm_int8_acc.restype = None
    lib.oracle_gemm_int8_acc.argtypes = [_P, _P, _I64, _I64, _I64, _P, _I64, _P]
    lib.oracle_epilogue_int8.restype = None
    lib.oracle_epilogue_int8.argtypes = [_P, _P, _P, _I64, _P, _I64, _P]
    lib.oracle_gemm_fp8.restype = None
    lib.oracle_gemm_fp8.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _P, _I64,
                                    _P, _P]
    lib.oracle_gemm_block_fp8.restype = None
    lib.oracle_gemm_block_fp8.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64,
                                          _I64, _P, _I64, _P, _P]
    lib.oracle_gemm_bf16.restype = None
    lib.oracle_gemm_bf16.argtypes = [_P, _P, _I64, _I64, _I64, _P, _I64, _P, _P]
    lib.oracle_bf16_encode_array.restype = None
    lib.oracle_bf16_encode_array.argtypes = [_P, _I64, _P]
    lib.oracle_e4m3_encode_array.restype = None
    lib.oracle_e4m3_encode_array.argtypes = [_P, _I64, _P]
    lib.oracle_e4m3_decode_array.restype = None
    lib.oracle_e4m3_decode_array.argtypes = [_P, _I64, _P]
    lib.oracle_e2m1_decode.restype = ctypes.c_double
    lib.oracle_e2m1_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e8m0_decode.restype = ctypes.c_double
    lib.oracle_e8m0_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e2m1_encode_array.restype = None
    lib.oracle_e2m1_encode_array.argtypes = [_P, _I64, _P]
    lib.oracle_quantize_mxfp4.restype = ctypes.c_int
    lib.oracle_quantize_mxfp4.argtypes = [_P, _I64, _I64, _P, _P]
    lib.oracle_gemm_mxfp4.restype = None
    lib.oracle_gemm_mxfp4.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _P, _I64,
                                      _P, _P]
    lib.oracle_int4_decode.restype = ctypes.c_int
    lib.oracle_int4_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_quantize_int4.restype = ctypes.c_int
    lib.oracle_quantize_int4.argtypes = [_P, _I64, _I64, _P, _P]
    lib.oracle_gemm_w4a16.restype = None
    lib.oracle_gemm_w4a16.argtypes = [_P, _P, _P, _I64, _I64, _I64, _P, _I64, _P, _P]
    lib.oracle_set_threads.restype = None
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _rows(M: int, rows) -> np.ndarray:
    if rows is None:
        return np.arange(M, dtype=np.int64)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if r.size and (r.min() < 0 or r.max() >= M):
        raise ValueError("row index out of range")
    return r


def num_threads() -> int:
    """OpenMP threads the oracle runs with."""
    return int(_load().oracle_num_threads())


def set_threads(n: int) -> None:
    """OpenMP threads for the oracle's loops from now on (timing runs)."""
    _load().oracle_set_threads(int(n))


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------

def e4m3_decode(codes) -> np.ndarray:
    """OCP e4m3fn codes (uint8) -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    out = np.empty(c.shape, dtype=np.float64)
    _load().oracle_e4m3_decode_array(_ptr(c), c.size, _ptr(out))
    return out


def e4m3_encode(values) -> np.ndarray:
    """float32 values with |v| <= 448 -> e4m3fn codes, round to nearest even
    (0xFF marks an input outside that domain)."""
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float32))
    out = np.empty(v.shape, dtype=np.uint8)
    _load().oracle_e4m3_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def bf16_encode(values) -> np.ndarray:
    """float32 values -> bfloat16 bit patterns (uint16), round to nearest even."""
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float32))
    out = np.empty(v.shape, dtype=np.uint16)
    _load().oracle_bf16_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def bf16_decode(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 values."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def e2m1_decode(codes) -> np.ndarray:
    """E2M1 codes (low 4 bits of uint8) -> float64 values."""
    c = np.asarray(codes, dtype=np.uint8)
    lib = _load()
    return np.vectorize(lambda v: lib.oracle_e2m1_decode(int(v) & 15),
                        otypes=[np.float64])(c)


def e2m1_encode(values) -> np.ndarray:
    """float64 values -> E2M1 codes, nearest with ties to even, saturating
    at 6, sign kept for zeros."""
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float64))
    out = np.empty(v.shape, dtype=np.uint8)
    _load().oracle_e2m1_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def e8m0_decode(codes) -> np.ndarray:
    """E8M0 scale codes -> float64 powers of two (NaN for 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8)
    lib = _load()
    return np.vectorize(lambda v: lib.oracle_e8m0_decode(int(v)),
                        otypes=[np.float64])(c)


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    """Packed E2M1 codes [..][K/2] -> one code per element [..][K] (element
    2j from bits 0-3 of byte j, element 2j+1 from bits 4-7)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


# --------------------------------------------------------------------------
# Quantizers
# --------------------------------------------------------------------------

def quantize_fp8(x_bf16_bits: np.ndarray, group: int | None = None):
    """Dynamic FP8 quantization of bf16 activations [M][K] (uint16 bits).

    group None / K: one scale per row (per token); 128: one per 1x128 group.
    Returns (codes uint8 [M][K], scales float32 [M][K/group]).
    """
    x = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16)
    M, K = x.shape
    G = K if group in (None, 0) else int(group)
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, K // G), dtype=np.float32)
    rc = _load().oracle_quantize_fp8(_ptr(x), M, K, G, _ptr(q), _ptr(s))
    if rc != 0:
        raise ValueError(f"oracle_quantize_fp8 failed ({rc}): non-finite input "
                         "or group does not divide K")
    return q, s


def quantize_fp8_block(w_bf16_bits: np.ndarray, block: int = 128):
    """Weight quantization with one scale per block x block tile of [N][K].
    Returns (codes uint8 [N][K], scales float32 [ceil(N/block)][K/block])."""
    w = np.ascontiguousarray(w_bf16_bits, dtype=np.uint16)
    N, K = w.shape
    q = np.empty((N, K), dtype=np.uint8)
    s = np.empty(((N + block - 1) // block, K // block), dtype=np.float32)
    rc = _load().oracle_quantize_fp8_block(_ptr(w), N, K, block, block, _ptr(q),
                                           _ptr(s))
    if rc != 0:
        raise ValueError(f"oracle_quantize_fp8_block failed ({rc})")
    return q, s


def quantize_mxfp4(x_bf16_bits: np.ndarray):
    """MXFP4 quantization of bf16 [M][K] (uint16 bits), one E8M0 scale per
    32 consecutive elements of a row.  Returns (packed codes uint8 [M][K/2],
    scale codes uint8 [M][K/32])."""
    x = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16)
    M, K = x.shape
    q = np.empty((M, K // 2), dtype=np.uint8)
    s = np.empty((M, K // 32), dtype=np.uint8)
    rc = _load().oracle_quantize_mxfp4(_ptr(x), M, K, _ptr(q), _ptr(s))
    if rc != 0:
        raise ValueError(f"oracle_quantize_mxfp4 failed ({rc}): non-finite input "
                         "or K not a multiple of 32")
    return q, s


def int4_decode(codes) -> np.ndarray:
    """4-bit two's complement codes (low 4 bits) -> int64 values."""
    c = np.asarray(codes, dtype=np.uint8)
    lib = _load()
    return np.vectorize(lambda v: lib.oracle_int4_decode(int(v) & 15),
                        otypes=[np.int64])(c)


def quantize_int4(w_bf16_bits: np.ndarray):
    """INT4 weight quantization of bf16 [N][K] (uint16 bits), one fp32 scale
    per 128 consecutive elements of a row.  Returns (packed codes uint8
    [N][K/2], scales float32 [N][K/128])."""
    w = np.ascontiguousarray(w_bf16_bits, dtype=np.uint16)
    N, K = w.shape
    q = np.empty((N, K // 2), dtype=np.uint8)
    s = np.empty((N, K // 128), dtype=np.float32)
    rc = _load().oracle_quantize_int4(_ptr(w), N, K, _ptr(q), _ptr(s))
    if rc != 0:
        raise ValueError(f"oracle_quantize_int4 failed ({rc}): non-finite input "
                         "or K not a multiple of 128")
    return q, s


# --------------------------------------------------------------------------
# GEMMs (A [M][K], B [N][K]; outputs [len(rows)][N])
# --------------------------------------------------------------------------

def gemm_int8_acc(A: np.ndarray, B: np.ndarray, rows=None) -> np.ndarray:
    """Exact int64 accumulators sum_k A[m][k] * B[n][k]."""
    A = np.ascontiguousarray(A, dtype=np.int8)
    B = np.ascontiguousarray(B, dtype=np.int8)
    M, K = A.shape
    N = B.shape[0]
    assert B.shape[1] == K
    r = _rows(M, rows)
    acc = np.empty((r.size, N), dtype=np.int64)
    _load().oracle_gemm_int8_acc(_ptr(A), _ptr(B), M, N, K, _ptr(r), r.size,
                                 _ptr(acc))
    return acc


def epilogue_int8(acc: np.ndarray, sa: np.ndarray, sb: np.ndarray,
                  rows=None) -> np.ndarray:
    """fp32 epilogue (float(acc) * sa[m]) * sb[n]; acc rows are `rows` of A."""
    acc = np.ascontiguousarray(acc, dtype=np.int64)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    sb = np.ascontiguousarray(sb, dtype=np.float32)
    nr, N = acc.shape
    r = _rows(sa.size, rows) if rows is not None else np.arange(nr, dtype=np.int64)
    assert r.size == nr and sb.size == N
    y = np.empty((nr, N), dtype=np.float32)
    _load().oracle_epilogue_int8(_ptr(acc), _ptr(sa), _ptr(sb), N, _ptr(r), nr,
                                 _ptr(y))
    return y


def gemm_w8a8_int8(A, B, sa, sb, rows=None):
    """W8A8 INT8 GEMM: returns (int64 accumulators, fp32 scaled output)."""
    acc = gemm_int8_acc(A, B, rows)
    return acc, epilogue_int8(acc, sa, sb, rows)


def gemm_fp8(A, B, sa, sb, rows=None, with_abs=False):
    """FP8 per-token x per-channel GEMM in fp64 (and sum of |terms|)."""
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    sa = np.ascontiguousarray(np.asarray(sa, dtype=np.float32).reshape(-1))
    sb = np.ascontiguousarray(np.asarray(sb, dtype=np.float32).reshape(-1))
    M, K = A.shape
    N = B.shape[0]
    assert B.shape[1] == K and sa.size == M and sb.size == N
    r = _rows(M, rows)
    ref = np.empty((r.size, N), dtype=np.float64)
    absref = np.empty((r.size, N), dtype=np.float64) if with_abs else None
    _load().oracle_gemm_fp8(_ptr(A), _ptr(B), _ptr(sa), _ptr(sb), M, N, K,
                            _ptr(r), r.size, _ptr(ref),
                            _ptr(absref) if with_abs else None)
    return (ref, absref) if with_abs else ref


def gemm_fp8_grouped(A, B, sa, sb, offsets, rows=None, with_abs=False):
    """Grouped (per-expert) FP8 GEMM in fp64: row m of A, with
    offsets[e] <= m < offsets[e+1], is multiplied by expert e's weights
    B[e] ([N][K]) and scaled by sa[m] and sb[e] ([N]) -- the per-channel FP8
    product of gemm_fp8, one expert at a time."""
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    sa = np.asarray(sa, dtype=np.float32).reshape(-1)
    sb = np.asarray(sb, dtype=np.float32)
    offsets = np.asarray(offsets, dtype=np.int64)
    M, K = A.shape
    E, N, K2 = B.shape
    assert K2 == K and sa.size == M and sb.shape == (E, N) and offsets.shape == (E + 1,)
    assert offsets[0] == 0 and offsets[E] == M and np.all(np.diff(offsets) >= 0)
    r = _rows(M, rows)
    ref = np.empty((r.size, N), dtype=np.float64)
    absref = np.empty((r.size, N), dtype=np.float64) if with_abs else None
    expert = np.searchsorted(offsets, r, side="right") - 1
    for e in range(E):
        sel = np.nonzero(expert == e)[0]
        if sel.size == 0:
            continue
        res = gemm_fp8(A, B[e], sa, sb[e], rows=r[sel], with_abs=with_abs)
        if with_abs:
            ref[sel], absref[sel] = res
        else:
            ref[sel] = res
    return (ref, absref) if with_abs else ref


def gemm_block_fp8(A, B, sa, sb, rows=None, with_abs=False, group: int = 128):
    """Block-FP8 GEMM (1 x group activation scales, group x group weight
    scales) in fp64."""
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    sb = np.ascontiguousarray(sb, dtype=np.float32)
    M, K = A.shape
    N = B.shape[0]
    assert B.shape[1] == K and K % group == 0
    assert sa.shape == (M, K // group)
    assert sb.shape == ((N + group - 1) // group, K // group)
    r = _rows(M, rows)
    ref = np.empty((r.size, N), dtype=np.float64)
    absref = np.empty((r.size, N), dtype=np.float64) if with_abs else None
    _load().oracle_gemm_block_fp8(_ptr(A), _ptr(B), _ptr(sa), _ptr(sb), M, N, K,
                                  group, _ptr(r), r.size, _ptr(ref),
                                  _ptr(absref) if with_abs else None)
    return (ref, absref) if with_abs else ref


def gemm_bf16(A_bits, B_bits, rows=None, with_abs=False):
    """bf16 GEMM (uint16 bit patterns in) in fp64."""
    A = np.ascontiguousarray(A_bits, dtype=np.uint16)
    B = np.ascontiguousarray(B_bits, dtype=np.uint16)
    M, K = A.shape
    N = B.shape[0]
    assert B.shape[1] == K
    r = _rows(M, rows)
    ref = np.empty((r.size, N), dtype=np.float64)
    absref = np.empty((r.size, N), dtype=np.float64) if with_abs else None
    _load().oracle_gemm_bf16(_ptr(A), _ptr(B), M, N, K, _ptr(r), r.size,
                             _ptr(ref), _ptr(absref) if with_abs else None)
    return (ref, absref) if with_abs else ref


def gemm_mxfp4(A, B, sa, sb, rows=None, with_abs=False):
    """MXFP4 GEMM in fp64: A [M][K/2], B [N][K/2] packed E2M1 codes, sa
    [M][K/32], sb [N][K/32] E8M0 scale codes; every element is its code's
    value times its block's power of two."""
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.uint8)
    sb = np.ascontiguousarray(sb, dtype=np.uint8)
    M, K2 = A.shape
    N = B.shape[0]
    K = 2 * K2
    assert B.shape[1] == K2 and K % 32 == 0
    assert sa.shape == (M, K // 32) and sb.shape == (N, K // 32)
    r = _rows(M, rows)
    ref = np.empty((r.size, N), dtype=np.float64)
    absref = np.empty((r.size, N), dtype=np.float64) if with_abs else None
    _load().oracle_gemm_mxfp4(_ptr(A), _ptr(B), _ptr(sa), _ptr(sb), M, N, K,
                              _ptr(r), r.size, _ptr(ref),
                              _ptr(absref) if with_abs else None)
    return (ref, absref) if with_abs else ref


def gemm_w4a16(A_bits, B, s, rows=None, with_abs=False):
    """INT4 weight-only GEMM in fp64: A bf16 [M][K] (uint16 bits), B packed
    int4 [N][K/2], s fp32 [N][K/128]; per 128-wide group the exact partial
    sum times the group scale."""
    A = np.ascontiguousarray(A_bits, dtype=np.uint16)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    M, K = A.shape
    N = B.shape[0]
    assert B.shape[1] == K // 2 and K % 128 == 0 and s.shape == (N, K // 128)
    r = _rows(M, rows)
    ref = np.empty((r.size, N), dtype=np.float64)
    absref = np.empty((r.size, N), dtype=np.float64) if with_abs else None
    _load().oracle_gemm_w4a16(_ptr(A), _ptr(B), _ptr(s), M, N, K, _ptr(r), r.size,
                              _ptr(ref), _ptr(absref) if with_abs else None)
    return (ref, absref) if with_abs else ref
