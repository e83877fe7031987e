"""Python binding of libqll.so, the MI355X (gfx950) scaled_mm library.

The functions here carry the same names as the C entry points declared in
``include/qll.h`` and only marshal arguments: they take torch tensors that
already live on the GPU, allocate outputs (and the Split-K workspace) when the
caller does not pass them, and hand raw device pointers plus the current HIP
stream to the library.  Every step of the computation runs in the library's
HIP kernels; there is no fallback of any kind -- a missing ``libqll.so``
raises.

Operations (see include/qll.h for the full contract):
  quantize_per_token_fp8, quantize_weight_block_fp8,
  gemm_w8a8_int8, gemm_fp8_scaled, gemm_block_fp8, gemm_bf16_batch_invariant,
  linear_fp8_dynamic (per-token quantization + FP8 GEMM in one call),
  gemm_fp8_grouped (per-expert FP8 GEMM over rows sorted by expert),
  quantize_mxfp4, gemm_mxfp4 (MXFP4: E2M1 codes packed two per byte, one
  E8M0 scale byte per 32 elements of a row; tensors as uint8),
  quantize_int4_weights, gemm_w4a16 (INT4 weight-only: int4 codes packed two
  per byte, an fp32 scale per 128-element group, bf16 activations).
"""
from __future__ import annotations

import ctypes
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqll.so")
TABLE_DIR = os.path.join(HERE, "tables")

QLL_OK = 0
STATUS = {0: "QLL_OK", 1: "QLL_ERR_INVALID_ARG", 2: "QLL_ERR_UNSUPPORTED",
          3: "QLL_ERR_MISALIGNED", 4: "QLL_ERR_WORKSPACE", 5: "QLL_ERR_NO_DEVICE",
          6: "QLL_ERR_TABLE", 7: "QLL_ERR_HIP"}
OUT = {"bf16": 0, "fp32": 1, "int32": 2}
OPS = {"int8": 0, "fp8": 1, "block_fp8": 2, "bf16_bi": 3, "mxfp4": 4, "w4a16": 5,
       "fp8_dynamic": 6}


class QllError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


class qll_cfg(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("splits", ctypes.c_int32)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_GEMM_ARGS = [_P, _P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _P,
              ctypes.c_size_t, _P]
_BF16_ARGS = [_P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _P, ctypes.c_size_t, _P]

_lib = None
_table_state = None


def load_library():
    """Load libqll.so (raises when it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m "
            "quantized_linear_layer_scaled_amd.build` (needs hipcc)")
    L = ctypes.CDLL(LIB_PATH)
    L.quantize_per_token_fp8.argtypes = [_P, _P, _P, _I64, _I64, _I64, _P]
    L.quantize_weight_block_fp8.argtypes = [_P, _P, _P, _I64, _I64, _P]
    for name in ("gemm_w8a8_int8", "gemm_fp8_scaled", "gemm_block_fp8"):
        getattr(L, name).argtypes = _GEMM_ARGS
        getattr(L, name + "_ex").argtypes = _GEMM_ARGS + [ctypes.POINTER(qll_cfg)]
    L.quantize_mxfp4.argtypes = [_P, _P, _P, _I64, _I64, _P]
    L.quantize_int4_weights.argtypes = [_P, _P, _P, _I64, _I64, _P]
    L.gemm_w4a16.argtypes = _BF16_ARGS[:2] + [_P] + _BF16_ARGS[2:]
    L.gemm_w4a16_ex.argtypes = _BF16_ARGS[:2] + [_P] + _BF16_ARGS[2:] + [ctypes.POINTER(qll_cfg)]
    L.gemm_mxfp4.argtypes = _GEMM_ARGS
    L.gemm_mxfp4_ex.argtypes = _GEMM_ARGS + [ctypes.POINTER(qll_cfg)]
    L.gemm_bf16_batch_invariant.argtypes = _BF16_ARGS
    L.gemm_bf16_batch_invariant_ex.argtypes = _BF16_ARGS + [ctypes.POINTER(qll_cfg)]
    _LIN = [_P, _P, _P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _P, ctypes.c_size_t, _P]
    L.linear_fp8_dynamic.argtypes = _LIN
    L.linear_fp8_dynamic_ex.argtypes = _LIN + [ctypes.POINTER(qll_cfg)]
    _GRP = [_P, _P, _P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _I64, _P]
    L.gemm_fp8_grouped.argtypes = _GRP
    L.gemm_fp8_grouped_ex.argtypes = _GRP + [ctypes.c_char_p]
    L.qll_grouped_select.argtypes = [_I64, _I64, ctypes.c_char_p, ctypes.c_size_t]
    L.qll_init.argtypes = [ctypes.c_char_p]
    L.qll_table_validate.argtypes = [ctypes.c_char_p, ctypes.c_char_p, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_char_p, ctypes.c_char_p,
                                     ctypes.c_size_t]
    L.qll_device_signature.argtypes = [ctypes.c_char_p, ctypes.c_size_t]
    L.gemm_fp8_scaled_noalloc.argtypes = _GEMM_ARGS[:9] + [_P]
    L.qll_select.argtypes = [ctypes.c_int, _I64, _I64, _I64, ctypes.POINTER(qll_cfg)]
    L.qll_workspace_bytes.argtypes = [ctypes.c_int, _I64, _I64, _I64,
                                      ctypes.POINTER(qll_cfg)]
    L.qll_workspace_bytes.restype = _I64
    L.qll_effective_splits.argtypes = [ctypes.c_int, _I64, ctypes.c_int32]
    L.qll_num_variants.argtypes = [ctypes.c_int]
    L.qll_variant_info.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_char_p,
                                   ctypes.c_size_t]
    L.qll_variant_index.argtypes = [ctypes.c_int, ctypes.c_char_p]
    L.qll_table_entries.argtypes = []
    L.qll_status_str.argtypes = [ctypes.c_int]
    L.qll_status_str.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(fn: str, rc: int):
    if rc != QLL_OK:
        raise QllError(fn, rc)


def default_table() -> str | None:
    """The packaged dispatch table for gfx950 (None if absent)."""
    p = os.path.join(TABLE_DIR, "gfx950.tsv")
    return p if os.path.exists(p) else None


def init(table: str | None = "default") -> int:
    """qll_init: load a dispatch table ("default" = $QLL_TABLE or the packaged
    table, None = heuristic only).  Returns the status (QLL_ERR_TABLE means
    the heuristic stays in force)."""
    global _table_state
    L = load_library()
    if table == "default":
        table = os.environ.get("QLL_TABLE") or default_table()
    rc = L.qll_init(table.encode() if table else None)
    _table_state = (table, rc)
    return rc


def _ensure_init():
    if _table_state is None:
        init()


# --------------------------------------------------------------------------
# marshalling helpers (plumbing only)
# --------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dev_ptr(t, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _on(stream):
    """Context in which the binding allocates what it hands to the library:
    the stream the kernels are enqueued on, so that torch's caching allocator
    never gives a temporary (the Split-K workspace) to other work before
    those kernels have used it."""
    import contextlib
    torch = _torch()
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _cfg(op: int, cfg):
    """cfg: None, a qll_cfg, or (variant name or index, splits)."""
    if cfg is None or isinstance(cfg, qll_cfg):
        return cfg
    v, s = cfg
    if isinstance(v, str):
        idx = load_library().qll_variant_index(op, v.encode())
        if idx < 0:
            raise ValueError(f"unknown variant {v!r}")
        v = idx
    return qll_cfg(int(v), int(s))


def _workspace(op, M, N, K, cfg, workspace):
    torch = _torch()
    L = load_library()
    need = L.qll_workspace_bytes(op, M, N, K, ctypes.byref(cfg) if cfg else None)
    if need < 0:
        raise QllError("qll_workspace_bytes", -need)
    if need == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device="cuda")
    nbytes = workspace.numel() * workspace.element_size()
    return workspace, nbytes


def _out(out, M, N, out_dtype, device):
    torch = _torch()
    dt = {"bf16": torch.bfloat16, "fp32": torch.float32, "int32": torch.int32}[out_dtype]
    if out is None:
        out = torch.empty((M, N), dtype=dt, device=device)
    elif out.dtype != dt or tuple(out.shape) != (M, N):
        raise ValueError(f"out must be {dt} of shape {(M, N)}")
    return out


def _bytes8(t, name):
    """fp8 / int8 tensors are passed as bytes."""
    torch = _torch()
    if t.dtype not in (torch.float8_e4m3fn, torch.uint8, torch.int8):
        raise TypeError(f"{name} must be float8_e4m3fn, uint8 or int8")
    return _dev_ptr(t, name)


def _f32(t, name, shape):
    """fp32 scales of the given shape; a vector of length L may also come as
    [L][1] (what the per-token quantizer returns)."""
    torch = _torch()
    ok = t.dtype == torch.float32 and (
        tuple(t.shape) == tuple(shape) or
        (len(shape) == 1 and tuple(t.shape) == (shape[0], 1)))
    if not ok:
        raise ValueError(f"{name} must be float32 of shape {tuple(shape)}")
    return _dev_ptr(t, name)


# --------------------------------------------------------------------------
# quantizers
# --------------------------------------------------------------------------

def quantize_per_token_fp8(x, group: int | None = None, q=None, scales=None,
                           stream=None):
    """bf16 [M][K] -> (e4m3 [M][K], fp32 scales [M][K/group]); group None =
    per token, 128 = per 1x128 group."""
    torch = _torch()
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be a 2-D bfloat16 tensor")
    M, K = x.shape
    G = K if group in (None, 0, K) else int(group)
    with _on(stream):
        if q is None:
            q = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=x.device)
        if scales is None:
            scales = torch.empty((M, K // G if G else 0), dtype=torch.float32,
                                 device=x.device)
    if tuple(q.shape) != (M, K) or tuple(scales.shape) != (M, K // G):
        raise ValueError("q / scales have the wrong shape")
    rc = load_library().quantize_per_token_fp8(
        _dev_ptr(x, "x"), _bytes8(q, "q"), _dev_ptr(scales, "scales"), M, K,
        0 if G == K else G, _stream(stream))
    _check("quantize_per_token_fp8", rc)
    return q, scales


def quantize_weight_block_fp8(w, q=None, scales=None, stream=None):
    """bf16 [N][K] -> (e4m3 [N][K], fp32 scales [ceil(N/128)][K/128])."""
    torch = _torch()
    if w.dtype != torch.bfloat16 or w.dim() != 2:
        raise ValueError("w must be a 2-D bfloat16 tensor")
    N, K = w.shape
    with _on(stream):
        if q is None:
            q = torch.empty((N, K), dtype=torch.float8_e4m3fn, device=w.device)
        if scales is None:
            scales = torch.empty(((N + 127) // 128, K // 128), dtype=torch.float32,
                                 device=w.device)
    rc = load_library().quantize_weight_block_fp8(
        _dev_ptr(w, "w"), _bytes8(q, "q"), _dev_ptr(scales, "scales"), N, K,
        _stream(stream))
    _check("quantize_weight_block_fp8", rc)
    return q, scales


# --------------------------------------------------------------------------
# GEMMs
# --------------------------------------------------------------------------

def _scaled_gemm(fn, op, A, B, sa, sb, sa_shape, sb_shape, out_dtype, out, cfg,
                 workspace, stream):
    _ensure_init()
    M, K = A.shape
    N, K2 = B.shape
    if K2 != K:
        raise ValueError(f"A is [M][{K}] but B is [N][{K2}]")
    pa, pb = _bytes8(A, "A"), _bytes8(B, "B")
    psa, psb = _f32(sa, "sa", sa_shape(M, N, K)), _f32(sb, "sb", sb_shape(M, N, K))
    c = _cfg(op, cfg)
    with _on(stream):
        out = _out(out, M, N, out_dtype, A.device)
        ws, wsb = _workspace(op, M, N, K, c, workspace)
        L = load_library()
        args = [pa, pb, psa, psb, _dev_ptr(out, "out"), OUT[out_dtype], M, N, K,
                ws.data_ptr() if ws is not None else None, wsb, _stream(stream)]
        rc = getattr(L, fn + "_ex")(*args, ctypes.byref(c)) if c else getattr(L, fn)(*args)
    _check(fn, rc)
    return out


def gemm_w8a8_int8(A, B, sa, sb, out_dtype="bf16", out=None, cfg=None,
                   workspace=None, stream=None):
    """int8 A [M][K] x int8 B [N][K] with fp32 sa [M], sb [N]."""
    return _scaled_gemm("gemm_w8a8_int8", 0, A, B, sa, sb,
                        lambda M, N, K: (M,), lambda M, N, K: (N,), out_dtype,
                        out, cfg, workspace, stream)


def gemm_fp8_scaled(A, B, sa, sb, out_dtype="bf16", out=None, cfg=None,
                    workspace=None, stream=None):
    """e4m3 A [M][K] x e4m3 B [N][K] with fp32 sa [M], sb [N]."""
    return _scaled_gemm("gemm_fp8_scaled", 1, A, B, sa, sb,
                        lambda M, N, K: (M,), lambda M, N, K: (N,), out_dtype,
                        out, cfg, workspace, stream)


def gemm_fp8_scaled_noalloc(A, B, sa, sb, out, out_dtype="bf16", stream=None):
    """gemm_fp8_scaled without a workspace (the library's static Split-K
    scratch array; nothing allocated): the caller passes the output too."""
    _ensure_init()
    M, K = A.shape
    N, K2 = B.shape
    if K2 != K:
        raise ValueError(f"A is [M][{K}] but B is [N][{K2}]")
    if out is None:
        raise ValueError("out must be given (this entry point allocates nothing)")
    out = _out(out, M, N, out_dtype, A.device)
    rc = load_library().gemm_fp8_scaled_noalloc(
        _bytes8(A, "A"), _bytes8(B, "B"), _f32(sa, "sa", (M,)), _f32(sb, "sb", (N,)),
        _dev_ptr(out, "out"), OUT[out_dtype], M, N, K, _stream(stream))
    _check("gemm_fp8_scaled_noalloc", rc)
    return out


def gemm_block_fp8(A, B, sa, sb, out_dtype="bf16", out=None, cfg=None,
                   workspace=None, stream=None):
    """e4m3 A [M][K] x e4m3 B [N][K], sa [M][K/128], sb [ceil(N/128)][K/128]."""
    return _scaled_gemm("gemm_block_fp8", 2, A, B, sa, sb,
                        lambda M, N, K: (M, K // 128),
                        lambda M, N, K: ((N + 127) // 128, K // 128), out_dtype,
                        out, cfg, workspace, stream)


def gemm_bf16_batch_invariant(A, B, out_dtype="bf16", out=None, cfg=None,
                              workspace=None, stream=None):
    """bf16 A [M][K] x bf16 B [N][K]; row m independent of M."""
    torch = _torch()
    _ensure_init()
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError("A and B must be bfloat16")
    M, K = A.shape
    N, K2 = B.shape
    if K2 != K:
        raise ValueError(f"A is [M][{K}] but B is [N][{K2}]")
    c = _cfg(3, cfg)
    with _on(stream):
        out = _out(out, M, N, out_dtype, A.device)
        ws, wsb = _workspace(3, M, N, K, c, workspace)
        L = load_library()
        args = [_dev_ptr(A, "A"), _dev_ptr(B, "B"), _dev_ptr(out, "out"),
                OUT[out_dtype], M, N, K, ws.data_ptr() if ws is not None else None,
                wsb, _stream(stream)]
        if c:
            rc = L.gemm_bf16_batch_invariant_ex(*args, ctypes.byref(c))
        else:
            rc = L.gemm_bf16_batch_invariant(*args)
    _check("gemm_bf16_batch_invariant", rc)
    return out


def _u8(t, name, shape):
    torch = _torch()
    if t.dtype != torch.uint8 or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be uint8 of shape {tuple(shape)}")
    return _dev_ptr(t, name)


def quantize_mxfp4(x, q=None, scales=None, stream=None):
    """bf16 [M][K] -> (packed E2M1 codes uint8 [M][K/2], E8M0 scale bytes
    uint8 [M][K/32]); K % 32 == 0."""
    torch = _torch()
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be a 2-D bfloat16 tensor")
    M, K = x.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    with _on(stream):
        if q is None:
            q = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
        if scales is None:
            scales = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device)
    rc = load_library().quantize_mxfp4(
        _dev_ptr(x, "x"), _u8(q, "q", (M, K // 2)), _u8(scales, "scales", (M, K // 32)),
        M, K, _stream(stream))
    _check("quantize_mxfp4", rc)
    return q, scales


def gemm_mxfp4(A, B, sa, sb, out_dtype="bf16", out=None, cfg=None, workspace=None,
               stream=None):
    """MXFP4 A [M][K/2] x B [N][K/2] (packed codes, uint8) with E8M0 scale
    bytes sa [M][K/32], sb [N][K/32] (uint8)."""
    _ensure_init()
    M, K2 = A.shape
    N, K2b = B.shape
    if K2b != K2:
        raise ValueError(f"A is [M][{K2}] but B is [N][{K2b}] bytes")
    K = 2 * K2
    pa, pb = _u8(A, "A", (M, K2)), _u8(B, "B", (N, K2))
    psa, psb = _u8(sa, "sa", (M, K // 32)), _u8(sb, "sb", (N, K // 32))
    c = _cfg(4, cfg)
    with _on(stream):
        out = _out(out, M, N, out_dtype, A.device)
        ws, wsb = _workspace(4, M, N, K, c, workspace)
        L = load_library()
        args = [pa, pb, psa, psb, _dev_ptr(out, "out"), OUT[out_dtype], M, N, K,
                ws.data_ptr() if ws is not None else None, wsb, _stream(stream)]
        rc = L.gemm_mxfp4_ex(*args, ctypes.byref(c)) if c else L.gemm_mxfp4(*args)
    _check("gemm_mxfp4", rc)
    return out


def quantize_int4_weights(w, q=None, scales=None, stream=None):
    """bf16 weights [N][K] -> (packed int4 codes uint8 [N][K/2], fp32 scales
    [N][K/128]); K % 128 == 0."""
    torch = _torch()
    if w.dtype != torch.bfloat16 or w.dim() != 2:
        raise ValueError("w must be a 2-D bfloat16 tensor")
    N, K = w.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    with _on(stream):
        if q is None:
            q = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
        if scales is None:
            scales = torch.empty((N, K // 128), dtype=torch.float32, device=w.device)
    rc = load_library().quantize_int4_weights(
        _dev_ptr(w, "w"), _u8(q, "q", (N, K // 2)), _f32(scales, "scales", (N, K // 128)),
        N, K, _stream(stream))
    _check("quantize_int4_weights", rc)
    return q, scales


def gemm_w4a16(A, B, scales, out_dtype="bf16", out=None, cfg=None, workspace=None,
               stream=None):
    """bf16 A [M][K] x packed int4 B [N][K/2] (uint8) with fp32 group scales
    [N][K/128]."""
    torch = _torch()
    _ensure_init()
    if A.dtype != torch.bfloat16 or A.dim() != 2:
        raise TypeError("A must be a 2-D bfloat16 tensor")
    M, K = A.shape
    N = B.shape[0]
    pb = _u8(B, "B", (N, K // 2))
    ps = _f32(scales, "scales", (N, K // 128))
    c = _cfg(5, cfg)
    with _on(stream):
        out = _out(out, M, N, out_dtype, A.device)
        ws, wsb = _workspace(5, M, N, K, c, workspace)
        L = load_library()
        args = [_dev_ptr(A, "A"), pb, ps, _dev_ptr(out, "out"), OUT[out_dtype], M, N, K,
                ws.data_ptr() if ws is not None else None, wsb, _stream(stream)]
        rc = L.gemm_w4a16_ex(*args, ctypes.byref(c)) if c else L.gemm_w4a16(*args)
    _check("gemm_w4a16", rc)
    return out


def linear_fp8_dynamic(x, B, sb, out_dtype="bf16", out=None, q=None, sa=None, cfg=None,
                       workspace=None, stream=None):
    """bf16 x [M][K] -> (out [M][N], q e4m3 [M][K], sa fp32 [M][1]): per-token
    quantization of x and the scaled FP8 GEMM with e4m3 B [N][K], sb [N]."""
    torch = _torch()
    _ensure_init()
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be a 2-D bfloat16 tensor")
    M, K = x.shape
    N, K2 = B.shape
    if K2 != K:
        raise ValueError(f"x is [M][{K}] but B is [N][{K2}]")
    # the quantizer writes M x K codes into q: its shape is checked before
    # anything is enqueued
    if q is not None and tuple(q.shape) != (M, K):
        raise ValueError(f"q must have shape {(M, K)}")
    c = _cfg(6, cfg)  # the FP8 GEMM variants, then the fused ones
    with _on(stream):
        if q is None:
            q = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=x.device)
        if sa is None:
            sa = torch.empty((M, 1), dtype=torch.float32, device=x.device)
        out = _out(out, M, N, out_dtype, x.device)
        ws, wsb = _workspace(6, M, N, K, c, workspace)
        L = load_library()
        args = [_dev_ptr(x, "x"), _bytes8(B, "B"), _f32(sb, "sb", (N,)), _bytes8(q, "q"),
                _f32(sa, "sa", (M,)), _dev_ptr(out, "out"), OUT[out_dtype], M, N, K,
                ws.data_ptr() if ws is not None else None, wsb, _stream(stream)]
        rc = (L.linear_fp8_dynamic_ex(*args, ctypes.byref(c)) if c
              else L.linear_fp8_dynamic(*args))
    _check("linear_fp8_dynamic", rc)
    return out, q, sa


def gemm_fp8_grouped(A, B, sa, sb, offsets, out_dtype="bf16", out=None, variant=None,
                     stream=None):
    """Grouped (per-expert) FP8 GEMM: A e4m3 [M][K] with rows sorted by
    expert, B e4m3 [E][N][K], sa fp32 [M], sb fp32 [E][N], offsets int32
    [E + 1] on the GPU (rows [offsets[e], offsets[e+1]) use expert e)."""
    torch = _torch()
    _ensure_init()
    M, K = A.shape
    E, N, K2 = B.shape
    if K2 != K:
        raise ValueError(f"A is [M][{K}] but B is [E][N][{K2}]")
    if offsets.dtype != torch.int32 or tuple(offsets.shape) != (E + 1,):
        raise ValueError(f"offsets must be int32 of shape ({E + 1},)")
    with _on(stream):
        out = _out(out, M, N, out_dtype, A.device)
    args = [_bytes8(A, "A"), _bytes8(B, "B"), _f32(sa, "sa", (M,)),
            _f32(sb, "sb", (E, N)), _dev_ptr(offsets, "offsets"), _dev_ptr(out, "out"),
            OUT[out_dtype], M, N, K, E, _stream(stream)]
    L = load_library()
    rc = (L.gemm_fp8_grouped_ex(*args, variant.encode()) if variant
          else L.gemm_fp8_grouped(*args))
    _check("gemm_fp8_grouped", rc)
    return out


def grouped_select(M: int, E: int) -> str:
    """The variant gemm_fp8_grouped picks for M rows over E experts."""
    buf = ctypes.create_string_buffer(64)
    _check("qll_grouped_select", load_library().qll_grouped_select(M, E, buf, 64))
    return buf.value.decode()


# --------------------------------------------------------------------------
# registry / dispatch introspection
# --------------------------------------------------------------------------

def variants(op: str | int) -> list[dict]:
    L = load_library()
    o = OPS[op] if isinstance(op, str) else op
    buf = ctypes.create_string_buffer(512)
    out = []
    for i in range(L.qll_num_variants(o)):
        _check("qll_variant_info", L.qll_variant_info(o, i, buf, 512))
        d = json.loads(buf.value.decode())
        d["index"] = i
        out.append(d)
    return out


def select(op: str | int, M: int, N: int, K: int) -> tuple[str, int]:
    """(variant name, requested splits) the entry point would use."""
    _ensure_init()
    L = load_library()
    o = OPS[op] if isinstance(op, str) else op
    c = qll_cfg()
    _check("qll_select", L.qll_select(o, M, N, K, ctypes.byref(c)))
    return variants(o)[c.variant]["name"], c.splits


def effective_splits(op: str | int, K: int, splits: int) -> int:
    o = OPS[op] if isinstance(op, str) else op
    return load_library().qll_effective_splits(o, K, splits)


def workspace_bytes(op: str | int, M: int, N: int, K: int, cfg=None) -> int:
    o = OPS[op] if isinstance(op, str) else op
    c = _cfg(o, cfg)
    n = load_library().qll_workspace_bytes(o, M, N, K, ctypes.byref(c) if c else None)
    if n < 0:
        raise QllError("qll_workspace_bytes", -n)
    return n


def table_entries() -> int:
    return load_library().qll_table_entries()


def parse_signature(sig: str) -> tuple[str, int, int, str]:
    """'<arch> <CUs> <MHz> <name>' -> (arch, cus, mhz, name); the name may be
    empty."""
    parts = sig.strip().split(None, 3)
    if len(parts) < 3:
        raise ValueError(f"bad device signature {sig!r}")
    return parts[0], int(parts[1]), int(parts[2]), (parts[3].strip() if len(parts) > 3 else "")


def table_signature(path: str) -> str | None:
    """The device signature on a table file's device line (None if absent)."""
    with open(path) as f:
        for line in f:
            t = line.strip()
            if t.startswith("device ") or t.startswith("device\t"):
                return t[len("device"):].strip()
    return None


def table_validate(path: str, signature: str):
    """(status, reason) of checking a table file against a device signature
    '<arch> <CUs> <MHz> <name>'."""
    arch, cus, mhz, name = parse_signature(signature)
    buf = ctypes.create_string_buffer(512)
    rc = load_library().qll_table_validate(path.encode(), arch.encode(), cus, mhz,
                                           name.encode(), buf, 512)
    return rc, buf.value.decode()


def device_signature() -> str:
    """The current device's signature, as a table's device line holds it."""
    buf = ctypes.create_string_buffer(512)
    _check("qll_device_signature", load_library().qll_device_signature(buf, 512))
    return buf.value.decode()
