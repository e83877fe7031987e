"""Seeded synthetic inputs for the scaled_mm workloads.

This module only draws random numbers and casts them to the storage types;
it holds none of the quantization or GEMM arithmetic.  Both the CPU oracle
(tests) and the HIP path (tests, bench) take their inputs from here, so both
sides see the same bytes.

Every array comes from ``numpy.random.default_rng([0, *key])`` (seed 0 for
every workload), is drawn and scaled in float32 and is then cast once, with
round-to-nearest-even, to bfloat16 by torch's CPU cast where a bf16 tensor is
wanted.  Shapes follow the layouts of the library: activations A are [M][K]
row-major, weights B are [N][K] row-major (the K x N operand stored
column-major, as a linear layer keeps it).

Workloads (the shapes of the pages' serving GEMMs: lm_head scale N=12288,
MLP down-projection N=2048 K=6144, attention projection N=4096, a large
vocabulary N=151936 and a square N=K=2048 weight):
  W8A8 INT8    M=16, N=K=2048; int8 uniform in [-127, 127]; fp32 scales
               uniform in [1e-3, 1e-2] per row of A and per row of B.
  FP8 dynamic  (N, K) in {(4096, 2048), (2048, 6144)}, M in FP8_M; A bf16
               N(0, 1) with round(0.01 K) outlier channels (the same columns in
               every row) multiplied by 20; W bf16 N(0, 0.02).
  Block-FP8    (N, K) in {(12288, 2048), (2048, 6144)}, M in BLOCK_M; A bf16
               N(0, 1); W bf16 N(0, 0.02).
  bf16 BI      (N, K) in {(2048, 2048), (4096, 2048)}, M in BI_M; A and B bf16
               N(0, 1) / sqrt(K); each M uses the first M rows of a 2048-row A.
  Vocab        N=151936, K=2048, M in VOCAB_M; A bf16 N(0, 1), W bf16
               N(0, 0.02); both the bf16 and the FP8 path on the same data.
  Grouped FP8  MOE_E = 64 experts of N=1536 x K=2048 weights (bf16 N(0, 0.02),
               quantized per output channel), T in MOE_T tokens routed to
               MOE_TOPK = 8 experts each with a skewed synthetic routing; the
               routed rows (bf16 N(0, 1) with outliers) are quantized per
               token.
  MXFP4        the FP8 dynamic shapes and M values on the same kind of data
               (A bf16 N(0, 1) with outlier channels, W bf16 N(0, 0.02)),
               both quantized to MXFP4; parity cases also draw packed codes
               uniformly over all 256 bytes and scale bytes uniform in a
               band around 2^0.
  INT4 W4A16   the FP8 dynamic shapes and M values: A bf16 N(0, 1) with
               outlier channels, W bf16 N(0, 0.02) quantized to int4 per
               128-element group; parity cases also draw packed codes over all
               256 bytes and fp32 group scales uniform in [1e-3, 1e-2].
"""
from __future__ import annotations

import os

import numpy as np

INT8_SHAPE = (16, 2048, 2048)  # M, N, K
FP8_SHAPES = [(4096, 2048), (2048, 6144)]  # (N, K)
FP8_M = [1, 4, 8, 16, 32, 64, 256, 512, 1024, 2048]
BLOCK_SHAPES = [(12288, 2048), (2048, 6144)]
BLOCK_M = [1, 16, 64, 256, 2048]
BI_SHAPES = [(2048, 2048), (4096, 2048)]
BI_M = [1, 4, 8, 16, 32, 64, 256, 512, 1024, 2048]
VOCAB_SHAPE = (151936, 2048)
VOCAB_M = [1, 8, 64, 512, 2048]
MAX_M = 2048
# grouped (per-expert) FP8 GEMM: E experts of [N][K] weights, T tokens each
# routed to TOPK distinct experts
MOE_E, MOE_TOPK = 64, 8
MOE_SHAPE = (1536, 2048)  # (N, K)
MOE_T = [16, 128, 1024]
# MXFP4 and INT4 weight-only: the FP8 dynamic (N, K) shapes and M values
MX_SHAPES = FP8_SHAPES
MX_M = FP8_M
W4_SHAPES = FP8_SHAPES
W4_M = FP8_M

# workload ids used in the seeds
W_INT8, W_FP8, W_BLOCK, W_BI, W_VOCAB, W_MOE, W_MX, W_W4, W_TEST = 1, 2, 3, 4, 5, 6, 7, 8, 9


def rng(*key) -> np.random.Generator:
    return np.random.default_rng([0, *[int(k) for k in key]])


def to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 array -> bfloat16 bit patterns (uint16), one RNE cast by torch."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def int8_uniform(shape, key) -> np.ndarray:
    """Integers uniform in [-127, 127] inclusive."""
    return rng(*key).integers(-127, 128, size=shape, dtype=np.int8)


def scales_uniform(n, key, lo=1e-3, hi=1e-2) -> np.ndarray:
    return rng(*key).uniform(lo, hi, size=n).astype(np.float32)


_CHUNK = 1 << 20  # elements per independently seeded block of rows


def normal_f32(shape, key, std=1.0) -> np.ndarray:
    """N(0, std) in float32.  Rows are drawn in blocks of about 2^20 elements,
    block j from rng(*key, j), on a few threads; the values depend only on
    the shape and the key."""
    shape = tuple(int(s) for s in shape)
    rows = shape[0] if len(shape) > 1 else 1
    cols = int(np.prod(shape[1:])) if len(shape) > 1 else int(np.prod(shape))
    x = np.empty((rows, cols), dtype=np.float32)
    per = max(1, _CHUNK // max(cols, 1))
    blocks = [(j, r, min(rows, r + per)) for j, r in enumerate(range(0, rows, per))]

    def fill(b):
        j, r0, r1 = b
        rng(*key, j).standard_normal(out=x[r0:r1], dtype=np.float32)
        if std != 1.0:
            np.multiply(x[r0:r1], np.float32(std), out=x[r0:r1])

    if len(blocks) > 4:
        import concurrent.futures as cf
        with cf.ThreadPoolExecutor(min(16, os.cpu_count() or 4)) as ex:
            list(ex.map(fill, blocks))
    else:
        for b in blocks:
            fill(b)
    return x.reshape(shape)


def bf16_normal(shape, key, std=1.0, inv_sqrt_k=False, outlier_frac=0.0,
                outlier_mult=20.0) -> np.ndarray:
    """bf16 bits of N(0, std) (optionally / sqrt(K)), with an optional set of
    outlier columns (round(outlier_frac * K) distinct columns, drawn without
    replacement, the same for every row) multiplied by outlier_mult."""
    x = normal_f32(shape, key, std)
    K = shape[-1]
    if inv_sqrt_k:
        x = x / np.float32(np.sqrt(np.float32(K)))
    if outlier_frac > 0.0:
        n_out = int(round(outlier_frac * K))
        cols = rng(*key, 1 << 30).choice(K, size=n_out, replace=False)
        x[..., cols] *= np.float32(outlier_mult)
    return to_bf16_bits(x)


# --------------------------------------------------------------------------
# Per-workload inputs
# --------------------------------------------------------------------------

def int8_inputs(M=16, N=2048, K=2048, key=(W_INT8,)):
    """A int8 [M][K], B int8 [N][K], sa fp32 [M], sb fp32 [N]."""
    return dict(A=int8_uniform((M, K), (*key, 0)),
                B=int8_uniform((N, K), (*key, 1)),
                sa=scales_uniform(M, (*key, 2)),
                sb=scales_uniform(N, (*key, 3)))


def fp8_activations(M, K, key=(W_FP8,)):
    """bf16 activations with 1% outlier channels x20 (first M rows of a
    MAX_M-row draw when M <= MAX_M, so every M shares its leading rows)."""
    rows = max(M, MAX_M)
    return bf16_normal((rows, K), (*key, K, 0), outlier_frac=0.01)[:M].copy()


def weights_bf16(N, K, key=(W_FP8,), std=0.02):
    return bf16_normal((N, K), (*key, N, K, 1), std=std)


def block_activations(M, K, key=(W_BLOCK,)):
    rows = max(M, MAX_M)
    return bf16_normal((rows, K), (*key, K, 0))[:M].copy()


def bi_inputs(N, K, key=(W_BI,)):
    """A_full bf16 [2048][K] and B bf16 [N][K], both N(0,1)/sqrt(K)."""
    return dict(A_full=bf16_normal((MAX_M, K), (*key, N, K, 0), inv_sqrt_k=True),
                B=bf16_normal((N, K), (*key, N, K, 1), inv_sqrt_k=True))


def vocab_activations(K=2048, key=(W_VOCAB,)):
    return bf16_normal((MAX_M, K), (*key, K, 0))


def vocab_weights(N=151936, K=2048, key=(W_VOCAB,)):
    return bf16_normal((N, K), (*key, N, K, 1), std=0.02)


def moe_routing(T, E=MOE_E, topk=MOE_TOPK, key=(W_MOE,)):
    """Synthetic routing: each of T tokens picks `topk` distinct experts with
    probabilities proportional to 1 / (rank + 1) over a seeded random order of
    the experts (a skewed load, some experts empty at small T).  Returns the
    expert offsets (int32 [E + 1]) of the rows sorted by expert: T * topk rows."""
    g = rng(*key, T, E, topk)
    order = g.permutation(E)
    p = 1.0 / (np.arange(E) + 1.0)
    p = p / p.sum()
    counts = np.zeros(E, dtype=np.int64)
    for _ in range(T):
        pick = g.choice(E, size=topk, replace=False, p=p)
        counts[order[pick]] += 1
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def moe_activations(rows, K, key=(W_MOE,)):
    """bf16 activations of the routed rows, distributed like the FP8 dynamic
    workload (N(0, 1) with outlier channels)."""
    return bf16_normal((rows, K), (*key, 1, rows, K), outlier_frac=0.01)


def moe_weights(E, N, K, key=(W_MOE,)):
    """bf16 expert weights [E][N][K], N(0, 0.02)."""
    return bf16_normal((E * N, K), (*key, 2, E, N, K), std=0.02).reshape(E, N, K)


def mx_activations(M, K, key=(W_MX,)):
    """bf16 activations of the MXFP4 workload (first M rows of a MAX_M-row
    draw, 1% outlier channels x20, like the FP8 dynamic workload)."""
    rows = max(M, MAX_M)
    return bf16_normal((rows, K), (*key, K, 0), outlier_frac=0.01)[:M].copy()


def mx_weights(N, K, key=(W_MX,)):
    return bf16_normal((N, K), (*key, N, K, 1), std=0.02)


def mx_codes(rows, K, key) -> np.ndarray:
    """Packed E2M1 codes [rows][K/2]: every byte uniform over 0..255."""
    return rng(*key).integers(0, 256, size=(rows, K // 2), dtype=np.uint8)


def mx_scale_bytes(rows, K, key, lo=118, hi=136) -> np.ndarray:
    """E8M0 scale bytes [rows][K/32] uniform in [lo, hi]."""
    return rng(*key).integers(lo, hi + 1, size=(rows, K // 32), dtype=np.uint8)


def w4_activations(M, K, key=(W_W4,)):
    """bf16 activations of the INT4 weight-only workload (first M rows of a
    MAX_M-row draw, 1% outlier channels x20)."""
    rows = max(M, MAX_M)
    return bf16_normal((rows, K), (*key, K, 0), outlier_frac=0.01)[:M].copy()


def w4_weights(N, K, key=(W_W4,)):
    return bf16_normal((N, K), (*key, N, K, 1), std=0.02)
