"""Helpers shared by the GPU parity tests: moving the seeded host arrays to
the device with the right dtype, and the floating-point acceptance rule.

Acceptance rule for floating-point outputs (the GPU accumulates in fp32 on the
matrix cores in an order of its own, so several results are correct):
  * normwise:  max|y - ref| / max|ref| <= 1e-2 (bf16 out) or 2e-3 (fp32 out);
  * elementwise a-priori bound, for every output element:
        |y - ref| <= c_out * |ref| + ((K + K/128 + 4) * 2^-23 + 2^-12) * absref
    where absref = sum_k |scale * a_k * b_k| (from the oracle), c_out = 2^-8
    (one bf16 rounding) or 2^-22 (the fp32 epilogue products), and 2^-23 is
    the fp32 unit roundoff doubled so that accumulation by truncation is
    covered as well as by rounding.  The 2^-12 term covers the matrix core's
    own sum inside one MFMA: gfx950's e4m3 x e4m3 MFMA (128 products per
    lane group) adds its products more coarsely than step-by-step fp32 -- at
    K = 256 every kernel, the plain tiled one included, showed errors up to
    2^-14 of absref, about twice the fp32-only term, and independent of K.
    The per-step errors add up to at most that fraction of absref, since the
    steps partition the K range.
"""
import numpy as np
import torch


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).cuda()


def dev_e4m3(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(
        torch.float8_e4m3fn).cuda()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_bits_bf16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host_codes(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.uint8).cpu().numpy()


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.float64).cpu().numpy()


def check_fp(y: np.ndarray, ref: np.ndarray, absref: np.ndarray, K: int,
             out_dtype: str, what: str = ""):
    y = np.asarray(y, np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    err = np.abs(y - ref)
    denom = max(np.max(np.abs(ref)), 1e-300)
    normwise = np.max(err) / denom if err.size else 0.0
    tol = 1e-2 if out_dtype == "bf16" else 2e-3
    assert normwise <= tol, f"{what}: normwise error {normwise:.3e} > {tol}"
    c_out = 2.0 ** -8 if out_dtype == "bf16" else 2.0 ** -22
    bound = c_out * np.abs(ref) + ((K + K // 128 + 4) * 2.0 ** -23 + 2.0 ** -12) * absref
    bad = err > bound * (1 + 1e-12) + 1e-30
    assert not np.any(bad), (
        f"{what}: {int(bad.sum())} elements outside the a-priori bound; worst "
        f"err {err[bad].max():.3e} at bound {bound[bad][np.argmax(err[bad])]:.3e}")
    return normwise


def sample_rows(M: int, n: int, seed: int = 0) -> np.ndarray:
    """First, last and a few random rows (sorted, unique)."""
    if M <= n:
        return np.arange(M, dtype=np.int64)
    g = np.random.default_rng([seed, M])
    r = set([0, M - 1]) | set(g.choice(M, size=n - 2, replace=False).tolist())
    return np.array(sorted(r), dtype=np.int64)
