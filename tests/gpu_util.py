"""Helpers shared by the GPU parity tests: moving the seeded host arrays to
the device with the right dtype, and the floating-point acceptance rule.

Acceptance rule for floating-point outputs (the GPU accumulates in fp32 on the
matrix cores in an order of its own, so several results are correct):
  * normwise:  max|y - ref| / max|ref| <= 1e-2 (bf16 out) or 2e-3 (fp32 out);
  * elementwise a-priori bound, for every output element:
        |y - ref| <= c_out * |ref| + ((K + K/128 + 4) * 2^-23 + t_mfma) * absref
    where absref = sum_k |scale * a_k * b_k| (from the oracle), c_out = 2^-8
    (one bf16 rounding) or 2^-22 (the fp32 epilogue products), and 2^-23 is
    the fp32 unit roundoff doubled so that accumulation by truncation is
    covered as well as by rounding.  t_mfma is the matrix core's own term,
    per instruction kind (MFMA_TERM; the measurement is pinned by
    test_gpu_mfma_precision.py at K = 256 and 2048): gfx950's e4m3 x e4m3
    steps (16x16x128 and 32x32x64 alike) add their products more coarsely
    than step-by-step fp32 -- errors up to 2^-13.2 of absref at K = 256,
    over three times the fp32-only term there, and no larger at K = 2048 --
    so the e4m3 ops carry t_mfma = 2^-12 (the per-step errors add up to at
    most that fraction of absref, the steps partitioning K); the bf16, MXFP4
    (scaled E2M1) and W4A16 (bf16 on widened int4) steps stay below 2^-22 of
    absref, well inside the fp32 term, and carry none.
"""
import numpy as np
import torch

from workloads import to_bf16_bits


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


# the matrix core's own term per instruction kind (see the module docstring)
MFMA_TERM = {"e4m3": 2.0 ** -12, "bf16": 0.0, "fp4": 0.0, "w4a16": 0.0}


def check_fp(y: np.ndarray, ref: np.ndarray, absref: np.ndarray, K: int,
             out_dtype: str, what: str = "", mfma: str = "e4m3"):
    y = np.asarray(y, np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    err = np.abs(y - ref)
    denom = max(np.max(np.abs(ref)), 1e-300)
    normwise = np.max(err) / denom if err.size else 0.0
    tol = 1e-2 if out_dtype == "bf16" else 2e-3
    assert normwise <= tol, f"{what}: normwise error {normwise:.3e} > {tol}"
    c_out = 2.0 ** -8 if out_dtype == "bf16" else 2.0 ** -22
    bound = c_out * np.abs(ref) + ((K + K // 128 + 4) * 2.0 ** -23 + MFMA_TERM[mfma]) * absref
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


def check_all_rows(y: torch.Tensor, ref: torch.Tensor, out_dtype: str, what: str = ""):
    """Every row of a full-size output against a float64 product computed on
    the device (decoded operands times scales, a test-only reference): all
    values finite and each row within the normwise bar of its own largest
    reference value.  The oracle's sampled rows carry the elementwise bound;
    this catches a tile that is misplaced or never written anywhere in the
    output."""
    yd = y.to(torch.float64)
    assert bool(torch.isfinite(yd).all()), f"{what}: non-finite output"
    tol = 1e-2 if out_dtype == "bf16" else 2e-3
    err = (yd - ref).abs().amax(dim=1)
    den = ref.abs().amax(dim=1).clamp_min(1e-300)
    worst = (err / den).max().item() if err.numel() else 0.0
    assert worst <= tol, f"{what}: a row's normwise error {worst:.3e} > {tol}"
    return worst


def fp8_product(q: torch.Tensor, qB: torch.Tensor, sa: torch.Tensor, sb: torch.Tensor):
    """float64 (q * sa) (qB * sb)^T on the device, per-token x per-channel."""
    f64 = torch.float64
    ref = q.float().to(f64) @ qB.float().to(f64).T
    return ref * sa.reshape(-1, 1).to(f64) * sb.reshape(1, -1).to(f64)


def block_fp8_product(q: torch.Tensor, qB: torch.Tensor, sa: torch.Tensor, sb: torch.Tensor):
    """float64 Block-FP8 product on the device: sum over 128-wide K groups of
    the group's partial times sa[m][g] * sb[n / 128][g]."""
    f64 = torch.float64
    M, K = q.shape
    N = qB.shape[0]
    a, b = q.float().to(f64), qB.float().to(f64)
    sbn = sb.to(f64).repeat_interleave(128, dim=0)[:N]
    ref = torch.zeros((M, N), dtype=f64, device=q.device)
    for g in range(K // 128):
        k = slice(128 * g, 128 * g + 128)
        ref += (a[:, k] @ b[:, k].T) * (sa.to(f64)[:, g, None] * sbn[None, :, g])
    return ref


def edge_rows(K, seed=22):
    """zeros, signed zeros, tiny values that round to +-0, bf16 subnormals,
    values at the clamp and scales on both sides of the reciprocal path's
    range, as rows of K elements"""
    g = np.random.default_rng(seed)
    rows = []
    r = np.zeros(K, np.uint16)
    rows.append(r.copy())                            # all zero
    r[:] = 0x8000
    rows.append(r.copy())                            # all -0.0
    big = to_bf16_bits(np.float32([448.0]))[0]
    for scale in (1.0, 1e-3, 2.0**-55, 2.0**-58, 2.0**-61, 1e-30, 2.0**68, 2.0**71, 1e37):
        v = (g.standard_normal(K) * scale).astype(np.float32)
        v[::7] *= np.float32(1e-6)
        b = to_bf16_bits(v)
        b[0] = big if scale == 1.0 else b[0]
        rows.append(b)
    sub = np.arange(1, K + 1, dtype=np.uint16) & 0x7F    # bf16 subnormals
    sub[1::2] |= 0x8000
    rows.append(sub)
    return np.stack(rows)
