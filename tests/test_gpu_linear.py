"""GPU parity of linear_fp8_dynamic, per-token quantization followed by the
scaled FP8 GEMM in one call ("FP8 dynamic quantization" of "Helion in vLLM:
A Unified Route to Tunable Linear Kernels", "What the integration changes").

Bars: the codes and scales it returns are bit-exact to the oracle's
quantizer; its output is bitwise the output of the two separate calls
(quantize_per_token_fp8 then gemm_fp8_scaled with the same configuration)
and within the floating-point rule of tests/gpu_util.py of the oracle.
"""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from gpu_util import check_fp, dev_bf16, dev_e4m3, dev, host_codes, host_f64  # noqa: E402


@pytest.fixture(scope="module")
def qll():
    import quantized_linear_layer_scaled_amd as q
    q.load_library()
    q.init()
    return q


def two_launch_cfg(qll, M, N, K):
    """The FP8 GEMM configuration whose output the dispatched linear layer
    reproduces bitwise: the fp8_dynamic entry itself, or for a fused variant
    f{HR}x16_w{W}_d{D} the W-wave decode GEMM k{HR}x16_w{W}."""
    name, splits = qll.select("fp8_dynamic", M, N, K)
    if name[0] == "f":
        v = next(x for x in qll.variants("fp8_dynamic") if x["name"] == name)
        return (f"k{v['bp']}x16_w{v['wp']}", 1)
    return (name, splits)


@pytest.mark.parametrize("N,K", [(4096, 2048), (2048, 6144), (520, 1040)])
def test_linear_equals_two_calls_and_oracle(qll, N, K):
    w = workloads.weights_bf16(N, K, key=(workloads.W_TEST, 40))
    B, sb = oracle.quantize_fp8(w)
    dB, dsb = dev_e4m3(B), dev(sb[:, 0].copy())
    x_all = workloads.fp8_activations(64, K, key=(workloads.W_TEST, 41))
    for M in (1, 5, 16, 17, 33, 64):
        x = x_all[:M].copy()
        qr, sr = oracle.quantize_fp8(x)
        ref, absref = oracle.gemm_fp8(qr, B, sr[:, 0].copy(), sb[:, 0].copy(), with_abs=True)
        dx = dev_bf16(x)
        for cfg in (None, ("k16x16_w8", 1), ("k16x16_w16", 1), ("k16x32_w8", 1),
                    ("k16x64_w8", 1), ("k16x16_w8", 2), ("p64x128_w2x2_k128_s4", 1)):
            for od in ("bf16", "fp32"):
                y, q, sa = qll.linear_fp8_dynamic(dx, dB, dsb, out_dtype=od, cfg=cfg)
                q2, sa2 = qll.quantize_per_token_fp8(dx)
                y2 = qll.gemm_fp8_scaled(q2, dB, sa2, dsb, out_dtype=od,
                                         cfg=cfg or two_launch_cfg(qll, M, N, K))
                torch.cuda.synchronize()
                assert np.array_equal(host_codes(q), qr), (M, cfg)
                assert np.array_equal(sa.cpu().numpy().view(np.uint32), sr.view(np.uint32))
                iv = torch.int16 if od == "bf16" else torch.int32
                assert torch.equal(y.view(iv), y2.view(iv)), (M, cfg, od)
                check_fp(host_f64(y), ref, absref, K, od, f"linear {cfg} M={M} {od}")


def test_linear_large_m_sampled(qll):
    N, K = 4096, 2048
    w = workloads.weights_bf16(N, K, key=(workloads.W_TEST, 42))
    B, sb = oracle.quantize_fp8(w)
    x = workloads.fp8_activations(512, K, key=(workloads.W_TEST, 43))
    qr, sr = oracle.quantize_fp8(x)
    rows = [0, 200, 511]
    ref, absref = oracle.gemm_fp8(qr, B, sr[:, 0].copy(), sb[:, 0].copy(), rows=rows,
                                  with_abs=True)
    y, q, sa = qll.linear_fp8_dynamic(dev_bf16(x), dev_e4m3(B), dev(sb[:, 0].copy()))
    torch.cuda.synchronize()
    assert np.array_equal(host_codes(q), qr)
    check_fp(host_f64(y)[rows], ref, absref, K, "bf16", "linear M=512")



@pytest.mark.parametrize("fn", ["gemm", "linear"])
def test_side_stream_split_k_workspace(qll, fn):
    # A forced Split-K call enqueued on a side stream while the default stream
    # stays current: the binding's temporary workspace belongs to the side
    # stream, so an allocation on the default stream right after the call
    # (filled at once) cannot take its memory before the reduction has read
    # it.  Bitwise equal to the same call on the default stream.
    N, K, M = 2048, 6144, 256
    w = workloads.weights_bf16(N, K, key=(workloads.W_TEST, 44))
    B, sb = oracle.quantize_fp8(w)
    dB, dsb = dev_e4m3(B), dev(sb[:, 0].copy())
    x = dev_bf16(workloads.fp8_activations(M, K, key=(workloads.W_TEST, 45)))
    q, sa = qll.quantize_per_token_fp8(x)
    cfg = ("p64x64_w2x2_k128_s2", 4)
    assert qll.workspace_bytes("fp8", M, N, K, cfg) > 0

    def call(stream=None):
        if fn == "gemm":
            return qll.gemm_fp8_scaled(q, dB, sa, dsb, cfg=cfg, stream=stream)
        return qll.linear_fp8_dynamic(x, dB, dsb, cfg=cfg, stream=stream)[0]

    want = call()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    nbytes = qll.workspace_bytes("fp8", M, N, K, cfg)
    for _ in range(3):
        side.wait_stream(torch.cuda.current_stream())
        got = call(stream=side)
        junk = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device="cuda")
        junk.add_(1)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))
        del junk


def fused_steps(K, W):
    """K steps of 128 the busiest of W waves handles (the decode GEMM's cut)."""
    T = -(-K // 128)
    TU = -(-T // 2)
    return max(min(T, 2 * ((w + 1) * TU // W)) - min(T, 2 * (w * TU // W)) for w in range(W))


@pytest.mark.parametrize("N,K", [(4096, 2048), (2048, 6144), (520, 1040), (300, 2064)])
def test_fused_equals_two_launches_and_oracle(qll, N, K):
    # the fused variants: codes and scales bitwise the quantizer's (oracle),
    # output bitwise the two launches with the 8-wave decode GEMM of the same
    # rows per workgroup, and within the bound of the oracle
    w = workloads.weights_bf16(N, K, key=(workloads.W_TEST, 50))
    B, sb = oracle.quantize_fp8(w)
    dB, dsb = dev_e4m3(B), dev(sb[:, 0].copy())
    x_all = workloads.fp8_activations(16, K, key=(workloads.W_TEST, 51))
    fused = [v for v in qll.variants("fp8_dynamic") if v.get("fused")]
    assert len(fused) >= 4
    ran = 0
    for v in fused:
        if fused_steps(K, v["wp"]) > v["ksteps"]:
            with pytest.raises(qll.QllError):
                qll.linear_fp8_dynamic(dev_bf16(x_all[:1]), dB, dsb, cfg=(v["name"], 1))
            continue
        for M in sorted({1, min(3, v["bq"]), v["bq"]}):
            x = x_all[:M].copy()
            qr, sr = oracle.quantize_fp8(x)
            ref, absref = oracle.gemm_fp8(qr, B, sr[:, 0].copy(), sb[:, 0].copy(), with_abs=True)
            dx = dev_bf16(x)
            for od in ("bf16", "fp32"):
                y, q, sa = qll.linear_fp8_dynamic(dx, dB, dsb, out_dtype=od, cfg=(v["name"], 1))
                y2, _, _ = qll.linear_fp8_dynamic(
                    dx, dB, dsb, out_dtype=od, cfg=(f"k{v['bp']}x16_w{v['wp']}", 1))
                torch.cuda.synchronize()
                assert np.array_equal(host_codes(q), qr), (v["name"], M)
                assert np.array_equal(sa.cpu().numpy()[:, 0].view(np.uint32),
                                      sr[:, 0].view(np.uint32)), (v["name"], M)
                iv = torch.int16 if od == "bf16" else torch.int32
                assert torch.equal(y.view(iv), y2.view(iv)), (v["name"], M, od)
                check_fp(host_f64(y), ref, absref, K, od, f"fused {v['name']} M={M} {od}")
                ran += 1
    assert ran > 0


def test_fused_edge_tokens(qll):
    # tokens with zeros, signed zeros, bf16 subnormals, values at the clamp
    # and scales on both sides of the quantizer's reciprocal range: codes and
    # scales bitwise the oracle's, the output bitwise the two launches' and
    # finite (an all-zero token gives scale 0, codes 0 and a zero row).  The
    # token scaled by 1e37 is left out of the finiteness check: the epilogue
    # multiplies left to right, (acc * s[m]) * sb[n], and acc * s[m]
    # (~1e6 * 8e34) overflows fp32 before sb[n] would bring it back -- the
    # same in both paths, which the bitwise check covers
    from gpu_util import edge_rows
    N, K = 520, 2048
    w = workloads.weights_bf16(N, K, key=(workloads.W_TEST, 53))
    B, sb = oracle.quantize_fp8(w)
    dB, dsb = dev_e4m3(B), dev(sb[:, 0].copy())
    x = edge_rows(K)[:16]
    qr, sr = oracle.quantize_fp8(x)
    for name in ("f16x16_w8_d2", "f8x16_w16_d2", "f16x8_w8_d2", "f16x4_w16_d2", "f16x2_w8_d2",
                 "f16x1_w8_d2"):
        v = next(t for t in qll.variants("fp8_dynamic") if t["name"] == name)
        for r0 in range(0, len(x), v["bq"]):
            # the edge rows in groups of the variant's tokens (the first group
            # holds the all-zero tokens)
            xs = x[r0:r0 + v["bq"]].copy()
            y, q, sa = qll.linear_fp8_dynamic(dev_bf16(xs), dB, dsb, out_dtype="fp32",
                                              cfg=(name, 1))
            y2, _, _ = qll.linear_fp8_dynamic(dev_bf16(xs), dB, dsb, out_dtype="fp32",
                                              cfg=(f"k{v['bp']}x16_w{v['wp']}", 1))
            torch.cuda.synchronize()
            assert np.array_equal(host_codes(q), qr[r0:r0 + v["bq"]]), (name, r0)
            assert np.array_equal(sa.cpu().numpy()[:, 0].view(np.uint32),
                                  sr[r0:r0 + v["bq"], 0].view(np.uint32)), (name, r0)
            assert torch.equal(y.view(torch.int32), y2.view(torch.int32)), (name, r0)
            huge = np.abs((xs.astype(np.uint32) << 16).view(np.float32)).max(axis=1) > 1e30
            assert bool(torch.isfinite(y[torch.from_numpy(~huge).cuda()]).all()), (name, r0)
            for i in range(len(xs)):
                if r0 + i < 2:  # the all-zero tokens: zero rows
                    assert bool((y[i] == 0).all()), (name, r0 + i)


def test_fused_refuses_more_than_its_tokens(qll):
    N, K = 520, 1040
    B = dev_e4m3(np.zeros((N, K), np.uint8))
    sb = torch.ones(N, device="cuda")
    x = dev_bf16(workloads.fp8_activations(17, K, key=(workloads.W_TEST, 52)))
    for name, tok in (("f16x16_w8_d2", 16), ("f16x8_w8_d2", 8), ("f16x4_w8_d2", 4),
                      ("f16x2_w8_d2", 2), ("f16x1_w8_d2", 1)):
        with pytest.raises(qll.QllError, match="UNSUPPORTED"):
            qll.linear_fp8_dynamic(x[:tok + 1], B, sb, cfg=(name, 1))
