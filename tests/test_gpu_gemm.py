"""GPU parity of the four GEMMs against the oracle, for every registered
kernel variant (ordinary and Swap-AB tiles) with and without Split-K, on
shapes that span several tiles and end in ragged M, N and K tails.

Operations: W8A8 INT8, FP8 (per-token x per-channel), Block-FP8 of "Helion in
vLLM: A Unified Route to Tunable Linear Kernels" ("What the integration
changes": ordinary GEMM, Split-K and Swap-AB compute the same product), and
the bf16 product of the batch-invariant matmul (vLLM PR #53446, "Summary").

Bars: INT8 int32 accumulators bit-exact (and the fp32/bf16 epilogue bit-exact,
since it is fully determined by acc and the scales); floating point within
the rule of tests/gpu_util.py; integer-valued FP8 / bf16 inputs bit-exact.
"""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from gpu_util import (check_fp, dev, dev_bf16, dev_e4m3, host_f64)  # noqa: E402


@pytest.fixture(scope="module")
def qll():
    import quantized_linear_layer_scaled_amd as q
    q.load_library()
    q.init(None)  # heuristic only: the variants are forced below anyway
    return q


def names(qll, op):
    return [v["name"] for v in qll.variants(op)]


INT8_SHAPES = [(1, 520, 1040), (37, 300, 2064), (130, 264, 512)]
FP8_SHAPES = [(1, 520, 1040), (37, 300, 2064), (130, 264, 512)]
BLOCK_SHAPES = [(1, 520, 1024), (37, 300, 2048), (130, 264, 512), (300, 648, 1024)]
BF16_SHAPES = [(1, 520, 1032), (37, 300, 2056), (130, 264, 512)]
SPLITS = [1, 3]


# ------------------------------------------------------------------ INT8
@pytest.fixture(scope="module")
def int8_cases():
    out = {}
    for (M, N, K) in INT8_SHAPES:
        d = workloads.int8_inputs(M, N, K, key=(workloads.W_TEST, 30, M, N, K))
        acc, y = oracle.gemm_w8a8_int8(d["A"], d["B"], d["sa"], d["sb"])
        out[(M, N, K)] = (d, acc, y)
    return out


@pytest.mark.parametrize("shape", INT8_SHAPES)
@pytest.mark.parametrize("splits", SPLITS)
def test_int8_all_variants_bit_exact(qll, int8_cases, shape, splits):
    d, acc, y = int8_cases[shape]
    A, B, sa, sb = dev(d["A"]), dev(d["B"]), dev(d["sa"]), dev(d["sb"])
    ybf = oracle.bf16_encode(y)
    for name in names(qll, "int8"):
        cfg = (name, splits)
        o32 = qll.gemm_w8a8_int8(A, B, sa, sb, out_dtype="int32", cfg=cfg)
        of = qll.gemm_w8a8_int8(A, B, sa, sb, out_dtype="fp32", cfg=cfg)
        ob = qll.gemm_w8a8_int8(A, B, sa, sb, out_dtype="bf16", cfg=cfg)
        torch.cuda.synchronize()
        assert np.array_equal(o32.cpu().numpy(), acc), f"{name} S={splits} acc"
        assert np.array_equal(of.cpu().numpy().view(np.uint32), y.view(np.uint32)), \
            f"{name} S={splits} fp32 epilogue"
        assert np.array_equal(ob.view(torch.int16).cpu().numpy().view(np.uint16), ybf), \
            f"{name} S={splits} bf16 epilogue"


def test_int8_closed_forms(qll):
    K = 2048
    for a, b, expect in [(127, -127, -16129 * K), (-128, -128, 16384 * K), (1, 1, K)]:
        A = torch.full((5, K), a, dtype=torch.int8, device="cuda")
        B = torch.full((70, K), b, dtype=torch.int8, device="cuda")
        one = torch.ones(5, device="cuda"), torch.ones(70, device="cuda")
        for name in names(qll, "int8"):
            o = qll.gemm_w8a8_int8(A, B, *one, out_dtype="int32", cfg=(name, 2))
            assert bool((o == expect).all()), (name, a, b)


# ------------------------------------------------------------------ FP8
def fp8_case(M, N, K, key):
    x = workloads.bf16_normal((M, K), (*key, 0), outlier_frac=0.01)
    w = workloads.bf16_normal((N, K), (*key, 1), std=0.02)
    A, sa = oracle.quantize_fp8(x)
    B, sb = oracle.quantize_fp8(w)
    ref, absref = oracle.gemm_fp8(A, B, sa, sb, with_abs=True)
    return A, B, sa[:, 0].copy(), sb[:, 0].copy(), ref, absref


@pytest.fixture(scope="module")
def fp8_cases():
    return {s: fp8_case(*s, key=(workloads.W_TEST, 31, *s)) for s in FP8_SHAPES}


@pytest.mark.parametrize("shape", FP8_SHAPES)
@pytest.mark.parametrize("splits", SPLITS)
def test_fp8_all_variants(qll, fp8_cases, shape, splits):
    A, B, sa, sb, ref, absref = fp8_cases[shape]
    M, N, K = shape
    dA, dB, dsa, dsb = dev_e4m3(A), dev_e4m3(B), dev(sa), dev(sb)
    for name in names(qll, "fp8"):
        for od in ("bf16", "fp32"):
            y = qll.gemm_fp8_scaled(dA, dB, dsa, dsb, out_dtype=od, cfg=(name, splits))
            torch.cuda.synchronize()
            check_fp(host_f64(y), ref, absref, K, od, f"fp8 {name} S={splits} {od}")


def test_fp8_integer_valued_exact(qll):
    # integers in [-16, 16] are exact in e4m3 and every partial sum stays
    # below 2^24, so with unit scales every summation order is exact
    g = np.random.default_rng(32)
    M, N, K = 33, 200, 2048
    ia = g.integers(-16, 17, (M, K)).astype(np.int8)
    ib = g.integers(-16, 17, (N, K)).astype(np.int8)
    A = oracle.e4m3_encode(ia.astype(np.float32))
    B = oracle.e4m3_encode(ib.astype(np.float32))
    exact = oracle.gemm_int8_acc(ia, ib).astype(np.float64)
    ones_m, ones_n = torch.ones(M, device="cuda"), torch.ones(N, device="cuda")
    for name in names(qll, "fp8"):
        for s in (1, 4):
            y = qll.gemm_fp8_scaled(dev_e4m3(A), dev_e4m3(B), ones_m, ones_n,
                                    out_dtype="fp32", cfg=(name, s))
            torch.cuda.synchronize()
            assert np.array_equal(host_f64(y), exact), (name, s)


# ------------------------------------------------------------------ Block-FP8
def block_case(M, N, K, key):
    x = workloads.bf16_normal((M, K), (*key, 0))
    w = workloads.bf16_normal((N, K), (*key, 1), std=0.02)
    A, sa = oracle.quantize_fp8(x, group=128)
    B, sb = oracle.quantize_fp8_block(w)
    ref, absref = oracle.gemm_block_fp8(A, B, sa, sb, with_abs=True)
    return A, B, sa, sb, ref, absref


@pytest.fixture(scope="module")
def block_cases():
    return {s: block_case(*s, key=(workloads.W_TEST, 33, *s)) for s in BLOCK_SHAPES}


@pytest.mark.parametrize("shape", BLOCK_SHAPES)
@pytest.mark.parametrize("splits", SPLITS)
def test_block_all_variants(qll, block_cases, shape, splits):
    A, B, sa, sb, ref, absref = block_cases[shape]
    M, N, K = shape
    dA, dB, dsa, dsb = dev_e4m3(A), dev_e4m3(B), dev(sa), dev(sb)
    for name in names(qll, "block_fp8"):
        for od in ("bf16", "fp32"):
            y = qll.gemm_block_fp8(dA, dB, dsa, dsb, out_dtype=od, cfg=(name, splits))
            torch.cuda.synchronize()
            check_fp(host_f64(y), ref, absref, K, od, f"block {name} S={splits} {od}")


def test_block_equal_scales_match_fp8_exactly(qll):
    # integer-valued codes and power-of-two scales that are equal along K:
    # Block-FP8 reduces to the per-channel FP8 product, exactly
    g = np.random.default_rng(34)
    M, N, K = 20, 256, 1024
    A = oracle.e4m3_encode(g.integers(-16, 17, (M, K)).astype(np.float32))
    B = oracle.e4m3_encode(g.integers(-16, 17, (N, K)).astype(np.float32))
    ra = (2.0 ** g.integers(-3, 4, M)).astype(np.float32)
    rb = (2.0 ** g.integers(-3, 4, N // 128)).astype(np.float32)
    sa = np.repeat(ra[:, None], K // 128, 1)
    sb = np.repeat(rb[:, None], K // 128, 1)
    ref = oracle.gemm_fp8(A, B, ra, np.repeat(rb, 128))
    for name in names(qll, "block_fp8"):
        y = qll.gemm_block_fp8(dev_e4m3(A), dev_e4m3(B), dev(sa), dev(sb),
                               out_dtype="fp32", cfg=(name, 2))
        torch.cuda.synchronize()
        assert np.array_equal(host_f64(y), ref), name


# ------------------------------------------------------------------ bf16
def bf16_case(M, N, K, key):
    A = workloads.bf16_normal((M, K), (*key, 0), inv_sqrt_k=True)
    B = workloads.bf16_normal((N, K), (*key, 1), inv_sqrt_k=True)
    ref, absref = oracle.gemm_bf16(A, B, with_abs=True)
    return A, B, ref, absref


@pytest.fixture(scope="module")
def bf16_cases():
    return {s: bf16_case(*s, key=(workloads.W_TEST, 35, *s)) for s in BF16_SHAPES}


@pytest.mark.parametrize("shape", BF16_SHAPES)
@pytest.mark.parametrize("splits", SPLITS)
def test_bf16_all_variants(qll, bf16_cases, shape, splits):
    A, B, ref, absref = bf16_cases[shape]
    M, N, K = shape
    dA, dB = dev_bf16(A), dev_bf16(B)
    for name in names(qll, "bf16_bi"):
        for od in ("bf16", "fp32"):
            y = qll.gemm_bf16_batch_invariant(dA, dB, out_dtype=od, cfg=(name, splits))
            torch.cuda.synchronize()
            check_fp(host_f64(y), ref, absref, K, od, f"bf16 {name} S={splits} {od}", mfma="bf16")


def test_bf16_integer_valued_exact(qll):
    g = np.random.default_rng(36)
    M, N, K = 17, 150, 1024
    ia = g.integers(-16, 17, (M, K)).astype(np.float32)
    ib = g.integers(-16, 17, (N, K)).astype(np.float32)
    A, B = workloads.to_bf16_bits(ia), workloads.to_bf16_bits(ib)
    exact = oracle.gemm_bf16(A, B)
    for name in names(qll, "bf16_bi"):
        for s in (1, 2):
            y = qll.gemm_bf16_batch_invariant(dev_bf16(A), dev_bf16(B), out_dtype="fp32",
                                              cfg=(name, s))
            torch.cuda.synchronize()
            assert np.array_equal(host_f64(y), exact), (name, s)


# ------------------------------------------------------------------ strategies
def test_splitk_and_swap_are_deterministic(qll, fp8_cases):
    A, B, sa, sb, ref, absref = fp8_cases[(37, 300, 2064)]
    dA, dB, dsa, dsb = dev_e4m3(A), dev_e4m3(B), dev(sa), dev(sb)
    for name in names(qll, "fp8"):
        first = qll.gemm_fp8_scaled(dA, dB, dsa, dsb, out_dtype="fp32", cfg=(name, 4))
        for _ in range(9):
            again = qll.gemm_fp8_scaled(dA, dB, dsa, dsb, out_dtype="fp32", cfg=(name, 4))
            assert torch.equal(first.view(torch.int32), again.view(torch.int32)), name


def test_zero_m_is_noop(qll):
    A = torch.empty((0, 256), dtype=torch.int8, device="cuda")
    B = torch.zeros((64, 256), dtype=torch.int8, device="cuda")
    out = qll.gemm_w8a8_int8(A, B, torch.empty(0, device="cuda"),
                             torch.ones(64, device="cuda"))
    assert out.shape == (0, 64)


def test_workspace_too_small_is_rejected(qll):
    A = torch.zeros((4, 2048), dtype=torch.int8, device="cuda")
    B = torch.zeros((64, 2048), dtype=torch.int8, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(qll.QllError) as e:
        qll.gemm_w8a8_int8(A, B, torch.ones(4, device="cuda"), torch.ones(64, device="cuda"),
                           cfg=("s64x16_w4x1_k256", 4), workspace=ws)
    assert e.value.status == 4


@pytest.mark.parametrize("op", ["bf16_bi", "fp8", "block_fp8"])
def test_swap_equals_ordinary_bitwise(qll, op, fp8_cases, bf16_cases, block_cases):
    # whether the Swap-AB orientation reproduces the ordinary one bit for bit
    # (same MFMA, operands exchanged); the batch-invariant dispatch only mixes
    # orientations if this holds
    if op == "fp8":
        A, B, sa, sb, _, _ = fp8_cases[(37, 300, 2064)]
        args = (dev_e4m3(A), dev_e4m3(B), dev(sa), dev(sb))
        fn = qll.gemm_fp8_scaled
    elif op == "block_fp8":
        A, B, sa, sb, _, _ = block_cases[(37, 300, 2048)]
        args = (dev_e4m3(A), dev_e4m3(B), dev(sa), dev(sb))
        fn = qll.gemm_block_fp8
    else:
        A, B, _, _ = bf16_cases[(37, 300, 2056)]
        args = (dev_bf16(A), dev_bf16(B))
        fn = qll.gemm_bf16_batch_invariant
    # fp8 and Block-FP8: the "k" skinny variants split K across waves and the
    # two-K-group tiles ("_g2") split it between two wave groups (another
    # summation order by design), every other variant accumulates K in one
    # accumulator (Block-FP8: one promotion per K group, in order).
    # bf16: every variant sums K in the same eight chunks, so all agree except
    # a skinny variant whose waves split K into another number of chunks.
    if op != "bf16_bi":
        single = [n for n in names(qll, op) if n[0] != "k" and not n.endswith("_g2")]
    else:
        single = [v["name"] for v in qll.variants(op)
                  if not (v["name"][0] == "k" and v["wp"] != 8)]
    outs = {n: fn(*args, out_dtype="fp32", cfg=(n, 1)) for n in single}
    torch.cuda.synchronize()
    ref = outs["n128x128_w2x2_k128"].view(torch.int32)
    diff = [n for n, y in outs.items() if not torch.equal(y.view(torch.int32), ref)]
    assert not diff, f"{op}: variants differing bitwise from n128x128: {diff}"


@pytest.mark.parametrize("op", ["fp8", "int8"])
def test_bf16_output_is_the_rounded_fp32_output(qll, op):
    # The per-token x per-channel epilogue computes (acc * sa[m]) * sb[n] in
    # fp32 and rounds it to bf16 (nearest even); the bf16 output must be the
    # fp32 output rounded, bit for bit, whichever path the kernel takes
    # (N a multiple of 8: scaled and rounded where the MFMA left it, paired
    # across lanes and staged as bf16; otherwise staged in fp32)
    g = np.random.default_rng(61)
    for M, N, K in [(300, 648, 1024), (257, 520, 2048), (130, 264, 512), (37, 300, 1024)]:
        if op == "fp8":
            A = g.integers(0, 256, (M, K)).astype(np.uint8)
            A[(A & 0x7F) == 0x7F] = 0
            B = g.integers(0, 256, (N, K)).astype(np.uint8)
            B[(B & 0x7F) == 0x7F] = 0
            dA, dB = dev_e4m3(A), dev_e4m3(B)
            fn = qll.gemm_fp8_scaled
        else:
            dA = dev(g.integers(-127, 128, (M, K)).astype(np.int8))
            dB = dev(g.integers(-127, 128, (N, K)).astype(np.int8))
            fn = qll.gemm_w8a8_int8
        sa = dev(g.uniform(1e-3, 1e-2, M).astype(np.float32))
        sb = dev(g.uniform(1e-3, 1e-2, N).astype(np.float32))
        for name in names(qll, op):
            if name[0] in "ks":
                continue  # decode kernels: their own epilogue, covered elsewhere
            y32 = fn(dA, dB, sa, sb, out_dtype="fp32", cfg=(name, 1))
            y16 = fn(dA, dB, sa, sb, out_dtype="bf16", cfg=(name, 1))
            torch.cuda.synchronize()
            assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16)), \
                (op, name, M, N, K)


@pytest.mark.parametrize("op", ["fp8", "int8"])
def test_k_groups_equal_split_k_two(qll, op):
    # A two-K-group tile ("_g2") sums its K range in two halves inside the
    # workgroup, the first group's partial plus the second's.  Where its
    # split point is Split-K's (K = 2048 and 4096: both halfway), it must be
    # bitwise the same tile run as two Split-K pieces added by the second
    # stage -- same halves, same order -- for every output kind.
    g = np.random.default_rng(67)
    ran = 0
    for M, N, K in [(130, 300, 2048), (37, 520, 4096)]:
        if op == "fp8":
            A = g.integers(0, 256, (M, K)).astype(np.uint8)
            A[(A & 0x7F) == 0x7F] = 0
            B = g.integers(0, 256, (N, K)).astype(np.uint8)
            B[(B & 0x7F) == 0x7F] = 0
            dA, dB = dev_e4m3(A), dev_e4m3(B)
            fn = qll.gemm_fp8_scaled
            kinds = ("fp32", "bf16")
        else:
            dA = dev(g.integers(-127, 128, (M, K)).astype(np.int8))
            dB = dev(g.integers(-127, 128, (N, K)).astype(np.int8))
            fn = qll.gemm_w8a8_int8
            kinds = ("int32", "fp32", "bf16")
        sa = dev(g.uniform(1e-3, 1e-2, M).astype(np.float32))
        sb = dev(g.uniform(1e-3, 1e-2, N).astype(np.float32))
        all_names = names(qll, op)
        for name in all_names:
            if not name.endswith("_g2"):
                continue
            # the same tile with one K group (any ring depth: same sums)
            prefix = name[:-3].rsplit("_s", 1)[0] + "_s"
            base = next(n for n in all_names if n.startswith(prefix) and not n.endswith("_g2"))
            for od in kinds:
                y1 = fn(dA, dB, sa, sb, out_dtype=od, cfg=(name, 1))
                y2 = fn(dA, dB, sa, sb, out_dtype=od, cfg=(base, 2))
                torch.cuda.synchronize()
                iv = torch.int16 if od == "bf16" else torch.int32
                assert torch.equal(y1.view(iv), y2.view(iv)), (op, name, base, od, M, N, K)
                ran += 1
    assert ran > 0


@pytest.mark.parametrize("op", ["block_fp8", "bf16_bi", "mxfp4", "w4a16"])
def test_unscaled_bf16_output_is_the_rounded_fp32_output(qll, op):
    # The ops whose accumulator is the output value (Block-FP8 after its
    # per-group promotion, bf16, MXFP4, W4A16): bf16 output must be the fp32
    # output rounded to nearest even, bit for bit, for every variant -- with
    # N a multiple of 8 the pipelined tiles round in the MFMA layout and
    # stage bf16x2 words, otherwise they stage fp32
    key = (workloads.W_TEST, 80)
    for M, N, K in [(257, 520, 2048), (130, 264, 512), (37, 300, 1024)]:
        x = dev_bf16(workloads.fp8_activations(M, K, key=(*key, M, K)))
        w = dev_bf16(workloads.weights_bf16(N, K, key=(*key, N, K)))
        if op == "block_fp8":
            qa, sa = qll.quantize_per_token_fp8(x, group=128)
            qb, sb = qll.quantize_weight_block_fp8(w)
            fn = lambda od, cfg: qll.gemm_block_fp8(qa, qb, sa, sb, out_dtype=od, cfg=cfg)
        elif op == "bf16_bi":
            fn = lambda od, cfg: qll.gemm_bf16_batch_invariant(x, w, out_dtype=od, cfg=cfg)
        elif op == "mxfp4":
            qa, sa = qll.quantize_mxfp4(x)
            qb, sb = qll.quantize_mxfp4(w)
            fn = lambda od, cfg: qll.gemm_mxfp4(qa, qb, sa, sb, out_dtype=od, cfg=cfg)
        else:
            qb, sb = qll.quantize_int4_weights(w)
            fn = lambda od, cfg: qll.gemm_w4a16(x, qb, sb, out_dtype=od, cfg=cfg)
        for name in names(qll, op):
            y32 = fn("fp32", (name, 1))
            y16 = fn("bf16", (name, 1))
            torch.cuda.synchronize()
            assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16)), \
                (op, name, M, N, K)
