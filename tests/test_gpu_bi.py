"""Batch invariance of gemm_bf16_batch_invariant (vLLM PR #53446, "Summary"
and "Test Plan": outputs must not change with the batch size).

Property (holds at any size): for fixed (N, K), row i of the output is
bitwise identical whether computed in a batch of M = 1 or of M = 2048 rows
(the first rows of A shared), whatever the other rows hold, and identical
over repeated runs.  The dispatch (table or heuristic) is used as shipped.
A negative control shows the comparison does catch an M-dependent K split.
"""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from gpu_util import check_fp, dev_bf16, host_f64, sample_rows  # noqa: E402


@pytest.fixture(scope="module")
def qll():
    import quantized_linear_layer_scaled_amd as q
    q.load_library()
    q.init()
    return q


@pytest.mark.parametrize("N,K", workloads.BI_SHAPES)
def test_rows_bitwise_equal_across_m(qll, N, K):
    d = workloads.bi_inputs(N, K)
    A_full, B = dev_bf16(d["A_full"]), dev_bf16(d["B"])
    full = qll.gemm_bf16_batch_invariant(A_full, B)
    for M in workloads.BI_M:
        y = qll.gemm_bf16_batch_invariant(A_full[:M].contiguous(), B)
        torch.cuda.synchronize()
        same = torch.equal(y.view(torch.int16), full[:M].view(torch.int16))
        assert same, f"N={N} K={K}: rows differ between M={M} and M=2048"
    # accuracy of the shared result against the oracle on sampled rows
    rows = sample_rows(2048, 12)
    ref, absref = oracle.gemm_bf16(d["A_full"], d["B"], rows=rows, with_abs=True)
    check_fp(host_f64(full)[rows], ref, absref, K, "bf16", f"BI N={N} K={K}", mfma="bf16")


def test_other_rows_do_not_matter(qll):
    N, K = 2048, 2048
    d = workloads.bi_inputs(N, K)
    A = dev_bf16(d["A_full"])
    B = dev_bf16(d["B"])
    for M in (64, 512):
        base = qll.gemm_bf16_batch_invariant(A[:M].contiguous(), B)
        mixed = A.clone()
        mixed[M:] = torch.randn_like(mixed[M:].float()).to(torch.bfloat16) * 7
        y = qll.gemm_bf16_batch_invariant(mixed, B)
        torch.cuda.synchronize()
        assert torch.equal(y[:M].view(torch.int16), base.view(torch.int16)), M


def test_repeat_runs_bitwise(qll):
    d = workloads.bi_inputs(4096, 2048)
    A, B = dev_bf16(d["A_full"][:256]), dev_bf16(d["B"])
    first = qll.gemm_bf16_batch_invariant(A, B, out_dtype="fp32")
    for _ in range(10):
        y = qll.gemm_bf16_batch_invariant(A, B, out_dtype="fp32")
        assert torch.equal(y.view(torch.int32), first.view(torch.int32))


def test_negative_control_m_dependent_split_is_caught(qll):
    # forcing a different K split at one M must break the bitwise property;
    # this shows the comparison above is able to fail
    d = workloads.bi_inputs(2048, 2048)
    A, B = dev_bf16(d["A_full"]), dev_bf16(d["B"])
    v = qll.select("bf16_bi", 2048, 2048, 2048)[0]
    full = qll.gemm_bf16_batch_invariant(A, B, out_dtype="fp32", cfg=(v, 1))
    small = qll.gemm_bf16_batch_invariant(A[:16].contiguous(), B, out_dtype="fp32",
                                          cfg=(v, 4))
    torch.cuda.synchronize()
    assert not torch.equal(small.view(torch.int32), full[:16].view(torch.int32))


def test_selected_configs_keep_the_k_split(qll):
    # what the dispatch picks for the BI op: one K split per (N, K) at every
    # M, and no variant whose waves split K into other than the fixed eight
    # chunks (orientation and tile may change with M: every other variant
    # reproduces the same sums bit for bit, see
    # test_swap_equals_ordinary_bitwise)
    for N, K in workloads.BI_SHAPES + [workloads.VOCAB_SHAPE]:
        picks = [qll.select("bf16_bi", M, N, K) for M in range(1, 4097, 37)]
        eff = {qll.effective_splits("bf16_bi", K, s) for _, s in picks}
        assert len(eff) == 1, (N, K, eff)
        vs = {v["name"]: v for v in qll.variants("bf16_bi")}
        assert not any(n[0] == "k" and vs[n]["wp"] != 8 for n, _ in picks), (N, K)
