"""The C-ABI calls only enqueue work on the caller's stream (no allocation,
no synchronization, no memset), so a caller can capture them into a HIP
graph: "What the integration changes" of "Helion in vLLM: A Unified Route to
Tunable Linear Kernels" recommends graph-covered execution for tuned kernels.

Each case captures a sequence of library calls (with and without Split-K,
every op family) into one graph, replays it several times with eager work in
between that overwrites the outputs and the workspace, and checks every
replay bitwise against the eager result of the same calls.
"""
import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from gpu_util import dev, dev_bf16  # noqa: E402


@pytest.fixture(scope="module")
def qll():
    import quantized_linear_layer_scaled_amd as q
    q.load_library()
    q.init()
    return q


def bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy().copy()


def check_graph(run, outs, scribble):
    """run() enqueues the calls (writing into outs); scribble() is eager work
    that overwrites outs and the workspaces between replays."""
    run()
    torch.cuda.synchronize()
    want = [bits(o) for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        scribble()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert np.array_equal(bits(o), w), f"replay {rep}"
    del g


def test_fp8_linear_and_splitk_in_a_graph(qll):
    M, N, K = 96, 1040, 2048
    x = dev_bf16(workloads.fp8_activations(M, K, key=(workloads.W_TEST, 90)))
    w = dev_bf16(workloads.weights_bf16(N, K, key=(workloads.W_TEST, 91)))
    B, sb = qll.quantize_per_token_fp8(w)
    sb = sb.view(-1).contiguous()
    q = torch.empty((M, K), dtype=torch.float8_e4m3fn, device="cuda")
    sa = torch.empty((M, 1), dtype=torch.float32, device="cuda")
    out1 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    out2 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    cfg = ("p64x64_w2x2_k128_s3", 4)
    ws = torch.empty(qll.workspace_bytes("fp8", M, N, K, cfg), dtype=torch.uint8, device="cuda")

    def run():
        qll.linear_fp8_dynamic(x, B, sb, out=out1, q=q, sa=sa)
        qll.gemm_fp8_scaled(q, B, sa, sb, out_dtype="fp32", out=out2, cfg=cfg, workspace=ws)

    def scribble():
        out1.fill_(7.0)
        out2.fill_(-3.0)
        ws.fill_(0x5A)
        q.view(torch.uint8).fill_(0x11)

    check_graph(run, [out1, out2], scribble)


def test_block_bi_int8_in_a_graph(qll):
    M, N, K = 80, 520, 1024
    xa = dev_bf16(workloads.block_activations(M, K, key=(workloads.W_TEST, 92)))
    wb = dev_bf16(workloads.weights_bf16(N, K, key=(workloads.W_TEST, 93)))
    Bq, Bs = qll.quantize_weight_block_fp8(wb)
    qa = torch.empty((M, K), dtype=torch.float8_e4m3fn, device="cuda")
    sa = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
    ob = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    obi = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    d = workloads.int8_inputs(M, N, K, key=(workloads.W_TEST, 94))
    Ai, Bi, sai, sbi = dev(d["A"]), dev(d["B"]), dev(d["sa"]), dev(d["sb"])
    oi = torch.empty((M, N), dtype=torch.int32, device="cuda")

    def run():
        qll.quantize_per_token_fp8(xa, group=128, q=qa, scales=sa)
        qll.gemm_block_fp8(qa, Bq, sa, Bs, out=ob)
        qll.gemm_bf16_batch_invariant(xa, wb, out=obi)
        qll.gemm_w8a8_int8(Ai, Bi, sai, sbi, out_dtype="int32", out=oi)

    def scribble():
        for t in (ob, obi):
            t.fill_(1.0)
        oi.fill_(-1)

    check_graph(run, [ob, obi, oi], scribble)


def test_mxfp4_w4a16_grouped_in_a_graph(qll):
    M, N, K = 64, 520, 1024
    x = dev_bf16(workloads.mx_activations(M, K, key=(workloads.W_TEST, 95)))
    w = dev_bf16(workloads.mx_weights(N, K, key=(workloads.W_TEST, 96)))
    qb, sbm = qll.quantize_mxfp4(w)
    qa = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    sam = torch.empty((M, K // 32), dtype=torch.uint8, device="cuda")
    omx = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    q4, s4 = qll.quantize_int4_weights(w)
    o4 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    E = 4
    off = torch.tensor([0, 10, 10, 40, M], dtype=torch.int32, device="cuda")
    Bg, sbg = qll.quantize_per_token_fp8(dev_bf16(workloads.weights_bf16(E * N, K,
                                                                      key=(workloads.W_TEST, 97))))
    qg = torch.empty((M, K), dtype=torch.float8_e4m3fn, device="cuda")
    sag = torch.empty((M, 1), dtype=torch.float32, device="cuda")
    og = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def run():
        qll.quantize_mxfp4(x, q=qa, scales=sam)
        qll.gemm_mxfp4(qa, qb, sam, sbm, out=omx)
        qll.gemm_w4a16(x, q4, s4, out=o4)
        qll.quantize_per_token_fp8(x, q=qg, scales=sag)
        qll.gemm_fp8_grouped(qg, Bg.view(E, N, K), sag, sbg.view(E, N), off, out=og)

    def scribble():
        for t in (omx, o4, og):
            t.fill_(2.0)
        qa.fill_(0x33)

    check_graph(run, [omx, o4, og], scribble)
