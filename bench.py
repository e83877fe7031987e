#!/usr/bin/env python3
"""Benchmark of the scaled_mm hot path on one MI355X.

Default workload (one "step"): the FP8 dynamic per-token sweep -- for
(N, K) in {(4096, 2048), (2048, 6144)} and M in {1, 4, 8, 16, 32, 64, 256,
512, 1024, 2048}: quantize the bf16 activations per token on the device
(quantize_per_token_fp8), then run the scaled FP8 GEMM (gemm_fp8_scaled) with
the configuration the dispatch picks, bf16 out; where the fp8_dynamic
dispatch names a fused variant for the shape, the problem is the one fused
call of linear_fp8_dynamic instead (quantizer and GEMM in one kernel).  Weights are quantized per
output channel on the device once, before timing.  Every (N, K, M) problem
has its own buffers (about 350 MB touched per step, more than the 256 MB
Infinity Cache), so a problem's weights come from HBM, not from a cache.

Timing (all on the one stream the library launches on):
  * value: after W warm-up steps, K steps launched from the host through the
    C ABI (prebuilt arguments, no per-call Python work) are timed between
    HIP events; value = GEMM flops of a step / step time (TFLOPS);
  * graph_value: the same step captured once into a HIP graph and replayed K
    times (graph-covered execution, the launch mode the pages recommend for
    tuned kernels);
  * per call: for every quantizer and GEMM call of the step, a HIP graph of
    back-to-back launches, each on its own copy of the call's buffers, with
    enough copies (>= 1 GiB per replay) that every launch reads from HBM,
    replayed --replays times between HIP events (median, p10, p90 of the
    per-launch time; the same call on one warm set of buffers as context):
    this gives the per-shape table and the roofline of the dominant kernel
    (the GEMM kernel with the most time per step among single-kernel calls);
  * eager per call: HIP events around each C-ABI call of a few extra eager
    steps (launch included);
  * dispatch: host-side costs of the C-ABI path (table load, the first step
    of the process, host enqueue time per call).
The line also carries the CPU oracle timed on a bounded sample of the same
workload, and, when the rocprofv3 counter CSVs are given (--fetch-csv,
--write-csv), the HBM traffic of the dominant kernel scaled by the same
counters read on a copy kernel of known size (--calib-copy runs that copy).
Without them the traffic comes from the workload's committed profile
(profiles/<workload>_sweep_bench_line.json) when that profile measured the
same kernel built from the same sources (a digest of the kernel and ABI
sources is stored with the counters), and is null otherwise.  --mfma-csv
(SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_MFMA, SQ_INSTS_VALU_MFMA_MOPS_*,
GRBM_GUI_ACTIVE) adds the matrix-core counters with their calibration (busy
cycles per instruction, MOPS against the algorithmic flops, the clock the
dispatch ran at); --kernel-trace-csv (a rocprofv3 --kernel-trace run of the
same command) adds the dominant kernel's traced duration over exactly the
launches the per-call timing times, and the roofline fraction at that
duration.  Both come from the committed profile under the same conditions
as the traffic when not given.

Other workloads (--workload int8|block|bi|vocab|vocab_bi|moe|mxfp4|w4a16) print the
same JSON shape; moe is the grouped (per-expert) FP8 GEMM of a 64-expert layer
with synthetic top-8 routing (per-token quantization + gemm_fp8_grouped);
mxfp4 is the FP8 sweep's shapes and data in MXFP4 (quantize_mxfp4 +
gemm_mxfp4); w4a16 is the same sweep with int4 weights and bf16 activations
(gemm_w4a16; the weights are quantized once, before timing).

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload fp8]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK = {"fp8": 5000.0, "int8": 5000.0, "bf16": 2500.0, "fp4": 10100.0}  # dense TFLOP/s (TOP/s)
# (W4A16 runs on the bf16 matrix cores: its peak is the bf16 one)
HBM_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="fp8",
                   choices=["fp8", "int8", "block", "bi", "vocab", "vocab_bi", "moe", "mxfp4",
                            "w4a16"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=2048,
                   help="rows per problem the CPU oracle computes (the default covers "
                        "every row of the FP8 and MXFP4 sweeps)")
    p.add_argument("--table", default="default",
                   help="dispatch table ('default', a path, or 'none')")
    p.add_argument("--fetch-csv", default=None,
                   help="rocprofv3 --pmc FETCH_SIZE counter_collection.csv of this command")
    p.add_argument("--write-csv", default=None,
                   help="rocprofv3 --pmc WRITE_SIZE counter_collection.csv of this command")
    p.add_argument("--kernel-trace-csv", default=None,
                   help="kernel trace CSV of a rocprofv3 --kernel-trace run of this same "
                        "command: the dominant kernel's duration over the launches the "
                        "per-call timing times, and its roofline fraction")
    p.add_argument("--mfma-csv", default=None,
                   help="rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE "
                        "counter_collection.csv of this command")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run a plain device copy of known size (counter calibration)")
    p.add_argument("--no-graph", action="store_true",
                   help="no graphs: eager steps only, no per-call timing (counter runs)")
    p.add_argument("--vendor", action="store_true",
                   help="also time the vendor library's GEMM on the same problems (context)")
    p.add_argument("--replays", type=int, default=5,
                   help="timed replays of each per-call timing graph (median, p10/p90)")
    return p.parse_args()


# --------------------------------------------------------------------------
# problems
# --------------------------------------------------------------------------

class Problem:
    """One (op, M, N, K) GEMM with its own device buffers and a prebuilt
    launch plan (raw pointers, so that the timed loop only makes the C calls)."""

    def __init__(self, op, M, N, K):
        self.op, self.M, self.N, self.K = op, M, N, K
        self.calls = []       # [(name, cfunc, args)]
        self.keep = []        # tensors that must stay alive
        self.tensors = {}     # kind -> (tensor dict, args builder)

    @property
    def flops(self):
        return 2.0 * self.M * self.N * self.K

    def algo_bytes(self):
        """Algorithmic HBM bytes of the GEMM: A + B + scales + bf16 out (the
        fused linear layer: bf16 tokens in, their codes and scales out too)."""
        M, N, K = self.M, self.N, self.K
        if getattr(self, "fused", False):
            return 2 * M * K + N * K + 4 * N + 2 * M * N + M * K + 4 * M
        if self.op == "bf16_bi":
            return 2 * M * K + 2 * N * K + 2 * M * N
        if self.op == "block_fp8":
            return M * K + N * K + 4 * M * (K // 128) + 4 * ((N + 127) // 128) * (K // 128) + 2 * M * N
        if self.op == "fp8_grouped":  # the weights of every expert that has rows
            return M * K + self.experts_used * (N * K + 4 * N) + 4 * M + 2 * M * N
        if self.op == "mxfp4":  # packed codes + one scale byte per 32 + bf16 out
            return (M + N) * (K // 2 + K // 32) + 2 * M * N
        if self.op == "w4a16":  # bf16 A + packed int4 B + fp32 group scales + bf16 out
            return 2 * M * K + N * K // 2 + 4 * N * (K // 128) + 2 * M * N
        return M * K + N * K + 4 * M + 4 * N + 2 * M * N

    def quant_bytes(self):
        if self.op == "mxfp4":
            return 2 * self.M * self.K + self.M * (self.K // 2 + self.K // 32)
        return 3 * self.M * self.K + 4 * self.M * max(1, self.K // (128 if self.op == "block_fp8" else self.K))


def dev_bf16(torch, bits):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def build_problems(torch, qll, workload):
    import numpy as np

    import workloads as W
    L = qll.load_library()
    stream = torch.cuda.current_stream().cuda_stream
    probs = []

    def ws_for(op, M, N, K):
        n = qll.workspace_bytes(op, M, N, K)
        if n == 0:
            return None, 0
        t = torch.empty(n, dtype=torch.uint8, device="cuda")
        return t, n

    def gemm_args(p, t):
        wsp = t["ws"].data_ptr() if t["ws"] is not None else None
        if p.op == "w4a16":
            return (t["A"].data_ptr(), t["B"].data_ptr(), t["sb"].data_ptr(),
                    t["out"].data_ptr(), 0, p.M, p.N, p.K, wsp, t["wsb"], stream)
        if p.op == "bf16_bi":
            return (t["A"].data_ptr(), t["B"].data_ptr(), t["out"].data_ptr(), 0, p.M, p.N,
                    p.K, wsp, t["wsb"], stream)
        return (t["A"].data_ptr(), t["B"].data_ptr(), t["sa"].data_ptr(), t["sb"].data_ptr(),
                t["out"].data_ptr(), 0, p.M, p.N, p.K, wsp, t["wsb"], stream)

    def add_gemm(p, fn, A, B, sa, sb):
        out = torch.empty((p.M, p.N), dtype=torch.bfloat16, device="cuda")
        ws, wsb = ws_for(p.op, p.M, p.N, p.K)
        t = dict(A=A, B=B, sa=sa, sb=sb, out=out, ws=ws, wsb=wsb)
        p.keep += [A, B, out] + [x for x in (sa, sb, ws) if x is not None]
        p.calls.append(("gemm", getattr(L, fn), gemm_args(p, t)))
        p.tensors["gemm"] = (t, gemm_args)
        p.variant, p.splits = qll.select(p.op, p.M, p.N, p.K)
        p.eff_splits = qll.effective_splits(p.op, p.K, p.splits)

    def add_quant(p, x, group):
        q = torch.empty((p.M, p.K), dtype=torch.float8_e4m3fn, device="cuda")
        G = p.K if group == 0 else group
        s = torch.empty((p.M, p.K // G), dtype=torch.float32, device="cuda")
        p.keep += [x, q, s]
        qargs = lambda p, t: (t["x"].data_ptr(), t["q"].data_ptr(), t["s"].data_ptr(), p.M,
                              p.K, group, stream)
        t = dict(x=x, q=q, s=s)
        p.calls.append(("quant", L.quantize_per_token_fp8, qargs(p, t)))
        p.tensors["quant"] = (t, qargs)
        return q, s

    def add_linear(p, x, B, sb, variant):
        # linear_fp8_dynamic on a fused configuration: quantizer and GEMM in
        # one kernel (timed and reported as the problem's "gemm" call)
        q = torch.empty((p.M, p.K), dtype=torch.float8_e4m3fn, device="cuda")
        sa = torch.empty((p.M, 1), dtype=torch.float32, device="cuda")
        out = torch.empty((p.M, p.N), dtype=torch.bfloat16, device="cuda")
        largs = lambda p, t: (t["x"].data_ptr(), t["B"].data_ptr(), t["sb"].data_ptr(),
                              t["q"].data_ptr(), t["sa"].data_ptr(), t["out"].data_ptr(), 0,
                              p.M, p.N, p.K, None, 0, stream)
        t = dict(x=x, B=B, sb=sb, q=q, sa=sa, out=out)
        p.keep += list(t.values())
        p.calls.append(("gemm", L.linear_fp8_dynamic, largs(p, t)))
        p.tensors["gemm"] = (t, largs)
        p.variant, p.splits, p.eff_splits = variant, 1, 1
        p.fused = True

    if workload in ("fp8", "vocab"):
        shapes = W.FP8_SHAPES if workload == "fp8" else [W.VOCAB_SHAPE]
        mlist = W.FP8_M if workload == "fp8" else W.VOCAB_M
        for N, K in shapes:
            if workload == "fp8":
                w = dev_bf16(torch, W.weights_bf16(N, K))
                x_all = dev_bf16(torch, W.fp8_activations(W.MAX_M, K))
            else:
                w = dev_bf16(torch, W.vocab_weights(N, K))
                x_all = dev_bf16(torch, W.vocab_activations(K))
            qw, sw = qll.quantize_per_token_fp8(w)
            del w
            for M in mlist:
                p = Problem("fp8", M, N, K)
                # own copy of the weights per problem (cold for every problem)
                dyn = qll.select("fp8_dynamic", M, N, K)[0]
                if dyn[0] == "f":
                    # the dispatch runs this linear layer fused: one call
                    add_linear(p, x_all[:M].clone(), qw.clone(), sw.clone(), dyn)
                else:
                    q, s = add_quant(p, x_all[:M].clone(), 0)
                    add_gemm(p, "gemm_fp8_scaled", q, qw.clone(), s, sw.clone())
                probs.append(p)
    elif workload == "mxfp4":
        for N, K in W.MX_SHAPES:
            qw, sw = qll.quantize_mxfp4(dev_bf16(torch, W.mx_weights(N, K)))
            x_all = dev_bf16(torch, W.mx_activations(W.MAX_M, K))
            for M in W.MX_M:
                p = Problem("mxfp4", M, N, K)
                x = x_all[:M].clone()
                q = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
                s = torch.empty((M, K // 32), dtype=torch.uint8, device="cuda")
                p.keep += [x, q, s]
                qargs = lambda p, t: (t["x"].data_ptr(), t["q"].data_ptr(), t["s"].data_ptr(),
                                      p.M, p.K, stream)
                t = dict(x=x, q=q, s=s)
                p.calls.append(("quant", L.quantize_mxfp4, qargs(p, t)))
                p.tensors["quant"] = (t, qargs)
                add_gemm(p, "gemm_mxfp4", q, qw.clone(), s, sw.clone())
                probs.append(p)
    elif workload == "w4a16":
        for N, K in W.W4_SHAPES:
            qw, sw = qll.quantize_int4_weights(dev_bf16(torch, W.w4_weights(N, K)))
            x_all = dev_bf16(torch, W.w4_activations(W.MAX_M, K))
            for M in W.W4_M:
                p = Problem("w4a16", M, N, K)
                add_gemm(p, "gemm_w4a16", x_all[:M].clone(), qw.clone(), None, sw.clone())
                probs.append(p)
    elif workload == "int8":
        M, N, K = W.INT8_SHAPE
        d = W.int8_inputs(M, N, K)
        for rep in range(8):
            p = Problem("int8", M, N, K)
            t = lambda a: torch.from_numpy(a).cuda()
            add_gemm(p, "gemm_w8a8_int8", t(d["A"]), t(d["B"]), t(d["sa"]), t(d["sb"]))
            probs.append(p)
    elif workload == "block":
        for N, K in W.BLOCK_SHAPES:
            w = dev_bf16(torch, W.weights_bf16(N, K, key=(W.W_BLOCK,)))
            qw, sw = qll.quantize_weight_block_fp8(w)
            x_all = dev_bf16(torch, W.block_activations(W.MAX_M, K))
            for M in W.BLOCK_M:
                p = Problem("block_fp8", M, N, K)
                q, s = add_quant(p, x_all[:M].clone(), 128)
                add_gemm(p, "gemm_block_fp8", q, qw.clone(), s, sw.clone())
                probs.append(p)
    elif workload == "moe":
        N, K = W.MOE_SHAPE
        E = W.MOE_E
        w = dev_bf16(torch, W.moe_weights(E, N, K).reshape(E * N, K))
        qw, sw = qll.quantize_per_token_fp8(w)
        del w

        def grouped_args(p, t):
            return (t["A"].data_ptr(), t["B"].data_ptr(), t["sa"].data_ptr(),
                    t["sb"].data_ptr(), t["off"].data_ptr(), t["out"].data_ptr(), 0,
                    p.M, p.N, p.K, E, stream)

        for T in W.MOE_T:
            off = W.moe_routing(T)
            M = int(off[-1])
            p = Problem("fp8_grouped", M, N, K)
            p.experts_used = int((np.diff(off) > 0).sum())
            q, s = add_quant(p, dev_bf16(torch, W.moe_activations(M, K)), 0)
            out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            t = dict(A=q, B=qw.clone().view(E, N, K), sa=s, sb=sw.clone().view(E, N),
                     off=torch.from_numpy(off).cuda(), out=out)
            p.keep += list(t.values())
            p.calls.append(("gemm", L.gemm_fp8_grouped, grouped_args(p, t)))
            p.tensors["gemm"] = (t, grouped_args)
            p.variant, p.splits, p.eff_splits = qll.grouped_select(M, E), 1, 1
            probs.append(p)
    elif workload == "vocab_bi":
        # the batch-invariant bf16 path on the large-vocabulary data (the FP8
        # path on the same data is --workload vocab)
        N, K = W.VOCAB_SHAPE
        w = dev_bf16(torch, W.vocab_weights(N, K))
        x_all = dev_bf16(torch, W.vocab_activations(K))
        for M in W.VOCAB_M:
            p = Problem("bf16_bi", M, N, K)
            add_gemm(p, "gemm_bf16_batch_invariant", x_all[:M].clone(), w.clone(), None, None)
            probs.append(p)
        del w
    elif workload == "bi":
        for N, K in W.BI_SHAPES:
            d = W.bi_inputs(N, K)
            a_full, b = dev_bf16(torch, d["A_full"]), dev_bf16(torch, d["B"])
            for M in W.BI_M:
                p = Problem("bf16_bi", M, N, K)
                add_gemm(p, "gemm_bf16_batch_invariant", a_full[:M].clone(), b.clone(),
                         None, None)
                probs.append(p)
    torch.cuda.synchronize()
    return probs


# --------------------------------------------------------------------------
# timing
# --------------------------------------------------------------------------

COLD_BYTES = 1 << 30  # buffers one per-call timing replay rotates through


def _graph_us(torch, fn, arg_sets, replays, stream):
    """A HIP graph of one launch per argument set, replayed once to warm up,
    then `replays` times, each replay between HIP events on the stream the
    graph runs on: the per-launch mean of every replay."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for args in arg_sets:
            fn(*args)
    g.replay()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(replays)]
    for e0, e1 in evs:
        e0.record()
        g.replay()
        e1.record()
    torch.cuda.synchronize()
    del g
    return [e0.elapsed_time(e1) * 1e3 / len(arg_sets) for e0, e1 in evs]


def _stats(xs):
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "n": int(a.size)}


def per_call_us(torch, probs, replays, stream, max_copies=256):
    """Every call timed on its own, cold: a HIP graph of back-to-back launches
    of the call, launch r on its own copy of all the call's buffers, with
    enough copies that one replay touches at least COLD_BYTES (more than the
    256 MB Infinity Cache and the L2s, so every launch reads from HBM); the
    median and p10/p90 over `replays` timed replays of the per-launch time
    (the GPU time of a replay divided by its launches: kernel time plus the
    in-graph gap between consecutive launches).  Context: the same number of
    launches on one warm set of buffers.  Returns ([[stats]], [[copies]])."""
    out, plan = [], []
    for p in probs:
        row, prow = [], []
        for kind, fn, _ in p.calls:
            base, make = p.tensors[kind]
            nbytes = sum(v.numel() * v.element_size() for v in base.values()
                         if isinstance(v, torch.Tensor))
            copies = max(8, min(max_copies, -(-COLD_BYTES // max(1, nbytes))))
            sets = []
            for _ in range(copies):
                t = {k: (v.clone() if isinstance(v, torch.Tensor) else v)
                     for k, v in base.items()}
                sets.append((t, make(p, t)))
            st = _stats(_graph_us(torch, fn, [a for _, a in sets], replays, stream))
            del sets
            st["warm"] = _stats(_graph_us(torch, fn, [make(p, base)] * copies, replays,
                                          stream))["median"]
            st["copies"] = copies
            row.append(st)
            prow.append(copies)
            torch.cuda.empty_cache()
        out.append(row)
        plan.append(prow)
    return out, plan


def vendor_us(torch, probs, replays, stream, max_copies=256):
    """Context only (not the product, not a target): the vendor library's
    GEMM on the same problems, timed like per_call_us (cold copies, graph
    replays, median per launch): torch._scaled_mm (hipBLASLt) with row-wise
    scales for the FP8 problems, torch.matmul for the bf16 ones; None where
    the op has no vendor counterpart or the call fails."""
    out = []
    for p in probs:
        t = p.tensors["gemm"][0]
        if p.op == "fp8":
            def call(A, B, sa, sb):
                return torch._scaled_mm(A, B.t(), scale_a=sa.view(-1, 1), scale_b=sb.view(1, -1),
                                        out_dtype=torch.bfloat16)
            # (a fused linear layer: the codes and scales its first run wrote)
            base = (t.get("A", t.get("q")), t["B"], t["sa"], t["sb"])
        elif p.op == "bf16_bi":
            def call(A, Bt):
                return torch.matmul(A, Bt)
            base = (t["A"], t["B"].t().contiguous())  # [K][N], no transposed view
        else:
            out.append(None)
            continue
        nbytes = sum(x.numel() * x.element_size() for x in base) + 2 * p.M * p.N
        copies = max(8, min(max_copies, -(-COLD_BYTES // max(1, nbytes))))
        try:
            sets = [tuple(x.clone() for x in base) for _ in range(copies)]
            call(*sets[0])
            out.append(_stats(_graph_us(torch, call, sets, replays, stream))["median"])
        except Exception as ex:  # the library may not take this shape
            print(f"# vendor GEMM failed for M={p.M} N={p.N} K={p.K}: {ex}", file=sys.stderr)
            out.append(None)
        sets = None
        torch.cuda.empty_cache()
    return out


def xcd_fill_bytes(M, N, kbytes, bp, bq, group=4):
    """Bytes the 8 XCD L2 caches must fetch for one pipelined launch when each
    XCD reads every A and B row its tiles touch once: the workgroup -> tile
    map of the kernel (consecutive workgroup ids go to the XCDs in turn; the
    tiles of one XCD form a contiguous run laid out `group` tile rows at a
    time) applied to every workgroup."""
    tp, tq = -(-M // bp), -(-N // bq)
    T = tp * tq
    per, rem = T >> 3, T & 7
    rows = [(set(), set()) for _ in range(8)]
    for bid in range(T):
        xcd, loc = bid & 7, bid >> 3
        t = xcd * (per + 1) + loc if xcd < rem else rem * (per + 1) + (xcd - rem) * per + loc
        span = group * tq
        first = (t // span) * group
        gsize = min(tp - first, group)
        p, q = first + (t % span) % gsize, (t % span) // gsize
        rows[xcd][0].add(p)
        rows[xcd][1].add(q)
    total = 0
    for a, b in rows:
        total += sum(min(bp, M - p * bp) for p in a) * kbytes
        total += sum(min(bq, N - q * bq) for q in b) * kbytes
    return total


def env_info():
    """ROCm version and the GPU's current shader and memory clocks as the
    driver's sysfs files report them (read, no program is started)."""
    import glob
    info = {}
    try:
        info["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        info["rocm"] = None
    clocks = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        for name in ("pp_dpm_sclk", "pp_dpm_mclk"):
            try:
                cur = [l.strip() for l in open(f"{dev}/{name}") if l.strip().endswith("*")]
            except OSError:
                continue
            if cur:
                clocks.setdefault(dev.split("/")[4], {})[name[-4:]] = cur[0]
    info["clocks"] = clocks or None
    return info


def run_step(probs, events=None):
    for i, p in enumerate(probs):
        for j, (_, fn, args) in enumerate(p.calls):
            if events is not None:
                events[i][j][0].record()
            rc = fn(*args)
            if events is not None:
                events[i][j][1].record()
            if rc != 0:
                raise RuntimeError(f"{fn.__name__} returned {rc} for M={p.M} N={p.N} K={p.K}")


def kernel_symbol(qll, op, variant):
    """The kernel's name as rocprofv3 prints it (for the skinny kernel, whose
    last template argument the registry does not list, the name up to it)."""
    grouped = op == "fp8_grouped"
    if grouped:
        op = "fp8"
    opn = {"int8": 0, "fp8": 1, "block_fp8": 2, "bf16_bi": 3, "mxfp4": 4, "w4a16": 5}[op]
    if op == "fp8" and variant[0] == "f":  # the fused linear layer
        v = next(x for x in qll.variants("fp8_dynamic") if x["name"] == variant)
        return (f"void qll::linear_fused_kernel<{v['bp']}, {v['wp']}, {v['ksteps']}, {v['bq']}>"
                "(qll::FusedArgs)")
    v = next(x for x in qll.variants(op) if x["name"] == variant)
    if variant[0] == "p" and "_k64_" in variant:  # the 32x32x64 deep-ring tiles
        st = variant.rsplit("_s", 1)[1]
        return (f"void qll::gemm_p32_kernel<{opn}, {v['bp']}, {v['bq']}, {v['wp']}, "
                f"{v['wq']}, {st}, false>(qll::GemmArgs)")
    if op == "w4a16":
        if variant[0] == "t":
            return (f"void qll::gemm_w4_tile_kernel<{v['bp']}, {v['bq']}, {v['wp']}, "
                    f"{v['wq']}>(qll::GemmArgs)")
        if variant[0] == "p":
            st = variant.rsplit("_s", 1)[1]
            return (f"void qll::gemm_w4_pipe_kernel<{v['bp']}, {v['bq']}, {v['wp']}, "
                    f"{v['wq']}, {st}>(qll::GemmArgs)")
        return f"void qll::gemm_w4_skinny_kernel<{v['bq'] // 16}, {v['wp']}, {v['bp']}, "
    if variant[0] == "p" and variant.rsplit("_", 1)[1][0] == "r":
        # "_r<RC>": operand copies through RC register stages
        rc = variant.rsplit("_r", 1)[1]
        return (f"void qll::gemm_pipe_rc_kernel<{opn}, {v['bp']}, {v['bq']}, {v['wp']}, "
                f"{v['wq']}, {v['kstage']}, {rc}, false>(qll::GemmArgs)")
    if variant[0] == "p":
        # "_g2": two K groups per workgroup (the kernel's last argument)
        kgrp = 2 if variant.endswith("_g2") else 1
        st = variant[:-3] if kgrp == 2 else variant
        st = st.rsplit("_s", 1)[1]
        return (f"void qll::gemm_pipe_kernel<{opn}, {v['bp']}, {v['bq']}, {v['wp']}, "
                f"{v['wq']}, {v['kstage']}, {st}, false, {'true' if grouped else 'false'}, "
                f"{kgrp}>(qll::GemmArgs)")
    if variant[0] in "kr":
        hr = v["bp"] if variant[0] == "k" else 16
        return (f"void qll::gemm_skinny_kernel<{opn}, {v['bq'] // 16}, {v['wp']}, {hr}, "
                f"{'true' if variant[0] == 'k' else 'false'}, ")
    return (f"void qll::gemm_tile_kernel<{opn}, {v['swap']}, {v['bp']}, {v['bq']}, "
            f"{v['wp']}, {v['wq']}, {v['kstage']}>(qll::GemmArgs)")


def cpu_baseline(workload, rows_cap):
    """Time the oracle (as it stands) on a bounded sample of the workload:
    the first min(M, rows_cap) rows of every problem, quantization included."""
    import numpy as np

    import oracle
    import workloads as W
    oracle.num_threads()
    flops = 0.0
    t_total = 0.0
    sample = []
    if workload in ("fp8", "vocab"):
        shapes = W.FP8_SHAPES if workload == "fp8" else [W.VOCAB_SHAPE]
        mlist = W.FP8_M if workload == "fp8" else W.VOCAB_M
        for N, K in shapes:
            w = W.weights_bf16(N, K) if workload == "fp8" else W.vocab_weights(N, K)
            x_all = W.fp8_activations(W.MAX_M, K) if workload == "fp8" else W.vocab_activations(K)
            B, sb = oracle.quantize_fp8(w)
            sb = sb[:, 0].copy()
            for M in mlist:
                r = min(M, rows_cap)
                t0 = time.perf_counter()
                A, sa = oracle.quantize_fp8(np.ascontiguousarray(x_all[:r]))
                oracle.gemm_fp8(A, B, sa[:, 0].copy(), sb)
                t_total += time.perf_counter() - t0
                flops += 2.0 * r * N * K
            sample.append(f"N={N},K={K}")
        desc = (f"first min(M,{rows_cap}) rows of every (N,K,M) problem "
                f"({', '.join(sample)}), per-token quantization + FP8 GEMM")
    elif workload == "mxfp4":
        for N, K in W.MX_SHAPES:
            B, sb = oracle.quantize_mxfp4(W.mx_weights(N, K))
            x_all = W.mx_activations(W.MAX_M, K)
            for M in W.MX_M:
                r = min(M, rows_cap)
                t0 = time.perf_counter()
                A, sa = oracle.quantize_mxfp4(np.ascontiguousarray(x_all[:r]))
                oracle.gemm_mxfp4(A, B, sa, sb)
                t_total += time.perf_counter() - t0
                flops += 2.0 * r * N * K
        desc = (f"first min(M,{rows_cap}) rows of every MXFP4 problem, "
                "MXFP4 quantization + GEMM")
    elif workload == "w4a16":
        for N, K in W.W4_SHAPES:
            B, sb = oracle.quantize_int4(W.w4_weights(N, K))
            x_all = W.w4_activations(W.MAX_M, K)
            for M in W.W4_M:
                r = min(M, rows_cap)
                t0 = time.perf_counter()
                oracle.gemm_w4a16(np.ascontiguousarray(x_all[:r]), B, sb)
                t_total += time.perf_counter() - t0
                flops += 2.0 * r * N * K
        desc = f"first min(M,{rows_cap}) rows of every W4A16 problem (GEMM only)"
    elif workload == "int8":
        M, N, K = W.INT8_SHAPE
        d = W.int8_inputs(M, N, K)
        t0 = time.perf_counter()
        for _ in range(4):
            oracle.gemm_w8a8_int8(d["A"], d["B"], d["sa"], d["sb"])
        t_total = time.perf_counter() - t0
        flops = 4 * 2.0 * M * N * K
        desc = "4 full W8A8 INT8 GEMMs M=16 N=K=2048"
    elif workload == "block":
        for N, K in W.BLOCK_SHAPES:
            w = W.weights_bf16(N, K, key=(W.W_BLOCK,))
            B, sb = oracle.quantize_fp8_block(w)
            x_all = W.block_activations(W.MAX_M, K)
            for M in W.BLOCK_M:
                r = min(M, rows_cap)
                t0 = time.perf_counter()
                A, sa = oracle.quantize_fp8(np.ascontiguousarray(x_all[:r]), group=128)
                oracle.gemm_block_fp8(A, B, sa, sb)
                t_total += time.perf_counter() - t0
                flops += 2.0 * r * N * K
        desc = f"first min(M,{rows_cap}) rows of every Block-FP8 problem"
    elif workload == "moe":
        N, K = W.MOE_SHAPE
        E = W.MOE_E
        w = W.moe_weights(E, N, K).reshape(E * N, K)
        B, sb = oracle.quantize_fp8(w)
        B, sb = B.reshape(E, N, K), sb[:, 0].reshape(E, N).copy()
        for T in W.MOE_T:
            off = W.moe_routing(T)
            M = int(off[-1])
            x = W.moe_activations(M, K)
            rows = np.arange(0, M, max(1, M // min(M, rows_cap)))[:rows_cap]
            t0 = time.perf_counter()
            A, sa = oracle.quantize_fp8(x)
            oracle.gemm_fp8_grouped(A, B, sa[:, 0].copy(), sb, off, rows=rows)
            t_total += time.perf_counter() - t0
            flops += 2.0 * rows.size * N * K
        desc = (f"min(M,{rows_cap}) evenly spaced rows of every grouped problem "
                "(all experts), per-token quantization of all rows + grouped FP8 GEMM")
    elif workload == "vocab_bi":
        N, K = W.VOCAB_SHAPE
        w = W.vocab_weights(N, K)
        x = W.vocab_activations(K)
        cap = min(rows_cap, 64)
        for M in W.VOCAB_M:
            r = min(M, cap)
            t0 = time.perf_counter()
            oracle.gemm_bf16(x[:r], w)
            t_total += time.perf_counter() - t0
            flops += 2.0 * r * N * K
        desc = f"first min(M,{cap}) rows of every vocabulary-size bf16 problem"
    else:
        for N, K in W.BI_SHAPES:
            d = W.bi_inputs(N, K)
            for M in W.BI_M:
                r = min(M, rows_cap)
                t0 = time.perf_counter()
                oracle.gemm_bf16(d["A_full"][:r], d["B"])
                t_total += time.perf_counter() - t0
                flops += 2.0 * r * N * K
        desc = f"first min(M,{rows_cap}) rows of every bf16 problem"
    cores = oracle.num_threads()
    # one single-thread timing on the W8A8 INT8 shape (median of 3 runs)
    M, N, K = W.INT8_SHAPE
    d = W.int8_inputs(M, N, K)
    oracle.set_threads(1)
    ts = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.gemm_w8a8_int8(d["A"], d["B"], d["sa"], d["sb"])
        ts.append(time.perf_counter() - t0)
    oracle.set_threads(cores)
    single = 2.0 * M * N * K / sorted(ts)[1] / 1e9
    cpu_model = None
    try:
        for l in open("/proc/cpuinfo"):
            if l.startswith("model name"):
                cpu_model = l.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(flops / t_total / 1e12, 6),
            "unit": "TOPS" if workload == "int8" else "TFLOPS",
            "cores": cores, "kind": "oracle", "sample": desc,
            "seconds": round(t_total, 2), "cpu_model": cpu_model,
            "cores_available": len(os.sched_getaffinity(0)),
            "single_thread_int8_gops": round(single, 3),
            "single_thread_shape": f"W8A8 INT8 M={M} N={N} K={K}, median of 3"}


CALIB_BYTES = 512 << 20  # the copy kernel moves this many bytes each way


def counter_per_dispatch(csv_path, counter):
    """{kernel name: [value per dispatch]} from a rocprofv3 counter CSV."""
    import csv
    out = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") == counter:
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def source_digest() -> str:
    """SHA-256 over the library's kernel and ABI sources (the build the
    counters describe)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_linear_layer_scaled_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc)
                   if f.endswith((".h", ".hip", ".cpp")))
    for path in files + [os.path.join(ROOT, "include", "qll.h")]:
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def hbm_traffic(fetch_csv, write_csv, kernel):
    """HBM bytes per launch of `kernel`: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by the ratio of known bytes to what the same
    counter reads for the calibration copy (CALIB_BYTES read and written)."""
    res = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        d = counter_per_dispatch(path, name)
        ks = [v for k, v in d.items() if k.startswith(kernel)]
        # the calibration kernel (torch.mul into a new buffer), not the
        # workload's own copies
        cal = [v for k, v in d.items() if "MulFunctor" in k]
        if not ks or not cal:
            return None
        vals = ks[0]
        cal_kib = max(max(c) for c in cal)   # the large calibration copy
        factor = CALIB_BYTES / (cal_kib * 1024.0)
        res[name] = (sum(vals) / len(vals)) * 1024.0 * factor
        res[name + "_factor"] = factor
    res["bytes_per_launch"] = res["FETCH_SIZE"] + res["WRITE_SIZE"]
    return res


XCDS = 8  # GRBM_GUI_ACTIVE adds up the busy cycles of the 8 XCDs


def dispatch_durations_ns(csv_path, kernel):
    """[(duration ns) per dispatch of `kernel`] from a rocprofv3 counter CSV
    (one row per counter: the first counter's rows), or [] without
    timestamps."""
    import csv
    out, first = [], None
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if not r.get("Kernel_Name", "").startswith(kernel):
                continue
            first = first or r.get("Counter_Name")
            if r.get("Counter_Name") != first:
                continue
            try:
                out.append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
            except (KeyError, ValueError):
                return []
    return out


def mfma_busy(csv_path, kernel, cus, flops_per_launch=None):
    """Matrix-core counters of `kernel`, each per dispatch (mean):
    SQ_VALU_MFMA_BUSY_CYCLES adds up, over every SIMD, the fixed number of
    busy cycles of each MFMA instruction issued (SQ_INSTS_MFMA counts them;
    the ratio is the cycles one instruction takes, e.g. 32 for the e4m3
    16x16x128 step), so for power-of-two shapes it is a power of two times
    that constant -- an exact count, not a sampled or saturated one.  The
    busy fraction is those cycles over the SIMD cycles of the dispatch
    (GRBM_GUI_ACTIVE / XCDS x 4 SIMDs x CUs); GRBM_GUI_ACTIVE / XCDS over the
    dispatch's duration is the engine clock the kernel ran at, and the
    SQ_INSTS_VALU_MFMA_MOPS_* counter x 512 its matrix-core operations (the
    algorithmic 2MNK plus the padding of partial tiles)."""
    def mean_of(counter):
        d = [v for k, v in counter_per_dispatch(csv_path, counter).items() if k.startswith(kernel)]
        return (sum(d[0]) / len(d[0]), len(d[0])) if d else (None, 0)
    b, n = mean_of("SQ_VALU_MFMA_BUSY_CYCLES")
    g, _ = mean_of("GRBM_GUI_ACTIVE")
    if b is None or g is None:
        return None
    res = {"mfma_busy_frac": round(b / (g / XCDS * 4 * cus), 4),
           "SQ_VALU_MFMA_BUSY_CYCLES": round(b), "GRBM_GUI_ACTIVE": round(g),
           "dispatches": n}
    inst, _ = mean_of("SQ_INSTS_MFMA")
    if inst:
        res["SQ_INSTS_MFMA"] = round(inst)
        res["busy_cycles_per_mfma"] = round(b / inst, 3)
    for dt in ("F8", "I8", "BF16", "F6F4"):
        mops, _ = mean_of(f"SQ_INSTS_VALU_MFMA_MOPS_{dt}")
        if mops:
            res[f"mops_{dt.lower()}_flops"] = round(mops * 512)
            if flops_per_launch:
                res["mops_over_algorithmic"] = round(mops * 512 / flops_per_launch, 4)
    durs = dispatch_durations_ns(csv_path, kernel)
    if durs:
        dur = sum(durs) / len(durs)
        res["dispatch_us"] = round(dur / 1e3, 3)
        # the counter's window is wider than the kernel by a few
        # microseconds, so the derived clock (and the busy fraction's
        # denominator) are inflated for short dispatches: the clock is given
        # for dispatches of 100 us and more only
        if dur >= 100e3:
            res["clock_ghz"] = round(g / XCDS / dur, 3)
    return res


def trace_timed_durations(csv_path, kernel, n_steps_dispatches, plan):
    """Durations (us) of the launches of `kernel` that the per-call timing
    times, from a rocprofv3 --kernel-trace CSV of a run of the same command.
    The kernel's dispatches come in this order: n_steps_dispatches from the
    first, warm-up, graph and eager steps; then per problem that uses it, in
    problem order, its per-call graph of `copies` launches replayed once
    untimed, `replays` times timed (these are the ones kept) and (1 +
    replays) times warm.  plan: [(problem index, copies, replays)].
    Returns {problem index: [durations]} or None when the counts disagree."""
    import csv
    durs = []
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r.get("Kernel_Name", "").startswith(kernel):
                durs.append((int(r["Start_Timestamp"]),
                             (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    durs.sort()
    d = [x for _, x in durs]
    need = n_steps_dispatches + sum(2 * (1 + rep) * c for _, c, rep in plan)
    if len(d) != need:
        return None
    out, at = {}, n_steps_dispatches
    for i, c, rep in plan:
        at += c  # the untimed replay
        out[i] = d[at:at + rep * c]
        at += rep * c + (1 + rep) * c  # the timed replays, then the warm graph
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the "
              "scaled_mm path is measured on a single MI355X and has no multi-GPU "
              "mode.", file=sys.stderr)
        sys.exit(2)
    import torch

    import quantized_linear_layer_scaled_amd as qll

    qll.load_library()
    t_init = time.perf_counter()
    rc = qll.init(None if args.table == "none" else args.table)
    init_ms = (time.perf_counter() - t_init) * 1e3
    table_used = qll.table_entries()
    props = torch.cuda.get_device_properties(0)
    print(f"# device {props.name} {getattr(props, 'gcnArchName', '?')} "
          f"{props.multi_processor_count} CUs; table entries {table_used} (init rc {rc})",
          file=sys.stderr, flush=True)

    # one stream for everything: the prebuilt calls, the events and the
    # graph capture all use it (default priority)
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    probs = build_problems(torch, qll, args.workload)
    env_before = env_info()
    print(f"# {len(probs)} problems built", file=sys.stderr, flush=True)

    # first step of the process: includes loading the kernels' code objects
    torch.cuda.synchronize()
    t_first = time.perf_counter()
    run_step(probs)
    torch.cuda.synchronize()
    first_step_ms = (time.perf_counter() - t_first) * 1e3
    for _ in range(args.warmup):
        run_step(probs)
    torch.cuda.synchronize()

    # ---- timed region 1: graph replays of the whole step -> value
    ms_graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            run_step(probs)
        graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        g0.record()
        for _ in range(args.steps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        ms_graph = g0.elapsed_time(g1) / args.steps
        print(f"# graph step {ms_graph * 1e3:.1f} us", file=sys.stderr, flush=True)

    # ---- timed region 2: eager steps (host launches, no graph)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    start.record()
    for step in range(args.steps):
        run_step(probs)
    end.record()
    host_enqueue_s = time.perf_counter() - t_wall0  # host time to enqueue K steps
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    ms_eager = start.elapsed_time(end) / args.steps
    n_calls = sum(len(p.calls) for p in probs)
    ms_per_step = ms_eager

    # ---- eager per-call wall time: HIP events around each C-ABI call
    eager_call = [[[] for _ in p.calls] for p in probs]
    if not args.no_graph:
        for _ in range(5):
            evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                    for _ in p.calls] for p in probs]
            run_step(probs, evs)
            torch.cuda.synchronize()
            for i, p in enumerate(probs):
                for j in range(len(p.calls)):
                    eager_call[i][j].append(evs[i][j][0].elapsed_time(evs[i][j][1]) * 1e3)

    # ---- timed region 3: every call on its own (graph of cold copies)
    if args.no_graph:  # counter-collection runs: launches only, no timing
        call_st = [[{"median": 1.0, "p10": 1.0, "p90": 1.0, "n": 1, "warm": 1.0, "copies": 1}
                    for _ in p.calls] for p in probs]
        call_plan = [[1 for _ in p.calls] for p in probs]
    else:
        call_st, call_plan = per_call_us(torch, probs, args.replays, stream)
    call_us = [[st["median"] for st in row] for row in call_st]
    vend = vendor_us(torch, probs, args.replays, stream) if args.vendor else None
    env_after = env_info()

    if args.calib_copy:
        # an elementwise kernel that reads CALIB_BYTES and writes CALIB_BYTES
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # per-call average durations (ms)
    per_shape = []
    kernels = {}  # symbol -> [total s, launches, flops, bytes, dtype, bounds, splits]
    gemm_flops_step = 0.0
    for i, p in enumerate(probs):
        rec = {"op": p.op, "M": p.M, "N": p.N, "K": p.K, "variant": p.variant,
               "splits": p.eff_splits}
        for j, (kind, _, _) in enumerate(p.calls):
            st = call_st[i][j]
            rec[f"{kind}_us"] = round(st["median"], 3)
            rec[f"{kind}_us_p10_p90"] = [round(st["p10"], 3), round(st["p90"], 3)]
            rec[f"{kind}_warm_us"] = round(st["warm"], 3)
            rec[f"{kind}_copies"] = st["copies"]
            if eager_call[i][j]:
                rec[f"{kind}_eager_us"] = round(sorted(eager_call[i][j])[len(eager_call[i][j]) // 2], 3)
        if getattr(p, "fused", False):
            rec["fused"] = True  # one kernel: quantizer and GEMM
        if vend is not None:
            rec["vendor_gemm_us"] = round(vend[i], 3) if vend[i] is not None else None
        t_gemm = rec["gemm_us"] * 1e-6
        dt = {"fp8": "fp8", "fp8_grouped": "fp8", "block_fp8": "fp8", "int8": "int8",
              "bf16_bi": "bf16", "mxfp4": "fp4", "w4a16": "bf16"}[p.op]
        t_mem = p.algo_bytes() / (HBM_GBS * 1e9)
        t_mfma = p.flops / (PEAK[dt] * 1e12)
        rec["tflops"] = round(p.flops / t_gemm / 1e12, 2)
        rec["gbs"] = round(p.algo_bytes() / t_gemm / 1e9, 1)
        rec["bound"] = "hbm" if t_mem >= t_mfma else "mfma"
        rec["roof_frac"] = round(max(t_mem, t_mfma) / t_gemm, 3)
        if "quant_us" in rec:
            rec["quant_gbs"] = round(p.quant_bytes() / (rec["quant_us"] * 1e-6) / 1e9, 1)
        per_shape.append(rec)
        gemm_flops_step += p.flops
        if p.eff_splits > 1:
            continue  # two kernels per call: not comparable with a kernel trace
        sym = kernel_symbol(qll, p.op, p.variant)
        k = kernels.setdefault(sym, [0.0, 0, 0.0, 0.0, dt, [], [], []])
        k[0] += t_gemm
        k[1] += 1
        k[2] += p.flops
        k[3] += p.algo_bytes()
        k[5].append(rec["bound"])
        k[6].append(p.eff_splits)
        k[7].append(rec["gemm_copies"])

    dom_sym, dom = max(kernels.items(), key=lambda kv: kv[1][0])
    avg_dur = dom[0] / dom[1]
    bound = "mfma" if dom[5].count("mfma") >= dom[5].count("hbm") else "hbm"
    if bound == "mfma":
        achieved = dom[2] / dom[1] / avg_dur / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK[dom[4]],
                "unit": "TFLOP/s", "frac": round(achieved / PEAK[dom[4]], 4)}
    else:
        achieved = dom[3] / dom[1] / avg_dur / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_GBS, 4)}
    roof["traffic"] = None
    digest = source_digest()
    if args.fetch_csv and args.write_csv and os.path.exists(args.fetch_csv) \
            and os.path.exists(args.write_csv):
        tr = hbm_traffic(args.fetch_csv, args.write_csv, dom_sym)
        if tr:
            roof["traffic"] = round(tr["bytes_per_launch"])
            roof["traffic_detail"] = {k: round(v, 4) for k, v in tr.items()}
            roof["traffic_detail"]["source_digest"] = digest
    else:
        # counters taken earlier by the profiling runs of this workload, used
        # only when they were taken on the same kernel built from the same
        # sources
        prof = os.path.join(ROOT, "profiles", f"{args.workload}_sweep_bench_line.json")
        try:
            with open(prof) as f:
                old = json.load(f)["roofline"]
        except (OSError, ValueError, KeyError):
            old = None
        if old and old.get("kernel") == dom_sym and old.get("traffic") and \
                (old.get("traffic_detail") or {}).get("source_digest") == digest:
            roof["traffic"] = old["traffic"]
            roof["traffic_detail"] = dict(old["traffic_detail"])
            roof["traffic_detail"]["from"] = (
                f"profiles/{args.workload}_sweep_traffic.md: rocprofv3 --pmc FETCH_SIZE and "
                "WRITE_SIZE runs of this workload on the same kernel and sources")
            # the matrix-core counters and the traced kernel duration of the
            # same profiling runs (same kernel, same sources)
            if old.get("mfma_counters") and not args.mfma_csv:
                roof["mfma_counters"] = dict(old["mfma_counters"])
                roof["mfma_counters"]["from"] = (
                    f"profiles/{args.workload}_sweep_traffic.md (rocprofv3 --pmc run)")
            kd = old.get("kernel_duration")
            if kd and "avg_us" in kd and not args.kernel_trace_csv:
                roof["kernel_duration"] = dict(kd)
                roof["kernel_duration"]["from"] = (
                    f"profiles/{args.workload}_sweep_kernel_stats.md: rocprofv3 --kernel-trace "
                    "run of this workload on the same kernel and sources (kernel only, no "
                    "in-graph gap)")
    if args.mfma_csv and os.path.exists(args.mfma_csv):
        mb = mfma_busy(args.mfma_csv, dom_sym, props.multi_processor_count,
                       flops_per_launch=dom[2] / dom[1])
        if mb:
            roof["mfma_counters"] = mb
    if args.kernel_trace_csv and os.path.exists(args.kernel_trace_csv):
        # the dominant kernel's own duration over the launches timed above
        # (kernel time only, without the in-graph gap the events include)
        users = [i for i, p in enumerate(probs) if p.eff_splits == 1 and
                 kernel_symbol(qll, p.op, p.variant) == dom_sym]
        steps_disp = len(users) * (1 + args.warmup + (1 + args.steps if not args.no_graph else 0)
                                   + args.steps + (5 if not args.no_graph else 0))
        gemm_j = {i: [k for k, _, _ in probs[i].calls].index("gemm") for i in users}
        plan = [(i, call_plan[i][gemm_j[i]], args.replays) for i in users]
        td = trace_timed_durations(args.kernel_trace_csv, dom_sym, steps_disp, plan)
        if td:
            t_k = sum(sum(v) / len(v) for v in td.values()) / len(td) * 1e-6
            ka = (dom[2] / dom[1] if bound == "mfma" else dom[3] / dom[1]) / t_k
            ka = ka / 1e12 if bound == "mfma" else ka / 1e9
            roof["kernel_duration"] = {
                "avg_us": round(t_k * 1e6, 3), "achieved": round(ka, 2),
                "frac": round(ka / roof["peak"], 4),
                "from": "rocprofv3 --kernel-trace of the same command: the durations of "
                        "the launches the per-call timing times (kernel only, no in-graph "
                        "gap)"}
        else:
            roof["kernel_duration"] = {"error": "the trace's dispatch count does not match "
                                                "this command's launch plan"}
    if dom_sym.startswith(("void qll::gemm_pipe_kernel", "void qll::gemm_pipe_rc_kernel")) \
            and ", true, " not in dom_sym and ", true>" not in dom_sym:
        # the fetch the XCD structure implies (each XCD's L2 reads the rows
        # of its tiles once), per launch, plus the bf16 output
        dp = [p for p in probs if p.eff_splits == 1 and
              kernel_symbol(qll, p.op, p.variant) == dom_sym]
        if dp:
            vv = {v["name"]: v for v in qll.variants(dp[0].op)}[dp[0].variant]
            kb = {"bf16_bi": 2, "mxfp4": 0.5}.get(dp[0].op, 1)
            model = [xcd_fill_bytes(p.M, p.N, int(p.K * kb), vv["bp"], vv["bq"]) + 2 * p.M * p.N
                     for p in dp]
            roof["traffic_xcd_model"] = round(sum(model) / len(model))
    roof["kernel"] = dom_sym
    roof["launches_per_step"] = dom[1]
    roof["avg_us"] = round(avg_dur * 1e6, 3)
    roof["algorithmic_per_launch"] = (round(dom[2] / dom[1]) if bound == "mfma"
                                      else round(dom[3] / dom[1]))
    roof["algorithmic_bytes_per_launch"] = round(dom[3] / dom[1])
    roof["timing"] = ("per call: HIP graph of back-to-back launches, each on its own copy "
                      "of the call's buffers (>= 1 GiB per replay: cold, from HBM), "
                      f"{args.replays} replays between HIP events, median per-launch time "
                      "(kernel time plus the in-graph gap to the next launch); the dominant "
                      "kernel is the one with the most time per step among calls that "
                      "launch a single kernel (no Split-K)")
    # the per-call timing launches of the dominant kernel, in trace order: for
    # each problem that uses it, (1 + replays) replays of `copies` cold
    # launches, then (1 + replays) replays of `copies` warm launches
    roof["per_call_plan"] = {"copies": dom[7], "replays": args.replays}

    value = gemm_flops_step / (ms_per_step * 1e-3) / 1e12
    names = {"fp8": "FP8 dynamic per-token sweep: (N,K) in {(4096,2048),(2048,6144)}, "
                    "M in {1,4,8,16,32,64,256,512,1024,2048}; per-token quantization + "
                    "scaled FP8 GEMM, bf16 out",
             "int8": "W8A8 INT8 GEMM M=16 N=2048 K=2048, bf16 out (8 independent copies)",
             "block": "Block-FP8 sweep: (N,K) in {(12288,2048),(2048,6144)}, "
                      "M in {1,16,64,256,2048}; 1x128 quantization + GEMM, bf16 out",
             "bi": "batch-invariant bf16 sweep: (N,K) in {(2048,2048),(4096,2048)}, "
                   "M in {1,4,...,2048}, bf16 out",
             "moe": "grouped FP8 GEMM (per-expert weights): 64 experts of N=1536 K=2048, "
                    "T in {16,128,1024} tokens routed to 8 experts each (skewed synthetic "
                    "routing); per-token quantization + gemm_fp8_grouped, bf16 out",
             "vocab": "large-vocab FP8 dynamic projection N=151936 K=2048, "
                      "M in {1,8,64,512,2048}",
             "vocab_bi": "large-vocab batch-invariant bf16 projection N=151936 K=2048, "
                         "M in {1,8,64,512,2048}, bf16 out",
             "w4a16": "INT4 weight-only sweep: (N,K) in {(4096,2048),(2048,6144)}, "
                      "M in {1,4,8,16,32,64,256,512,1024,2048}; bf16 activations x int4 "
                      "weights (scale per 128-element group), bf16 out",
             "mxfp4": "MXFP4 sweep: (N,K) in {(4096,2048),(2048,6144)}, "
                      "M in {1,4,8,16,32,64,256,512,1024,2048}; MXFP4 quantization of the "
                      "activations + MXFP4 GEMM (E8M0 scale per 32), bf16 out"}
    dtype = {"fp8": "fp8e4m3", "vocab": "fp8e4m3", "block": "fp8e4m3", "int8": "int8",
             "moe": "fp8e4m3", "mxfp4": "fp4e2m1", "w4a16": "bf16 x int4",
             "bi": "bf16", "vocab_bi": "bf16"}[args.workload]
    line = {
        "metric": "TFLOPS/TOPS + % of HBM or MFMA roofline per (M,N,K), FP8/INT8 scaled_mm",
        "value": round(value, 3),
        "unit": "TOPS" if args.workload == "int8" else "TFLOPS",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype, "data": "synthetic (seeded, shapes and distributions of the workload)",
        "config": {"workload": names[args.workload],
                   "problems_per_step": len(probs),
                   "dispatch": "table" if table_used else "heuristic",
                   "timing": "eager C-ABI launches (graph replay in graph_value)",
                   "cold_weights": True},
        "graph_ms_per_step": round(ms_graph, 4) if ms_graph is not None else None,
        "graph_value": (round(gemm_flops_step / (ms_graph * 1e-3) / 1e12, 3)
                        if ms_graph is not None else None),
        "roofline": roof,
        "cpu_baseline": None,
        # host side of the C-ABI path: table load, the first step of the
        # process (code-object loading included), and the host time to
        # enqueue one call (ctypes + argument checks + dispatch + launch)
        "dispatch": {"init_ms": round(init_ms, 3),
                     "first_step_ms": round(first_step_ms, 3),
                     "calls_per_step": n_calls,
                     "host_us_per_call": round(host_enqueue_s * 1e6 / (args.steps * n_calls), 2),
                     "host_us_per_step": round(host_enqueue_s * 1e6 / args.steps, 1)},
        "wall_s_timed": round(wall, 3),
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "arch": getattr(props, "gcnArchName", "?"), "rocm": env_before["rocm"],
                   "torch": torch.__version__, "clocks_before": env_before["clocks"],
                   "clocks_after": env_after["clocks"]},
        "per_shape": per_shape,
    }
    if vend is not None:
        both = [(r["gemm_us"], r["vendor_gemm_us"]) for r in per_shape
                if r.get("vendor_gemm_us")]
        line["vendor_context"] = {
            "library": "torch._scaled_mm (hipBLASLt), row-wise scales"
                       if args.workload not in ("bi", "vocab_bi") else "torch.matmul (hipBLASLt)",
            "problems": len(both),
            "sum_gemm_us_ours": round(sum(a for a, _ in both), 2),
            "sum_gemm_us_vendor": round(sum(b for _, b in both), 2),
            "note": "context only: the same per-call method (cold copies, graph replays); "
                    "GEMM only, the quantizer is not part of the vendor call"}
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        cb = cpu_baseline(args.workload, args.cpu_rows)
        cb["gpu_over_cpu"] = round(value / cb["value"], 1) if cb["value"] else None
        line["cpu_baseline"] = cb
    for r in per_shape:
        print(f"#  {r['op']:9s} M={r['M']:5d} N={r['N']:6d} K={r['K']:5d} {r['variant']:24s} "
              f"S={r['splits']} gemm {r['gemm_us']:8.2f} us {r['tflops']:8.1f} TFLOPS "
              f"{r['gbs']:7.0f} GB/s {r['bound']} {100 * r['roof_frac']:5.1f}%"
              + (f"  quant {r['quant_us']:6.2f} us" if 'quant_us' in r else ""),
              file=sys.stderr)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
