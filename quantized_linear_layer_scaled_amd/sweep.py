"""Offline on-device sweep that fills the dispatch table.

This is the ahead-of-time search of "Helion in vLLM: A Unified Route to
Tunable Linear Kernels" ("What the integration changes": the algorithm --
ordinary, Split-K, Swap-AB -- is chosen per shape together with its tile
configuration), done on the device the table will serve, as in vLLM PR
#53446 (per-device tables; per-bucket winners kept, "Re-benchmark" section).

For every (op, N, K) and every M bucket (powers of two) it runs each
registered kernel variant with each Split-K factor through the C entry
point with a forced configuration, checks the result against a reference
configuration of the same op (bit-exact for the INT8 int32 accumulators,
normwise 1e-2 otherwise -- the oracle parity is the test suite's job), times
the whole call (tile kernel plus Split-K reduction) by replaying a HIP graph
of back-to-back calls that rotate through enough copies of the weights to
exceed the 256 MB Infinity Cache (cold weights, as in serving, where every
layer's weights come from HBM; the activations stay the same, as when the
previous kernel has just written them), and keeps the fastest configuration
per bucket.  The batch-invariant op only
considers configurations without a cross-workgroup K split and whose waves,
if they split K, split it into the op's fixed eight chunks, so the table it
produces is accepted by the loader.

    python -m quantized_linear_layer_scaled_amd.sweep --out tables/gfx950.tsv
    python -m quantized_linear_layer_scaled_amd.sweep --ops fp8 --shapes 4096x2048 --report

The output is an append-free text table: one "device <arch> <CUs>" line and
"op N K bucket variant splits  # us tflops" lines.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

# The serving shapes the library ships a table for: (op, N, K) and M list.
DEFAULT_M = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048]
DEFAULT_SHAPES = {
    "int8": [(2048, 2048)],
    "fp8": [(4096, 2048), (2048, 6144), (151936, 2048)],
    "block_fp8": [(12288, 2048), (2048, 6144)],
    "bf16_bi": [(2048, 2048), (4096, 2048), (151936, 2048)],
    "mxfp4": [(4096, 2048), (2048, 6144)],
    "w4a16": [(4096, 2048), (2048, 6144)],
}
SPLITS = [1, 2, 4, 8]
WS_LIMIT = 1 << 30
COLD_BYTES = 384 << 20  # weights touched per timing replay: > the 256 MB Infinity Cache


def _inputs(torch, op, M, N, K, copies):
    g = torch.Generator(device="cuda")
    g.manual_seed(1234 + N + K)

    def e4m3(shape):
        # random finite e4m3 codes of moderate magnitude
        c = torch.randint(0, 0x70, shape, device="cuda", dtype=torch.uint8, generator=g)
        sign = torch.randint(0, 2, shape, device="cuda", dtype=torch.uint8, generator=g) << 7
        return (c | sign).view(torch.float8_e4m3fn)

    if op == "int8":
        A = torch.randint(-127, 128, (M, K), device="cuda", dtype=torch.int8, generator=g)
        Bs = [torch.randint(-127, 128, (N, K), device="cuda", dtype=torch.int8, generator=g)
              for _ in range(copies)]
        sa = torch.rand(M, device="cuda", generator=g) * 9e-3 + 1e-3
        sb = torch.rand(N, device="cuda", generator=g) * 9e-3 + 1e-3
    elif op == "fp8":
        A = e4m3((M, K))
        Bs = [e4m3((N, K)) for _ in range(copies)]
        sa = torch.rand(M, device="cuda", generator=g) * 1e-2 + 1e-3
        sb = torch.rand(N, device="cuda", generator=g) * 1e-4 + 1e-5
    elif op == "mxfp4":
        # random packed E2M1 codes, scale bytes around 2^0
        A = torch.randint(0, 256, (M, K // 2), device="cuda", dtype=torch.uint8, generator=g)
        Bs = [torch.randint(0, 256, (N, K // 2), device="cuda", dtype=torch.uint8, generator=g)
              for _ in range(copies)]
        sa = torch.randint(120, 134, (M, K // 32), device="cuda", dtype=torch.uint8, generator=g)
        sb = torch.randint(120, 134, (N, K // 32), device="cuda", dtype=torch.uint8, generator=g)
    elif op == "w4a16":
        A = (torch.randn((M, K), device="cuda", generator=g)).to(torch.bfloat16)
        Bs = [torch.randint(0, 256, (N, K // 2), device="cuda", dtype=torch.uint8, generator=g)
              for _ in range(copies)]
        sa = None
        sb = torch.rand((N, K // 128), device="cuda", generator=g) * 9e-3 + 1e-3
    elif op == "block_fp8":
        A = e4m3((M, K))
        Bs = [e4m3((N, K)) for _ in range(copies)]
        sa = torch.rand((M, K // 128), device="cuda", generator=g) * 1e-2 + 1e-3
        sb = torch.rand(((N + 127) // 128, K // 128), device="cuda", generator=g) * 1e-4 + 1e-5
    else:
        A = (torch.randn((M, K), device="cuda", generator=g) / math.sqrt(K)).to(torch.bfloat16)
        Bs = [(torch.randn((N, K), device="cuda", generator=g) / math.sqrt(K)).to(torch.bfloat16)
              for _ in range(copies)]
        sa = sb = None
    return A, Bs, sa, sb


def _call(qll, op, A, B, sa, sb, out_dtype, cfg, ws, out=None):
    kw = dict(out_dtype=out_dtype, cfg=cfg, workspace=ws, out=out)
    if op == "int8":
        return qll.gemm_w8a8_int8(A, B, sa, sb, **kw)
    if op == "fp8":
        return qll.gemm_fp8_scaled(A, B, sa, sb, **kw)
    if op == "block_fp8":
        return qll.gemm_block_fp8(A, B, sa, sb, **kw)
    if op == "mxfp4":
        return qll.gemm_mxfp4(A, B, sa, sb, **kw)
    if op == "w4a16":
        return qll.gemm_w4a16(A, B, sb, **kw)
    return qll.gemm_bf16_batch_invariant(A, B, **kw)


def candidates(qll, op, M, N, K):
    """(variant, splits) pairs worth timing for this shape."""
    out = []
    for v in qll.variants(op):
        name = v["name"]
        if op == "bf16_bi" and name[0] == "k" and v["wp"] != 8:
            continue  # its waves split K into other chunks than the fixed eight
        if name[0] in "kr" and M > 128:
            continue  # skinny kernels hold all tokens of a tile in registers
        if name[0] in "np" and M <= 8 and v["bp"] >= 64 and not v["swap"]:
            continue  # 64+ token rows per tile for a handful of tokens
        for s in SPLITS:
            if op == "bf16_bi" and s != 1:
                continue
            if s > 1 and qll.effective_splits(op, K, s) != s:
                continue
            if qll.workspace_bytes(op, M, N, K, (name, s)) > WS_LIMIT:
                continue
            out.append((name, s))
    return out


def time_config(torch, qll, op, A, Bs, sa, sb, cfg, ws, reps):
    """GPU time per call: `reps` calls (rotating the weight copies) are
    captured into one HIP graph and the graph replay is timed, so the number
    is kernel time plus the in-graph launch gaps, free of host overhead."""
    M, N = A.shape[0], Bs[0].shape[0]
    outs = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    for i in range(2):  # warm up outside the capture
        _call(qll, op, A, Bs[i % len(Bs)], sa, sb, "bf16", cfg, ws, outs[i % 2])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            _call(qll, op, A, Bs[i % len(Bs)], sa, sb, "bf16", cfg, ws, outs[i % 2])
    g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    g.replay()
    g.replay()
    e.record()
    torch.cuda.synchronize()
    del g
    return s.elapsed_time(e) * 1e3 / (2 * reps), outs[0]


def sweep_shape(torch, qll, op, N, K, mlist, reps, log):
    row_bytes = {"bf16_bi": 2 * K, "mxfp4": K // 2, "w4a16": K // 2}.get(op, K)
    # rotate through at least COLD_BYTES of weights per graph replay
    copies = max(2, min(64, -(-COLD_BYTES // max(1, N * row_bytes))))
    reps = max(reps, copies)
    Mmax = max(mlist)
    A_all, Bs, sa_all, sb = _inputs(torch, op, Mmax, N, K, copies)
    results = {}
    for M in mlist:
        A = A_all[:M].contiguous()
        sa = sa_all[:M].contiguous() if sa_all is not None else None
        cands = candidates(qll, op, M, N, K)
        need = max(qll.workspace_bytes(op, M, N, K, c) for c in cands)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        # reference: the plain heuristic choice without Split-K
        ref_cfg = (qll.select(op, M, N, K)[0], 1)
        if op == "int8":
            ref = _call(qll, op, A, Bs[0], sa, sb, "int32", ref_cfg, ws)
        else:
            ref = _call(qll, op, A, Bs[0], sa, sb, "fp32", ref_cfg, ws).double()
        rows = []
        for cfg in cands:
            if op == "int8":
                got = _call(qll, op, A, Bs[0], sa, sb, "int32", cfg, ws)
                ok = torch.equal(got, ref)
            else:
                got = _call(qll, op, A, Bs[0], sa, sb, "fp32", cfg, ws).double()
                den = ref.abs().max().item() or 1.0
                ok = (got - ref).abs().max().item() / den <= 1e-4
            if not ok:
                log(f"  PARITY FAIL {op} M={M} N={N} K={K} {cfg}")
                continue
            us, _ = time_config(torch, qll, op, A, Bs, sa, sb, cfg, ws, reps)
            rows.append((us, cfg))
        rows.sort()
        best_us, best = rows[0]
        tflops = 2.0 * M * N * K / best_us / 1e6
        results[M] = (best, best_us, tflops, rows[:5])
        log(f"  {op} N={N} K={K} M={M}: best {best[0]} S={best[1]} {best_us:.2f} us "
            f"{tflops:.1f} TFLOPS; next: " +
            ", ".join(f"{c[0]}/S{c[1]} {u:.2f}" for u, c in rows[1:4]))
        del ws
    return results


def main(argv=None):
    ap = argparse.ArgumentParser(description="fill the scaled_mm dispatch table")
    ap.add_argument("--ops", default="int8,fp8,block_fp8,bf16_bi,mxfp4,w4a16")
    ap.add_argument("--shapes", default=None, help="NxK[,NxK...] (default: the shipped set)")
    ap.add_argument("--m", default=None, help="M values (default: 1..2048 powers of two)")
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--out", default=None, help="table path to write")
    ap.add_argument("--json", default=None, help="also write all timings as JSON")
    args = ap.parse_args(argv)

    import torch

    import quantized_linear_layer_scaled_amd as qll
    qll.load_library()
    qll.init(None)  # sweep against the heuristic, never a stale table
    props = torch.cuda.get_device_properties(0)
    arch = getattr(props, "gcnArchName", "gfx950").split(":")[0]
    cus = props.multi_processor_count
    mlist = [int(x) for x in args.m.split(",")] if args.m else DEFAULT_M
    log = lambda s: print(s, flush=True)
    log(f"# sweep on {arch} with {cus} CUs")
    lines = [f"# scaled_mm dispatch table, written by quantized_linear_layer_scaled_amd.sweep",
             f"# {time.strftime('%Y-%m-%d %H:%M:%S')}; reps {args.reps}",
             f"device {arch} {cus}"]
    dump = {}
    for op in args.ops.split(","):
        shapes = DEFAULT_SHAPES[op]
        if args.shapes:
            shapes = [tuple(int(v) for v in s.split("x")) for s in args.shapes.split(",")]
        for N, K in shapes:
            res = sweep_shape(torch, qll, op, N, K, mlist, args.reps, log)
            for M, (best, us, tf, top) in res.items():
                lines.append(f"{op} {N} {K} {M} {best[0]} {best[1]}  # {us:.2f} us {tf:.1f} TFLOPS")
                dump[f"{op} {N} {K} {M}"] = [[c[0], c[1], u] for u, c in top]
            torch.cuda.empty_cache()
    text = "\n".join(lines) + "\n"
    if args.out:
        os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
        with open(args.out, "w") as f:
            f.write(text)
        log(f"# wrote {args.out}")
    else:
        sys.stdout.write(text)
    if args.json:
        with open(args.json, "w") as f:
            json.dump(dump, f, indent=1)


if __name__ == "__main__":
    main()
