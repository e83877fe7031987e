"""Offline on-device sweep that fills the dispatch table.

This is the ahead-of-time search of "Helion in vLLM: A Unified Route to
Tunable Linear Kernels" ("What the integration changes": the algorithm --
ordinary, Split-K, Swap-AB -- is chosen per shape together with its tile
configuration), done on the device the table will serve, as in vLLM PR
#53446 (per-device tables; per-bucket winners kept, "Re-benchmark" section).

For every (op, N, K) and every M bucket (powers of two) it runs each
registered kernel variant with each Split-K factor through the C entry
point with a forced configuration, checks the result against an independent
reference -- a float64 product of the decoded operands and scales computed
with torch on the device (exact integer accumulators for INT8; normwise
within 2e-3 for the fp32 output of the other ops) --, times the whole call
(tile kernel plus Split-K reduction) by replaying a HIP graph of
back-to-back calls that rotate through enough copies of the weights to
exceed the 256 MB Infinity Cache (cold weights, as in serving, where every
layer's weights come from HBM; the activations stay the same, as when the
previous kernel has just written them), and keeps the fastest configuration
per bucket.  The batch-invariant op only considers configurations without a
cross-workgroup K split and whose waves, if they split K, split it into the
op's fixed eight chunks, so the table it produces is accepted by the loader.

Searches like this take long ("The costs behind the gains": ahead-of-time
searches can take hours), so every finished (shape, M, configuration) is
appended to a log as one JSON line the moment it is measured, and a run
given the same log skips what the log already holds: a killed sweep resumes
where it stopped.  The table is written from the log at the end.

    python -m quantized_linear_layer_scaled_amd.sweep --out tables/gfx950.tsv
    python -m quantized_linear_layer_scaled_amd.sweep --ops fp8 --shapes 4096x2048 --report

The table is plain text: one "device <arch> <CUs> <MHz> <name>" line (the
device signature the library matches it against) and
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
    # the FP8 dynamic linear layer (quantizer + GEMM in two launches, or the
    # fused decode kernel), swept where the fused kernel can run
    "fp8_dynamic": [(4096, 2048), (2048, 6144), (151936, 2048)],
}
DYN_M = [1, 2, 4, 8, 16]
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
    elif op == "fp8_dynamic":
        A = torch.randn((M, K), device="cuda", generator=g).to(torch.bfloat16)
        Bs = [e4m3((N, K)) for _ in range(copies)]
        sa = None
        sb = torch.rand(N, device="cuda", generator=g) * 1e-3 + 1e-4
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


_DYN_BUFS = {}


def _call(qll, op, A, B, sa, sb, out_dtype, cfg, ws, out=None):
    kw = dict(out_dtype=out_dtype, cfg=cfg, workspace=ws, out=out)
    if op == "fp8_dynamic":
        import torch
        key = (A.shape[0], A.shape[1])
        if key not in _DYN_BUFS:  # codes and scales outside any graph capture
            _DYN_BUFS[key] = (torch.empty(key, dtype=torch.float8_e4m3fn, device="cuda"),
                              torch.empty((key[0], 1), dtype=torch.float32, device="cuda"))
        q, s = _DYN_BUFS[key]
        return qll.linear_fp8_dynamic(A, B, sb, q=q, sa=s, **kw)[0]
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


def fused_steps(K, W):
    """K steps of 128 elements the busiest of W waves of a fused decode
    workgroup handles (the cut of the W-wave decode GEMM)."""
    T = -(-K // 128)
    TU = -(-T // 2)
    return max(min(T, 2 * ((w + 1) * TU // W)) - min(T, 2 * (w * TU // W)) for w in range(W))


def candidates(qll, op, M, N, K):
    """(variant, splits) pairs worth timing for this shape."""
    out = []
    for v in qll.variants(op):
        name = v["name"]
        if v.get("fused"):
            # the fused linear layer: at most its tokens, K within its chunk
            if M <= v["bq"] and fused_steps(K, v["wp"]) <= v["ksteps"]:
                out.append((name, 1))
            continue
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


_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def reference(torch, op, A, B, sa, sb):
    """The op's product in float64 from the decoded operands and scales, on
    the device: the acceptance check of every timed configuration (exact for
    INT8, whose int32 accumulators it holds as integers)."""
    f64 = torch.float64
    if op == "int8":
        return A.to(f64) @ B.to(f64).T
    if op == "bf16_bi":
        return A.to(f64) @ B.to(f64).T
    if op == "fp8":
        ref = A.float().to(f64) @ B.float().to(f64).T
        return ref * sa.to(f64)[:, None] * sb.to(f64)[None, :]
    if op == "block_fp8":
        M, K = A.shape
        N = B.shape[0]
        a, b = A.float().to(f64), B.float().to(f64)
        sbn = sb.to(f64).repeat_interleave(128, dim=0)[:N]  # [N][K/128]
        ref = torch.zeros((M, N), dtype=f64, device=A.device)
        for g in range(K // 128):
            k = slice(128 * g, 128 * g + 128)
            ref += (a[:, k] @ b[:, k].T) * (sa.to(f64)[:, g, None] * sbn[None, :, g])
        return ref
    if op == "mxfp4":
        lut = torch.tensor(_E2M1 + [-v for v in _E2M1], dtype=f64, device=A.device)

        def dec(codes, scales):
            lo, hi = (codes & 15).long(), (codes >> 4).long()
            v = torch.stack([lut[lo], lut[hi]], dim=-1).reshape(codes.shape[0], -1)
            s = torch.exp2(scales.to(f64) - 127.0).repeat_interleave(32, dim=1)
            return v * s
        return dec(A, sa) @ dec(B, sb).T
    if op == "fp8_dynamic":
        import quantized_linear_layer_scaled_amd as qll
        q, s = qll.quantize_per_token_fp8(A)
        return reference(torch, "fp8", q, B, s[:, 0], sb)
    if op == "w4a16":
        lo, hi = (B & 15).to(torch.int16), (B >> 4).to(torch.int16)
        v = torch.stack([lo, hi], dim=-1).reshape(B.shape[0], -1)
        v = torch.where(v >= 8, v - 16, v).to(f64)
        w = v * sb.to(f64).repeat_interleave(128, dim=1)
        return A.to(f64) @ w.T
    raise ValueError(op)


def accept(torch, op, got, ref):
    """INT8: the int32 accumulators equal the exact ones; otherwise the fp32
    output is within 1e-3 of the float64 product, normwise (a broken
    configuration -- a tile, split or K range handled wrongly -- is off by
    O(1))."""
    if op == "int8":
        return bool(torch.equal(got.to(torch.float64), ref))
    den = ref.abs().max().item() or 1.0
    return bool(torch.isfinite(got).all()) and \
        (got.double() - ref).abs().max().item() / den <= 1e-3


def read_log(path):
    """Entries of an append-only sweep log: key -> record.  A line cut short
    by a kill is skipped (its configuration is measured again)."""
    done = {}
    if not path or not os.path.exists(path):
        return done
    with open(path) as f:
        for line in f:
            try:
                r = json.loads(line)
                done[r["key"]] = r
            except (ValueError, KeyError):
                continue
    return done


def entry_key(op, N, K, M, cfg):
    return f"{op} {N} {K} {M} {cfg[0]} {cfg[1]}"


def sweep_shape(torch, qll, op, N, K, mlist, reps, log, done=None, record=None):
    """Best configuration per M for one (op, N, K).  `done` holds log records
    of configurations measured before (skipped here); `record` receives each
    new one as it is measured."""
    done = {} if done is None else done
    record = record or (lambda r: None)
    row_bytes = {"bf16_bi": 2 * K, "mxfp4": K // 2, "w4a16": K // 2}.get(op, K)
    if op == "fp8_dynamic":
        mlist = [m for m in mlist if m <= max(DYN_M)]
    # rotate through at least COLD_BYTES of weights per graph replay
    copies = max(2, min(64, -(-COLD_BYTES // max(1, N * row_bytes))))
    reps = max(reps, copies)
    Mmax = max(mlist)
    state = {}

    def inputs():
        if not state:
            state["all"] = _inputs(torch, op, Mmax, N, K, copies)
        return state["all"]

    results = {}
    timed = 0
    for M in mlist:
        cands = candidates(qll, op, M, N, K)
        todo = [c for c in cands if entry_key(op, N, K, M, c) not in done]
        rows = [(done[entry_key(op, N, K, M, c)]["us"], c) for c in cands
                if entry_key(op, N, K, M, c) in done and done[entry_key(op, N, K, M, c)]["ok"]]
        if todo:
            A_all, Bs, sa_all, sb = inputs()
            A = A_all[:M].contiguous()
            sa = sa_all[:M].contiguous() if sa_all is not None else None
            need = max(qll.workspace_bytes(op, M, N, K, c) for c in todo)
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
            ref = reference(torch, op, A, Bs[0], sa, sb)
            for cfg in todo:
                got = _call(qll, op, A, Bs[0], sa, sb, "int32" if op == "int8" else "fp32",
                            cfg, ws)
                ok = accept(torch, op, got, ref)
                us = None
                if ok:
                    us, _ = time_config(torch, qll, op, A, Bs, sa, sb, cfg, ws, reps)
                    rows.append((us, cfg))
                else:
                    log(f"  PARITY FAIL {op} M={M} N={N} K={K} {cfg}")
                rec = {"key": entry_key(op, N, K, M, cfg), "ok": ok, "us": us}
                done[rec["key"]] = rec
                record(rec)
                timed += 1
            del ws, ref
        if not rows:
            log(f"  {op} N={N} K={K} M={M}: no configuration passed")
            continue
        rows.sort()
        best_us, best = rows[0]
        tflops = 2.0 * M * N * K / best_us / 1e6
        results[M] = (best, best_us, tflops, rows[:5])
        log(f"  {op} N={N} K={K} M={M}: best {best[0]} S={best[1]} {best_us:.2f} us "
            f"{tflops:.1f} TFLOPS; next: " +
            ", ".join(f"{c[0]}/S{c[1]} {u:.2f}" for u, c in rows[1:4]))
    state.clear()
    return results, timed


def main(argv=None):
    ap = argparse.ArgumentParser(description="fill the scaled_mm dispatch table")
    ap.add_argument("--ops", default="int8,fp8,block_fp8,bf16_bi,mxfp4,w4a16")
    ap.add_argument("--shapes", default=None, help="NxK[,NxK...] (default: the shipped set)")
    ap.add_argument("--m", default=None, help="M values (default: 1..2048 powers of two)")
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--out", default=None, help="table path to write")
    ap.add_argument("--log", default=None,
                    help="append-only log of every measured configuration; a run "
                         "given an existing log resumes from it (default: <out>.log.jsonl)")
    ap.add_argument("--json", default=None, help="also write all timings as JSON")
    args = ap.parse_args(argv)

    import torch

    import quantized_linear_layer_scaled_amd as qll
    qll.load_library()
    qll.init(None)  # sweep against the heuristic, never a stale table
    sig = qll.device_signature()
    mlist = [int(x) for x in args.m.split(",")] if args.m else DEFAULT_M
    log = lambda s: print(s, flush=True)
    log_path = args.log or (args.out + ".log.jsonl" if args.out else None)
    done = read_log(log_path)
    if done:
        log(f"# resuming: {len(done)} configurations already measured in {log_path}")
    logf = open(log_path, "a") if log_path else None
    if logf and logf.tell() > 0:
        with open(log_path, "rb") as f:
            f.seek(-1, os.SEEK_END)
            if f.read(1) != b"\n":
                logf.write("\n")  # a record cut short by a kill stays on its own line

    def record(rec):
        if logf:
            logf.write(json.dumps(rec) + "\n")
            logf.flush()
            os.fsync(logf.fileno())

    log(f"# sweep on {sig}")
    lines = [f"# scaled_mm dispatch table, written by quantized_linear_layer_scaled_amd.sweep",
             f"# {time.strftime('%Y-%m-%d %H:%M:%S')}; reps {args.reps}",
             f"device {sig}"]
    dump = {}
    timed = 0
    for op in args.ops.split(","):
        shapes = DEFAULT_SHAPES[op]
        if args.shapes:
            shapes = [tuple(int(v) for v in s.split("x")) for s in args.shapes.split(",")]
        for N, K in shapes:
            res, n = sweep_shape(torch, qll, op, N, K, mlist, args.reps, log, done, record)
            timed += n
            for M, (best, us, tf, top) in res.items():
                lines.append(f"{op} {N} {K} {M} {best[0]} {best[1]}  # {us:.2f} us {tf:.1f} TFLOPS")
                dump[f"{op} {N} {K} {M}"] = [[c[0], c[1], u] for u, c in top]
            torch.cuda.empty_cache()
    if logf:
        logf.close()
    text = "\n".join(lines) + "\n"
    if args.out:
        os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
        tmp = args.out + ".tmp"
        with open(tmp, "w") as f:
            f.write(text)
        os.replace(tmp, args.out)
        log(f"# wrote {args.out} ({timed} configurations measured in this run)")
    else:
        sys.stdout.write(text)
    if args.json:
        with open(args.json, "w") as f:
            json.dump(dump, f, indent=1)
    return {"timed": timed, "entries": len(lines) - 3}


if __name__ == "__main__":
    main()
