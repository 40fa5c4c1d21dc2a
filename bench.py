#!/usr/bin/env python3
"""Benchmark: complete-sketch throughput of SparseStack on one MI355X.

Step = one complete FP16-accumulate SparseStack sketch of the scale
workload (A 2^20 x 256 FP32 N(0,1), zeta = 4, d = 512 = 2n) with A already
resident in HBM: one sk_sketch_f16acc call, whose fused kernel draws the
Philox metadata in-kernel and keeps its partials in registers, followed by
the reduce kernel that writes (and so initializes) B (FP16 sketching page
§V-A: complete sketch time includes initialization, map generation and
application).

value = the bytes the complete sketch moves (A read once + the FP16
sketch written once) per step / step time, in GB/s; value_with_metadata
adds the metadata bytes (8 per row and stack block) that the metric's byte
count includes and the stored-metadata path writes and reads, which the
fused call draws in-kernel instead.  The roofline block divides the same
moved bytes by the call's time (fused kernel + reduce), measured with HIP
events on its stream.  Every addition of the FP16 sketch is an FP16
nearest-even addition, the reduce's combine of the row-chunk partials
included (the SK_COMBINE_F32 leg adds those partials in FP32).  The same run
times the comparison legs: the stored-metadata FP16 sketch (sk_meta_generate
+ the register or the LDS apply), the flat FP32 scatter (one global atomic per
contribution), the LDS and fused FP32 sketches, the page's flat FP16
design, the headline again under the FP16 page's protocol (medians over 11
repetitions and sketch seeds 1..10), the complete sketch-and-solve, the
coherence sweep (U = orth of the coherent 2^20 x 128 workload, zeta in
{1, 2, 4, 8} x d in {256, 512, 1024}: times and E_OSE), and BlockPerm-SJLT
on its own workload (A 2^21 x 512, d = 1024, M = 64, kappa = 4, s = 1)
through sk_apply_blockperm_ex (register kernel) and sk_apply_blockperm
(component kernel).  cpu_baseline times the CPU oracle on the same
workload's rows, one thread.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
    python bench.py --profile-pass   # short fixed run for rocprofv3 --pmc
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0                      # MI355X HBM3E, published
M_ROWS, N_COLS, D_ROWS, ZETA = 1 << 20, 256, 512, 4
BP_M, BP_N, BP_D, BP_BLOCKS, BP_KAPPA = 1 << 21, 512, 1024, 64, 4
SEED = 1
# The dominant call's kernels.
HEADLINE_KERNELS = ("k_stack_fused<AccF16,2,128,32,1,false,false>",
                    "k_stack_reduce<AccF16,false>")
# HBM bytes one complete fused FP16 step moves, from rocprofv3 --pmc
# FETCH_SIZE and WRITE_SIZE passes over bench.py --profile-pass (KiB per
# dispatch, averaged over the pass's three calls; FETCH_SIZE x 2.0 and
# WRITE_SIZE x 1.0, the factors a 1 GiB device copy reads on the same
# counters: 524,305 KiB fetched and 1,048,576 KiB written per GiB).  Valid for
# the kernels named here only (the summary under profiles/ gives the commands).
TRAFFIC = {"kernels": HEADLINE_KERNELS,
           "fetch_kib": [524683, 32801],     # fused kernel (A once), reduce (partials)
           "write_kib": [65536, 256],        # fused kernel (partials), reduce (sketch)
           "fetch_scale": 2.0, "write_scale": 1.0}


def sparsestack_bytes(m, n, d, zeta, out_elem):
    """A read once (4mn) + metadata row_idx/val (8 m zeta) + sketch (d n)."""
    return 4 * m * n + 8 * m * zeta + out_elem * d * n


def fused_bytes(m, n, d, out_elem):
    """What the fused path must move: A once and the sketch once."""
    return 4 * m * n + out_elem * d * n


def blockperm_bytes(m, n, d):
    return 4 * m * n + 4 * d * n


def traffic_bytes():
    """HBM bytes per complete fused step measured by the PMC counters (None
    when they were not taken on the current kernels)."""
    t = TRAFFIC
    if t is None or tuple(t["kernels"]) != HEADLINE_KERNELS:
        return None
    kib = t["fetch_scale"] * sum(t["fetch_kib"]) + t["write_scale"] * sum(t["write_kib"])
    return int(kib * 1024)


def timed(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps            # ms per call


def timed_median(fn, steps, warmup, stream, blocks=3):
    """Median over `blocks` timed regions of `steps` calls each (ms per call)."""
    return median([timed(fn, steps, warmup, stream) for _ in range(blocks)])


def timed_reps(fn, reps, warmup, stream):
    """Per-repetition times (ms) of fn, each bracketed by its own events."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for i in range(reps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]


def median(xs):
    ys = sorted(xs)
    k = len(ys) // 2
    return ys[k] if len(ys) % 2 else 0.5 * (ys[k - 1] + ys[k])


def cpu_baseline(A_host, sample_rows, emul_rows, outputs):
    """The CPU oracle on the scale workload's rows (a host copy of the device
    input), single-threaded: metadata + fp64 sketch of the first sample_rows
    rows (the timed baseline, bytes per second of the same algorithmic-byte
    count) and, separately, its RN-emulation FP16 sketch of the first
    emul_rows rows.  When the fp64 sketch covers every row, the GPU sketches
    in `outputs` (name -> host array) are checked against it (relative
    Frobenius error)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    sample_rows = min(sample_rows, A_host.shape[0])
    emul_rows = min(emul_rows, A_host.shape[0])
    A = A_host[:sample_rows]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        ri, v = oracle.meta_ref(SEED, sample_rows, D_ROWS, ZETA)
        B = oracle.sketch_f64(A, ri, v, D_ROWS, ZETA)
        t1 = time.perf_counter()
        Ae = A_host[:emul_rows]
        t2 = time.perf_counter()
        rie, ve = oracle.meta_ref(SEED, emul_rows, D_ROWS, ZETA)
        Be = oracle.sketch_f16_rn_emul(Ae, rie, ve, D_ROWS, ZETA)
        t3 = time.perf_counter()
    assert np.isfinite(B).all() and np.isfinite(Be.astype(np.float64)).all()
    sec, sec_e = t1 - t0, t3 - t2
    gbs = sparsestack_bytes(sample_rows, N_COLS, D_ROWS, ZETA, 4) / sec / 1e9
    gbs_e = sparsestack_bytes(emul_rows, N_COLS, D_ROWS, ZETA, 2) / sec_e / 1e9
    check = None
    if sample_rows == A_host.shape[0]:
        check = {name: float(oracle.rel_frob(np.asarray(x, dtype=np.float64), B))
                 for name, x in outputs.items()}
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"oracle metadata + fp64 sketch of the first {sample_rows} of {M_ROWS} "
                      f"rows (n={N_COLS}, zeta={ZETA}, d={D_ROWS}), {sec:.2f} s, 1 thread; "
                      f"host reports {os.cpu_count()} cpus, affinity "
                      f"{len(os.sched_getaffinity(0))}",
            "rn_emulation": {"value": round(gbs_e, 5), "unit": "GB/s", "seconds": round(sec_e, 2),
                             "sample": f"oracle metadata + RN-emulated FP16 sketch (flat order) "
                                       f"of the first {emul_rows} rows, 1 thread"},
            "oracle_rel_frob": check}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-sample-rows", type=int, default=M_ROWS)
    ap.add_argument("--cpu-emul-rows", type=int, default=M_ROWS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-blockperm", action="store_true")
    ap.add_argument("--no-coherence", action="store_true")
    ap.add_argument("--no-range", action="store_true")
    ap.add_argument("--profile-pass", action="store_true",
                    help="few fixed launches of the dominant kernels and a 1 GiB copy, no JSON")
    ap.add_argument("--profile-legs", default="headline",
                    help="with --profile-pass: comma list of headline, atomics, lds, narrow, "
                         "blockperm, solve")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "sharding over several GPUs is described, not implemented", file=sys.stderr)
        sys.exit(2)

    import torch

    from sparse_sketching_amd import binding as b
    from sparse_sketching_amd import inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    b.load()
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    m, n, d, zeta = M_ROWS, N_COLS, D_ROWS, ZETA
    A = inputs.gaussian_torch(m, n, seed=0)
    ri = torch.empty(m * zeta, dtype=torch.int32, device=dev)
    val = torch.empty(m * zeta, dtype=torch.float32, device=dev)
    B16 = torch.empty((d, n), dtype=torch.float16, device=dev)
    B32 = torch.empty((d, n), dtype=torch.float32, device=dev)

    ws16 = b.workspace(A, d, zeta, "f16acc")
    ws32 = b.workspace(A, d, zeta, "f32")
    wsr16 = b.workspace(A, d, zeta, "f16acc", b.SK_VARIANT_REG)
    wsr32 = b.workspace(A, d, zeta, "f32", b.SK_VARIANT_REG)
    wsf16 = b.sketch_workspace(A, d, zeta, "f16acc")
    wsf32 = b.sketch_workspace(A, d, zeta, "f32")

    def meta():
        b.sk_meta_generate(SEED, 0, m, d, zeta, ri, val, sp)

    def f16(flags=0, ws=ws16):
        b.sk_apply_f16acc_ws(A, m, n, n, ri, val, zeta, B16, d, n, flags, ws, 0, sp)

    def f32(flags=0, ws=ws32):
        b.sk_apply_f32_ws(A, m, n, n, ri, val, zeta, B32, d, n, flags, ws, 0, sp)

    def fused16(flags=0, seed=SEED):
        b.sk_sketch_f16acc(seed, 0, A, m, n, n, d, zeta, B16, n, flags, wsf16, 0, sp)

    def fused32(flags=0, seed=SEED):
        b.sk_sketch_f32(seed, 0, A, m, n, n, d, zeta, B32, n, flags, wsf32, 0, sp)

    if args.profile_pass:
        legs = set(args.profile_legs.split(","))
        done = []
        if "headline" in legs:
            for _ in range(3):
                fused16()
            for _ in range(3):
                fused32()
            meta()
            for _ in range(3):
                f16(b.SK_VARIANT_LDS)
            for _ in range(3):
                f16(b.SK_VARIANT_REG, wsr16)
            src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)                          # 1 GiB read + 1 GiB write
            del src, dst
            done.append("3 x fused f16 sketch, 3 x fused f32 sketch, 3 x f16 LDS apply + "
                        "reduce, 3 x f16 register apply + reduce, 3 x 1 GiB copy")
        if "atomics" in legs:
            meta()
            for _ in range(2):
                f32(b.SK_VARIANT_FLAT, None)
            for _ in range(2):
                f16(b.SK_VARIANT_FLAT, None)
            for _ in range(2):
                f16(b.SK_VARIANT_LDS, None)
            for _ in range(2):
                f32(b.SK_VARIANT_LDS, None)
            done.append("2 x flat f32, 2 x flat f16, 2 x LDS f16 / f32 apply with the atomic "
                        "flush")
        if "lds" in legs:
            meta()
            for _ in range(3):
                f16(b.SK_VARIANT_LDS)
            for _ in range(3):
                f32(b.SK_VARIANT_LDS)
            done.append("3 x LDS f16 apply + reduce, 3 x LDS f32 apply + reduce")
        if "narrow" in legs:
            mc, nc = m, 128
            U = inputs.gaussian_torch(mc, nc, seed=2)
            for zc, dc in ((8, 1024), (4, 512)):
                Bc = torch.empty((dc, nc), dtype=torch.float16, device=dev)
                wsc = b.sketch_workspace(U, dc, zc, "f16acc")
                for _ in range(2):
                    b.sk_sketch_f16acc(SEED, 0, U, mc, nc, nc, dc, zc, Bc, nc, 0, wsc, 0, sp)
                del Bc, wsc
            del U
            g4 = torch.Generator(device=dev).manual_seed(0)
            Ac = torch.randn((4194304, 64), device=dev, generator=g4)
            Bc = torch.empty((128, 64), dtype=torch.float16, device=dev)
            wsc = b.sketch_workspace(Ac, 128, 4, "f16acc")
            for _ in range(2):
                b.sk_sketch_f16acc(SEED, 0, Ac, 4194304, 64, 64, 128, 4, Bc, 64, 0, wsc, 0, sp)
            B32 = torch.empty((128, 64), dtype=torch.float32, device=dev)
            ws32c = b.sketch_workspace(Ac, 128, 4, "f32")
            for _ in range(2):
                b.sk_sketch_f32(SEED, 0, Ac, 4194304, 64, 64, 128, 4, B32, 64, 0, ws32c, 0, sp)
            del Ac, Bc, wsc, B32, ws32c
            R2 = torch.zeros((m, 2), dtype=torch.float32, device=dev)
            Bc = torch.empty((d, 2), dtype=torch.float16, device=dev)
            wsc = b.sketch_workspace(R2, d, zeta, "f16acc")
            for _ in range(2):
                b.sk_sketch_f16acc(SEED, 0, R2, m, 2, 2, d, zeta, Bc, 2, 0, wsc, 0, sp)
            del R2, Bc, wsc
            done.append("2 x fused f16 sketch of 2^20 x 128 at (zeta, d) = (8, 1024) and "
                        "(4, 512), of 4,194,304 x 64 at (4, 128) (and 2 x fused f32), and of "
                        "2^20 x 2 at (4, 512)")
        if "solve" in legs:
            gq = torch.Generator(device=dev).manual_seed(0)
            SA = torch.randn((2 * n, n), device=dev, generator=gq)
            Sb = torch.randn(2 * n, device=dev, generator=gq)
            xq = torch.empty(n, dtype=torch.float32, device=dev)
            wsq = torch.empty(b.sk_lstsq_workspace_size(2 * n, n), dtype=torch.uint8, device=dev)
            for _ in range(3):
                b.sk_lstsq_qr_f32(SA, 2 * n, n, n, Sb, xq, wsq, 0, sp)
            del SA, Sb, xq, wsq
            done.append(f"3 x FP32 QR solve of a {2 * n} x {n} system (d = 2n)")
        if "headline" in legs or "blockperm" in legs:
            del A, ri, val, ws16, ws32, wsr16, wsr32, wsf16, wsf32
            torch.cuda.empty_cache()
            Abp = inputs.gaussian_torch(BP_M, BP_N, seed=0)
            Y = torch.empty((BP_D, BP_N), dtype=torch.float32, device=dev)
            wsbp = torch.empty(b.sk_blockperm_workspace_size(BP_M, BP_N, BP_D, BP_BLOCKS,
                                                             BP_KAPPA, 1, b.SK_WIRING_SHIFT),
                               dtype=torch.uint8, device=dev)
            for _ in range(3):
                b.sk_apply_blockperm_ex(Abp, BP_M, BP_N, BP_N, BP_D, BP_BLOCKS, BP_KAPPA, 1,
                                        b.SK_WIRING_SHIFT, SEED, Y, BP_N, 0, wsbp, wsbp.numel(),
                                        sp)
            for _ in range(3):
                b.sk_apply_blockperm(Abp, BP_M, BP_N, BP_N, BP_D, BP_BLOCKS, BP_KAPPA, 1, SEED, Y,
                                     BP_N, 0, sp)
            ws2 = torch.empty(b.sk_blockperm_workspace_size(BP_M, BP_N, BP_D, BP_BLOCKS,
                                                            BP_KAPPA, 2, b.SK_WIRING_SHIFT),
                              dtype=torch.uint8, device=dev)
            for _ in range(3):
                b.sk_apply_blockperm_ex(Abp, BP_M, BP_N, BP_N, BP_D, BP_BLOCKS, BP_KAPPA, 2,
                                        b.SK_WIRING_SHIFT, SEED, Y, BP_N, 0, ws2, ws2.numel(), sp)
            done.append("3 x BlockPerm register kernel + reduce, 3 x BlockPerm without workspace, "
                        "3 x BlockPerm register kernel + reduce at s = 2")
        torch.cuda.synchronize()
        print("profile pass done: " + "; ".join(done), flush=True)
        return

    K, W = args.steps, args.warmup
    bytes16 = sparsestack_bytes(m, n, d, zeta, 2)
    bytes32 = sparsestack_bytes(m, n, d, zeta, 4)

    # bring clocks and caches to a steady state before any timed region
    for _ in range(max(20, W)):
        fused16()
        meta()
        f16(b.SK_VARIANT_REG, wsr16)
        f16(b.SK_VARIANT_LDS)
        f32(b.SK_VARIANT_FLAT, None)
    torch.cuda.synchronize()

    # headline step: complete FP16-accumulate sketch in one fused call
    ms16 = timed(fused16, K, W, stream)
    print(f"[bench] f16acc complete sketch (fused) {ms16:.4f} ms", file=sys.stderr, flush=True)
    out16 = B16.cpu().numpy()
    ms16_c32 = timed(lambda: fused16(b.SK_COMBINE_F32), K, W, stream)
    out16_c32 = B16.cpu().numpy()
    ms32_fused = timed(fused32, K, W, stream)
    out32 = B32.cpu().numpy()
    # the stored-metadata sketch through sk_meta_generate + sk_apply_*: the
    # register apply (the fused kernel reading the metadata; the default
    # with a workspace) and the LDS apply, both with the store-and-reduce
    # flush that also initializes B
    ms16_meta_reg = timed(lambda: (meta(), f16(b.SK_VARIANT_REG, wsr16)), K, W, stream)
    out16_reg = B16.cpu().numpy()
    ms16_meta = timed(lambda: (meta(), f16(b.SK_VARIANT_LDS)), K, W, stream)
    print(f"[bench] f32 fused {ms32_fused:.4f} ms, f16acc meta+register apply "
          f"{ms16_meta_reg:.4f} ms, meta+LDS apply {ms16_meta:.4f} ms",
          file=sys.stderr, flush=True)
    ms16_atomic = timed(lambda: (meta(), f16(b.SK_VARIANT_LDS, None)), K, W, stream)
    ms32_flat = timed(lambda: (meta(), f32(b.SK_VARIANT_FLAT, None)), K, W, stream)
    ms32_lds = timed(lambda: (meta(), f32(b.SK_VARIANT_LDS)), K, W, stream)
    ms32_reg = timed(lambda: (meta(), f32(b.SK_VARIANT_REG, wsr32)), K, W, stream)
    ms16_flat = timed(lambda: (meta(), f16(b.SK_VARIANT_FLAT, None)), max(1, K // 4), 1, stream)
    print(f"[bench] f16 lds+atomic flush {ms16_atomic:.4f} ms, f32 flat {ms32_flat:.4f} ms, "
          f"f32 lds {ms32_lds:.4f} ms, f32 register {ms32_reg:.4f} ms, f16 flat "
          f"{ms16_flat:.4f} ms", file=sys.stderr, flush=True)
    # the apply alone (apply kernel + its reduce), and the metadata kernel alone
    ms_kernel_reg = timed(lambda: f16(b.SK_ACCUMULATE | b.SK_VARIANT_REG, wsr16), K, W, stream)
    ms_kernel = timed(lambda: f16(b.SK_ACCUMULATE | b.SK_VARIANT_LDS), K, W, stream)
    ms_kernel_atomic = timed(lambda: f16(b.SK_ACCUMULATE | b.SK_VARIANT_LDS, None), K, W, stream)
    ms_meta = timed(meta, K, W, stream)
    # device copy bandwidth for context
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    ms_copy = timed(lambda: dst.copy_(src), K, 2, stream)
    copy_gbs = 2 * src.numel() * 4 / ms_copy / 1e6
    del src, dst
    print(f"[bench] register apply+reduce {ms_kernel_reg:.4f} ms, LDS apply+reduce "
          f"{ms_kernel:.4f} ms, LDS apply(atomic flush) {ms_kernel_atomic:.4f} ms, "
          f"meta {ms_meta:.4f} ms, copy {copy_gbs:.0f} GB/s", file=sys.stderr, flush=True)

    # the FP16 sketching page's protocol (§V-A): per sketch seed 1..10, 3
    # warm-ups and 11 timed repetitions, the median per seed, then the
    # median over seeds
    proto = {}
    for name, fn in (("fp16", fused16), ("fp32", fused32)):
        per_seed = [median(timed_reps(lambda: fn(0, sd), 11, 3, stream)) for sd in range(1, 11)]
        proto[name] = median(per_seed)
    proto_out = {"protocol": "median over sketch seeds 1..10 of the median of 11 repetitions "
                             "(3 warm-ups), each repetition one complete sketch call",
                 "fp16_ms": round(proto["fp16"], 5), "fp32_ms": round(proto["fp32"], 5),
                 "fp16_GBps": round(bytes16 / proto["fp16"] / 1e6, 2),
                 "fp16_hbm_frac": round(bytes16 / proto["fp16"] / 1e6 / HBM_PEAK_GBS, 4),
                 "speedup_fp16_vs_fp32": round(proto["fp32"] / proto["fp16"], 3)}
    print(f"[bench] pages' protocol: fp16 {proto['fp16']:.4f} ms, fp32 {proto['fp32']:.4f} ms",
          file=sys.stderr, flush=True)

    # downstream: complete sketch-and-solve (shared-map SA and Sb, then the
    # library's FP32 QR, projection and triangular solve, sk_lstsq_qr_f32)
    # with FP16 and FP32 sketches, d = 2n
    from sparse_sketching_amd import solve
    g = torch.Generator(device=dev).manual_seed(5)
    x0 = torch.randn(n, device=dev, generator=g)
    rhs = A @ x0 + 0.1 * torch.randn(m, device=dev, generator=g)
    ls = {}
    for prec in ("f16acc", "f32"):
        ls[prec] = timed(lambda: solve.solve_sketched(*solve.sketch_pair(A, rhs, d, zeta, SEED, prec)),
                         K, W, stream)
    res = {p: solve.sketch_and_solve(A, rhs, d, zeta, SEED, p)[1] for p in ("f16acc", "f32")}
    res["f16acc_combine_f32"] = solve.sketch_and_solve(A, rhs, d, zeta, SEED, "f16acc",
                                                       combine="f32")[1]
    SA_ls, Sb_ls = solve.sketch_pair(A, rhs, d, zeta, SEED, "f32")
    ms_qr = timed(lambda: solve.solve_sketched(SA_ls, Sb_ls), K, W, stream)
    ls_out = {"workload": f"least squares A 2^20 x {n}, b = A x0 + 0.1 N(0,1), d = {d}, zeta = {zeta}",
              "fp16_ms": round(ls["f16acc"], 4), "fp32_ms": round(ls["f32"], 4),
              "speedup": round(ls["f32"] / ls["f16acc"], 3),
              "fp16_residual": round(res["f16acc"], 6), "fp32_residual": round(res["f32"], 6),
              "fp16_combine_f32_residual": round(res["f16acc_combine_f32"], 6),
              "qr_solve_ms": round(ms_qr, 4)}
    print(f"[bench] sketch-and-solve fp16 {ls['f16acc']:.4f} ms fp32 {ls['f32']:.4f} ms "
          f"(QR solve {ms_qr:.4f} ms), residuals {res['f16acc']:.6f} / {res['f32']:.6f} "
          f"(fp16 with fp32 combine {res['f16acc_combine_f32']:.6f})", file=sys.stderr, flush=True)
    del rhs, x0, SA_ls, Sb_ls

    # coherence sweep: U = orth(A) of the coherent 2^20 x 128 workload,
    # zeta in {1, 2, 4, 8} x d in {256, 512, 1024}; complete fused sketch
    # times and the sketches' subspace distortion E_OSE = ||(SU)^T SU - I||_2
    c3 = []
    if not args.no_coherence:
        nc = 128
        U = inputs.orth_torch(inputs.coherent_torch(m, nc, seed=0))
        for zc in (1, 2, 4, 8):
            for dc in (256, 512, 1024):
                row = {"zeta": zc, "d": dc}
                for prec, dt in (("fp16", torch.float16), ("fp32", torch.float32)):
                    Bc = torch.empty((dc, nc), dtype=dt, device=dev)
                    wsc = b.sketch_workspace(U, dc, zc, "f16acc" if prec == "fp16" else "f32")
                    call = b.sk_sketch_f16acc if prec == "fp16" else b.sk_sketch_f32
                    ms = timed(lambda: call(SEED, 0, U, m, nc, nc, dc, zc, Bc, nc, 0, wsc, 0, sp),
                               K, W, stream)
                    row[f"{prec}_ms"] = round(ms, 5)
                    row[f"{prec}_GBps"] = round(
                        sparsestack_bytes(m, nc, dc, zc, 2 if prec == "fp16" else 4) / ms / 1e6, 1)
                    row[f"{prec}_ose"] = round(solve.ose_error(Bc.float()), 5)
                    row[f"{prec}_sv_ratio"] = round(solve.sv_ratio(Bc.float()), 5)
                    del Bc, wsc
                c3.append(row)
        del U
        print("[bench] coherence sweep (zeta, d, fp16 ms, fp16 E_OSE, fp32 E_OSE): " +
              ", ".join(f"({r['zeta']},{r['d']},{r['fp16_ms']:.4f},{r['fp16_ose']:.4f},"
                        f"{r['fp32_ose']:.4f})" for r in c3), file=sys.stderr, flush=True)

    A_host = None if args.no_cpu_baseline else A.cpu().numpy()

    # range configuration: A 4,194,304 x 64 of N(0,1) rows times
    # exp(2Z) row scales (drawn on the device, seeded), zeta = 4, d = 128:
    # the complete FP32 and FP16 sketches and the conversion variants of the
    # page's flat FP16 design (apply only, metadata stored); accuracy is in
    # the GPU tests
    c4 = None
    if not args.no_range:
        mc, nc, dc, zc = 4194304, 64, 128, 4
        g4 = torch.Generator(device=dev).manual_seed(0)
        Ac = torch.randn((mc, nc), device=dev, generator=g4)
        Ac *= torch.exp(2.0 * torch.randn((mc, 1), device=dev, generator=g4))
        ric = torch.empty(mc * zc, dtype=torch.int32, device=dev)
        vc = torch.empty(mc * zc, dtype=torch.float32, device=dev)
        b.sk_meta_generate(SEED, 0, mc, dc, zc, ric, vc, sp)
        Bc16 = torch.empty((dc, nc), dtype=torch.float16, device=dev)
        Bc32 = torch.empty((dc, nc), dtype=torch.float32, device=dev)
        wc16, wc32 = b.sketch_workspace(Ac, dc, zc, "f16acc"), b.sketch_workspace(Ac, dc, zc, "f32")
        t = {"fp32_fused": timed(lambda: b.sk_sketch_f32(SEED, 0, Ac, mc, nc, nc, dc, zc, Bc32, nc,
                                                         0, wc32, 0, sp), K, W, stream),
             "fp16_two_level": timed(lambda: b.sk_sketch_f16acc(SEED, 0, Ac, mc, nc, nc, dc, zc,
                                                                Bc16, nc, 0, wc16, 0, sp),
                                     K, W, stream)}
        for name, fmt, conv in (("fp16_rn_flat", b.SK_FORMAT_F16, b.SK_CONVERT_RN),
                                ("fp16_sr_flat", b.SK_FORMAT_F16, b.SK_CONVERT_SR),
                                ("bf16_rn_flat", b.SK_FORMAT_BF16, b.SK_CONVERT_RN)):
            t[name] = timed(lambda: b.sk_apply_lowp(Ac, mc, nc, nc, ric, vc, zc, Bc16, dc, nc,
                                                    fmt, conv, 1, 0, 0, None, 0, sp),
                            max(1, K // 4), 1, stream)
        nlw = b.sk_apply_workspace_size(b.SK_PRECISION_LOWP, mc, nc, dc, zc, b.SK_VARIANT_REG)
        wlw = torch.empty(nlw, dtype=torch.uint8, device=dev)
        for name, fmt, conv in (("fp16_rn_two_level_apply", b.SK_FORMAT_F16, b.SK_CONVERT_RN),
                                ("fp16_sr_two_level_apply", b.SK_FORMAT_F16, b.SK_CONVERT_SR),
                                ("bf16_rn_two_level_apply", b.SK_FORMAT_BF16, b.SK_CONVERT_RN)):
            t[name] = timed(lambda: b.sk_apply_lowp(Ac, mc, nc, nc, ric, vc, zc, Bc16, dc, nc,
                                                    fmt, conv, 1, 0, b.SK_VARIANT_REG, wlw, nlw,
                                                    sp), max(1, K // 4), 1, stream)
        del wlw
        c4 = {"workload": "A 4,194,304 x 64 N(0,1) x exp(2Z) row scales, zeta = 4, d = 128",
              **{k + "_ms": round(v, 4) for k, v in t.items()},
              "fp16_two_level_GBps": round(sparsestack_bytes(mc, nc, dc, zc, 2)
                                           / t["fp16_two_level"] / 1e6, 1),
              "note": "fp32/fp16 two-level are complete sketches (metadata drawn in the call); "
                      "the flat and *_two_level_apply variants are the apply alone (stored "
                      "metadata; the two-level applies convert each contribution per hit)"}
        print("[bench] range config: " + ", ".join(f"{k} {v:.4f} ms" for k, v in t.items()),
              file=sys.stderr, flush=True)
        del Ac, ric, vc, Bc16, Bc32, wc16, wc32

    bp = None
    if not args.no_blockperm:
        del A, ri, val, ws16, ws32, wsr16, wsr32, wsf16, wsf32
        torch.cuda.empty_cache()
        Abp = inputs.gaussian_torch(BP_M, BP_N, seed=0)
        Y = torch.empty((BP_D, BP_N), dtype=torch.float32, device=dev)
        nbp = b.sk_blockperm_workspace_size(BP_M, BP_N, BP_D, BP_BLOCKS, BP_KAPPA, 1,
                                            b.SK_WIRING_SHIFT)
        wsbp = torch.empty(nbp, dtype=torch.uint8, device=dev)
        # (each leg: the median of three timed regions of K calls, steadier
        # than one region right after the 4 GiB input is drawn)
        ms_bp = timed_median(lambda: b.sk_apply_blockperm_ex(
            Abp, BP_M, BP_N, BP_N, BP_D, BP_BLOCKS, BP_KAPPA, 1, b.SK_WIRING_SHIFT, SEED, Y, BP_N,
            0, wsbp, nbp, sp), K, W, stream)
        ms_bpc = timed_median(lambda: b.sk_apply_blockperm(Abp, BP_M, BP_N, BP_N, BP_D, BP_BLOCKS,
                                                    BP_KAPPA, 1, SEED, Y, BP_N, 0, sp), K, W,
                       stream)
        # the general options on the same workload: affine wiring, s = 2
        var = {}
        for name, s_rows, wiring in (("affine", 1, b.SK_WIRING_AFFINE),
                                     ("s2", 2, b.SK_WIRING_SHIFT)):
            nv = b.sk_blockperm_workspace_size(BP_M, BP_N, BP_D, BP_BLOCKS, BP_KAPPA, s_rows,
                                               wiring)
            wsv = torch.empty(nv, dtype=torch.uint8, device=dev)
            var[name] = timed_median(lambda: b.sk_apply_blockperm_ex(
                Abp, BP_M, BP_N, BP_N, BP_D, BP_BLOCKS, BP_KAPPA, s_rows, wiring, SEED, Y, BP_N,
                0, wsv, nv, sp), K, W, stream)
            del wsv
        gbs_bp = blockperm_bytes(BP_M, BP_N, BP_D) / ms_bp / 1e6
        bp = {"workload": f"BlockPerm-SJLT m=2^21 n={BP_N} d={BP_D} M={BP_BLOCKS} "
                          f"kappa={BP_KAPPA} s=1", "path": "sk_apply_blockperm_ex (register kernel)",
              "ms": round(ms_bp, 4), "GBps": round(gbs_bp, 1),
              "hbm_frac": round(gbs_bp / HBM_PEAK_GBS, 4),
              "component_kernel_ms": round(ms_bpc, 4),
              "affine_wiring_ms": round(var["affine"], 4), "s2_ms": round(var["s2"], 4)}
        print(f"[bench] blockperm {ms_bp:.4f} ms {gbs_bp:.0f} GB/s (component kernel "
              f"{ms_bpc:.4f} ms, affine {var['affine']:.4f} ms, s=2 {var['s2']:.4f} ms)",
              file=sys.stderr, flush=True)
        del Abp, Y, wsbp

    fbytes16 = fused_bytes(m, n, d, 2)
    moved_gbs = fbytes16 / ms16 / 1e6
    gbs16 = bytes16 / ms16 / 1e6
    out = {
        "metric": "complete-sketch SA GB/s and % HBM roofline, zeta=4, d=2n, FP16-acc vs FP32",
        "value": round(moved_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms16, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic N(0,1) A drawn on device with a seeded generator",
        "config": {"workload": f"SparseStack m=2^20 n={n} zeta={zeta} d={d} (d=2n), dense N(0,1)",
                   "m": m, "n": n, "d": d, "zeta": zeta, "seed": SEED,
                   "precision": "FP32 products, each rounded to FP16 (nearest-even), every "
                                "addition an FP16 nearest-even addition (row-chunk partials in "
                                "registers, then combined by FP16 additions in a fixed order)",
                   "path": "sk_sketch_f16acc (Philox metadata drawn in-kernel)",
                   "value_bytes": fbytes16,
                   "value_bytes_are": "A read once + FP16 sketch written once (what the call "
                                      "moves)"},
        "hbm_frac": round(moved_gbs / HBM_PEAK_GBS, 4),
        "value_with_metadata": {"GBps": round(gbs16, 2), "hbm_frac": round(gbs16 / HBM_PEAK_GBS, 4),
                                "bytes": bytes16,
                                "bytes_are": "A + metadata (8 bytes per row and stack block) + "
                                             "sketch, the metric's count; the fused call draws "
                                             "the metadata instead of moving it"},
        "fp16_combine_f32_ms": round(ms16_c32, 5),
        "fp32_flat_ms": round(ms32_flat, 5),
        "fp32_flat_GBps": round(bytes32 / ms32_flat / 1e6, 2),
        "fp32_lds_ms": round(ms32_lds, 5),
        "fp32_fused_ms": round(ms32_fused, 5),
        "fp32_fused_GBps": round(fused_bytes(m, n, d, 4) / ms32_fused / 1e6, 2),
        "fp16_meta_reg_ms": round(ms16_meta_reg, 5),
        "fp16_meta_reg_GBps": round(bytes16 / ms16_meta_reg / 1e6, 2),
        "fp16_meta_reg_hbm_frac": round(bytes16 / ms16_meta_reg / 1e6 / HBM_PEAK_GBS, 4),
        "fp16_meta_lds_ms": round(ms16_meta, 5),
        "fp16_meta_lds_GBps": round(bytes16 / ms16_meta / 1e6, 2),
        "fp32_meta_reg_ms": round(ms32_reg, 5),
        "fp16_flat_ms": round(ms16_flat, 5),
        "fp16_lds_atomic_flush_ms": round(ms16_atomic, 5),
        "speedup_vs_fp32_flat": round(ms32_flat / ms16, 3),
        "speedup_vs_fp32_lds": round(ms32_lds / ms16, 3),
        "speedup_vs_fp32_fused": round(ms32_fused / ms16, 3),
        "fp16_reg_apply_ms": round(ms_kernel_reg, 5),
        "fp16_lds_apply_ms": round(ms_kernel, 5),
        "meta_ms": round(ms_meta, 5),
        "copy_GBps": round(copy_gbs, 1),
        "pages_protocol": proto_out,
        "blockperm": bp,
        "sketch_and_solve": ls_out,
        "coherence_sweep": {"workload": "U = orth(coherent 2^20 x 128), seed 1", "rows": c3},
        "range_config": c4,
        "roofline": {"bound": "hbm", "achieved": round(moved_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(moved_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_bytes(),
                     "kernel": " + ".join(HEADLINE_KERNELS),
                     "call_ms": round(ms16, 5), "algorithmic_bytes": fbytes16,
                     "apply_atomic_flush_ms": round(ms_kernel_atomic, 5)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(
            A_host, args.cpu_sample_rows, args.cpu_emul_rows,
            {"fp16_fused": out16, "fp16_fused_combine_f32": out16_c32, "fp32_fused": out32,
             "fp16_meta_register": out16_reg})
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
