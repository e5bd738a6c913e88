"""Benchmark of the W12 hot path on one MI355X.

Step = one exact verification pass over one 27B-class dense decoder layer (hidden 5120):
the four W12 GEMMs qkv [7168x5120], o_proj [5120x5120], gate_up [34816x5120] and
down [5120x17408] against X [16 rows] (a 16-position drafted block).  Inputs are synthetic
(seeded Gaussian x per-channel lognormal weights, see w12_synth) and resident in HBM before
the timed region.  Three encoded copies of the layer (1.49 GB of W12) are rotated so the
256 MB Infinity Cache cannot serve repeated weight reads.

value = weight-GB/s = BF16-equivalent weight bytes (2*N*K per matrix) per second over the
timed steps.  Extra legs (same JSON line): the tree-verify M sweep, per-launch roofline of
the dominant kernel (gate_up), load-time encode/verify throughput, and the CPU oracle
timed on the host cores.

    python bench.py [--gpus 1] [--steps 50] [--warmup 50]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import lossless_bit_weight_encode_amd as w12  # noqa: E402
import w12_synth as S  # noqa: E402

HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def alg_bytes(n, k, m, e):
    """Algorithmic bytes of one GEMM: records, bases, pointers, escapes, X and Y."""
    return 1.5 * n * k + n + 4 * (n + 1) + 4 * e + 2 * m * k + 4 * m * n


BF16_PEAK_TFLOPS = 2500.0


def byte_floor_us(n, k, m, e):
    """The pages' floor for a kernel: the larger of its FLOP time at 60% of the dense BF16 peak
    and its byte time at 90% of the HBM peak (SpecPilot summary page, the ceiling bullet
    attributed to section 3.1)."""
    return max(2.0 * m * n * k / (0.6 * BF16_PEAK_TFLOPS * 1e6), alg_bytes(n, k, m, e) / (0.9 * HBM_PEAK_GBPS * 1e3))


def dev_bits(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def clone_tensor(t: w12.W12Tensor) -> w12.W12Tensor:
    return w12.W12Tensor(t.n, t.k, t.base.clone(), t.hi.clone(), t.lo.clone(), t.esc_ptr.clone(), t.esc.clone())


def timed(fn, iters, stream):
    """Average milliseconds per call of fn over iters calls, HIP events on `stream`."""
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(iters):
        fn(i)
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / iters


def timed_blocks(fn, iters, stream, blocks=5):
    """Average milliseconds per call over iters calls (one synchronisation on each side), plus the
    per-call means of `blocks` consecutive blocks of calls, from events recorded between blocks."""
    nb = max(1, min(blocks, iters))
    bounds = [round(i * iters / nb) for i in range(nb + 1)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for b in range(nb):
        for i in range(bounds[b], bounds[b + 1]):
            fn(i)
        ev[b + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[b].elapsed_time(ev[b + 1]) / (bounds[b + 1] - bounds[b]) for b in range(nb)]
    return ev[0].elapsed_time(ev[nb]) / iters, per


READ_SIZES = {"o_proj_39MB": 39_340_032, "down_134MB": 133_693_440, "gate_up_267MB": 267_386_880,
              "1GiB": 1 << 30}
# the read-probe shape the default run reports (the fastest of the --read-probe sweep)
READ_BEST = (8, 1)   # (loads in flight per lane, 256-thread work-groups per CU)


def read_ceiling(dev, stream, variants, sizes=READ_SIZES, reps=20):
    """Plain streaming reads (w12_read_probe) of each size, rotating over a 2 GiB buffer so the
    256 MB Infinity Cache cannot serve a repeat; per-launch HIP events on the launch stream.
    Returns {size: {"U<u>_G<g>": {"us": median, "GBps": bytes / median}}}."""
    buf = torch.ones(2 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(16 * 1024, dtype=torch.int32, device=dev)
    out = {}
    for name, nb in sizes.items():
        nb = nb // 256 * 256
        slots = max(1, (buf.numel() - nb) // nb + 1)
        res = {}
        for u, g in variants:
            for i in range(3):
                w12.read_probe(buf, nb, u, g, sink, offset=(i % slots) * nb, stream=stream)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            torch.cuda.synchronize()
            for i in range(reps):
                ev[i][0].record(stream)
                w12.read_probe(buf, nb, u, g, sink, offset=((i + 3) % slots) * nb, stream=stream)
                ev[i][1].record(stream)
            torch.cuda.synchronize()
            us = float(np.median([a.elapsed_time(b) * 1e3 for a, b in ev]))
            res[f"U{u}_G{g}"] = {"us": round(us, 2), "GBps": round(nb / us / 1e3, 1)}
        out[name] = res
    del buf, sink
    return out


def ci95(samples):
    """Median and the half-width of a t-based 95% confidence interval of the mean."""
    import statistics
    n = len(samples)
    med = statistics.median(samples)
    if n < 2:
        return med, None
    t = {2: 12.71, 3: 4.30, 4: 3.18, 5: 2.78, 6: 2.57, 7: 2.45, 8: 2.36, 9: 2.31, 10: 2.26}.get(n, 2.0)
    return med, t * statistics.stdev(samples) / n ** 0.5


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-legs", action="store_true",
                    help="only the oracle on the host cores, for the tiny case, the tree-verify M sweep, the batched "
                         "M and heavy-tail matrices, and the full model streamed one layer at a time (no GPU; "
                         "several minutes); prints one JSON line")
    ap.add_argument("--summarize-cpu-legs", nargs="+", metavar="JSON",
                    help="turn the JSON lines of --cpu-legs runs (the other legs, and the full model in parts) into "
                         "profiles/cpu_oracle_legs.md")
    ap.add_argument("--cpu-layers", nargs=2, type=int, metavar=("FIRST", "END"),
                    help="with --cpu-legs: only the full-model leg, over layers FIRST..END-1 (so the whole model can "
                         "be timed in parts whose totals add up)")
    ap.add_argument("--no-full-model", action="store_true", help="skip the 64-layer weight stream")
    ap.add_argument("--model-layers", type=int, default=S.FULL_MODEL_LAYERS)
    ap.add_argument("--only-layer", action="store_true", help="time only the layer steps (for profiling)")
    ap.add_argument("--only-group", action="store_true",
                    help="time only the grouped layer steps, one w12_gemm_group launch each (for profiling)")
    ap.add_argument("--summarize-group-counters", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "ALG_BYTES"),
                    help="turn FETCH_SIZE / WRITE_SIZE rocprofv3 runs of --only-group --copy-probe into the grouped "
                         "launch's traffic summary under profiles/")
    ap.add_argument("--summarize-group-trace", nargs=3, metavar=("STATS_CSV", "TRACE_CSV", "COMMAND"),
                    help="turn a rocprofv3 --kernel-trace --stats run of --only-group into the grouped-launch "
                         "kernel-time summary under profiles/")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after the layer steps, run one torch elementwise kernel that reads and writes exactly "
                         "256 MiB (the plain kernel of known size against which HBM byte counters are scaled)")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("STATS_CSV", "TRACE_CSV", "COMMAND"),
                    help="turn a rocprofv3 --kernel-trace --stats run of --only-layer into the kernel-time "
                         "summary under profiles/ (COMMAND is the profiled command line, recorded verbatim)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE run, WRITE_SIZE run of "
                         "--only-layer --copy-probe) into the per-launch traffic summary under profiles/")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="only the batched-verify GEMMs (gate_up and down at M=256 and 512, three launches "
                         "each on rotating copies), for MFMA counters; prints their event times as JSON")
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("PMC_CSV", "PROBE_JSON"),
                    help="turn a rocprofv3 --pmc run of --mfma-probe (SQ_VALU_MFMA_BUSY_CYCLES, "
                         "SQ_INSTS_VALU_MFMA_MOPS_BF16, GRBM_GUI_ACTIVE) and the probe's own output into the "
                         "MFMA summary under profiles/")
    ap.add_argument("--summarize-wide-lds", nargs=2, metavar=("PMC_CSV", "PROBE_JSON"),
                    help="turn a rocprofv3 --pmc run of --mfma-probe (SQ_INSTS_LDS, SQ_LDS_BANK_CONFLICT, "
                         "SQ_LDS_IDX_ACTIVE, SQ_WAIT_INST_LDS) and the probe's own output into the wide-tile LDS "
                         "summary under profiles/")
    ap.add_argument("--valu-probe", action="store_true",
                    help="only gate_up at M=1, 8, 16, 32, 48 and 64 (three launches each on rotating copies), for "
                         "the VALU instruction and stall counters; prints their event times as JSON")
    ap.add_argument("--summarize-valu", nargs=2, metavar=("PMC_CSV", "PROBE_JSON"),
                    help="turn a rocprofv3 --pmc run of --valu-probe (SQ_WAVES, SQ_INSTS_VALU, SQ_INSTS_MFMA, "
                         "SQ_INSTS_SALU, SQ_INSTS_LDS, GRBM_GUI_ACTIVE) and the probe's own output into the "
                         "VALU-budget summary under profiles/")
    ap.add_argument("--summarize-stalls", nargs=2, metavar=("PMC_CSV", "PROBE_JSON"),
                    help="turn a rocprofv3 --pmc run of --valu-probe (SQ_WAVES, SQ_WAIT_ANY, SQ_WAIT_INST_ANY, "
                         "SQ_ACTIVE_INST_ANY, SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE, SQ_BUSY_CYCLES, "
                         "GRBM_GUI_ACTIVE) and the probe's own output into the wave-stall summary under profiles/")
    ap.add_argument("--summarize-encode-lds", nargs=2, metavar=("PMC_CSV", "FETCH_CSV"),
                    help="turn two rocprofv3 --pmc runs of --valu-probe (LDS counters; FETCH_SIZE) into the "
                         "encode-kernel LDS summary under profiles/")
    ap.add_argument("--read-probe", action="store_true",
                    help="sweep the plain streaming-read kernel (loads in flight x work-groups per CU) and exit")
    ap.add_argument("--probe-reps", type=int, default=3,
                    help="launches per case of --valu-probe (the counter summaries expect 3)")
    ap.add_argument("--timeline", action="store_true",
                    help="with libw12_timeline.so (build --timeline): per-work-group timelines of the gate_up and "
                         "down launches at M = 16 (and M = 1); writes the phase summary under profiles/")
    ap.add_argument("--sweep-probe", action="store_true",
                    help="gate_up and down at M = 1..64 (the default paths), --probe-reps launches each, for a "
                         "kernel trace (--summarize-sweep-trace)")
    ap.add_argument("--read-trace-probe", action="store_true",
                    help="the plain streaming read at the matrices' sizes and 1 GiB (best launch shape), for a "
                         "kernel trace (--summarize-read-trace)")
    ap.add_argument("--summarize-read-trace", nargs=3, metavar=("TRACE_CSV", "PROBE_JSON", "COMMAND"),
                    help="turn a rocprofv3 --kernel-trace run of --read-trace-probe into the read-ceiling summary "
                         "under profiles/")
    ap.add_argument("--r13-probe", action="store_true",
                    help="gate_up and down at M = 1..8, once through the wavefront GEMV (W12_GEMV_MAX_M=8) and once "
                         "through the 16-row MFMA tiles (W12_GEMV_MAX_M=0), --probe-reps launches each; prints the "
                         "event times as JSON")
    ap.add_argument("--summarize-r13-trace", nargs=3, metavar=("TRACE_CSV", "PROBE_JSON", "COMMAND"),
                    help="turn a rocprofv3 --kernel-trace run of --r13-probe into the GEMV-vs-MFMA summary under "
                         "profiles/")
    ap.add_argument("--encode-probe", action="store_true",
                    help="encode the layer's four matrices and the two heavy-tail matrices with each emit form "
                         "(auto, blocks, rows), --probe-reps encodes each, for a kernel trace "
                         "(--summarize-encode-trace)")
    ap.add_argument("--summarize-encode-trace", nargs=3, metavar=("TRACE_CSV", "PROBE_JSON", "COMMAND"),
                    help="turn a rocprofv3 --kernel-trace run of --encode-probe into the encode kernel-time "
                         "summary under profiles/")
    ap.add_argument("--summarize-sweep-trace", nargs=3, metavar=("TRACE_CSV", "PROBE_JSON", "COMMAND"),
                    help="turn a rocprofv3 --kernel-trace run of --valu-probe into the per-M kernel-time summary "
                         "under profiles/")
    args = ap.parse_args()
    if args.summarize_sweep_trace:
        summarize_sweep_trace(*args.summarize_sweep_trace)
        return
    if args.summarize_encode_trace:
        summarize_encode_trace(*args.summarize_encode_trace)
        return
    if args.summarize_r13_trace:
        summarize_r13_trace(*args.summarize_r13_trace)
        return
    if args.summarize_cpu_legs:
        summarize_cpu_legs(args.summarize_cpu_legs)
        return
    if args.summarize_read_trace:
        summarize_read_trace(*args.summarize_read_trace)
        return
    if args.summarize_encode_lds:
        summarize_encode_lds(*args.summarize_encode_lds)
        return
    if args.summarize_stalls:
        summarize_stalls(*args.summarize_stalls)
        return
    if args.summarize_valu:
        summarize_valu(*args.summarize_valu)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma)
        return
    if args.summarize_wide_lds:
        summarize_wide_lds(*args.summarize_wide_lds)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_group_trace:
        summarize_group_trace(*args.summarize_group_trace)
        return
    if args.summarize_group_counters:
        summarize_group_counters(*args.summarize_group_counters)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the W12 path is built and timed on a single MI355X); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    if args.cpu_legs:
        rng = tuple(args.cpu_layers) if args.cpu_layers else None
        print(json.dumps(cpu_legs(args.model_layers, rng)))
        return
    if args.timeline:
        import lossless_bit_weight_encode_amd._lib as L
        L.LIB_PATH = os.path.join(ROOT, "lossless_bit_weight_encode_amd", "libw12_timeline.so")
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.init()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    m_step = 16
    if args.mfma_probe:
        mfma_probe(dev, stream)
        return
    if args.valu_probe:
        gemm_probe(dev, stream, VALU_PROBE_MATS, VALU_PROBE_M, args.probe_reps)
        return
    if args.sweep_probe:
        gemm_probe(dev, stream, ("gate_up", "down"), VALU_PROBE_M, args.probe_reps)
        return
    if args.encode_probe:
        encode_probe(dev, stream, args.probe_reps)
        return
    if args.read_trace_probe:
        res = read_ceiling(dev, stream, [READ_BEST])
        print(json.dumps({"sizes": READ_SIZES, "variant": list(READ_BEST), "warmup": 3, "reps": 20, "read": res}))
        return
    if args.timeline:
        timeline_leg(dev, stream, " ".join(["python3", "bench.py"] + sys.argv[1:]))
        return
    if args.r13_probe:
        gemm_probe(dev, stream, R13_MATS, R13_M, args.probe_reps, gemv_max=(8, 0))
        return
    if args.read_probe:
        variants = [(u, g) for u in (1, 2, 4, 8, 16) for g in (1, 2, 4, 8)]
        res = read_ceiling(dev, stream, variants)
        for nm, r in res.items():
            best = max(r, key=lambda v: r[v]["GBps"])
            log(f"[read] {nm}: best {best} {r[best]['GBps']} GB/s")
        print(json.dumps({"what": "plain streaming read (w12_read_probe), median of per-launch events",
                          "read": res}))
        return

    # ---- inputs (synthetic, seeded; host-generated so bits do not depend on the GPU) ----
    t0 = time.time()
    layer = S.layer(0)
    log(f"[bench] generated layer 0 in {time.time() - t0:.1f}s")
    names = list(S.LAYER_ORDER)
    w_dev = {nm: dev_bits(layer[nm]) for nm in names}
    x_dev = {}
    for nm in names:
        n, k = S.LAYER_SHAPES[nm]
        x_dev[(nm, m_step)] = dev_bits(S.activations(m_step, k, S.x_seed(m_step, k)))

    # ---- load-time leg: encode + verify per matrix ----
    enc, load_leg = {}, {}
    for nm in names:
        w = w_dev[nm]
        n, k = w.shape
        enc[nm] = w12.encode(w)   # untimed: the first launch of each kernel loads its code
        t_enc = timed(lambda i: w12.encode(w), 3, stream)
        res = torch.empty(2, dtype=torch.int64, device=dev)
        w12.verify_async(enc[nm], w, res)
        t_ver = timed(lambda i: w12.verify_async(enc[nm], w, res), 5, stream)
        cnt, first = res.cpu().tolist()
        assert cnt == 0, f"load-time check failed on {nm}: {cnt} mismatches (first {first})"
        load_leg[nm] = {
            "encode_ms": round(t_enc, 4), "encode_GBps": round(2 * n * k / t_enc / 1e6, 1),
            "verify_ms": round(t_ver, 4),
            "verify_GBps": round((3.5 * n * k + 5 * n + 4 * enc[nm].num_escapes) / t_ver / 1e6, 1),
            "escapes": enc[nm].num_escapes, "bits_per_weight": round(enc[nm].bits_per_weight(), 5),
        }
        log(f"[bench] {nm}: E={enc[nm].num_escapes} bpw={enc[nm].bits_per_weight():.4f} "
            f"encode {t_enc:.3f} ms verify {t_ver:.3f} ms")
    # ---- checkpoint leg: the layer's W12 file streamed back, checked against the BF16 source ----
    out_ckpt = checkpoint_leg(enc, w_dev, names)
    # the caching allocator keeps this memory: returning it to the driver right before the timed
    # steps slows the first few hundred launches after it
    del w_dev

    copies = [enc] + [{nm: clone_tensor(enc[nm]) for nm in names} for _ in range(args.copies - 1)]
    y_dev = {nm: torch.empty(m_step, S.LAYER_SHAPES[nm][0], dtype=torch.float32, device=dev) for nm in names}
    ws = {nm: w12.gemm_workspace(m_step, *S.LAYER_SHAPES[nm]) for nm in names}
    if args.only_group:
        xs_o = [x_dev[(nm, m_step)] for nm in names]
        ys_o = [y_dev[nm] for nm in names]
        ws_o = w12.gemm_group_workspace(m_step, [enc[nm] for nm in names])

        def group_only(i):
            c = copies[i % len(copies)]
            w12.gemm_group(xs_o, [c[nm] for nm in names], ys_o, ws=ws_o, stream=stream)

        for i in range(args.warmup):
            group_only(i)
        t_o = timed(group_only, args.steps, stream)
        moved_o = sum(alg_bytes(*S.LAYER_SHAPES[nm], m_step, enc[nm].num_escapes) for nm in names)
        if args.copy_probe:
            a = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
            b = torch.empty_like(a)
            torch.cuda.synchronize()
            torch.bitwise_not(a, out=b)   # one elementwise kernel: reads and writes 256 MiB
            torch.cuda.synchronize()
        print(json.dumps({"what": "grouped layer step (qkv, o_proj, gate_up, down at M=16, one launch)",
                          "ms_per_step": round(t_o, 5), "bytes_moved_GBps": round(moved_o / t_o / 1e6, 1),
                          "alg_bytes_per_launch": int(moved_o)}))
        return

    # HIP events bracket every gate_up launch of the roofline pass (same stream as the launch);
    # the host enqueues a step in well under the step's GPU time, so the stream is never idle
    # between an event and its kernel.
    ev_pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.steps)]
    rec = {"on": False}

    def layer_step(i):
        c = copies[i % len(copies)]
        for nm in names:
            if rec["on"] and nm == "gate_up":
                ev_pairs[i][0].record(stream)
                w12.gemm(x_dev[(nm, m_step)], c[nm], y=y_dev[nm], ws=ws[nm], stream=stream)
                ev_pairs[i][1].record(stream)
            else:
                w12.gemm(x_dev[(nm, m_step)], c[nm], y=y_dev[nm], ws=ws[nm], stream=stream)

    for i in range(args.warmup):
        layer_step(i)
    torch.cuda.synchronize()
    # the headline: K steps with nothing but the GEMM launches on the stream (events only at the
    # boundaries of 5 consecutive blocks of steps, for the spread)
    t_step, block_ms = timed_blocks(layer_step, args.steps, stream)
    # then K more steps with HIP events around every gate_up launch, for the per-launch roofline
    # (each event record is a marker packet on the stream and lengthens the step it sits in)
    rec["on"] = True
    t_step_instr = timed(layer_step, args.steps, stream)
    rec["on"] = False
    # Y of the last timed step, kept on the host for the oracle check after all timing
    torch.cuda.synchronize()
    y_timed = {nm: y_dev[nm].cpu().numpy() for nm in names}
    gate_us = [a.elapsed_time(b) * 1e3 for a, b in ev_pairs]
    weight_bytes = sum(2 * n * k for n, k in (S.LAYER_SHAPES[nm] for nm in names))
    moved = sum(alg_bytes(*S.LAYER_SHAPES[nm], m_step, enc[nm].num_escapes) for nm in names)
    value = weight_bytes / t_step / 1e6
    log(f"[bench] layer step {t_step * 1e3:.1f} us -> {value:.1f} weight-GB/s, "
        f"{moved / t_step / 1e6:.1f} GB/s moved")

    out = {
        "metric": "w12_gemm weight-GB/s and % of HBM peak at M=1..64; bits/weight",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "one 27B-class dense decoder layer (hidden 5120): qkv 7168x5120, o_proj 5120x5120, "
                        "gate_up 34816x5120, down 5120x17408; W12 weights, M=16 BF16 verify rows",
            "M": m_step,
            "weights_bf16_bytes": weight_bytes,
            "bytes_moved_per_step": int(moved),
            "bytes_moved_GBps": round(moved / t_step / 1e6, 1),
            "bytes_moved_frac_of_8TBps": round(moved / t_step / 1e6 / HBM_PEAK_GBPS, 4),
            "bits_per_weight": round(sum(enc[nm].nbytes() for nm in names) * 8 / (weight_bytes / 2), 5),
            "byte_floor_us": round(sum(byte_floor_us(*S.LAYER_SHAPES[nm], m_step, enc[nm].num_escapes)
                                       for nm in names), 2),
            "ms_per_step_with_gate_up_events": round(t_step_instr, 5),
            "ms_per_step_block_median": round(ci95(block_ms)[0], 5),
            "ms_per_step_ci95_halfwidth": None if ci95(block_ms)[1] is None else round(ci95(block_ms)[1], 5),
            "step_blocks": len(block_ms),
            "rotated_copies": len(copies),
            "inputs_sha256": {nm: S.sha256(layer[nm])[:16] for nm in names},
        },
    }
    if args.only_layer:
        if args.copy_probe:
            a = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
            b = torch.empty_like(a)
            torch.cuda.synchronize()
            torch.bitwise_not(a, out=b)   # one elementwise kernel: reads and writes 256 MiB
            torch.cuda.synchronize()
        print(json.dumps(out))
        return

    # ---- roofline of the dominant kernel: the gate_up GEMM launch, from the timed steps ----
    nm = "gate_up"
    n, k = S.LAYER_SHAPES[nm]
    t_g = float(np.mean(gate_us)) / 1e3   # ms
    ab = alg_bytes(n, k, m_step, enc[nm].num_escapes)
    plan = w12.gemm_plan(m_step, n, k)
    out["roofline"] = {
        "bound": "hbm", "achieved": round(ab / t_g / 1e6, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
        "frac": round(ab / t_g / 1e6 / HBM_PEAK_GBPS, 4), "traffic": None,
        "kernel": kernel_name(plan, m_step),
        "launch": f"gate_up {n}x{k} M={m_step}, grid={plan['grid']}, segments/tile<={plan['splits']}",
        "avg_launch_us": round(t_g * 1e3, 2), "median_launch_us": round(float(np.median(gate_us)), 2),
        "alg_bytes_per_launch": int(ab),
    }
    out["roofline"].update(traffic_from_profile(ab))
    out["load_time"] = load_leg
    out["checkpoint"] = out_ckpt

    # ---- the same four products in one grouped launch (w12_gemm_group) ----
    xs_g = [x_dev[(nm, m_step)] for nm in names]
    ys_g = [y_dev[nm] for nm in names]
    ws_g = w12.gemm_group_workspace(m_step, [enc[nm] for nm in names])

    def group_step(i):
        c = copies[i % len(copies)]
        w12.gemm_group(xs_g, [c[nm] for nm in names], ys_g, ws=ws_g, stream=stream)

    for i in range(args.warmup):
        group_step(i)
    torch.cuda.synchronize()
    t_grp = timed(group_step, args.steps, stream)
    out["grouped"] = {
        "what": "the same four independent products (qkv, o_proj, gate_up, down at M=16) in one stream-K "
                "launch (w12_gemm_group); valid where the products do not depend on one another",
        "ms_per_step": round(t_grp, 5), "weight_GBps": round(weight_bytes / t_grp / 1e6, 1),
        "bytes_moved_GBps": round(moved / t_grp / 1e6, 1),
        "bytes_moved_frac_of_8TBps": round(moved / t_grp / 1e6 / HBM_PEAK_GBPS, 4),
    }
    log(f"[bench] grouped layer step {t_grp * 1e3:.1f} us -> {weight_bytes / t_grp / 1e6:.1f} weight-GB/s, "
        f"{moved / t_grp / 1e6:.1f} GB/s moved")

    # ---- the Q pass (nested 8-bit view, hi plane only) of the same layer step ----
    def q_step(i):
        c = copies[i % len(copies)]
        for nm in names:
            w12.gemm(x_dev[(nm, m_step)], c[nm], y=y_dev[nm], ws=ws[nm], stream=stream, qpass=True)

    for i in range(args.warmup):
        q_step(i)
    torch.cuda.synchronize()
    t_q = timed(q_step, args.steps, stream)
    moved_q = sum(alg_bytes(*S.LAYER_SHAPES[nm], m_step, enc[nm].num_escapes) - 0.5 * S.LAYER_SHAPES[nm][0] *
                  S.LAYER_SHAPES[nm][1] for nm in names)
    out["qpass"] = {
        "what": "the same layer step through w12_gemm_q (hi plane only: 1 B/weight, escapes exact)",
        "ms_per_step": round(t_q, 5), "weight_GBps": round(weight_bytes / t_q / 1e6, 1),
        "bytes_moved_GBps": round(moved_q / t_q / 1e6, 1),
        "bytes_moved_frac_of_8TBps": round(moved_q / t_q / 1e6 / HBM_PEAK_GBPS, 4),
    }
    log(f"[bench] Q-pass layer step {t_q * 1e3:.1f} us -> {weight_bytes / t_q / 1e6:.1f} weight-GB/s")

    # ---- hot cache: each layer GEMM at M=16 re-reading one copy (labelled; not the headline) ----
    hot = {}
    for nm in names:
        n, k = S.LAYER_SHAPES[nm]
        f = lambda i: w12.gemm(x_dev[(nm, m_step)], enc[nm], y=y_dev[nm], ws=ws[nm], stream=stream)
        for i in range(3):
            f(i)
        t = timed(f, 30, stream)
        ab = alg_bytes(n, k, m_step, enc[nm].num_escapes)
        hot[nm] = {"us": round(t * 1e3, 2), "moved_GBps": round(ab / t / 1e6, 1),
                   "w12_MB": round(enc[nm].nbytes() / 1e6, 1)}
    out["hot_cache"] = {"what": "the same encoded copy launched 30 times in a row at M=16: matrices under the "
                                "256 MB Infinity Cache are served from it", **hot}

    # encoded copies of one matrix rotated by the sweep legs: at least 1 GiB, so no launch finds
    # its weights in the 256 MB Infinity Cache
    rot = {}
    if not args.no_sweep:
        for nm in ("gate_up", "down"):
            cs = [c[nm] for c in copies]
            while sum(t.nbytes() for t in cs) < (1 << 30):
                cs.append(clone_tensor(enc[nm]))
            rot[nm] = cs

    # ---- tree-verify M sweep on gate_up and down ----
    if not args.no_sweep:
        sweep = {"rotated_MB": {nm: round(sum(t.nbytes() for t in cs) / 1e6, 1) for nm, cs in rot.items()}}
        for nm in ("gate_up", "down"):
            n, k = S.LAYER_SHAPES[nm]
            cs = rot[nm]
            for m in S.TREE_M_SWEEP + (16,):
                x = dev_bits(S.activations(m, k, S.x_seed(m, k)))
                y = torch.empty(m, n, dtype=torch.float32, device=dev)
                wsm = w12.gemm_workspace(m, n, k)
                for i in range(3):
                    w12.gemm(x, cs[i % len(cs)], y=y, ws=wsm)
                t = timed(lambda i: w12.gemm(x, cs[i % len(cs)], y=y, ws=wsm), 30, stream)
                ab = alg_bytes(n, k, m, enc[nm].num_escapes)
                fl = byte_floor_us(n, k, m, enc[nm].num_escapes)
                sweep[f"{nm}_M{m}"] = {
                    "us": round(t * 1e3, 2), "weight_GBps": round(2 * n * k / t / 1e6, 1),
                    "moved_GBps": round(ab / t / 1e6, 1), "frac": round(ab / t / 1e6 / HBM_PEAK_GBPS, 4),
                    "byte_floor_us": round(fl, 2), "floor_over_time": round(fl / (t * 1e3), 4),
                    "splits": w12.gemm_plan(m, n, k)["splits"],
                }
                log(f"[bench] {nm} M={m}: {t * 1e3:.1f} us, {ab / t / 1e6:.0f} GB/s moved")
        out["tree_sweep"] = sweep

    # ---- batched verify on gate_up and down (MFMA-bound tiles) ----
    if not args.no_sweep:
        batched = {"rotated_MB": {nm: round(sum(t.nbytes() for t in cs) / 1e6, 1) for nm, cs in rot.items()}}
        for nm in ("gate_up", "down"):
            n, k = S.LAYER_SHAPES[nm]
            cs = rot[nm]
            for m in S.BATCHED_M:
                x = dev_bits(S.activations(m, k, S.x_seed(m, k)))
                y = torch.empty(m, n, dtype=torch.float32, device=dev)
                wsm = w12.gemm_workspace(m, n, k)
                for i in range(3):
                    w12.gemm(x, cs[i % len(cs)], y=y, ws=wsm)
                t = timed(lambda i: w12.gemm(x, cs[i % len(cs)], y=y, ws=wsm), 10, stream)
                fl = byte_floor_us(n, k, m, enc[nm].num_escapes)
                plan = w12.gemm_plan(m, n, k)
                batched[f"{nm}_M{m}"] = {
                    "us": round(t * 1e3, 2), "TFLOPs": round(2 * m * n * k / t / 1e9, 1),
                    "frac_of_bf16_peak": round(2 * m * n * k / t / 1e9 / BF16_PEAK_TFLOPS, 4),
                    "weight_GBps": round(2 * n * k / t / 1e6, 1), "byte_floor_us": round(fl, 2),
                    "floor_over_time": round(fl / (t * 1e3), 4), "kernel": kernel_name(plan, m),
                }
                log(f"[bench] batched {nm} M={m}: {t * 1e3:.1f} us, {2 * m * n * k / t / 1e9:.0f} TFLOP/s")
        out["batched_verify"] = batched

    # ---- escape stress: heavy-tailed weights with 2% out-of-window values (gate_up, down) ----
    if not args.no_sweep:
        out["heavy_tail"] = heavy_tail_leg(dev, stream, out.get("tree_sweep", {}), out.get("batched_verify", {}))

    # ---- full-model weight stream: 64 layers resident, 256 GEMMs at M=32 from cold weights ----
    if not args.no_full_model:
        del copies, rot
        torch.cuda.empty_cache()
        out["full_model"] = full_model_leg(dev, stream, args.model_layers, 32)

    # ---- practical HBM ceilings (context for frac): the hand-written streaming read at the
    # matrices' sizes, and a plain torch copy ----
    rd = read_ceiling(dev, stream, [READ_BEST])
    key = f"U{READ_BEST[0]}_G{READ_BEST[1]}"
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    bcp = torch.empty_like(a)
    t_cp = timed(lambda i: bcp.copy_(a), 10, stream)
    out["hbm_reference"] = {
        "what": "w12_read_probe: plain streaming read, %d loads in flight per lane, %d work-groups per CU; "
                "median of 20 launches rotating over 2 GiB" % READ_BEST,
        "read_GBps": {nm: r[key]["GBps"] for nm, r in rd.items()},
        "read_us": {nm: r[key]["us"] for nm, r in rd.items()},
        "copy_1GiB_GBps": round(2 * a.numel() / t_cp / 1e6, 1)}
    log(f"[bench] plain read {out['hbm_reference']['read_GBps']} GB/s, copy {2 * a.numel() / t_cp / 1e6:.0f} GB/s")
    del a, bcp

    # ---- CPU oracle on the host cores (a reported baseline, not the target) ----
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(layer, enc, y_timed)
    print(json.dumps(out))


MFMA_PROBE_M = (256, 512)
MFMA_PROBE_MATS = ("gate_up", "down")


VALU_PROBE_M = (1, 8, 16, 32, 48, 64)
VALU_PROBE_MATS = ("gate_up",)


def mfma_probe(dev, stream):
    """gate_up and down at M = 256 and 512 (the batched-verify tiles)."""
    gemm_probe(dev, stream, MFMA_PROBE_MATS, MFMA_PROBE_M)


def gemm_probe(dev, stream, mats, ms, reps=3, gemv_max=(None,)):
    """Layer 0's matrices in ``mats`` at every M of ``ms``, ``reps`` launches each on three rotating
    encoded copies, in a fixed order (matrix-major, then W12_GEMV_MAX_M values, then M); prints
    the per-launch event times.  A gemv_max of None keeps the default GEMV / MFMA boundary."""
    layer = S.layer(0, which=mats)
    res = {}
    for nm in mats:
        n, k = S.LAYER_SHAPES[nm]
        e0 = w12.encode(dev_bits(layer[nm]))
        cs = [e0, clone_tensor(e0), clone_tensor(e0)]
        for gv, m in [(gv, m) for gv in gemv_max for m in ms]:
            if gv is None:
                os.environ.pop("W12_GEMV_MAX_M", None)
            else:
                os.environ["W12_GEMV_MAX_M"] = str(gv)
            x = dev_bits(S.activations(m, k, S.x_seed(m, k)))
            y = torch.empty(m, n, dtype=torch.float32, device=dev)
            ws = w12.gemm_workspace(m, n, k)
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            for i, (a, b) in enumerate(evs):
                a.record(stream)
                w12.gemm(x, cs[i % len(cs)], y=y, ws=ws, stream=stream)
                b.record(stream)
            torch.cuda.synchronize()
            plan = w12.gemm_plan(m, n, k)
            key = f"{nm}_M{m}" if gv is None else f"{nm}_M{m}_gemvmax{gv}"
            res[key] = {"kernel": kernel_name(plan, m), "launch_us": [round(a.elapsed_time(b) * 1e3, 2)
                                                                     for a, b in evs],
                        "flops": 2 * m * n * k, "grid": plan["grid"], "m_tile": plan["m_tile"],
                        "escapes": e0.num_escapes}
        os.environ.pop("W12_GEMV_MAX_M", None)
        del cs, e0
        torch.cuda.empty_cache()
    print(json.dumps(res))




def encode_cases():
    """(label, n, k, BF16 bits) of the encode probe: layer 0's four matrices, then the heavy-tail
    gate_up and down (seeds 1000 / 1001, as in the parity tests)."""
    layer = S.layer(0)
    for nm in S.LAYER_ORDER:
        yield nm, layer[nm]
    for nm, seed in (("gate_up", 1000), ("down", 1001)):
        n, k = S.LAYER_SHAPES[nm]
        yield f"heavy_{nm}", S.heavy_tail_weights(seed, n, k)


def encode_probe(dev, stream, reps=3):
    """Each matrix of encode_cases: one checked encode, then ``reps`` count passes (count + scan)
    back to back, ``reps`` emits back to back (the kernels in steady state), and ``reps`` whole
    encodes, each with its read-back of E (timed with events: the load-time cost).  Prints the
    case order, escape counts and the whole-encode times as JSON; the kernel times come from the
    trace."""
    res = []
    for label, bits in encode_cases():
        n, k = bits.shape
        w = dev_bits(bits)
        t = w12.encode(w, stream=stream)
        assert w12.verify(t, w, stream=stream) == (0, -1), f"{label}: encode does not verify"
        e = t.num_escapes
        base, esc_ptr = torch.empty_like(t.base), torch.empty_like(t.esc_ptr)
        for _ in range(reps):
            w12.encode_count(w, base, esc_ptr, stream=stream)
        for _ in range(reps):
            w12.encode_emit(w, t, stream=stream)
        torch.cuda.synchronize()
        assert w12.verify(t, w, stream=stream) == (0, -1), f"{label}: repeated emit does not verify"
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in evs:
            a.record(stream)
            w12.encode(w, stream=stream)
            b.record(stream)
        torch.cuda.synchronize()
        res.append({"matrix": label, "n": n, "k": k, "reps": reps, "escapes": e,
                    "encode_us": [round(a.elapsed_time(b) * 1e3, 1) for a, b in evs]})
        del t, w, base, esc_ptr
        torch.cuda.empty_cache()
    print(json.dumps({"cases": res}))


def encode_bytes(n, k, e):
    """Algorithmic bytes of the three encode kernels: the count reads W and writes the bases and
    escape counts; the scan reads and writes the counts; the emit reads W, the bases and pointers
    and writes both planes (padding included) and the escapes."""
    hib, lob = w12.layout_bytes(n, k)
    return {"count": 2 * n * k + n + 4 * n, "scan": 8 * n + 4,
            "emit": 2 * n * k + n + 4 * (n + 1) + hib + lob + 4 * e}


def summarize_encode_trace(trace_csv, probe_json, command):
    """rocprofv3 kernel durations of the --encode-probe runs: per matrix the medians of the count,
    scan and emit kernels launched back to back (steady state), the encode's algorithmic bytes
    over the sum of the medians against 8 TB/s, and the whole encode with its read-back of E
    (event time, median)."""
    import csv
    with open(trace_csv) as f:
        trace = sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))
    names = ("k_encode_count", "k_scan_counts", "k_encode_emit")
    enc = [r for r in trace if any(kn in r["Kernel_Name"] for kn in names)]
    with open(probe_json) as f:
        probe = json.loads([ln for ln in f.read().splitlines() if ln.startswith("{")][-1])
    dur = lambda rs: float(np.median([(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rs]))
    lines = ["# W12 encode kernel times (count, scan, emit) on the layer's matrices and the heavy-tail ones, "
             "MI355X", "", "Command (run from the repository root):", "", "```", command, "```", "",
             f"Kernel sources: `csrc/` sha256 {source_stamp()}.", "",
             "Kernel trace durations (`k_encode_count`, `k_scan_counts`, `k_encode_emit`), medians over R launches "
             "of each kernel back to back (after one checked encode). Bytes are algorithmic: the count reads W "
             "(2NK) and writes 5 B per channel; the scan reads and writes the counts; the emit reads W, bases and "
             "pointers and writes the padded planes and 4 B per escape. The last three columns are the whole encode "
             "as the library runs it at load time (count, scan, read-back of E, emit): the same kernels' durations "
             "inside that sequence (count / scan / emit, medians of R), their sum against 8 TB/s, and the whole "
             "encode's event time (median of R), read-back and host work included.", "",
             "| matrix | N x K | escapes | count us | scan us | emit us | kernels us | count GB/s | emit GB/s | "
             "encode GB/s | of 8 TB/s | in sequence us | of 8 TB/s | whole encode us |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    i = 0
    for c in probe["cases"]:
        r = c["reps"]
        per = 3 + 2 * r + r + 3 * r
        rows = enc[i:i + per]
        i += per
        assert len(rows) == per, "trace ends early"
        counts, emits = rows[3:3 + 2 * r], rows[3 + 2 * r:3 + 3 * r]
        assert all(names[j % 2] in x["Kernel_Name"] for j, x in enumerate(counts)), f"unexpected order at {c}"
        assert all(names[2] in x["Kernel_Name"] for x in emits), f"unexpected order at {c}"
        seq = rows[3 + 3 * r:]
        assert all(names[j % 3] in x["Kernel_Name"] for j, x in enumerate(seq)), f"unexpected order at {c}"
        med = {"count": dur(counts[0::2]), "scan": dur(counts[1::2]), "emit": dur(emits)}
        in_seq = [dur(seq[j::3]) for j in range(3)]
        by = encode_bytes(c["n"], c["k"], c["escapes"])
        tot_us = sum(med.values())
        tot_b = sum(by.values())
        lines.append(f"| {c['matrix']} | {c['n']} x {c['k']} | {c['escapes']} | "
                     f"{med['count']:.1f} | {med['scan']:.1f} | {med['emit']:.1f} | {tot_us:.1f} | "
                     f"{by['count'] / med['count'] / 1e3:.0f} | {by['emit'] / med['emit'] / 1e3:.0f} | "
                     f"{tot_b / tot_us / 1e3:.0f} | {tot_b / tot_us / 1e3 / HBM_PEAK_GBPS:.3f} | "
                     f"{in_seq[0]:.1f} / {in_seq[1]:.1f} / {in_seq[2]:.1f} = {sum(in_seq):.1f} | "
                     f"{tot_b / sum(in_seq) / 1e3 / HBM_PEAK_GBPS:.3f} | {float(np.median(c['encode_us'])):.1f} |")
    assert i == len(enc), f"{len(enc) - i} encode kernels in the trace are not in the probe"
    path = os.path.join(ROOT, "profiles", "encode_layer_kernel_trace.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


TIMELINE_CASES = (("gate_up", 16), ("down", 16), ("gate_up", 1), ("o_proj", 16))


def timeline_leg(dev, stream, command, launches=6):
    """Per-work-group timelines (measurement build) of single GEMM launches on the layer
    matrices, over >= 1 GiB of rotated encoded copies; summarised per phase into
    profiles/gemm_M16_workgroup_timeline.md."""
    import ctypes
    import lossless_bit_weight_encode_amd._lib as L
    lib = L.lib()
    lib.w12_timeline_copy.restype = ctypes.c_int
    lib.w12_timeline_copy.argtypes = [ctypes.c_void_p, ctypes.c_uint64]
    layer = S.layer(0, which=tuple(sorted({nm for nm, _ in TIMELINE_CASES})))
    res = {}
    P = lambda a, q: float(np.percentile(a, q))
    for nm, m in TIMELINE_CASES:
        n, k = S.LAYER_SHAPES[nm]
        e0 = w12.encode(dev_bits(layer[nm]))
        cs = [e0]
        while sum(t.nbytes() for t in cs) < (1 << 30):
            cs.append(clone_tensor(e0))
        x = dev_bits(S.activations(m, k, S.x_seed(m, k)))
        y = torch.empty(m, n, dtype=torch.float32, device=dev)
        ws = w12.gemm_workspace(m, n, k)
        plan = w12.gemm_plan(m, n, k)
        G = plan["grid"]
        for i in range(6):
            w12.gemm(x, cs[i % len(cs)], y=y, ws=ws, stream=stream)
        runs = []
        for i in range(launches):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record(stream)
            w12.gemm(x, cs[i % len(cs)], y=y, ws=ws, stream=stream)
            b.record(stream)
            torch.cuda.synchronize()
            buf = np.zeros(G * 16, dtype=np.uint64)
            assert lib.w12_timeline_copy(buf.ctypes.data, buf.nbytes) == 0
            t = buf.reshape(G, 16).astype(np.int64)
            rel = lambda c: (t[:, c] - t[:, 0].min()) / 100.0   # us
            nseg = t[:, 13]
            two = nseg >= 2
            last_loop = np.where(two, rel(4), rel(2))
            last_stores = np.where(two, rel(10), rel(7))
            busy = last_loop - rel(1) - np.where(two, rel(3) - rel(2), 0.0)
            first_wave = np.arange(G) < min(G, 256)
            r = {"event_us": a.elapsed_time(b) * 1e3, "span_us": float(rel(11).max()),
                 "start_skew_us": P(rel(0), 100), "prologue_us": P(rel(1) - rel(0), 50),
                 "seg_end_wait_us": P(rel(5) - rel(2), 50), "reduce_us": P(rel(6) - rel(5), 50),
                 "stores_us": P(rel(7) - rel(6), 50),
                 "switch_us": P((rel(3) - rel(2))[two], 50) if two.any() else None,
                 "fixup_us": P(rel(11) - last_stores, 50), "fixup_p90_us": P(rel(11) - last_stores, 90),
                 "busy_p0_us": P(busy, 0), "busy_p50_us": P(busy, 50), "busy_p100_us": P(busy, 100),
                 "busy_first_wave_us": float(busy[first_wave].mean()),
                 "busy_second_wave_us": float(busy[~first_wave].mean()) if (~first_wave).any() else None,
                 "end_p0_us": P(rel(11), 0), "end_p50_us": P(rel(11), 50), "end_p100_us": P(rel(11), 100),
                 "segments": {int(a_): int(b_) for a_, b_ in zip(*np.unique(nseg, return_counts=True))}}
            runs.append(r)
        med = {key: (float(np.median([r[key] for r in runs])) if runs[0][key] is not None and
                     not isinstance(runs[0][key], dict) else runs[0][key]) for key in runs[0]}
        moved = alg_bytes(n, k, m, e0.num_escapes)
        med["grid"] = G
        med["alg_bytes"] = int(moved)
        res[f"{nm}_M{m}"] = med
        log(f"[timeline] {nm} M={m}: {json.dumps({k_: (round(v, 2) if isinstance(v, float) else v) for k_, v in med.items()})}")
        del cs, e0
        torch.cuda.empty_cache()
    lines = ["# Per-work-group timeline of the streaming GEMM (MI355X)", "",
             "Measurement build (`python -m lossless_bit_weight_encode_amd.build --timeline`, the same kernels with "
             "thread 0 of every work-group stamping the 100 MHz real-time counter; include/w12_timeline.h), then:",
             "", "```", command, "```", "", f"Kernel sources: `csrc/` sha256 {source_stamp()}.", "",
             f"Medians over {launches} launches (>= 1 GiB of rotated encoded copies). Per launch: the median over "
             "work-groups of each phase; `busy` is a work-group's time in its step loops (switch excluded); "
             "`first wave` / `second wave` are work-groups 0..255 / 256.. (dispatched breadth-first: the first "
             "and the second work-group of each compute unit). Times in us from the earliest work-group start. "
             "`event` brackets one launch on an idle GPU (the timeline is read back after every launch), so it "
             "includes the idle-to-busy dispatch latency that back-to-back launches hide; `span` is first "
             "work-group start to last work-group end.", "",
             "| case | grid | event | span | start skew | prologue | seg end wait | reduce | stores | switch | "
             "fixup (p50 / p90) | busy p0 / p50 / p100 | busy 1st / 2nd wave | end p0 / p50 / p100 |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    f2 = lambda v: "-" if v is None else f"{v:.2f}"
    for key, r in res.items():
        lines.append(f"| {key} | {r['grid']} | {f2(r['event_us'])} | {f2(r['span_us'])} | {f2(r['start_skew_us'])} | "
                     f"{f2(r['prologue_us'])} | {f2(r['seg_end_wait_us'])} | {f2(r['reduce_us'])} | "
                     f"{f2(r['stores_us'])} | {f2(r['switch_us'])} | {f2(r['fixup_us'])} / {f2(r['fixup_p90_us'])} | "
                     f"{f2(r['busy_p0_us'])} / {f2(r['busy_p50_us'])} / {f2(r['busy_p100_us'])} | "
                     f"{f2(r['busy_first_wave_us'])} / {f2(r['busy_second_wave_us'])} | "
                     f"{f2(r['end_p0_us'])} / {f2(r['end_p50_us'])} / {f2(r['end_p100_us'])} |")
    # written under profiles/ and, when the run has one, under gpurun_out/ as well
    for d in ("profiles", "gpurun_out"):
        if os.path.isdir(os.path.join(ROOT, d)):
            with open(os.path.join(ROOT, d, "gemm_M16_workgroup_timeline.md"), "w") as f:
                f.write("\n".join(lines) + "\n")
    print(json.dumps(res))


def summarize_read_trace(trace_csv, probe_json, command):
    """rocprofv3 kernel durations of the --read-trace-probe launches (warm-up launches dropped):
    the plain streaming read's bytes per second at each size, the practical HBM read ceiling."""
    import csv
    with open(trace_csv) as f:
        trace = sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))
    rd = [r for r in trace if "k_read_probe" in r["Kernel_Name"]]
    with open(probe_json) as f:
        probe = json.loads([ln for ln in f.read().splitlines() if ln.startswith("{")][-1])
    u, g = probe["variant"]
    lines = ["# Plain streaming read (practical HBM read ceiling), MI355X", "",
             "Command (run from the repository root):", "", "```", command, "```", "",
             f"Kernel sources: `csrc/` sha256 {source_stamp()}.", "",
             f"`w12_read_probe`: {g} work-groups of 256 threads per compute unit, each reading a contiguous share "
             f"with 16-byte loads, {u} loads in flight per lane; every launch reads a different part of a 2 GiB "
             "buffer (so the 256 MB Infinity Cache cannot serve it). Kernel trace durations over the timed "
             "launches of each size.", "",
             "| size | bytes | launches | median us | min us | GB/s (median) | of 8 TB/s |",
             "|---|---|---|---|---|---|---|"]
    i = 0
    for name, nb in probe["sizes"].items():
        nb = nb // 256 * 256
        rows = rd[i + probe["warmup"]:i + probe["warmup"] + probe["reps"]]
        i += probe["warmup"] + probe["reps"]
        d = np.array([(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows])
        med = float(np.median(d))
        lines.append(f"| {name} | {nb} | {len(d)} | {med:.2f} | {d.min():.2f} | {nb / med / 1e3:.0f} | "
                     f"{nb / med / 1e3 / HBM_PEAK_GBPS:.3f} |")
    assert i == len(rd), f"{len(rd) - i} read launches in the trace are not in the probe"
    path = os.path.join(ROOT, "profiles", "read_probe_ceiling_kernel_trace.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


R13_MATS = ("gate_up", "down")
R13_M = tuple(range(1, 9))


def summarize_r13_trace(trace_csv, probe_json, command):
    """rocprofv3 kernel durations of the --r13-probe launches: the wavefront GEMV (GemvPath<M>)
    against the 16-row MFMA tile (MfmaPath<1>) at M = 1..8 on gate_up and down, first launch of
    each case dropped."""
    import csv
    with open(trace_csv) as f:
        trace = sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))
    gemm = [r for r in trace if "k_gemm" in r["Kernel_Name"]]
    with open(probe_json) as f:
        probe = json.loads([ln for ln in f.read().splitlines() if ln.startswith("{")][-1])
    med = {}
    i = 0
    for nm in R13_MATS:
        for gv in (8, 0):
            for m in R13_M:
                info = probe[f"{nm}_M{m}_gemvmax{gv}"]
                reps = len(info["launch_us"])
                rows = gemm[i:i + reps][1:]
                i += reps
                assert all(info["kernel"].split("<")[1][:4] in r["Kernel_Name"] for r in rows), "trace out of order"
                d = np.array([(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows])
                med[(nm, gv, m)] = (float(np.median(d)), float(d.mean()), len(d), info["escapes"])
    assert i == len(gemm), f"{len(gemm) - i} GEMM launches in the trace are not in the probe"
    lines = ["# Wavefront GEMV against 16-row MFMA tiles at M = 1..8 (gate_up 34816 x 5120, down 5120 x 17408), "
             "MI355X", "", "Command (run from the repository root):", "", "```", command, "```", "",
             f"Kernel sources: `csrc/` sha256 {source_stamp()}.", "",
             "Kernel trace durations (median and mean over the launches of each case, the first dropped; three "
             "rotating encoded copies). `GemvPath<M>` is the FP32 dot2 wavefront GEMV (W12_GEMV_MAX_M=8), "
             "`MfmaPath<1>` the bf16 MFMA 16-row tile (W12_GEMV_MAX_M=0). Fraction = algorithmic bytes of the "
             "launch / median / 8 TB/s.", "",
             "| matrix | M | GEMV median us | GEMV frac | MFMA median us | MFMA frac | faster |",
             "|---|---|---|---|---|---|---|"]
    for nm in R13_MATS:
        n, k = S.LAYER_SHAPES[nm]
        for m in R13_M:
            g, f = med[(nm, 8, m)], med[(nm, 0, m)]
            ab = alg_bytes(n, k, m, g[3])
            lines.append(f"| {nm} | {m} | {g[0]:.2f} | {ab / g[0] / 1e3 / HBM_PEAK_GBPS:.3f} | {f[0]:.2f} | "
                         f"{ab / f[0] / 1e3 / HBM_PEAK_GBPS:.3f} | {'GEMV' if g[0] < f[0] else 'MFMA'} "
                         f"({abs(g[0] - f[0]) / max(g[0], f[0]) * 100:.1f}%) |")
    path = os.path.join(ROOT, "profiles", "gemm_gemv_vs_mfma_M1_M8_kernel_trace.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_mfma(pmc_csv, probe_json):
    """MFMA busy fraction and BF16 MFMA FLOP rate of the --mfma-probe GEMM launches.  Per
    dispatch: util = SQ_VALU_MFMA_BUSY_CYCLES (summed over SIMDs) / (GPU-active cycles x SIMDs),
    where the GPU-active cycles are GRBM_GUI_ACTIVE / XCDs (the CSV sums the counter over the
    XCDs); MFMA flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; the rate uses the probe's own event
    time of the launch (the middle one of each three, in the fixed launch order).  SIMD and XCD
    counts come from the run's agent info."""
    rows = _counter_rows(pmc_csv)
    by_disp = {}
    for r in rows:
        if "k_gemm" not in r["Kernel_Name"]:
            continue
        d = by_disp.setdefault(int(r["Dispatch_Id"]), {"kernel": r["Kernel_Name"]})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    disp = [by_disp[i] for i in sorted(by_disp)]
    with open(probe_json) as f:
        probe = json.loads([ln for ln in f.read().splitlines() if ln.startswith("{")][-1])
    import csv
    agent_csv = os.path.join(os.path.dirname(pmc_csv), os.path.basename(pmc_csv).replace("counter_collection",
                                                                                         "agent_info"))
    simds, xcds = 1024, 8
    if os.path.exists(agent_csv):
        with open(agent_csv) as f:
            for r in csv.DictReader(f):
                if r.get("Name", "").startswith("gfx"):
                    simds, xcds = int(r["Simd_Count"]), int(r["Num_Xcc"])
    out = {"commands": [
        "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 GRBM_GUI_ACTIVE -f csv "
        "-d gpurun_out/pmc_mfma -o run -- python3 bench.py --mfma-probe",
        "python3 bench.py --mfma-probe > gpurun_out/mfma_probe.json",
        f"python3 bench.py --summarize-mfma {pmc_csv} {probe_json}"],
        "simds": simds, "xcds": xcds, "peak_bf16_dense_TFLOPs": 2500.0, "launches": {}}
    i = 0
    for nm in MFMA_PROBE_MATS:
        for m in MFMA_PROBE_M:
            key = f"{nm}_M{m}"
            ds = disp[i:i + 3]
            i += 3
            mid = ds[1]
            t_us = probe[key]["launch_us"][1]
            util = mid["SQ_VALU_MFMA_BUSY_CYCLES"] / (mid["GRBM_GUI_ACTIVE"] / xcds * simds)
            mflops = mid["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
            out["launches"][key] = {
                "kernel": probe[key]["kernel"], "grid": probe[key]["grid"], "m_tile": probe[key]["m_tile"],
                "launch_us": t_us, "mfma_busy_frac": round(util, 4),
                "mfma_flops": mflops, "useful_flops": probe[key]["flops"],
                "mfma_TFLOPs": round(mflops / t_us / 1e6, 1),
                "useful_TFLOPs": round(probe[key]["flops"] / t_us / 1e6, 1),
                "frac_of_bf16_peak": round(probe[key]["flops"] / t_us / 1e6 / 2500.0, 4)}
    path = os.path.join(ROOT, "profiles", "gemm_M256_M512_mfma_counters.txt")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def summarize_wide_lds(pmc_csv, probe_json):
    """LDS counters of the --mfma-probe wide-tile launches (summed over the GPU per dispatch; each
    case is the middle of its three launches, in the probe's fixed launch order)."""
    rows = _counter_rows(pmc_csv)
    by_disp = {}
    for r in rows:
        if "k_gemm" not in r["Kernel_Name"]:
            continue
        d = by_disp.setdefault(int(r["Dispatch_Id"]), {"kernel": r["Kernel_Name"]})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    disp = [by_disp[i] for i in sorted(by_disp)]
    command = ("rocprofv3 --pmc SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_WAIT_INST_LDS -f csv "
               "-d gpurun_out/pmc_lds -o run -- python3 bench.py --mfma-probe")
    lines = ["# LDS counters of the wide-tile GEMM (batched verify, M = 256 / 512), MI355X", "",
             "Command (run from the repository root), then the summary:", "", "```", command,
             "python3 bench.py --mfma-probe > gpurun_out/mfma_probe.json",
             f"python3 bench.py --summarize-wide-lds {pmc_csv} {probe_json}", "```", "",
             f"Kernel sources: `csrc/` sha256 {source_stamp()}.", "",
             "Counters are summed over the GPU; each row is the middle of the three launches of a case.", "",
             "| case | kernel | SQ_INSTS_LDS | SQ_LDS_BANK_CONFLICT | SQ_LDS_IDX_ACTIVE | conflict / active | "
             "SQ_WAIT_INST_LDS |", "|---|---|---|---|---|---|---|"]
    i = 0
    for nm in MFMA_PROBE_MATS:
        for m in MFMA_PROBE_M:
            mid = disp[i + 1]
            i += 3
            act = mid["SQ_LDS_IDX_ACTIVE"]
            lines.append(f"| {nm} M={m} | `{mid['kernel'].split('(')[0]}` | {mid['SQ_INSTS_LDS']:.0f} | "
                         f"{mid['SQ_LDS_BANK_CONFLICT']:.0f} | {act:.0f} | "
                         f"{mid['SQ_LDS_BANK_CONFLICT'] / act if act else 0.0:.3f} | {mid['SQ_WAIT_INST_LDS']:.0f} |")
    lines += ["", "SQ_INSTS_LDS is within 1.3% of 16 operand reads per wave and 32-k stage (4 X fragments, 2 hi "
              "and 2 lo reads per k16 step, two steps), e.g. 21,760 work-group stages x 8 waves x 16 = 2.79 M for "
              "gate_up at M = 256; the rest are escape-slice reads and the epilogue's."]
    path = os.path.join(ROOT, "profiles", "gemm_wide_M256_M512_lds_counters.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_valu(pmc_csv, probe_json):
    """VALU budget of the streaming GEMM (gate_up at M = 1, 8, 16, 32 from --valu-probe).

    The counters are summed over the GPU per dispatch; each case uses the middle of its three
    launches and the probe's own event time for it.  A wave64 VALU instruction occupies a 16-lane
    SIMD for 4 cycles, so the VALU issue floor of a launch is SQ_INSTS_VALU x 4 cycles spread over
    every SIMD at 2.4 GHz (MFMA instructions are counted apart and excluded from it).  Lane-ops per
    weight = (SQ_INSTS_VALU - SQ_INSTS_MFMA) x 64 / (N K); the chip issues 1024 SIMDs x 16 lanes x
    2.4 GHz = 39.3 T lane-ops/s, i.e. 9.2 lane-ops per weight when weights stream at 6.4 TB/s
    (1.5 bytes each)."""
    rows = _counter_rows(pmc_csv)
    by_disp = {}
    for r in rows:
        if "k_gemm" not in r["Kernel_Name"]:
            continue
        d = by_disp.setdefault(int(r["Dispatch_Id"]), {"kernel": r["Kernel_Name"]})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    disp = [by_disp[i] for i in sorted(by_disp)]
    with open(probe_json) as f:
        probe = json.loads([ln for ln in f.read().splitlines() if ln.startswith("{")][-1])
    simds, clock = 1024, 2.4e9
    lane_rate = simds * 16 * clock
    out = {"commands": [
        "rocprofv3 --pmc SQ_WAVES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_SALU SQ_INSTS_LDS GRBM_GUI_ACTIVE -f csv "
        "-d gpurun_out/pmc_valu -o run -- python3 bench.py --valu-probe",
        "python3 bench.py --valu-probe > gpurun_out/valu_probe.json",
        f"python3 bench.py --summarize-valu {pmc_csv} {probe_json}"],
        "simds": simds, "clock_GHz": clock / 1e9, "valu_lane_ops_per_s": lane_rate,
        "budget_lane_ops_per_weight_at_6.4TBps": round(lane_rate / (6.4e12 / 1.5), 2), "launches": {}}
    i = 0
    for nm in VALU_PROBE_MATS:
        n, k = S.LAYER_SHAPES[nm]
        for m in VALU_PROBE_M:
            key = f"{nm}_M{m}"
            ds = disp[i:i + 3]
            i += 3
            mid = ds[1]
            t_us = probe[key]["launch_us"][1]
            valu = mid["SQ_INSTS_VALU"] - mid["SQ_INSTS_MFMA"]
            floor_us = valu * 4 / simds / clock * 1e6
            out["launches"][key] = {
                "kernel": probe[key]["kernel"], "grid": probe[key]["grid"], "launch_us": t_us,
                "waves": int(mid["SQ_WAVES"]), "valu_insts": int(valu), "mfma_insts": int(mid["SQ_INSTS_MFMA"]),
                "salu_insts": int(mid["SQ_INSTS_SALU"]), "lds_insts": int(mid["SQ_INSTS_LDS"]),
                "valu_lane_ops_per_weight": round(valu * 64 / (n * k), 3),
                "valu_issue_floor_us": round(floor_us, 2), "valu_floor_over_time": round(floor_us / t_us, 3)}
    path = os.path.join(ROOT, "profiles", "gemm_gate_up_M1_M64_valu_counters.txt")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def _probe_dispatches(pmc_csv):
    rows = _counter_rows(pmc_csv)
    by_disp = {}
    for r in rows:
        if "k_gemm" not in r["Kernel_Name"]:
            continue
        d = by_disp.setdefault(int(r["Dispatch_Id"]), {"kernel": r["Kernel_Name"]})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [by_disp[i] for i in sorted(by_disp)]


def summarize_stalls(pmc_csv, probe_json):
    """Where the waves of the streaming GEMM spend their time (gate_up at M = 1..64 from
    --valu-probe; the middle launch of each case).  The kernel's cycles are GRBM_GUI_ACTIVE / XCDs
    and every wave lives about that long, so wave-cycles = SQ_WAVES x kernel cycles; SQ_WAIT_ANY and
    SQ_WAIT_INST_ANY count quad-cycles (x 4), SQ_ACTIVE_INST_ANY cycles.  The LDS conflict share is
    SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE."""
    disp = _probe_dispatches(pmc_csv)
    with open(probe_json) as f:
        probe = json.loads([ln for ln in f.read().splitlines() if ln.startswith("{")][-1])
    xcds = 8
    out = {"commands": [
        "rocprofv3 --pmc SQ_WAVES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_LDS_BANK_CONFLICT "
        "SQ_LDS_IDX_ACTIVE SQ_BUSY_CYCLES GRBM_GUI_ACTIVE -f csv -d gpurun_out/pmc_stall -o run -- "
        "python3 bench.py --valu-probe",
        "python3 bench.py --valu-probe > gpurun_out/valu_probe.json",
        f"python3 bench.py --summarize-stalls {pmc_csv} {probe_json}"], "launches": {}}
    i = 0
    for nm in VALU_PROBE_MATS:
        for m in VALU_PROBE_M:
            key = f"{nm}_M{m}"
            mid = disp[i + 1]
            i += 3
            cyc = mid["GRBM_GUI_ACTIVE"] / xcds
            wave_cycles = mid["SQ_WAVES"] * cyc
            lds = mid["SQ_LDS_IDX_ACTIVE"]
            out["launches"][key] = {
                "kernel": probe[key]["kernel"], "grid": probe[key]["grid"], "launch_us": probe[key]["launch_us"][1],
                "waves": int(mid["SQ_WAVES"]), "kernel_cycles": int(cyc),
                "wait_any_frac": round(4 * mid["SQ_WAIT_ANY"] / wave_cycles, 3),
                "wait_inst_issue_frac": round(4 * mid["SQ_WAIT_INST_ANY"] / wave_cycles, 3),
                "active_inst_frac": round(mid["SQ_ACTIVE_INST_ANY"] / wave_cycles, 3),
                "lds_conflict_over_active": round(mid["SQ_LDS_BANK_CONFLICT"] / lds, 3) if lds else None}
    path = os.path.join(ROOT, "profiles", "gemm_gate_up_M1_M64_stall_counters.txt")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def summarize_sweep_trace(trace_csv, probe_json, command):
    """rocprofv3 kernel durations of the --valu-probe GEMM launches (gate_up at M = 1..64, in probe
    order, R launches per M), the first launch of each M dropped; weight-GB/s = 2NK / t and the
    fraction of 8 TB/s from the algorithmic bytes of each M."""
    import csv
    with open(trace_csv) as f:
        trace = sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))
    gemm = [r for r in trace if "k_gemm" in r["Kernel_Name"]]
    with open(probe_json) as f:
        probe = json.loads([ln for ln in f.read().splitlines() if ln.startswith("{")][-1])
    mats = [nm for nm in S.LAYER_ORDER if any(key.startswith(nm + "_M") for key in probe)]
    lines = ["# W12 GEMM kernel times over the M sweep: " +
             ", ".join(f"{nm} {S.LAYER_SHAPES[nm][0]} x {S.LAYER_SHAPES[nm][1]}" for nm in mats) + ", MI355X", "",
             "Command (run from the repository root):", "", "```", command, "```", "",
             f"Kernel sources: `csrc/` sha256 {source_stamp()}.", "",
             "Kernel trace durations; each M runs R launches on three rotating encoded copies (the first is "
             "dropped).", "Moved bytes are the algorithmic bytes of the launch (records, bases, pointers, "
             "escapes, X, Y).", "",
             "| matrix | M | kernel | launches | avg us | median us | min us | weight-GB/s (median) | "
             "moved GB/s (median) | of 8 TB/s |", "|---|---|---|---|---|---|---|---|---|---|"]
    i = 0
    for nm in mats:
        n, k = S.LAYER_SHAPES[nm]
        for m in VALU_PROBE_M:
            info = probe[f"{nm}_M{m}"]
            reps = len(info["launch_us"])
            rows = gemm[i:i + reps][1:]
            i += reps
            d = np.array([(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows])
            med = float(np.median(d))
            moved = alg_bytes(n, k, m, info["escapes"])
            lines.append(f"| {nm} | {m} | `{info['kernel']}` | {len(d)} | {d.mean():.2f} | {med:.2f} | {d.min():.2f} | "
                         f"{2 * n * k / med / 1e3:.0f} | {moved / med / 1e3:.0f} | "
                         f"{moved / med / 1e3 / HBM_PEAK_GBPS:.3f} |")
    assert i == len(gemm), f"{len(gemm) - i} GEMM launches in the trace are not in the probe"
    path = os.path.join(ROOT, "profiles", "gemm_" + "_".join(mats) + "_M1_M64_kernel_trace.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_encode_lds(pmc_csv, fetch_csv):
    """LDS use of the encode kernels on gate_up (the --valu-probe run encodes it once: count, scan,
    emit).  Kernel cycles = GRBM_GUI_ACTIVE / 8 XCDs; the LDS-busy share is SQ_LDS_IDX_ACTIVE /
    (256 CUs x kernel cycles); FETCH_SIZE is scaled by the copy-probe factor of the layer-step
    traffic runs (2.00)."""
    def by_kernel(path):
        agg = {}
        for r in _counter_rows(path):
            for kn in ("k_encode_count", "k_encode_emit"):
                if kn in r["Kernel_Name"]:
                    d = agg.setdefault(kn, {})
                    d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        return agg
    a, f = by_kernel(pmc_csv), by_kernel(fetch_csv)
    cmds = [
        "rocprofv3 --pmc SQ_WAVES SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_WAIT_INST_LDS SQ_INSTS_VALU "
        "SQ_BUSY_CYCLES GRBM_GUI_ACTIVE -f csv -d gpurun_out/pmc_cnt -o run -- python3 bench.py --valu-probe",
        "rocprofv3 --pmc FETCH_SIZE -f csv -d gpurun_out/pmc_cnt2 -o run -- python3 bench.py --valu-probe",
        f"python3 bench.py --summarize-encode-lds {pmc_csv} {fetch_csv}"]
    lines = ["# LDS counters of the encode kernels (gate_up 34816 x 5120), MI355X", "",
             "Commands (run from the repository root):", "", "```"] + cmds + ["```", "",
             "The probe encodes gate_up once. Counters are summed over the GPU. Kernel cycles = GRBM_GUI_ACTIVE / 8",
             "XCDs; the LDS-busy share is SQ_LDS_IDX_ACTIVE / (256 CUs x kernel cycles). FETCH_SIZE is scaled by the",
             "copy-probe factor of the layer-step traffic runs (2.00).", "",
             "| kernel | waves | kernel cycles | LDS instructions per wave | LDS busy share per CU | "
             "conflict cycles / LDS-active cycles | VALU instructions per wave | HBM fetch (MB) |",
             "|---|---|---|---|---|---|---|---|"]
    for kn, c in a.items():
        cyc = c["GRBM_GUI_ACTIVE"] / 8
        lines.append(f"| `{kn}` | {int(c['SQ_WAVES'])} | {int(cyc)} | {c['SQ_INSTS_LDS'] / c['SQ_WAVES']:.0f} | "
                     f"{c['SQ_LDS_IDX_ACTIVE'] / (256 * cyc):.3f} | "
                     f"{c['SQ_LDS_BANK_CONFLICT'] / c['SQ_LDS_IDX_ACTIVE']:.3f} | "
                     f"{c['SQ_INSTS_VALU'] / c['SQ_WAVES']:.0f} | "
                     f"{f.get(kn, {}).get('FETCH_SIZE', 0.0) * 1024 * 2.0 / 1e6:.1f} |")
    path = os.path.join(ROOT, "profiles", "encode_gate_up_lds_counters.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def checkpoint_leg(enc, w_dev, names, reps=3):
    """One layer's W12 checkpoint (w12_file_write), streamed back with w12_file_load through a
    64 MiB pinned staging buffer, with and without the load-time check of each matrix against its
    BF16 source enqueued during the load.  The file was just written, so it is read from the page
    cache: this is the host-to-HBM path, not a disk."""
    import tempfile
    d = tempfile.mkdtemp(prefix="w12ckpt_")
    path = os.path.join(d, "layer0.w12")
    t0 = time.perf_counter()
    w12.save(path, {nm: enc[nm] for nm in names})
    t_save = time.perf_counter() - t0
    file_bytes = os.path.getsize(path)
    staging = torch.empty(64 << 20, dtype=torch.uint8, pin_memory=True)
    res = {}
    for label, refs in (("load_only", None), ("load_and_check", {nm: w_dev[nm] for nm in names})):
        times = []
        for _ in range(reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            got, chk = w12.load(path, refs=refs, staging=staging)
            torch.cuda.synchronize()
            times.append(time.perf_counter() - t0)
            if refs:
                assert chk[:, 0].sum().item() == 0, "checkpoint load-time check failed"
            del got
        t = float(np.median(times))
        res[label] = {"s": round(t, 4), "file_GBps": round(file_bytes / t / 1e9, 2)}
    os.remove(path)
    os.rmdir(d)
    log(f"[bench] checkpoint {file_bytes / 1e6:.0f} MB: load {res['load_only']['file_GBps']} GB/s, "
        f"load + check {res['load_and_check']['file_GBps']} GB/s")
    return {"what": "one layer's W12 file (w12_file_write) streamed to HBM with w12_file_load through 64 MiB of "
                    "pinned staging; the check compares each matrix with its BF16 source during the load; "
                    "the file is read from the page cache", "file_bytes": file_bytes,
            "save_s": round(t_save, 3), **res}


def full_model_leg(dev, stream, n_layers, m, reps=5):
    """The full-model weight stream: n_layers decoder layers (each drawn from its own seed on
    the GPU's generator, see w12_synth.layer_device), encoded (one read-back of the escape counts
    per layer, w12.encode_many) and checked bit for bit at load time, then all 4 n_layers GEMMs
    launched back to back at M=m.  Before every timed pass a
    1 GiB buffer is written, so the pass starts from cold weights (the W12 model is far larger
    than the 256 MB Infinity Cache in any case)."""
    names = list(S.LAYER_ORDER)
    model, res = [], torch.zeros(n_layers, len(names), 2, dtype=torch.int64, device=dev)
    t_enc = t_ver = 0.0
    wbytes = 0
    for li in range(n_layers):
        lay = S.layer_device(li, dev)
        torch.cuda.synchronize()
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record(stream)
        enc = dict(zip(names, w12.encode_many([lay[nm] for nm in names], stream=stream)))
        e1.record(stream)
        for i, nm in enumerate(names):
            w12.verify_async(enc[nm], lay[nm], res[li, i], stream=stream)
        e2.record(stream)
        torch.cuda.synchronize()
        t_enc += e0.elapsed_time(e1)
        t_ver += e1.elapsed_time(e2)
        wbytes += sum(2 * lay[nm].numel() for nm in names)
        model.append(enc)
        del lay
    bad = int(res[:, :, 0].sum().item())
    assert bad == 0, f"full-model load-time check: {bad} mismatching weights"
    # the freed BF16 layers stay in torch's cache: returning memory to the driver right before
    # the timed passes slows the launches that follow it
    escapes = sum(enc[nm].num_escapes for enc in model for nm in names)
    w12_bytes = sum(enc[nm].nbytes() for enc in model for nm in names)
    log(f"[bench] full model: {n_layers} layers, {w12_bytes / 1e9:.2f} GB W12, encode {t_enc:.1f} ms, "
        f"verify {t_ver:.1f} ms")

    xs = {k: dev_bits(S.activations(m, k, S.x_seed(m, k))) for k in {S.LAYER_SHAPES[nm][1] for nm in names}}
    ys = {nm: torch.empty(m, S.LAYER_SHAPES[nm][0], dtype=torch.float32, device=dev) for nm in names}
    wss = {nm: w12.gemm_workspace(m, *S.LAYER_SHAPES[nm]) for nm in names}
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    def one_pass():
        for enc in model:
            for nm in names:
                w12.gemm(xs[S.LAYER_SHAPES[nm][1]], enc[nm], y=ys[nm], ws=wss[nm], stream=stream)

    # grouped: every product of the model in one launch (w12_gemm_group; the argument blocks go
    # to the workspace), and, for comparison, 16 layers (64 products) and 2 layers (8 products,
    # the kernel-argument form) per launch
    ts_all = [enc[nm] for enc in model for nm in names]
    xg = [xs[S.LAYER_SHAPES[nm][1]] for _ in model for nm in names]
    yg = [torch.empty(m, S.LAYER_SHAPES[nm][0], dtype=torch.float32, device=dev) for _ in model for nm in names]
    wsg = w12.gemm_group_workspace(m, ts_all)

    def grouped_pass():
        w12.gemm_group(xg, ts_all, yg, ws=wsg, stream=stream)

    def by_layers(per):
        wsp = w12.gemm_group_workspace(m, ts_all[:4 * per])

        def run():
            for l0 in range(0, len(ts_all), 4 * per):
                w12.gemm_group(xg[l0:l0 + 4 * per], ts_all[l0:l0 + 4 * per], yg[l0:l0 + 4 * per], ws=wsp,
                               stream=stream)
        return run

    def time_pass(fn):
        fn()   # warm-up (code objects, first-touch of the outputs)
        times = []
        for _ in range(reps):
            flush.fill_(reps)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        return times

    times = time_pass(one_pass)
    times_g = time_pass(grouped_pass)
    times_by = {per: time_pass(by_layers(per)) for per in (16, 2) if per < len(model)}
    del flush
    t = float(np.median(times))
    t_g = float(np.median(times_g))
    moved = sum(alg_bytes(enc[nm].n, enc[nm].k, m, enc[nm].num_escapes) for enc in model for nm in names)
    log(f"[bench] full model GEMM pass M={m}: {t:.3f} ms, {wbytes / t / 1e6:.0f} weight-GB/s, "
        f"{moved / t / 1e6:.0f} GB/s moved")
    out = {
        "what": f"{n_layers} decoder layers (4 GEMMs each) resident in HBM, all {4 * n_layers} GEMMs launched "
                f"back to back at M={m} from cold weights; weights drawn on the GPU generator",
        "layers": n_layers, "M": m, "weights_bf16_bytes": wbytes, "w12_bytes": w12_bytes, "escapes": escapes,
        "bits_per_weight": round(w12_bytes * 8 / (wbytes / 2), 5),
        "gemm_pass_ms_median": round(t, 4), "gemm_pass_ms_min": round(min(times), 4), "reps": reps,
        "weight_GBps": round(wbytes / t / 1e6, 1), "bytes_moved_GBps": round(moved / t / 1e6, 1),
        "bytes_moved_frac_of_8TBps": round(moved / t / 1e6 / HBM_PEAK_GBPS, 4),
        "encode_ms": round(t_enc, 3), "encode_GBps": round(wbytes / t_enc / 1e6, 1),
        "verify_ms": round(t_ver, 3), "verify_GBps": round((1.75 * wbytes + 4 * escapes) / t_ver / 1e6, 1),
        "grouped": {
            "what": f"the same {4 * n_layers} products in one launch (w12_gemm_group)",
            "gemm_pass_ms_median": round(t_g, 4), "gemm_pass_ms_min": round(min(times_g), 4),
            "weight_GBps": round(wbytes / t_g / 1e6, 1), "bytes_moved_GBps": round(moved / t_g / 1e6, 1),
            "bytes_moved_frac_of_8TBps": round(moved / t_g / 1e6 / HBM_PEAK_GBPS, 4),
        },
    }
    for per, tp in times_by.items():
        tm = float(np.median(tp))
        out[f"grouped_by_{per}_layers"] = {
            "what": f"the same {4 * n_layers} products, {4 * per} per launch (w12_gemm_group, {per} layers each)",
            "gemm_pass_ms_median": round(tm, 4), "gemm_pass_ms_min": round(min(tp), 4),
            "bytes_moved_frac_of_8TBps": round(moved / tm / 1e6 / HBM_PEAK_GBPS, 4),
        }
    log(f"[bench] full model grouped pass M={m}: {t_g:.3f} ms in one launch, {moved / t_g / 1e6:.0f} GB/s moved; " +
        ", ".join(f"{np.median(tp):.3f} ms at {4 * per} products per launch" for per, tp in times_by.items()))
    del model
    torch.cuda.empty_cache()
    return out


def kernel_name(plan, m, dense=False):
    """Name of the GEMM kernel variant a plan launches (exact pass), as rocprofv3 lists it; dense:
    the escape-window instantiation that escape-dense tensors run (GEMV M <= 4, 16-row tiles, wide
    tiles)."""
    if plan["path"] == 3:
        return f"w12::k_gemm_wide<{plan['m_tile'] // 64}, false, {'true' if dense else 'false'}>"
    path = f"GemvPath<{m}>" if plan["path"] == 1 else f"MfmaPath<{plan['m_tile'] // 16}>"
    dense = dense and (m <= 4 if plan["path"] == 1 else plan["m_tile"] == 16)
    return f"w12::k_gemm<w12::{path}, false, {'true' if dense else 'false'}>"


def traffic_from_profile(alg):
    """HBM bytes per gate_up launch from the committed rocprofv3 counter summary, when it
    matches the current kernel source (else null)."""
    path = os.path.join(ROOT, "profiles", "gemm_gate_up_M16_counters.txt")
    if not os.path.exists(path):
        return {"traffic": None}
    with open(path) as f:
        d = json.load(f)
    src = os.path.join(ROOT, "lossless_bit_weight_encode_amd", "csrc", "w12_gemm.hip")
    import hashlib
    with open(src, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    if d.get("kernel_source_sha256") != digest:
        return {"traffic": None, "traffic_note": "counters predate the current kernel source"}
    return {"traffic": d["hbm_bytes_per_launch"], "traffic_over_alg": round(d["hbm_bytes_per_launch"] / alg, 4)}


def source_stamp() -> str:
    """SHA-256 (first 16 hex digits) of the kernel sources and headers, for the summaries under
    profiles/: a summary whose stamp differs from the tree's predates a kernel change."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "lossless_bit_weight_encode_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def summarize_trace(stats_csv, trace_csv, command):
    """Kernel-time summary of a profiled --only-layer run: rocprofv3's per-kernel stats, plus the
    GEMM durations split by matrix (the four layer GEMMs share one kernel name and are launched
    in layer order)."""
    import csv
    with open(stats_csv) as f:
        stats = list(csv.DictReader(f))
    with open(trace_csv) as f:
        trace = sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))
    gemm = [r for r in trace if "k_gemm" in r["Kernel_Name"]]
    lines = ["# W12 GEMM kernel times: one dense decoder layer (hidden 5120), M=16, MI355X", "",
             "Command (run from the repository root):", "", "```", command, "```", "",
             f"Kernel sources: `csrc/` sha256 {source_stamp()}.", "",
             "## rocprofv3 --stats (all kernels of the run)", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    lines += ["", "## GEMM launches by matrix (kernel trace, layer order qkv, o_proj, gate_up, down)", "",
              "| matrix | kernel | launches | avg us | median us | min us | max us |", "|---|---|---|---|---|---|---|"]
    for i, nm in enumerate(S.LAYER_ORDER):
        rows = gemm[i::len(S.LAYER_ORDER)]
        d = np.array([(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows])
        lines.append(f"| {nm} | `{rows[0]['Kernel_Name'].split('(')[0]}` | {len(d)} | {d.mean():.2f} | "
                     f"{np.median(d):.2f} | {d.min():.2f} | {d.max():.2f} |")
    path = os.path.join(ROOT, "profiles", "gemm_layer_M16_kernel_trace.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_group_trace(stats_csv, trace_csv, command):
    """Kernel-time summary of a profiled --only-group run: rocprofv3's per-kernel stats and the
    grouped GEMM launches (one per layer step: qkv, o_proj, gate_up and down together)."""
    import csv
    with open(stats_csv) as f:
        stats = list(csv.DictReader(f))
    with open(trace_csv) as f:
        trace = sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))
    grp = [r for r in trace if "k_gemm_group" in r["Kernel_Name"]]
    d = np.array([(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in grp])
    moved = 0
    for nm in S.LAYER_ORDER:
        n, k = S.LAYER_SHAPES[nm]
        moved += 1.5 * n * k   # the records dominate; exact bytes are in the bench line
    lines = ["# W12 grouped GEMM: one dense decoder layer (hidden 5120) in one launch, M=16, MI355X", "",
             "Command (run from the repository root):", "", "```", command, "```", "",
             "## rocprofv3 --stats (all kernels of the run)", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    lines += ["", "## Grouped launches (kernel trace)", "",
              "| kernel | launches | avg us | median us | min us | max us | record bytes / avg time |",
              "|---|---|---|---|---|---|---|",
              f"| `{grp[0]['Kernel_Name'].split('(')[0]}` | {len(d)} | {d.mean():.2f} | {np.median(d):.2f} | "
              f"{d.min():.2f} | {d.max():.2f} | {moved / d.mean() / 1e3:.0f} GB/s |"]
    path = os.path.join(ROOT, "profiles", "gemm_group_layer_M16_kernel_trace.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_group_counters(fetch_csv, write_csv, alg_bytes_str):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the grouped layer launches, each scaled by the
    same counter's reading for the 256 MiB torch copy of the same run, against the launch's
    algorithmic bytes."""
    copy_bytes = 256 << 20
    res = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in _counter_rows(path) if r.get("Counter_Name") == name]
        rows.sort(key=lambda r: int(r.get("Dispatch_Id", 0)))
        grp = [float(r["Counter_Value"]) for r in rows if "k_gemm_group" in r["Kernel_Name"]]
        probe = [float(r["Counter_Value"]) for r in rows if "elementwise" in r["Kernel_Name"].lower()]
        if not grp or not probe:
            raise SystemExit(f"{path}: no grouped GEMM or elementwise probe dispatch found")
        scale = copy_bytes / (probe[-1] * 1024.0)
        res[name] = float(np.median(grp)) * 1024 * scale
    alg = float(alg_bytes_str)
    out = {"kernel": "w12::k_gemm_group<w12::MfmaPath<1>> (qkv, o_proj, gate_up and down at M=16 in one launch)",
           "fetch_bytes_per_launch": res["FETCH_SIZE"], "write_bytes_per_launch": res["WRITE_SIZE"],
           "hbm_bytes_per_launch": res["FETCH_SIZE"] + res["WRITE_SIZE"], "alg_bytes_per_launch": alg,
           "traffic_over_alg": round((res["FETCH_SIZE"] + res["WRITE_SIZE"]) / alg, 4),
           "commands": [f"rocprofv3 --pmc {c} -f csv -d gpurun_out/gpmc_{c.split('_')[0].lower()} -o run -- "
                        "python3 bench.py --only-group --steps 3 --warmup 1 --copy-probe"
                        for c in ("FETCH_SIZE", "WRITE_SIZE")],
           "scaling": "each counter is scaled by 256 MiB / (its reading for the probe's elementwise kernel, "
                      "which reads and writes exactly 256 MiB)"}
    path = os.path.join(ROOT, "profiles", "gemm_group_layer_M16_counters.txt")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def _counter_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_counters(fetch_csv, write_csv):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the gate_up GEMM launches, each scaled by
    the same counter's reading for the 256 MiB torch copy of the same run."""
    import hashlib
    copy_bytes = 256 << 20
    res = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in _counter_rows(path) if r.get("Counter_Name") == name]
        rows.sort(key=lambda r: int(r.get("Dispatch_Id", 0)))
        # the layer step launches qkv, o_proj, gate_up, down in that order
        gemms = [float(r["Counter_Value"]) for r in rows if "k_gemm" in r["Kernel_Name"]]
        gate = gemms[S.LAYER_ORDER.index("gate_up")::len(S.LAYER_ORDER)]
        probe = [float(r["Counter_Value"]) for r in rows if "elementwise" in r["Kernel_Name"].lower()]
        if not gate or not probe:
            raise SystemExit(f"{path}: no gate_up GEMM or elementwise probe dispatch found")
        # the probe reads (FETCH) and writes (WRITE) exactly copy_bytes
        scale = copy_bytes / (probe[-1] * 1024.0)
        res[name] = {"gemm_kib_per_dispatch": gate, "copy_kib": probe[-1], "scale": scale}
    layer_gemms = res["FETCH_SIZE"]["gemm_kib_per_dispatch"]
    fetch = float(np.median(res["FETCH_SIZE"]["gemm_kib_per_dispatch"])) * 1024 * res["FETCH_SIZE"]["scale"]
    write = float(np.median(res["WRITE_SIZE"]["gemm_kib_per_dispatch"])) * 1024 * res["WRITE_SIZE"]["scale"]
    src = os.path.join(ROOT, "lossless_bit_weight_encode_amd", "csrc", "w12_gemm.hip")
    with open(src, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    out = {"kernel": "w12::k_gemm<w12::MfmaPath<1>, false, false> (M=16 launches of the layer step)",
           "dispatches": len(layer_gemms), "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
           "hbm_bytes_per_launch": fetch + write,
           "fetch_scale": res["FETCH_SIZE"]["scale"], "write_scale": res["WRITE_SIZE"]["scale"],
           "kernel_source_sha256": digest,
           "commands": [f"rocprofv3 --pmc {c} -f csv -d gpurun_out/pmc_{c.split('_')[0].lower()} -o run -- "
                        "python3 bench.py --only-layer --steps 3 --warmup 1 --copy-probe"
                        for c in ("FETCH_SIZE", "WRITE_SIZE")] +
                       [f"python3 bench.py --summarize-counters {fetch_csv} {write_csv}"],
           "scaling": "each counter is scaled by 256 MiB / (its reading for the probe's elementwise kernel, "
                      "which reads and writes exactly 256 MiB)"}
    path = os.path.join(ROOT, "profiles", "gemm_gate_up_M16_counters.txt")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


HEAVY_M = (16, 256, 512)


def heavy_tail_leg(dev, stream, sweep, batched):
    """GEMM times on the heavy-tail matrices (Student-t weights, 2% values 12..19 binades above the
    bulk; seeds 1000 / 1001 as in the parity tests) at M = 16, 256, 512, over >= 1 GiB of rotated
    encoded copies, with the ratio to the Gaussian matrix of the same shape and M."""
    res = {}
    for nm, seed in (("gate_up", 1000), ("down", 1001)):
        n, k = S.LAYER_SHAPES[nm]
        w = dev_bits(S.heavy_tail_weights(seed, n, k))
        t0 = w12.encode(w)
        del w
        cs = [t0]
        while sum(t.nbytes() for t in cs) < (1 << 30):
            cs.append(clone_tensor(t0))
        e = t0.num_escapes
        res[nm] = {"escapes": e, "escape_frac": round(e / (n * k), 5), "bits_per_weight": round(t0.bits_per_weight(), 4),
                   "rotated_MB": round(sum(t.nbytes() for t in cs) / 1e6, 1)}
        for m in HEAVY_M:
            x = dev_bits(S.activations(m, k, S.x_seed(m, k)))
            y = torch.empty(m, n, dtype=torch.float32, device=dev)
            wsm = w12.gemm_workspace(m, n, k)
            for i in range(3):
                w12.gemm(x, cs[i % len(cs)], y=y, ws=wsm)
            t = timed(lambda i: w12.gemm(x, cs[i % len(cs)], y=y, ws=wsm), 10 if m > 64 else 30, stream)
            ab = alg_bytes(n, k, m, e)
            g = sweep.get(f"{nm}_M{m}") or batched.get(f"{nm}_M{m}")
            res[nm][f"M{m}"] = {
                "us": round(t * 1e3, 2), "weight_GBps": round(2 * n * k / t / 1e6, 1),
                "moved_GBps": round(ab / t / 1e6, 1), "frac": round(ab / t / 1e6 / HBM_PEAK_GBPS, 4),
                "over_gaussian": None if not g else round(t * 1e3 / g["us"], 3),
            }
            log(f"[bench] heavy {nm} M={m}: {t * 1e3:.1f} us ({res[nm][f'M{m}']['over_gaussian']} x gaussian)")
        del cs, t0
        torch.cuda.empty_cache()
    return res


def cpu_baseline(layer, enc, y_timed):
    """The oracle's decode + FP64 GEMM of gate_up at M=16 (the whole matrix), timed 3 times on all
    host cores, once on one thread; and the oracle's encode and decode-compare (decode, then a
    bit-for-bit comparison with the BF16 source) of the same matrix, timed once each.

    The same leg checks the GPU's Y of the last timed layer step (untimed): every gate_up output
    against the reference just computed, and 256 sampled channels of each other matrix."""
    from oracle import w12_oracle as O
    w = layer["gate_up"]
    n, k = w.shape
    log("[bench] cpu baseline: oracle encode of gate_up")
    t0 = time.perf_counter()
    ref = O.encode(w)
    t_enc = time.perf_counter() - t0
    x = S.activations(16, k, S.x_seed(16, k))
    log("[bench] cpu baseline: oracle decode-compare of gate_up")
    t0 = time.perf_counter()
    same = bool(np.array_equal(O.decode(ref), w))
    t_cmp = time.perf_counter() - t0
    assert same, "oracle round trip failed"

    last = {}

    def run():
        t0 = time.perf_counter()
        wd = O.decode(ref)
        last["ya"] = O.gemm_reference(x, wd)
        return time.perf_counter() - t0

    times = []
    for _ in range(3):
        times.append(run())
        log(f"[bench] cpu baseline rep {times[-1]:.2f}s")
    t = float(np.median(times))
    # the timed GPU outputs against the oracle (after all timing)
    y_ref, a_ref = last.pop("ya")
    checked = {"gate_up": {"outputs": int(y_ref.size),
                           "bad": int((~O.within_tolerance(y_timed["gate_up"], y_ref, a_ref)).sum())}}
    del y_ref, a_ref
    rng = np.random.default_rng(7)
    for nm in ("qkv", "o_proj", "down"):
        wn = layer[nm]
        rows = np.sort(rng.choice(wn.shape[0], 256, replace=False))
        xn = S.activations(16, wn.shape[1], S.x_seed(16, wn.shape[1]))
        bad, _ = O.gemm_check(xn, wn[rows], y_timed[nm][:, rows])
        checked[nm] = {"outputs": 16 * len(rows), "bad": int(bad)}
    log(f"[bench] timed outputs against the oracle: {checked}")
    assert all(c["bad"] == 0 for c in checked.values()), f"timed GEMM outputs fail the oracle check: {checked}"
    blas_threads, t1 = None, None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        with threadpool_limits(limits=1):
            t1 = run()
        log(f"[bench] cpu baseline one thread {t1:.2f}s")
    except Exception:
        pass
    return {
        "value": round(2 * n * k / t / 1e9, 3), "unit": "GB/s", "cores": len(os.sched_getaffinity(0)),
        "blas_threads": blas_threads, "kind": "oracle",
        "sample": f"gate_up {n}x{k}, M=16: oracle decode + FP64 GEMM, median of 3 runs ({t:.2f} s each)",
        "one_thread": None if t1 is None else {"s": round(t1, 3), "GBps": round(2 * n * k / t1 / 1e9, 3)},
        "oracle_encode": {"s": round(t_enc, 3), "GBps": round(2 * n * k / t_enc / 1e9, 3)},
        "oracle_decode_compare": {"s": round(t_cmp, 3), "GBps": round(2 * n * k / t_cmp / 1e9, 3)},
        "timed_outputs_checked": checked,
    }


def cpu_legs(n_layers, layer_range=None):
    """The oracle on all host cores for the other workloads (BASELINE plan): the tiny case
    (encode, decode-compare, GEMM at M=1), the tree-verify M sweep and the batched M on gate_up
    and down (decode + FP64 GEMM, median of 3), the heavy-tail matrices (encode + decode + GEMM
    at M=16), and the full model streamed one layer at a time (generate, encode, decode-compare,
    FP64 GEMM at M=32 for each of the four matrices; the real total over n_layers layers, with
    the generation time reported apart)."""
    from oracle import w12_oracle as O

    def med3(f):
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            f()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts))

    res = {"cores": len(os.sched_getaffinity(0)), "kind": "oracle", "unit": "s"}
    try:
        from threadpoolctl import threadpool_info
        res["blas_threads"] = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        res["blas_threads"] = None
    if layer_range is not None:
        res["full_model"] = full_model_cpu(*layer_range)
        return res
    w = S.tiny_weights(0)
    x = S.activations(1, w.shape[1], S.x_seed(1, w.shape[1]))
    ref = O.encode(w)
    res["tiny"] = {"encode": med3(lambda: O.encode(w)),
                   "decode_compare": med3(lambda: np.array_equal(O.decode(ref), w)),
                   "gemm_M1": med3(lambda: O.gemm_reference(x, O.decode(ref)))}
    log(f"[cpu] tiny {res['tiny']}")
    lay = S.layer(0, which=("gate_up", "down"))
    for leg, ms in (("tree_sweep", S.TREE_M_SWEEP), ("batched", S.BATCHED_M)):
        res[leg] = {}
        for nm in ("gate_up", "down"):
            wn = lay[nm]
            refn = O.encode(wn)
            for m in ms:
                xm = S.activations(m, wn.shape[1], S.x_seed(m, wn.shape[1]))
                res[leg][f"{nm}_M{m}"] = med3(lambda: O.gemm_reference(xm, O.decode(refn)))
                log(f"[cpu] {leg} {nm} M={m}: {res[leg][f'{nm}_M{m}']:.2f} s")
    del lay
    res["heavy_tail"] = {}
    for nm, seed in (("gate_up", 1000), ("down", 1001)):
        n, k = S.LAYER_SHAPES[nm]
        wh = S.heavy_tail_weights(seed, n, k)
        xh = S.activations(16, k, S.x_seed(16, k))
        t0 = time.perf_counter()
        refh = O.encode(wh)
        t_enc = time.perf_counter() - t0
        res["heavy_tail"][nm] = {"escapes": int(refh.num_escapes), "encode": t_enc,
                                 "gemm_M16": med3(lambda: O.gemm_reference(xh, O.decode(refh)))}
        log(f"[cpu] heavy {nm} {res['heavy_tail'][nm]}")
        del wh, refh
    res["full_model"] = full_model_cpu(0, n_layers)
    return res


def summarize_cpu_legs(paths):
    """profiles/cpu_oracle_legs.md from --cpu-legs JSON lines: the legs of one run, and the full
    model summed over runs that cover disjoint layer ranges (all 64 layers between them)."""
    runs = []
    for p in paths:
        with open(p) as f:
            runs.append(json.loads([ln for ln in f.read().splitlines() if ln.startswith("{")][-1]))
    legs = next(r for r in runs if "tree_sweep" in r)
    parts = [r["full_model"] for r in runs if r.get("full_model", {}).get("layers", [0, 0])[1] >
             r.get("full_model", {}).get("layers", [0, 0])[0]]
    layers = sorted(i for a, b in (p["layers"] for p in parts) for i in range(a, b))
    assert len(layers) == len(set(layers)), "the layer ranges overlap"
    cores = {r["cores"] for r in runs}
    gbps = lambda nm, t: 2 * S.LAYER_SHAPES[nm][0] * S.LAYER_SHAPES[nm][1] / t / 1e9
    lines = ["# The CPU oracle on the other workloads (host cores of the MI355X box)", "",
             "Commands (run from the repository root; the full model in two parts whose layer ranges cover 0..63):",
             "", "```", "python3 bench.py --cpu-legs --model-layers 0", "python3 bench.py --cpu-legs --cpu-layers 0 16",
             "python3 bench.py --cpu-legs --cpu-layers 16 64",
             "python3 bench.py --summarize-cpu-legs <the three JSON outputs>", "```", "",
             f"The oracle as it stands (numpy, FP64 GEMM through the BLAS), {sorted(cores)} cores, "
             f"{legs.get('blas_threads')} BLAS threads. GEMM legs: decode + FP64 GEMM (+ the sum of |x w|), median "
             "of 3; GB/s = BF16 bytes of W (2NK) per second. A reported baseline, not a target.", "",
             "| leg | case | seconds | GB/s (2NK / t) |", "|---|---|---|---|"]
    t = legs["tiny"]
    lines.append(f"| tiny 256x512 | encode / decode-compare / GEMM M=1 | {t['encode']:.4f} / "
                 f"{t['decode_compare']:.4f} / {t['gemm_M1']:.4f} | - |")
    for leg in ("tree_sweep", "batched"):
        for key, v in legs[leg].items():
            nm = key.split("_M")[0]
            lines.append(f"| {leg} | {key} | {v:.3f} | {gbps(nm, v):.3f} |")
    for nm, v in legs["heavy_tail"].items():
        lines.append(f"| heavy_tail | {nm} (E = {v['escapes']}): encode / GEMM M=16 | {v['encode']:.3f} / "
                     f"{v['gemm_M16']:.3f} | {gbps(nm, v['gemm_M16']):.3f} (GEMM) |")
    if layers:
        tot = sum(p["oracle_s"] for p in parts)
        gen = sum(p["generation_s"] for p in parts)
        wb = len(layers) * sum(2 * n * k for n, k in S.LAYER_SHAPES.values())
        lines += ["", f"Full model, one layer at a time: layers {layers[0]}..{layers[-1]} "
                      f"({len(layers)} layers{'' if layers == list(range(len(layers))) else ', with gaps'}), per layer "
                      "the oracle's encode, decode-compare and FP64 GEMM at M = 32 of qkv, o_proj, gate_up and down: "
                      f"**{tot:.1f} s** in all ({wb / tot / 1e9:.3f} GB/s of BF16 weights), plus {gen:.1f} s to draw "
                      "the layers (not counted)."]
    path = os.path.join(ROOT, "profiles", "cpu_oracle_legs.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def full_model_cpu(first, end):
    """The oracle over layers first..end-1 of the full model, one layer at a time."""
    from oracle import w12_oracle as O
    t_gen = t_work = 0.0
    for seed in range(first, end):
        t0 = time.perf_counter()
        lay = S.layer(seed)
        t_gen += time.perf_counter() - t0
        t0 = time.perf_counter()
        for nm in S.LAYER_ORDER:
            wn = lay[nm]
            r = O.encode(wn)
            assert np.array_equal(O.decode(r), wn)
            O.gemm_reference(S.activations(32, wn.shape[1], S.x_seed(32, wn.shape[1])), O.decode(r))
        t_work += time.perf_counter() - t0
        log(f"[cpu] full model layer {seed}: {t_work:.1f} s so far")
    return {"layers": [first, end], "M": 32, "oracle_s": t_work, "generation_s": t_gen,
            "what": "encode + decode-compare + FP64 GEMM of qkv, o_proj, gate_up, down per layer"}


if __name__ == "__main__":
    main()
