#!/usr/bin/env python3
"""Benchmark of the fused SwiGLU + MXFP8 cast on one MI355X.

A step is one pass of the hot path over one batch: the fused forward and
the fused backward, each emitting both scale layouts (rowwise 1x32 and
colwise 32x1) in one launch, on 131072 x 8192 activations (gate/up the two
halves of a 131072 x 16384 bf16 w13 tensor, dh 131072 x 8192; N(0, 1)
synthetic values).  Throughput is achieved HBM bandwidth: algorithmic bytes
(inputs read once, E4M3 data and E8M0 scales written once per layout) over
time, the accounting the pages' tables use ("Add swiglu + MXFP8 fused CuTe
DSL kernel", Performance).  Inputs are resident in HBM before timing.

Prints ONE JSON line.  Extra fields: `roofline` (dominant kernel, HIP-event
timing on the launch stream), `cpu_baseline` (the CPU oracle on a bounded
sample of the same workload), `detail` (each op and layout alone, the other
gated activations, the MX GEMM consumer against the fp8 MFMA peak, the 3D
expert cast, and the streaming ceilings: a plain streaming kernel timed at
each call's read:write byte mix, with each call's share of it).  Before
timing, random 32-row slabs of the outputs are checked against the oracle
(`validation`: scale-mismatch and one-code rates per direction and layout).

`--sweep` prints instead a markdown table over the pages' shapes: every
direction and layout, fused and unfused (the activation written as bf16,
then the plain cast), with the pages' columns ("Add swiglu + MXFP8 fused
CuTe DSL kernel", Performance), and the 3D expert cast over 1 to 64 experts
of 8192 x 5120 ("[mxfp8 moe training] update 3d quant colwise scaling
kernel to use single input/output TMA descriptors", Performance).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused SwiGLU+MXFP8 cast achieved HBM GB/s (% of peak), fwd/bwd, both scales"
M_ROWS, N_COLS = 131072, 8192
WORKLOAD = "swiglu_131072x8192_w13"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_swiglu_131072x8192_bench.txt")


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--cpu-slabs", type=int, default=512,
                   help="32-row slabs of the workload the CPU oracle processes on all host cores")
    p.add_argument("--cpu-slabs-1t", type=int, default=48, help="slabs for the single-thread oracle figure")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    p.add_argument("--no-detail", action="store_true", help="skip the per-op breakdown")
    p.add_argument("--detail-set", choices=("full", "core"), default="full",
                   help="core: only the per-layout casts, the gated casts and the streaming ceilings "
                        "(shorter runs under counter collection)")
    p.add_argument("--validate-slabs", type=int, default=64,
                   help="random 32-row slabs checked against the oracle before timing (0: none)")
    p.add_argument("--sweep", action="store_true", help="print the per-shape table instead of the JSON line")
    return p.parse_args()


def kernel_source_hash() -> str:
    from swiglu_activation_cast_amd._build import kernel_source_hash as h

    return h()


def measured_traffic(src_hash: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (rocprofv3 FETCH_SIZE and WRITE_SIZE, calibrated on a device copy), or
    None when that summary was taken with different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    fields = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if not line.startswith("#") and ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_hash") != src_hash:
        return None
    v = fields.get(f"{kernel}_hbm_bytes_per_launch")
    return int(v) if v is not None else None


# Spin cycles that hold the stream while the host queues a timed series
# (a few milliseconds at the shader clock): far longer than the host needs
# to enqueue 20 launches with their events.
BACKLOG_CYCLES = 5_000_000


def time_launches(fn, iters, warmup, backlog=False):
    """Average and median duration (s) of fn's launch, HIP events on torch's
    current stream (the stream the binding launches on).

    With backlog, the stream first runs a short spin kernel, so every launch
    and event of the series is queued before the first one starts and the
    launches run back to back: the events then time the kernels alone.
    Without it, a launch shorter than the host's time per call (about 14 us
    from Python) is timed with the host's gap before it."""
    import torch

    for _ in range(warmup):
        fn()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    torch.cuda.synchronize()
    if backlog:
        torch.cuda._sleep(BACKLOG_CYCLES)
    for i in range(iters):
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    ms = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    return sum(ms) / len(ms) / 1e3, ms[len(ms) // 2] / 1e3


def host_threads() -> int:
    """Threads for host-side oracle work: the CPU share the process is given
    (OMP_NUM_THREADS when set, else the usable cores), at most 16."""
    env = os.environ.get("OMP_NUM_THREADS")
    n = int(env) if env and env.isdigit() else len(os.sched_getaffinity(0))
    return max(1, min(16, n))


def _slab_bits(inp, slabs):
    """Host copies (bf16 bits) of gate, up and dh for each 32-row slab."""
    import numpy as np
    import torch

    def bits(t):
        return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    return {sb: tuple(bits(t[sb * 32:sb * 32 + 32]) for t in (inp.gate, inp.up, inp.dh)) for sb in slabs}


def _oracle_step(host):
    """The oracle on one slab: fused forward and backward, both layouts."""
    import oracle

    g, u, dh = host
    oracle.swiglu_fwd(g, u, oracle.BOTH)
    oracle.swiglu_bwd(dh, g, u, oracle.BOTH)


def cpu_baseline(inp, n_slabs: int, n_slabs_1t: int):
    """The oracle as it stands (plain single-threaded C) on a random sample of
    32-row slabs of the workload, fused forward + backward, both layouts:
    once spread over the host cores (one slab per call, calls from a thread
    pool; the C code releases the interpreter lock), once on one thread."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    from swiglu_activation_cast_amd import metrics

    rng = np.random.default_rng(1234)
    slabs = sorted(rng.choice(M_ROWS // 32, size=n_slabs, replace=False).tolist())
    host = _slab_bits(inp, slabs)
    threads = host_threads()
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as pool:
        list(pool.map(_oracle_step, host.values()))
    dt = time.perf_counter() - t0
    t0 = time.perf_counter()
    for sb in slabs[:n_slabs_1t]:
        _oracle_step(host[sb])
    dt1 = time.perf_counter() - t0
    rows, rows1 = 32 * len(slabs), 32 * min(n_slabs_1t, len(slabs))
    per_row = (metrics.swiglu_fwd_bytes(1, N_COLS, 3) + metrics.swiglu_bwd_bytes(1, N_COLS, 3))
    return {
        "value": round(metrics.gbps(per_row * rows, dt), 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{len(slabs)} random 32-row slabs ({rows} of {M_ROWS} rows) of the {M_ROWS}x{N_COLS} workload, "
                  f"fused fwd + bwd, both layouts: {dt:.1f} s on {threads} threads",
        "seconds": round(dt, 3),
        "single_thread": {"value": round(metrics.gbps(per_row * rows1, dt1), 4), "unit": "GB/s",
                          "rows": rows1, "seconds": round(dt1, 3)},
        "cpu": _cpu_model(),
        "host_cores_visible": os.cpu_count(),
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def validate(inp, fwd_out, bwd_out, n_slabs: int):
    """Random 32-row slabs of the benchmark's own outputs (forward and
    backward, both layouts in one launch each) against the oracle, with the
    fused casts' bar (oracle/parity.py): codes within one E4M3 step, scales
    bit-exact except next to a power-of-two boundary, such blocks at most
    1e-4 of all.  Runs before timing; returns the rates per direction and
    layout."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch

    import oracle
    from oracle.parity import compare_fused, layout_parts
    import swiglu_activation_cast_amd as mx

    mx.mxfp8_swiglu_fwd(inp.gate, inp.up, rowwise=True, colwise=True, out=fwd_out)
    mx.mxfp8_swiglu_bwd(inp.dh, inp.gate, inp.up, rowwise=True, colwise=True, out=bwd_out)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4321)
    slabs = sorted(set(rng.choice(M_ROWS // 32, size=n_slabs, replace=False).tolist()) | {0, M_ROWS // 32 - 1})
    host = _slab_bits(inp, slabs)

    def ref(sb):
        g, u, dh = host[sb]
        dg, du = oracle.swiglu_bwd_values(dh, g, u)
        return sb, (oracle.swiglu_fwd(g, u, oracle.BOTH), oracle.swiglu_fwd_values(g, u)), \
            (oracle.swiglu_bwd(dh, g, u, oracle.BOTH), np.concatenate([dg, du], axis=1))

    with ThreadPoolExecutor(max_workers=host_threads()) as pool:
        refs = list(pool.map(ref, slabs))
    totals = {}
    for sb, *per_dir in refs:
        r0, r1 = sb * 32, sb * 32 + 32
        for direction, outs, (orc, vals) in zip(("fwd", "bwd"), (fwd_out, bwd_out), per_dir):
            q_row, q_col, s_row, s_col = outs
            gpu = (q_row[r0:r1].cpu().numpy(), s_row[r0:r1].cpu().numpy(), q_col[:, r0:r1].cpu().numpy(),
                   s_col[:, sb:sb + 1].cpu().numpy())
            try:
                st = compare_fused(oracle, f"{direction}/slab{sb}", gpu, orc, vals, 3)
            except AssertionError as e:
                raise SystemExit(f"validation failed: {e}")
            for lay, part in layout_parts(st).items():
                key = f"{direction}_{lay}"
                totals[key] = totals[key].merge(part) if key in totals else part
    res = {"slabs": len(slabs), "rows": 32 * len(slabs)}
    for key, st in totals.items():
        if st.scale_mismatch_rate > 1e-4:
            raise SystemExit(f"validation failed: {key} scale mismatch rate {st.scale_mismatch_rate:.2e} > 1e-4")
        res[key] = {"blocks": st.blocks, "scale_mismatch_rate": st.scale_mismatch_rate,
                    "one_code_rate": st.one_code_rate}
    print(f"bench: validated {len(slabs)} slabs against the oracle", file=sys.stderr, flush=True)
    return res


SWEEP_SHAPES = ((128, 128), (4096, 2048), (4096, 7168), (16384, 7168), (131072, 8192))
SWEEP_EXPERTS = (1, 2, 4, 8, 16, 32, 64)


def run_sweep():
    """The pages' table on MI355X: fused and unfused time, speedup and
    achieved HBM GB/s for every shape, direction and layout; then the 3D
    expert cast.  Inputs: gate/up the halves of one N(0, 1) bf16 w13 tensor,
    dh N(0, 1); experts N(0, 0.02).  Times are medians of 20 launches run
    back to back behind a spin kernel (kernel time; at the small shapes one
    stalled launch would move a mean by a third); the last column times the
    same fused call launched from Python one at a time, the host's
    overhead included."""
    import torch

    import swiglu_activation_cast_amd as mx
    from swiglu_activation_cast_amd import metrics, synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    print("| input_shape (M, K) | direction | scales | unfused µs | fused µs | speedup | fused GB/s | % of 8 TB/s "
          "| fused µs per call from Python |")
    print("|---|---|---|---|---|---|---|---|---|")
    for M, N in SWEEP_SHAPES:
        inp = synth.swiglu_inputs(M, N, seed=5, std=1.0, packed=True, device=dev)
        outs = {"forward": mx.alloc_outputs(M, N, mx.BOTH, dev), "backward": mx.alloc_outputs(M, 2 * N, mx.BOTH, dev)}
        vals = {"forward": torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                "backward": torch.empty((M, 2 * N), dtype=torch.bfloat16, device=dev)}
        for direction in ("forward", "backward"):
            out, v = outs[direction], vals[direction]
            for lay, lname in ((mx.ROWWISE, "rowwise"), (mx.COLWISE, "colwise"), (mx.BOTH, "both")):
                fl = dict(rowwise=bool(lay & 1), colwise=bool(lay & 2))
                if direction == "forward":
                    fused = lambda: mx.mxfp8_swiglu_fwd(inp.gate, inp.up, out=out, stream=stream, **fl)

                    def unfused():
                        mx.mxfp8_swiglu_fwd_bf16(inp.gate, inp.up, out=v, stream=stream)
                        mx.mxfp8_quant_2d(v, out=out, stream=stream, **fl)
                    nbytes = metrics.swiglu_fwd_bytes(M, N, lay)
                else:
                    fused = lambda: mx.mxfp8_swiglu_bwd(inp.dh, inp.gate, inp.up, out=out, stream=stream, **fl)

                    def unfused():
                        mx.mxfp8_swiglu_bwd_bf16(inp.dh, inp.gate, inp.up, out=v, stream=stream)
                        mx.mxfp8_quant_2d(v, out=out, stream=stream, **fl)
                    nbytes = metrics.swiglu_bwd_bytes(M, N, lay)
                _, tu = time_launches(unfused, 20, 10, backlog=True)
                _, tf = time_launches(fused, 20, 10, backlog=True)
                _, tc = time_launches(fused, 20, 10)
                gbps = metrics.gbps(nbytes, tf)
                print(f"| ({M}, {N}) | {direction} | {lname} | {tu * 1e6:.2f} | {tf * 1e6:.2f} | {tu / tf:.2f}× | "
                      f"{gbps:.1f} | {100 * gbps / metrics.HBM_PEAK_GBPS:.1f}% | {tc * 1e6:.2f} |", flush=True)
        del inp, outs, vals
        torch.cuda.empty_cache()
    print()
    print("| experts (E, 8192, 5120) | 3D colwise µs | GB/s | % of 8 TB/s |")
    print("|---|---|---|---|")
    for E in SWEEP_EXPERTS:
        w = synth.expert_weights(E, 8192, 5120, seed=3 + E, device=dev)
        q = torch.empty((E, 5120, 8192), dtype=torch.uint8, device=dev)
        sc = torch.empty((E, 5120, 256), dtype=torch.uint8, device=dev)
        _, t = time_launches(lambda: mx.mxfp8_quant_3d_colwise(w, out=(q, sc), stream=stream), 20, 10, backlog=True)
        gbps = metrics.gbps(metrics.quant_3d_bytes(E, 8192, 5120), t)
        print(f"| ({E}, 8192, 5120) | {t * 1e6:.2f} | {gbps:.1f} | {100 * gbps / metrics.HBM_PEAK_GBPS:.1f}% |", flush=True)
        del w, q, sc
        torch.cuda.empty_cache()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the cast shards rows or experts "
              "across GPUs with no exchange, so the one-GPU number is the per-GPU figure.", file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        run_sweep()
        return

    import torch

    import swiglu_activation_cast_amd as mx
    from swiglu_activation_cast_amd import metrics, synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    print(f"bench: generating {WORKLOAD} on {torch.cuda.get_device_name(dev)}", file=sys.stderr, flush=True)
    inp = synth.workload(WORKLOAD, device=dev)

    M, N = M_ROWS, N_COLS
    fwd_out = mx.alloc_outputs(M, N, mx.BOTH, dev)
    bwd_out = mx.alloc_outputs(M, 2 * N, mx.BOTH, dev)
    stream = torch.cuda.current_stream(dev)
    validation = validate(inp, fwd_out, bwd_out, args.validate_slabs) if args.validate_slabs > 0 else None

    def fwd():
        mx.mxfp8_swiglu_fwd(inp.gate, inp.up, rowwise=True, colwise=True, out=fwd_out, stream=stream)

    def bwd():
        mx.mxfp8_swiglu_bwd(inp.dh, inp.gate, inp.up, rowwise=True, colwise=True, out=bwd_out, stream=stream)

    fwd_bytes = metrics.swiglu_fwd_bytes(M, N, mx.BOTH)
    bwd_bytes = metrics.swiglu_bwd_bytes(M, N, mx.BOTH)
    step_bytes = fwd_bytes + bwd_bytes

    # ---- the step: warmup, then exactly K timed steps between synchronizations
    for _ in range(args.warmup):
        fwd()
        bwd()
    ev_f = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    ev_b = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev_f[i][0].record(stream)
        fwd()
        ev_f[i][1].record(stream)
        ev_b[i][0].record(stream)
        bwd()
        ev_b[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"bench: {args.steps} steps done", file=sys.stderr, flush=True)
    fwd_s = sum(a.elapsed_time(b) for a, b in ev_f) / args.steps / 1e3
    bwd_s = sum(a.elapsed_time(b) for a, b in ev_b) / args.steps / 1e3
    step_s = wall / args.steps
    value = metrics.gbps(step_bytes, step_s)

    # ---- roofline of the dominant kernel (the backward, both layouts)
    dom_bytes, dom_s, dom_name = (bwd_bytes, bwd_s, "k_tiled<OpBwd, rowwise+colwise>")
    if fwd_s > bwd_s:
        dom_bytes, dom_s, dom_name = (fwd_bytes, fwd_s, "k_tiled<OpFwd, rowwise+colwise>")
    achieved = metrics.gbps(dom_bytes, dom_s)
    src_hash = kernel_source_hash()
    traffic = measured_traffic(src_hash, "bwd_both" if dom_bytes == bwd_bytes else "fwd_both")
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": metrics.HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / metrics.HBM_PEAK_GBPS, 4),
        "traffic": traffic,
        "kernel": dom_name,
        "algorithmic_bytes": dom_bytes,
        "avg_launch_us": round(dom_s * 1e6, 2),
    }

    detail = {}
    if not args.no_detail:
        detail = run_detail(inp, fwd_out, bwd_out, stream, core_only=args.detail_set == "core")
        mix = CALL_MIX["bwd_both" if dom_bytes == bwd_bytes else "fwd_both"]
        ceil = detail["stream_ceilings"][mix]["GB/s"]
        roofline["stream_ceiling"] = {"mix": mix, "GB/s": ceil, "frac_of_ceiling": round(achieved / ceil, 4)}

    cpu = None
    if not args.no_cpu:
        print("bench: timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(inp, args.cpu_slabs, args.cpu_slabs_1t)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "fused SwiGLU fwd + bwd, rowwise+colwise MXFP8 in one pass each, M=131072, N=8192, "
                        "gate/up halves of a bf16 w13 [131072, 16384], dh [131072, 8192], N(0,1)",
            "M": M,
            "N": N,
            "layout": "both",
            "step_bytes": step_bytes,
            "fraction_of_peak": round(value / metrics.HBM_PEAK_GBPS, 4),
            "fwd_us": round(fwd_s * 1e6, 2),
            "bwd_us": round(bwd_s * 1e6, 2),
            "kernel_source_hash": src_hash,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "validation": validation,
        "detail": detail,
    }
    print(json.dumps(out), flush=True)


# read:write byte mix of each call (inputs : outputs per element): forward
# 4 : 1.03 per layout, backward 6 : 2.06 per layout, the plain casts 2 : 1.03
from swiglu_activation_cast_amd.metrics import STREAM_CONFIGS  # noqa: E402

STREAM_MIXES = {"4:1": (4, 1), "2:1": (2, 1), "3:1": (3, 1), "3:2": (3, 2), "1:1": (1, 1)}
CALL_MIX = {"fwd_row": "4:1", "fwd_col": "4:1", "fwd_both": "2:1", "bwd_row": "3:1", "bwd_col": "3:1",
            "bwd_both": "3:2", "quant2d_row": "2:1", "quant2d_col": "2:1", "quant3d_E64": "2:1",
            "bwd_both_grouped_g8": "3:2", "quant2d_col_grouped_g8": "2:1",
            **{f"{a}_{d}_both": m for a in ("gelu_tanh", "gelu", "relu") for d, m in (("fwd", "2:1"), ("bwd", "3:2"))}}


def stream_ceilings(inp, bwd_out, stream):
    """What plain streaming reaches at each read:write mix: the probe kernel
    (nontemporal 16-byte accesses, as the casts use) over 1 GiB buffers, the
    best of a few grid sizes and accesses in flight.  Inputs are 1 GiB slices
    of the w13 tensor, outputs slices of the backward's rowwise output."""
    import torch

    from swiglu_activation_cast_amd import metrics, stream_probe

    gib = 1 << 30
    src = inp.w13.view(torch.uint8).view(-1)
    dst = bwd_out[0].view(-1)
    ins = [src[i * gib:(i + 1) * gib] for i in range(4)]
    outs = [dst[:gib], dst[gib:2 * gib]]
    res = {}
    for name, (nr, nw) in STREAM_MIXES.items():
        best = None
        for unroll, grid in STREAM_CONFIGS:
            fn = lambda: stream_probe.mix(ins[:nr], outs[:nw], gib, unroll=unroll, grid=grid, stream=stream)
            t, _ = time_launches(fn, 5, 2)
            gbps = metrics.gbps((nr + nw) * gib, t)
            if best is None or gbps > best[0]:
                best = (gbps, unroll, grid, t)
        res[name] = {"GB/s": round(best[0], 1), "frac": round(best[0] / metrics.HBM_PEAK_GBPS, 4),
                     "unroll": best[1], "grid": best[2], "us": round(best[3] * 1e6, 2)}
    print("bench: stream ceilings done", file=sys.stderr, flush=True)
    return res


def run_detail(inp, fwd_out, bwd_out, stream, core_only=False):
    """Each op and layout alone at the same size, the 3D expert cast, and a
    device copy of the w13 tensor as a bandwidth ceiling."""
    import torch

    import swiglu_activation_cast_amd as mx
    from swiglu_activation_cast_amd import metrics, synth

    M, N = M_ROWS, N_COLS
    res = {}
    for lay, name in ((mx.ROWWISE, "row"), (mx.COLWISE, "col"), (mx.BOTH, "both")):
        fl = dict(rowwise=bool(lay & 1), colwise=bool(lay & 2))
        f = lambda: mx.mxfp8_swiglu_fwd(inp.gate, inp.up, out=fwd_out, stream=stream, **fl)
        b = lambda: mx.mxfp8_swiglu_bwd(inp.dh, inp.gate, inp.up, out=bwd_out, stream=stream, **fl)
        for op, fn, nbytes in (("fwd", f, metrics.swiglu_fwd_bytes(M, N, lay)),
                               ("bwd", b, metrics.swiglu_bwd_bytes(M, N, lay))):
            avg, med = time_launches(fn, 10, 2)
            res[f"{op}_{name}"] = {"us": round(avg * 1e6, 2), "GB/s": round(metrics.gbps(nbytes, avg), 1),
                                   "frac": round(metrics.gbps(nbytes, avg) / metrics.HBM_PEAK_GBPS, 4)}
    print("bench: per-layout timing done", file=sys.stderr, flush=True)
    # the other gated activations, both layouts in one pass, same inputs
    for act in ("gelu_tanh", "gelu", "relu"):
        f = lambda: mx.mxfp8_gated_fwd(inp.gate, inp.up, act=act, rowwise=True, colwise=True, out=fwd_out,
                                       stream=stream)
        b = lambda: mx.mxfp8_gated_bwd(inp.dh, inp.gate, inp.up, act=act, rowwise=True, colwise=True, out=bwd_out,
                                       stream=stream)
        for op, fn, nbytes in (("fwd", f, metrics.swiglu_fwd_bytes(M, N, mx.BOTH)),
                               ("bwd", b, metrics.swiglu_bwd_bytes(M, N, mx.BOTH))):
            avg, _ = time_launches(fn, 10, 2)
            res[f"{act}_{op}_both"] = {"us": round(avg * 1e6, 2), "GB/s": round(metrics.gbps(nbytes, avg), 1),
                                       "frac": round(metrics.gbps(nbytes, avg) / metrics.HBM_PEAK_GBPS, 4)}
    print("bench: gated activations done", file=sys.stderr, flush=True)
    if core_only:
        res["stream_ceilings"] = stream_ceilings(inp, bwd_out, stream)
        return res
    # the unfused two-kernel pipeline (bf16 activation written, then the plain
    # cast of it), both layouts: the pages' baseline structure
    h = torch.empty((M, N), dtype=torch.bfloat16, device=inp.gate.device)
    y = torch.empty((M, 2 * N), dtype=torch.bfloat16, device=inp.gate.device)

    def unfused_fwd():
        mx.mxfp8_swiglu_fwd_bf16(inp.gate, inp.up, out=h, stream=stream)
        mx.mxfp8_quant_2d(h, rowwise=True, colwise=True, out=fwd_out, stream=stream)

    def unfused_bwd():
        mx.mxfp8_swiglu_bwd_bf16(inp.dh, inp.gate, inp.up, out=y, stream=stream)
        mx.mxfp8_quant_2d(y, rowwise=True, colwise=True, out=bwd_out, stream=stream)

    for name, fn, fused in (("unfused_fwd_both", unfused_fwd, "fwd_both"), ("unfused_bwd_both", unfused_bwd, "bwd_both")):
        avg, _ = time_launches(fn, 10, 2)
        res[name] = {"us": round(avg * 1e6, 2), "fused_speedup": round(avg * 1e6 / res[fused]["us"], 3)}
    del h, y
    torch.cuda.empty_cache()
    # plain 2D cast of the gate half (colwise, the "dim1" cast) and rowwise
    for lay, name in ((mx.ROWWISE, "row"), (mx.COLWISE, "col")):
        fl = dict(rowwise=bool(lay & 1), colwise=bool(lay & 2))
        fn = lambda: mx.mxfp8_quant_2d(inp.dh, out=fwd_out, stream=stream, **fl)
        avg, _ = time_launches(fn, 10, 2)
        nb = metrics.quant_2d_bytes(M, N, lay)
        res[f"quant2d_{name}"] = {"us": round(avg * 1e6, 2), "GB/s": round(metrics.gbps(nb, avg), 1),
                                  "frac": round(metrics.gbps(nb, avg) / metrics.HBM_PEAK_GBPS, 4)}
    # streaming ceilings at the calls' read:write byte mixes (libmxstream.so),
    # and each call's share of the ceiling at its own mix
    res["stream_ceilings"] = stream_ceilings(inp, bwd_out, stream)
    for name, mix in CALL_MIX.items():
        if name in res and "GB/s" in res[name]:
            res[name]["mix"] = mix
            res[name]["frac_of_stream_ceiling"] = round(res[name]["GB/s"] / res["stream_ceilings"][mix]["GB/s"], 4)
    # torch's device copy of the 4 GiB w13 tensor (context only: a copy kernel
    # of known size, not a ceiling)
    dst = torch.empty_like(inp.w13)
    avg, _ = time_launches(lambda: dst.copy_(inp.w13), 10, 2)
    res["torch_copy_w13"] = {"us": round(avg * 1e6, 2), "GB/s": round(metrics.gbps(2 * inp.w13.numel() * 2, avg), 1)}
    del dst
    torch.cuda.empty_cache()
    # the consumer: MX GEMM C = A B^T on cast outputs, 16384 x 8192 x 5120
    # (A the rowwise cast of activations, B of weights); fp8 MFMA roofline
    gm, gn, gk = 16384, 8192, 5120
    x = synth.normal_bf16((gm, gk), 1.0, seed=70, device=inp.gate.device)
    w = synth.normal_bf16((gn, gk), 0.02, seed=71, device=inp.gate.device)
    qa, _, sa, _ = mx.mxfp8_quant_2d(x, rowwise=True, stream=stream)
    qb, _, sb, _ = mx.mxfp8_quant_2d(w, rowwise=True, stream=stream)
    del x, w
    cg = torch.empty((gm, gn), dtype=torch.float32, device=inp.gate.device)
    # 10 warm-up launches: after the pause for its inputs the GPU's clocks
    # take a few launches of this compute-bound kernel to come back up
    avg, med = time_launches(lambda: mx.mxfp8_gemm(qa, sa, qb, sb, out=cg, stream=stream), 20, 10)
    tflops = 2.0 * gm * gn * gk / avg / 1e12
    res["gemm_16384x8192x5120"] = {"us": round(avg * 1e6, 2), "TFLOP/s": round(tflops, 1),
                                   "frac": round(tflops / metrics.MFMA_FP8_PEAK_TFLOPS, 4),
                                   "median_us": round(med * 1e6, 2)}
    del qa, qb, sa, sb, cg
    torch.cuda.empty_cache()
    # grouped form at the pages' shape: 16640 tokens over 4 experts of 8192 x
    # 5120 ("[mxfp8 moe training] add compile support", Perf analysis)
    gm, gn, gk, ng = 16640, 8192, 5120, 4
    x = synth.normal_bf16((gm, gk), 1.0, seed=72, device=inp.gate.device)
    w = synth.normal_bf16((ng * gn, gk), 0.02, seed=73, device=inp.gate.device)
    qa, _, sa, _ = mx.mxfp8_quant_2d(x, rowwise=True, stream=stream)
    qb, _, sb, _ = mx.mxfp8_quant_2d(w, rowwise=True, stream=stream)
    del x, w
    offs = torch.arange(1, ng + 1, dtype=torch.int32, device=inp.gate.device) * (gm // ng)
    cg = torch.empty((gm, gn), dtype=torch.float32, device=inp.gate.device)
    qb3, sb3 = qb.view(ng, gn, gk), sb.view(ng, gn, gk // 32)
    avg, med = time_launches(lambda: mx.mxfp8_grouped_gemm(qa, sa, qb3, sb3, offs, out=cg, stream=stream), 20, 10)
    tflops = 2.0 * gm * gn * gk / avg / 1e12
    res["grouped_gemm_16640x8192x5120_g4"] = {"us": round(avg * 1e6, 2), "TFLOP/s": round(tflops, 1),
                                              "frac": round(tflops / metrics.MFMA_FP8_PEAK_TFLOPS, 4),
                                              "median_us": round(med * 1e6, 2)}
    del qa, qb, sa, sb, qb3, sb3, cg
    torch.cuda.empty_cache()
    # the input gradient at the same shape, its expert operand the 3D cast's
    # output as written: dx [16640, 5120] = dy [16640, 8192] W_g [8192, 5120]
    dy = synth.normal_bf16((gm, gn), 1.0, seed=74, device=inp.gate.device)
    w3 = synth.expert_weights(ng, gn, gk, seed=75, std=0.02, device=inp.gate.device)
    qa, _, sa, _ = mx.mxfp8_quant_2d(dy, rowwise=True, stream=stream)
    q3, s3 = mx.mxfp8_quant_3d_colwise(w3, stream=stream)
    del w3
    cg = torch.empty((gm, gk), dtype=torch.float32, device=inp.gate.device)
    avg, med = time_launches(lambda: mx.mxfp8_grouped_gemm(qa, sa, q3, s3, offs, out=cg, stream=stream), 20, 10)
    tflops = 2.0 * gm * gn * gk / avg / 1e12
    res["dgrad_grouped_gemm_16640x5120x8192_g4"] = {"us": round(avg * 1e6, 2), "TFLOP/s": round(tflops, 1),
                                                    "frac": round(tflops / metrics.MFMA_FP8_PEAK_TFLOPS, 4),
                                                    "median_us": round(med * 1e6, 2)}
    del qa, sa, q3, s3, cg
    # the weight gradient: dW_g [8192, 5120] = dy_g^T x_g over each expert's
    # tokens, operands the grouped colwise casts (per-group padded scales)
    # (uneven groups whose token counts are multiples of 128, as padded
    # mixture-of-experts token groups are: every group's tokens start on a
    # 128-byte boundary of the operand rows)
    x = synth.normal_bf16((gm, gk), 1.0, seed=76, device=inp.gate.device)
    ends = torch.tensor([3072, 7168, 11776, 16640], dtype=torch.int32, device=inp.gate.device)
    _, qa, _, sa = mx.mxfp8_quant_2d_grouped(dy, ends, stream=stream)
    _, qb, _, sb = mx.mxfp8_quant_2d_grouped(x, ends, stream=stream)
    del dy, x
    cw = torch.empty((ng, gn, gk), dtype=torch.float32, device=inp.gate.device)
    avg, med = time_launches(lambda: mx.mxfp8_grouped_gemm_k(qa, sa, qb, sb, ends, out=cw, stream=stream), 20, 10)
    tflops = 2.0 * gm * gn * gk / avg / 1e12
    res["wgrad_grouped_gemm_k_8192x5120_t16640_g4"] = {"us": round(avg * 1e6, 2), "TFLOP/s": round(tflops, 1),
                                                       "frac": round(tflops / metrics.MFMA_FP8_PEAK_TFLOPS, 4),
                                                       "median_us": round(med * 1e6, 2)}
    del qa, sa, qb, sb, cw, offs, ends
    torch.cuda.empty_cache()
    # the grouped casts at 131072 x 8192 (8 token groups): colwise scales in
    # the per-group padded layout, the same bytes as the plain casts
    ends = torch.arange(1, 9, dtype=torch.int32, device=inp.gate.device) * (M // 8)
    bo = mx.alloc_outputs(M, 2 * N, mx.BOTH, inp.gate.device, 8)
    qo = mx.alloc_outputs(M, N, mx.COLWISE, inp.gate.device, 8)
    for name, fn, nbytes in (
            ("bwd_both_grouped_g8", lambda: mx.mxfp8_gated_bwd_grouped(inp.dh, inp.gate, inp.up, ends, out=bo,
                                                                        stream=stream),
             metrics.swiglu_bwd_bytes(M, N, mx.BOTH)),
            ("quant2d_col_grouped_g8", lambda: mx.mxfp8_quant_2d_grouped(inp.dh, ends, out=qo, stream=stream),
             metrics.quant_2d_bytes(M, N, mx.COLWISE))):
        avg, _ = time_launches(fn, 10, 2)
        res[name] = {"us": round(avg * 1e6, 2), "GB/s": round(metrics.gbps(nbytes, avg), 1),
                     "frac": round(metrics.gbps(nbytes, avg) / metrics.HBM_PEAK_GBPS, 4)}
    del bo, qo, ends
    torch.cuda.empty_cache()
    # 3D expert cast, 64 experts of 8192 x 5120 (inputs 5.4 GB)
    w = synth.expert_workload(64, device=inp.gate.device)
    q = torch.empty((64, 5120, 8192), dtype=torch.uint8, device=w.device)
    s = torch.empty((64, 5120, 256), dtype=torch.uint8, device=w.device)
    avg, _ = time_launches(lambda: mx.mxfp8_quant_3d_colwise(w, out=(q, s), stream=stream), 10, 2)
    nb = metrics.quant_3d_bytes(64, 8192, 5120)
    res["quant3d_E64"] = {"us": round(avg * 1e6, 2), "GB/s": round(metrics.gbps(nb, avg), 1),
                          "frac": round(metrics.gbps(nb, avg) / metrics.HBM_PEAK_GBPS, 4)}
    del w, q, s
    torch.cuda.empty_cache()
    print("bench: detail done", file=sys.stderr, flush=True)
    return res


if __name__ == "__main__":
    main()
