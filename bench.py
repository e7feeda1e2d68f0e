"""Benchmark of the fused vocabulary CE forward + backward on one MI355X.

One step = one ce_fused_fwd_bwd call over one batch of synthetic input (the
whole hot path: row statistics, per-row loss, gradient, segment sums). Inputs
are resident in HBM before timing starts. Each step uses the next of
``--rotate`` input/output buffer sets, so a step never finds its logits in
the 256 MB last-level cache from the previous use of the same buffers.

Prints ONE JSON line with the metric, the roofline object for the row kernel
(algorithmic bytes / measured kernel time, against 8 TB/s HBM), and the fp64
CPU reference timed on a sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# The headline: the largest workload (CE + z-loss + segment sums, 65536 x
# 201088 bf16). Beside it, the shape the pages measure (16384 x 128256 bf16,
# in place; torchtitan PR #5661, revised PR description, the H100 table).
DEFAULT_WORKLOAD = "cezseg_bf16_T65536_V201088_seg512"
EXTRA_WORKLOAD = "ce_bf16_T16384_V128256_zipf_inplace"
HBM_PEAK_GBPS = 8000.0
METRIC = "fused CE fwd+bwd logit elems/sec + achieved HBM GB/s (% of peak)"
METRIC_FORWARD = "CE forward + logsumexp + entropy logit elems/sec + achieved HBM GB/s (% of peak)"
METRIC_DISTILL = "fused CE + distillation (KL to a teacher matrix) fwd+bwd logit elems/sec + achieved HBM GB/s (% of peak)"
METRIC_FORWARD_LSE = "CE forward + logsumexp logit elems/sec + achieved HBM GB/s (% of peak)"


def kernel_source_sha(src="ce_fused.hip"):
    with open(os.path.join(ROOT, "loss_vocab_amd", "csrc", src), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profiles(workload, prefix="traffic", src="ce_fused.hip"):
    """HBM bytes per launch from committed rocprofv3 counter summaries, or None
    when none exists or the kernel source changed since they were taken."""
    path = os.path.join(ROOT, "profiles", f"{prefix}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha") != kernel_source_sha(src):
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None where absent)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, rows, threads, forward=False, min_seconds=10.0, kl_beta=None):
    """Time the fp64 oracle on ``rows`` rows of the workload recipe (generated
    on the host), split in 256-row blocks over a thread pool, repeating the
    sample until ``min_seconds`` have passed. ``forward``: loss, logsumexp and
    entropy without the gradient. A segmented recipe keeps its minimum segment
    length, with fewer segments when the sample is short. ``kl_beta``: the
    distillation oracle against a second draw of the recipe as teacher."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    from oracle import ce_oracle, distill_oracle, row_entropy
    from workloads import make_inputs

    sample = wl.scaled(T=rows) if rows != wl.T else wl
    if wl.num_segments and rows < wl.num_segments * wl.seg_min_len * 2:
        sample = wl.scaled(T=rows, num_segments=max(1, rows // (2 * wl.seg_min_len)))
    inp = make_inputs(sample, device="cpu")
    z = inp["logits"]
    t = inp["targets"].numpy()
    seg = inp["segment_ids"].numpy() if inp["segment_ids"] is not None else None
    teacher = None if kl_beta is None else make_inputs(sample, device="cpu", seed_offset=100)["logits"]
    blocks = [(r0, min(rows, r0 + 256)) for r0 in range(0, rows, 256)]

    def work(b):
        r0, r1 = b
        zb = z[r0:r1].double().numpy()
        if teacher is not None:
            return distill_oracle(zb, teacher[r0:r1].double().numpy(), t[r0:r1],
                                  z_alpha=inp["z_alpha"], kl_beta=kl_beta,
                                  grad_scale=inp["grad_scale"])["loss"].sum()
        out = ce_oracle(zb, t[r0:r1], z_alpha=inp["z_alpha"], grad_scale=inp["grad_scale"],
                        segment_ids=None if seg is None else seg[r0:r1],
                        num_segments=inp["num_segments"], segment_mean=False,
                        want_grad=not forward)["loss"].sum()
        if forward:
            out += row_entropy(zb, t[r0:r1])[0].sum()
        return out

    passes = 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while True:
            tot = sum(ex.map(work, blocks))
            assert np.isfinite(tot)
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                break
    what = "loss+logsumexp+entropy" if forward else "loss+gradient"
    segs = f", {sample.num_segments} segments" if sample.num_segments else ""
    if teacher is not None:
        what, segs = "CE+KL loss and gradient against a second draw as teacher", ""
    return {"value": passes * rows * wl.V / dt, "unit": "logit elems/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(), "seconds": round(dt, 3),
            "sample": f"{rows} rows x V={wl.V} of the same recipe{segs} generated on the host, "
                      f"{passes} passes; fp64 numpy {what} in 256-row blocks on {threads} threads"}


MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC_LMHEAD = "fused LM-head + CE fwd+bwd tokens/sec + achieved matrix-core TFLOP/s (% of bf16 peak)"
DEFAULT_LMHEAD = "lmhead_bf16_T16384_V128256_H4096"


def cpu_baseline_lmhead(wl, rows, threads, min_seconds):
    """The oracle on the first ``rows`` rows (the whole weight): logits, loss,
    dX and dW of those rows in fp64, 8-row blocks over a thread pool, repeated
    until ``min_seconds`` have passed."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    from oracle import lmhead_ce
    from workloads import make_lmhead_inputs

    inp = make_lmhead_inputs(wl, device="cpu", rows=rows)
    X = inp["hidden"].double().numpy()
    W = inp["weight"].double().numpy()
    t = inp["targets"].numpy()
    blocks = [(r0, min(rows, r0 + 8)) for r0 in range(0, rows, 8)]

    def work(b):
        out = lmhead_ce(X[b[0]:b[1]], W, t[b[0]:b[1]], grad_scale=inp["grad_scale"])
        return float(np.nansum(out["loss"])) + float(out["dweight"][0, 0])

    passes = 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while True:
            list(ex.map(work, blocks))
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                break
    return {"value": passes * rows / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "seconds": round(dt, 3),
            "sample": f"{rows} rows of the recipe (whole weight V={wl.V} x H={wl.H}) generated on "
                      f"the host, {passes} passes; fp64 numpy logits, loss, dX and dW in 8-row "
                      f"blocks on {threads} threads"}


def bench_lmhead(args):
    """One step = one ce_lmhead_fwd_bwd call (forward statistics, finish, and
    the chunked backward with dX and dW) on resident inputs."""
    from workloads import LMHEAD_WORKLOADS, lmhead_flops

    name = args.workload if args.workload in LMHEAD_WORKLOADS else DEFAULT_LMHEAD
    wl = LMHEAD_WORKLOADS[name]
    cpu = None
    if not args.no_cpu_baseline:
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
        cpu = cpu_baseline_lmhead(wl, args.cpu_rows or 32, threads, args.cpu_seconds)

    import torch

    import loss_vocab_amd as L
    from workloads import make_lmhead_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_lmhead_inputs(wl, device=dev)
    X, W, t = inp["hidden"], inp["weight"], inp["targets"]
    loss = torch.empty(wl.T, dtype=torch.float32, device=dev)
    lse = torch.empty(wl.T, dtype=torch.float32, device=dev)
    dh = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((wl.V, wl.H), dtype=torch.float32, device=dev)
    p = L.make_lmhead(X, W, dhidden_dtype=torch.bfloat16)
    ws = torch.empty(L._lib.lmhead_workspace_bytes(p, True), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        L.ce_lmhead_fwd_bwd(X, W, t, None, inp["z_alpha"], inp["grad_scale"], loss, lse, dh, dw,
                            workspace=ws, stream=stream.cuda_stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    per_call = sorted(a.elapsed_time(b) for a, b in ev)
    avg_call = sum(per_call) / len(per_call)
    # The method's own matrix work is 6 T V H (the logit product forward, dX
    # and dW backward); the backward also recomputes the logit product, so
    # 8 T V H flops are executed. The roofline counts the 6.
    flops = lmhead_flops(wl, recompute=False)
    flops_exec = lmhead_flops(wl)
    achieved = flops / (avg_call * 1e-3) / 1e12
    achieved_exec = flops_exec / (avg_call * 1e-3) / 1e12
    out = {
        "metric": METRIC_LMHEAD,
        "value": wl.T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "V": wl.V, "H": wl.H,
                   "ignored_rows": wl.n_masked, "dhidden_dtype": "bf16", "dweight_dtype": "f32",
                   "flops_per_step": flops, "flops_executed_per_step": flops_exec,
                   "path": "lmhead"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "basis": "6 T V H (algorithmic)",
                     "executed_TFLOPs": achieved_exec,
                     "executed_frac": achieved_exec / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": None, "call_ms_avg": avg_call,
                     "call_ms_median": per_call[len(per_call) // 2]},
        "cpu_baseline": cpu,
        "wall_s_timed": wall,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--rotate", type=int, default=0,
                    help="input/output buffer sets used in turn (0: 3 below 2 GiB of logits, else 2)")
    ap.add_argument("--extra-workload", default=EXTRA_WORKLOAD,
                    help="fused path: a second workload timed after the headline one and "
                         "reported under 'extra' ('none' to skip)")
    ap.add_argument("--cpu-rows", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum time of the CPU oracle baseline (the sample is repeated)")
    ap.add_argument("--no-entropy", action="store_true",
                    help="forward path: logsumexp only, no entropy output")
    ap.add_argument("--copy-probe-mib", type=int, default=1024,
                    help="size of the plain device copy timed after the run (0: skip)")
    ap.add_argument("--path", choices=["fused", "split", "forward", "lmhead", "distill"],
                    default="fused",
                    help="fused: one ce_fused_fwd_bwd call per step; split: per-shard statistics, "
                         "finish, per-shard gradient (the vocabulary-parallel form on one GPU); "
                         "forward: one ce_fused_forward call with logsumexp and entropy outputs "
                         "(another metric: no gradient); lmhead: ce_lmhead_fwd_bwd from hidden "
                         "states and the head weight (another metric: matrix-core bound); "
                         "distill: ce_fused_distill with a second draw of the recipe as teacher "
                         "(another metric: two matrices read)")
    ap.add_argument("--kl-beta", type=float, default=0.5)
    ap.add_argument("--shards", type=int, default=2)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(rows shard across GPUs with no exchange beyond a token count; "
              "see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.path == "lmhead":
        return bench_lmhead(args)

    from workloads import WORKLOADS, alg_bytes

    wl = WORKLOADS[args.workload]

    # CPU reference first, before the GPU is touched.
    cpu = None
    if not args.no_cpu_baseline:
        avail = len(os.sched_getaffinity(0))
        threads = max(1, min(16, avail))
        rows = args.cpu_rows or min(wl.T, max(256, int(3e8 // wl.V) // 256 * 256))
        cpu = cpu_baseline(wl, rows, threads, forward=args.path == "forward",
                           min_seconds=args.cpu_seconds,
                           kl_beta=args.kl_beta if args.path == "distill" else None)
        cpu["cores_available"] = avail
        cpu["cores_online"] = os.cpu_count()

    import torch

    import loss_vocab_amd as L

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    res = bench_workload(wl, args, dev, stream, main=True)

    extra = None
    if args.path == "fused" and args.extra_workload not in ("", "none") and \
            args.extra_workload != wl.name:
        # the pages' measured shape beside the headline, same timing rules
        ew = WORKLOADS[args.extra_workload]
        e = bench_workload(ew, args, dev, stream, main=False)
        extra = {"workload": ew.name, "T": ew.T, "V": ew.V, "value": e["value"],
                 "unit": "logit elems/s", "ms_per_step": e["ms_per_step"],
                 "alg_bytes_per_step": e["nbytes"], "alg_GBps": e["achieved"],
                 "frac": e["achieved"] / HBM_PEAK_GBPS, "timing": e["timing"],
                 "traffic": e["traffic"]}

    # A plain device-to-device copy of known size, after the timed regions:
    # the same box's practical read+write ceiling, and the calibration kernel
    # for the HBM byte counters.
    copy_probe = None
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        reps = 5
        c0.record(stream)
        for _ in range(reps):
            dst.copy_(src)
        c1.record(stream)
        torch.cuda.synchronize()
        cms = c0.elapsed_time(c1) / reps
        copy_probe = {"bytes_read": n, "bytes_written": n, "ms": cms, "GBps": 2 * n / (cms * 1e-3) / 1e9}
        del src, dst

    metric = {"fused": METRIC, "split": METRIC, "distill": METRIC_DISTILL,
              "forward": METRIC_FORWARD_LSE if args.no_entropy else METRIC_FORWARD}[args.path]
    nbytes, achieved = res["nbytes"], res["achieved"]
    out = {
        "metric": metric,
        "value": res["value"],
        "unit": "logit elems/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "T": wl.T, "V": wl.V, "logits_dtype": wl.dtype,
            "grad_dtype": "bf16" if wl.grad_torch_dtype == torch.bfloat16 else "f32",
            "in_place": wl.grad == "inplace", "z_alpha": wl.z_alpha,
            "ignored_rows": wl.n_masked,
            "segments": 0 if args.path == "distill" else wl.num_segments,
            "rotating_buffer_sets": res["rotate"], "alg_bytes_per_step": nbytes,
            "path": args.path, "timing": res["timing"],
            **({"entropy": not args.no_entropy} if args.path == "forward" else {}),
            **({"kl_beta": args.kl_beta, "teacher": "second draw of the recipe, seed offset 100"}
               if args.path == "distill" else {}),
        },
        "alg_GBps": nbytes / (res["ms_per_step"] * 1e-3) / 1e9,
        "pct_of_hbm_peak": 100.0 * nbytes / (res["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS, "traffic": res["traffic"],
            "kernel_ms_avg": res["avg_call_ms"],
            "single_call_ms_median_with_events": res["single_call_ms_median"],
        },
        "cpu_baseline": cpu,
        "copy_probe": copy_probe,
        "split": res["split"],
        "extra": extra,
        "wall_s_timed": res["wall"],
    }
    print(json.dumps(out), flush=True)


def bench_workload(wl, args, dev, stream, main=True):
    """Inputs resident in HBM, W warmup steps, K timed steps of the chosen
    path on ``wl``. Returns the timing and the algorithmic bytes per step.

    Timing: K steps back to back between two events on the launch stream,
    bracketed by synchronisation, nothing else enqueued between the calls (an
    event around every call costs ~9 us per call on MI355X: the next kernel
    waits for the marker). A workload whose gradient overwrites its logits
    (in place) runs in rounds of back-to-back steps, one per buffer set, each
    round between two events, with every set's logits restored from a
    pristine copy before the round (outside the events), so that every step
    computes on the recipe's logits. One call per step, so the figure is the
    average launch duration of the fused call."""
    import torch

    import loss_vocab_amd as L
    from workloads import alg_bytes, make_inputs

    in_place = wl.grad == "inplace" and args.path != "forward"
    logit_bytes = wl.T * wl.V * (4 if wl.dtype == "f32" else 2)
    rotate = args.rotate or (3 if logit_bytes < (2 << 30) else 2)
    if in_place and not args.rotate:
        # in place: enough sets (each with a pristine copy) for runs of
        # back-to-back steps between restores, within about 40 GB
        rotate = max(2, min(args.steps, int(40e9 // (2 * logit_bytes))))
    sets = []
    for i in range(rotate):
        inp = make_inputs(wl, device=dev, seed_offset=i)
        loss = torch.empty(wl.T, dtype=torch.float32, device=dev)
        if args.path == "forward":
            grad = None
        elif in_place:
            grad = inp["logits"]
        else:
            grad = torch.empty((wl.T, wl.V), dtype=wl.grad_torch_dtype, device=dev)
        seg = (torch.empty(wl.num_segments, dtype=torch.float32, device=dev)
               if wl.num_segments else None)
        ws_n = L.workspace_bytes(inp["logits"], num_segments=wl.num_segments)
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)
        pristine = inp["logits"].clone() if in_place else None
        sets.append((inp, loss, grad, seg, ws, pristine))
    torch.cuda.synchronize()

    bounds = L.shard_bounds(wl.V, args.shards, 8 if wl.dtype == "bf16" else 4)
    split_bufs = []
    if args.path == "split":
        for _ in sets:
            split_bufs.append((torch.empty((len(bounds), wl.T, 3), dtype=torch.float32, device=dev),
                               torch.empty((wl.T, 8), dtype=torch.float32, device=dev)))
    phase_ev = []   # split path: (stats, finish, grad) event quadruples per step
    teachers = []
    if args.path == "distill":
        for i in range(len(sets)):
            teachers.append((make_inputs(wl, device=dev, seed_offset=100 + i)["logits"],
                             torch.empty(wl.T, dtype=torch.float32, device=dev)))
        torch.cuda.synchronize()
    fwd_bufs = []
    if args.path == "forward":
        for _ in sets:
            fwd_bufs.append((torch.empty(wl.T, dtype=torch.float32, device=dev),
                             torch.empty(wl.T, dtype=torch.float32, device=dev)))

    def restore(i):
        inp, *_, pristine = sets[i % len(sets)]
        inp["logits"].copy_(pristine)

    def step(i):
        inp, loss, grad, seg, ws, _ = sets[i % len(sets)]
        if args.path == "fused":
            L.ce_fused_fwd_bwd(inp["logits"], inp["targets"], None, inp["segment_ids"],
                               inp["z_alpha"], inp["grad_scale"], loss, seg, grad,
                               num_segments=wl.num_segments, segment_mean=inp["segment_mean"],
                               workspace=ws, stream=stream.cuda_stream)
            return
        if args.path == "distill":
            teacher, kl = teachers[i % len(sets)]
            L.ce_fused_distill(inp["logits"], teacher, inp["targets"], None, inp["z_alpha"],
                               args.kl_beta, inp["grad_scale"], loss, kl, grad,
                               stream=stream.cuda_stream)
            return
        if args.path == "forward":
            lse, ent = fwd_bufs[i % len(sets)]
            L.ce_fused_forward(inp["logits"], inp["targets"], None, inp["segment_ids"],
                               inp["z_alpha"], loss, seg, lse, None if args.no_entropy else ent,
                               num_segments=wl.num_segments,
                               workspace=ws, stream=stream.cuda_stream)
            return
        stats, row_state = split_bufs[i % len(sets)]
        z, t = inp["logits"], inp["targets"]
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record(stream)
        for k, (a, b) in enumerate(bounds):
            L.ce_shard_stats(z[:, a:b], t, None, stats[k], v0=a, stream=stream.cuda_stream)
        ev[1].record(stream)
        L.ce_rows_finish(len(bounds), stats, t, None, inp["segment_ids"], inp["z_alpha"], loss,
                         seg, row_state, vocab=wl.V, num_segments=wl.num_segments,
                         segment_mean=inp["segment_mean"], workspace=ws, stream=stream.cuda_stream)
        ev[2].record(stream)
        for a, b in bounds:
            L.ce_shard_grad(z[:, a:b], t, row_state, inp["grad_scale"], grad[:, a:b], v0=a,
                            stream=stream.cuda_stream)
        ev[3].record(stream)
        phase_ev.append(ev)

    for i in range(args.warmup):
        if in_place:
            restore(i)
        step(i)
    torch.cuda.synchronize()

    if in_place:
        # Rounds of back-to-back steps, one per buffer set, between two events;
        # before each round every set's logits are restored from its pristine
        # copy (outside the events), so every step computes on the recipe.
        total_ms, done, wall = 0.0, 0, 0.0
        while done < args.steps:
            n = min(len(sets), args.steps - done)
            for i in range(n):
                restore(i)
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            wall0 = time.perf_counter()
            a.record(stream)
            for i in range(n):
                step(i)
            b.record(stream)
            torch.cuda.synchronize()
            wall += time.perf_counter() - wall0
            total_ms += a.elapsed_time(b)
            done += n
        ms_per_step = total_ms / args.steps
        timing = (f"rounds of up to {len(sets)} back-to-back steps (one per buffer set) between "
                  "two events; logits restored from pristine copies before each round, outside "
                  "the events")
        for i in range(min(20, len(sets))):
            restore(i)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(min(20, len(sets)))]
        for i, (a, b) in enumerate(ev):
            a.record(stream)
            step(i)
            b.record(stream)
        torch.cuda.synchronize()
        per_call_ms = sorted(a.elapsed_time(b) for a, b in ev)
    else:
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        t_start.record(stream)
        for i in range(args.steps):
            step(i)
        t_end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        ms_per_step = t_start.elapsed_time(t_end) / args.steps
        timing = "two events around the K back-to-back steps"
        # The spread of single calls, after the timed region: events around
        # each of up to 20 calls (these include the event overhead).
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(min(20, args.steps))]
        for i, (a, b) in enumerate(ev):
            a.record(stream)
            step(args.steps + i)
            b.record(stream)
        torch.cuda.synchronize()
        per_call_ms = sorted(a.elapsed_time(b) for a, b in ev)
    avg_call_ms = ms_per_step

    nbytes = alg_bytes(wl)
    achieved = nbytes / (avg_call_ms * 1e-3) / 1e9
    traffic = traffic_from_profiles(wl.name)
    split_info = None
    if args.path == "split":
        # The split form reads each valid row twice (statistics, then
        # gradient); its dominant kernels are the gradient passes.
        timed = phase_ev[args.warmup:args.warmup + args.steps]
        ms = [sum(e[j].elapsed_time(e[j + 1]) for e in timed) / len(timed) for j in range(3)]
        b_in = 4 if wl.dtype == "f32" else 2
        b_out = 4 if wl.grad_torch_dtype == torch.float32 else 2
        read = wl.n_valid * wl.V * b_in
        grad_bytes = read + wl.T * wl.V * b_out + 8 * wl.T + 16 * wl.T
        stats_bytes = read + 8 * wl.T + 12 * wl.T * len(bounds)
        split_info = {"shards": [list(b) for b in bounds], "stats_ms": ms[0], "finish_ms": ms[1],
                      "grad_ms": ms[2], "stats_GBps": stats_bytes / (ms[0] * 1e-3) / 1e9,
                      "grad_GBps": grad_bytes / (ms[2] * 1e-3) / 1e9,
                      "split_alg_bytes_per_step": stats_bytes + grad_bytes}
        achieved = grad_bytes / (ms[2] * 1e-3) / 1e9
        avg_call_ms = ms[2]
        traffic = None
    if args.path == "distill":
        # Valid rows of both matrices read once; every gradient row written;
        # targets read, loss and KL written.
        b_in = 4 if wl.dtype == "f32" else 2
        b_out = 4 if wl.grad_torch_dtype == torch.float32 else 2
        nbytes = wl.n_valid * wl.V * 2 * b_in + wl.T * wl.V * b_out + wl.T * (8 + 2 * 4)
        achieved = nbytes / (avg_call_ms * 1e-3) / 1e9
        traffic = traffic_from_profiles(wl.name, "traffic_distill", "distill_ce.hip")
    if args.path == "forward":
        # Valid rows read once; targets read, loss / lse / entropy written
        # (the segment terms of the fused call stay the same).
        b_in = 4 if wl.dtype == "f32" else 2
        nbytes = wl.n_valid * wl.V * b_in + wl.T * (8 + (2 if args.no_entropy else 3) * 4)
        if wl.num_segments:
            nbytes += wl.T * (4 + 8) + wl.num_segments * 4
        achieved = nbytes / (avg_call_ms * 1e-3) / 1e9
        # counters were taken on the default (entropy) forward kernel
        traffic = None if args.no_entropy else traffic_from_profiles(wl.name, "traffic_forward")
    out = {"value": wl.T * wl.V / (ms_per_step * 1e-3), "ms_per_step": ms_per_step,
           "avg_call_ms": avg_call_ms, "nbytes": nbytes, "achieved": achieved,
           "traffic": traffic, "split": split_info, "wall": wall, "timing": timing,
           "rotate": rotate, "single_call_ms_median": per_call_ms[len(per_call_ms) // 2]}
    del sets, split_bufs, teachers, fwd_bufs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
