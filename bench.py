#!/usr/bin/env python3
"""bench.py -- time the bf16 delta-sync hot path on one MI355X.

One step is one sync of the resident snapshots of a parameter list in the
sparse mode, the quantity the metric names (weights diffed, compacted and
applied):
  1. delta_diff_many  (sender: bitwise change detection + compaction)
  2. delta_apply_many (receiver: in-place scatter into its snapshot)
Steps alternate the forward delta (old -> new) and the reverse one
(new -> old), so the receiver's snapshot moves back and forth and every step
does identical work without any reset.  The XOR mode (xor_mask on the sender,
xor_apply on the receiver) is timed the same way as its own loop and reported
under "xor_mode"; every kernel's time, bytes and fraction of peak is listed
under "kernels", and the memory-system ceilings under "ceilings_gbs".

Default workload: the Llama-7B-shaped list (291 tensors, 6,738,415,616 bf16
elements), weights N(0, 0.02), bf16-resident step at lr 1e-6 (about 1 %
changed).  Inputs are generated on the GPU and resident in HBM before timing.
Other modes: --config tensor1m / qwen3_0p6b (smaller lists), sweep256m (the
density sweep), llama405b_share (the 405B-shaped 10-layer share, streamed
layer by layer, in place), --shards W, --receiver, --wire.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, GB/s
METRIC = "GB/s of bf16 weights diffed+compacted and applied; % of MI355X HBM peak"
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "sparse_bf16_delta_amd", "csrc")
# HBM bytes measured by rocprofv3 counters, per kernel and launch, for a
# workload (profiles/<workload>_traffic.json); valid only while the kernel
# sources hash to the recorded value.
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "delta_diff_many": ("diff.hip", "sbd_internal.h"),
    "delta_apply_many": ("apply.hip", "sbd_internal.h"),
    "xor_mask": ("xor.hip", "sbd_internal.h"),
    "xor_apply": ("xor.hip", "sbd_internal.h"),
}


def source_hash(kernel):
    import hashlib

    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload_key):
    """{kernel: bytes per launch} from the committed counter summary of the
    workload, for the kernels whose sources are unchanged since the counters
    were taken."""
    try:
        with open(os.path.join(PROFILES, workload_key.split(":")[0] + "_traffic.json")) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return {}
    if rec.get("workload_key") != workload_key:
        return {}
    out = {}
    for k, v in rec.get("kernels", {}).items():
        if k in KERNEL_SOURCES and v.get("source_sha256") == source_hash(k):
            out[k] = v.get("hbm_bytes_per_launch")
    return out


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="llama7b",
                    choices=["tensor1m", "qwen3_0p6b", "llama7b", "sweep256m", "llama405b_share"],
                    help="llama7b (default): the 7B-shaped list; tensor1m, qwen3_0p6b: smaller "
                         "lists; sweep256m: density sweep on one flat 2^28-element tensor (table "
                         "on stderr); llama405b_share: the 405B-shaped 10-layer share, streamed "
                         "layer by layer")
    ap.add_argument("--lr", type=float, default=None)
    ap.add_argument("--mode", default=None, choices=[None, "fp32_master", "bf16_resident"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU-time budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--torch-cpu-seconds", type=float, default=5.0,
                    help="time budget of the second CPU point: the sources' own torch-CPU "
                         "formulation on every host core (0 skips it)")
    ap.add_argument("--wire", action="store_true",
                    help="time the wire encoding of the list's delta: positions block encode, "
                         "decode and the flush hashes")
    ap.add_argument("--receiver", action="store_true",
                    help="time the receiver with the delta and the XOR mask in pinned host "
                         "memory: copy only, copy then apply, and the streamed pipeline")
    ap.add_argument("--chunks", type=int, default=8,
                    help="--receiver: parameter chunks of the streamed sparse receiver")
    ap.add_argument("--sweep-case", default=None,
                    help="sweep256m: run one case only, as pattern:density (e.g. uniform:0.01), "
                         "so a profiler sees that case alone")
    ap.add_argument("--shards", type=int, default=0,
                    help="W > 0: time delta_diff_many_sharded for each rank of a W-way Shard(0) "
                         "split of the list, one rank after another (table on stderr)")
    return ap.parse_args()


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path; each rank "
              "would run it on its own shard (asked for "
              f"--gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_bf16_delta_amd as sbd
    from sparse_bf16_delta_amd.plan import ApplyPlan, DiffPlan
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    sbd.load()
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    if args.config == "sweep256m":
        density_sweep(args, props)
        return
    if args.config == "llama405b_share":
        layer_stream_run(args, props)
        return
    if args.shards > 0:
        sharded_run(args, props)
        return
    if args.receiver:
        receiver_run(args, props)
        return
    if args.wire:
        wire_run(args, props)
        return
    cfg = workloads.CONFIGS[args.config]
    lr = args.lr if args.lr is not None else (1e-6 if cfg.key == "llama7b" else cfg.lrs[0])
    mode = args.mode or cfg.mode
    numels = cfg.numels
    n_model = sum(numels)
    offs, n_alloc = workloads.flat_layout(numels)
    log(f"[bench] device {props.name} ({getattr(props, 'gcnArchName', '?')}), "
        f"{props.multi_processor_count} CUs, {props.total_memory / 2**30:.0f} GiB")
    log(f"[bench] workload {cfg.key}: {len(numels)} tensors, {n_model:,} elements, "
        f"lr {lr:g}, {mode}")

    # ---- resident inputs: one flat arena per snapshot, 256-byte aligned params
    t0 = time.perf_counter()
    old = torch.zeros(n_alloc, dtype=torch.bfloat16, device=dev)
    new = torch.zeros(n_alloc, dtype=torch.bfloat16, device=dev)
    for t, (o, n) in enumerate(zip(offs, numels)):
        sw, su = workloads.seeds(cfg.seed_family, t)
        workloads.fill_step_pair_(old[o:o + n], new[o:o + n], sw, su, lr, mode)
    snap = old.clone()
    mask = torch.empty(n_alloc, dtype=torch.int16, device=dev)
    olds = [old[o:o + n] for o, n in zip(offs, numels)]
    news = [new[o:o + n] for o, n in zip(offs, numels)]
    snaps = [snap[o:o + n] for o, n in zip(offs, numels)]
    torch.cuda.synchronize()
    log(f"[bench] generated inputs in {time.perf_counter() - t0:.1f} s")

    # ---- plans: capacity from one untimed sizing pass.  The forward plan
    # diffs (old, new), the reverse plan (new, old): applied in turn they move
    # the receiver's snapshot old -> new -> old, so every step is a real sync
    # and no reset is needed.
    cap = n_model // 8 + 65536
    dplan = DiffPlan(olds, news, cap)
    dplan.run()
    nnz_total = dplan.changed()
    if nnz_total > cap:
        cap = nnz_total + 65536
        dplan = DiffPlan(olds, news, cap)
        dplan.run()
        nnz_total = dplan.changed()
    rplan = DiffPlan(news, olds, cap)
    rplan.run()
    if rplan.changed() != nnz_total:
        print("bench.py: forward and reverse deltas differ in size", file=sys.stderr)
        sys.exit(1)
    aplan = ApplyPlan(snaps)
    density = nnz_total / n_model
    log(f"[bench] changed {nnz_total:,} of {n_model:,} (density {density:.4%}, "
        f"sparsity {1 - density:.4%})")

    # correctness of both modes before timing.  The receiver knows the delta's
    # entry count (it travels with the delta), so apply is launched for it.
    aplan.run(dplan.idx, dplan.val, dplan.offsets, nnz_total)
    ok_apply = torch.equal(snap.view(torch.int16), new.view(torch.int16))
    aplan.run(rplan.idx, rplan.val, rplan.offsets, nnz_total)
    ok_rev = torch.equal(snap.view(torch.int16), old.view(torch.int16))
    sbd.xor_mask(old, new, out=mask)
    sbd.xor_apply_(snap, mask)
    ok_xor = torch.equal(snap.view(torch.int16), new.view(torch.int16))
    sbd.xor_apply_(snap, mask)
    ok_xor = ok_xor and torch.equal(snap.view(torch.int16), old.view(torch.int16))
    if not (ok_apply and ok_rev and ok_xor):
        print(f"bench.py: step check failed (apply {ok_apply}, reverse {ok_rev}, xor {ok_xor})",
              file=sys.stderr)
        sys.exit(1)

    # ---- algorithmic bytes per launch
    nnz_dev = dplan.nnz
    segs64 = None
    if nnz_total:
        poff = torch.tensor(offs, dtype=torch.int64, device=dev)
        base = torch.repeat_interleave(poff, nnz_dev)
        pos = dplan.idx[:nnz_total].long() + base
        lines128 = int(((pos >> 6)[1:] != (pos >> 6)[:-1]).sum().item()) + 1
        s64 = pos >> 5
        keep = torch.ones_like(s64, dtype=torch.bool)
        keep[1:] = s64[1:] != s64[:-1]
        segs64 = s64[keep].contiguous()
        lines64 = segs64.numel()
        del base, pos, s64, keep
    else:
        lines128 = lines64 = 0
    b_diff = 4 * n_model + 6 * nnz_total
    b_apply = 6 * nnz_total + 2 * 128 * lines128
    b_apply64 = 6 * nnz_total + 2 * 64 * lines64
    b_xor = 6 * n_alloc
    # xor_apply reads the mask and rewrites only the 128-byte snapshot lines
    # where it is nonzero, the lines holding a changed element (line model)
    b_xor_apply = 2 * n_alloc + 2 * 128 * lines128

    stream = torch.cuda.current_stream(dev)
    names = ["delta_diff_many", "delta_apply_many", "xor_mask", "xor_apply"]

    def sparse_step(k, ev=None):
        plan = dplan if k % 2 == 0 else rplan
        if ev is not None:
            ev[0].record(stream)
        plan.run()
        if ev is not None:
            ev[1].record(stream)
        aplan.run(plan.idx, plan.val, plan.offsets, nnz_total)
        if ev is not None:
            ev[2].record(stream)

    def xor_step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        sbd.xor_mask(old, new, out=mask)
        if ev is not None:
            ev[1].record(stream)
        sbd.xor_apply_(snap, mask)
        if ev is not None:
            ev[2].record(stream)

    def timed_loop(step, nev):
        for k in range(args.warmup):
            step(k)
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)]
                  for _ in range(args.steps)]
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for k in range(args.steps):
            step(k, events[k])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        samples = [sorted(events[k][i].elapsed_time(events[k][i + 1]) for k in range(args.steps))
                   for i in range(nev - 1)]
        return 1e3 * wall / args.steps, samples

    # the timed step: one sync in the sparse mode (diff on the sender, apply
    # on the receiver); an even number of warm-up steps leaves the snapshot
    # at `old` when the timed steps start
    if args.warmup % 2:
        args.warmup += 1
    ms_step, sparse_samples = timed_loop(sparse_step, 3)
    if args.steps % 2:
        aplan.run(rplan.idx, rplan.val, rplan.offsets, nnz_total)  # back to old
    if not torch.equal(snap.view(torch.int16), old.view(torch.int16)):
        print("bench.py: timed sparse steps left a wrong snapshot", file=sys.stderr)
        sys.exit(1)
    if dplan.changed() != nnz_total or rplan.changed() != nnz_total:
        print("bench.py: timed steps changed the delta", file=sys.stderr)
        sys.exit(1)
    # the XOR mode, timed the same way as its own loop (xor_apply toggles the
    # snapshot between old and new)
    xor_ms_step, xor_samples = timed_loop(lambda k, ev=None: xor_step(ev), 3)
    want = old if (args.warmup + args.steps) % 2 == 0 else new
    if not torch.equal(snap.view(torch.int16), want.view(torch.int16)):
        print("bench.py: timed XOR steps left a wrong snapshot", file=sys.stderr)
        sys.exit(1)
    if (args.warmup + args.steps) % 2:
        sbd.xor_apply_(snap, mask)

    samples = sparse_samples + xor_samples
    op_ms = [sum(x) / args.steps for x in samples]  # the mean: what a step spends
    alg = [b_diff, b_apply, b_xor, b_xor_apply]
    workload_key = f"{cfg.key}:{mode}:{lr:g}"
    traffic = measured_traffic(workload_key)
    kernels = []
    for name, ms, b, x in zip(names, op_ms, alg, samples):
        gbs = b / (ms * 1e-3) / 1e9
        t = traffic.get(name)
        kk = {"kernel": name, "ms": round(ms, 4), "ms_median": round(x[len(x) // 2], 4),
              "ms_min": round(x[0], 4), "alg_bytes": b,
              "achieved_gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
              "weights_gbs": round(2 * n_model / (ms * 1e-3) / 1e9, 1),
              "traffic": t,
              "moved_frac": round(t / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4) if t else None}
        if name == "delta_apply_many":
            # the same launch on the 64-byte model: the unit the kernel rewrites
            kk["alg_bytes_64B"] = b_apply64
            kk["frac_64B"] = round(b_apply64 / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        kernels.append(kk)
    for kk in kernels:
        log(f"[bench] {kk['kernel']:17s} {kk['ms']:8.3f} ms (median {kk['ms_median']:.3f}, min "
            f"{kk['ms_min']:.3f})  {kk['achieved_gbs']:8.1f} GB/s "
            f"({100 * kk['frac']:.1f} % of peak)  weights {kk['weights_gbs']:.1f} GB/s")
    # the dominant kernel of the timed (sparse) step
    dom = 0 if op_ms[0] >= op_ms[1] else 1
    roofline = {"bound": "hbm", "kernel": names[dom],
                "achieved": kernels[dom]["achieved_gbs"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": kernels[dom]["frac"], "traffic": traffic.get(names[dom])}

    # ---- memory-system ceilings on the same arenas, from the reference
    # kernels of libsbd_ceiling (one snapshot's bytes per operand)
    ceilings = measure_ceilings(torch, stream, old, new, snap, mask, segs64)
    del segs64

    result = {
        "metric": METRIC,
        "value": round(2 * n_model / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.title}: {len(numels)} tensors, {n_model} bf16 elements, "
                        f"{mode} step lr {lr:g}",
            "tensors": len(numels), "elements": n_model, "lr": lr, "step_model": mode,
            "changed": nnz_total, "density": round(density, 6),
            "sparsity": round(1 - density, 6), "wire_bytes": 6 * nnz_total,
            "touched_lines_128B": lines128, "touched_lines_64B": lines64,
            "step": "one sparse-mode sync: delta_diff_many on the sender, delta_apply_many "
                    "into the receiver's snapshot (forward and reverse deltas alternate); "
                    "value = one snapshot's bytes per step time",
            "workload_key": workload_key,
        },
        "roofline": roofline,
        "kernels": kernels,
        "xor_mode": {"ms_per_step": round(xor_ms_step, 4),
                     "weights_gbs": round(2 * n_model / (xor_ms_step * 1e-3) / 1e9, 2),
                     "step": "xor_mask + xor_apply, timed as its own loop of the same steps"},
        "ceilings_gbs": ceilings,
        "copy_ceiling_gbs": ceilings.get("copy"),
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", None),
                   "cus": props.multi_processor_count, "torch": torch.__version__},
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, cfg, olds, news, dplan, nnz_total)
        if args.torch_cpu_seconds > 0:
            result["cpu_torch"] = cpu_torch_formulation(args, olds, news, dplan)
    print(json.dumps(result), flush=True)


def measure_ceilings(torch, stream, old, new, snap, scratch, segs64, reps=3):
    """What the memory system sustains on these arenas (GB/s, bytes moved per
    second), timed with HIP events on the launch stream: a 16-byte
    nontemporal copy of one snapshot, a read of two snapshots, an in-place
    rewrite of one, and the read-and-rewrite of the touched 64-byte segments
    of this delta (its time in ms too: the floor under the segment-rewrite
    apply, which also has to find the segments and patch them)."""
    import ctypes

    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_bf16_delta_amd", "libsbd_ceiling.so"))
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.sbd_ceiling_copy.argtypes = [vp, vp, i64, vp]
    lib.sbd_ceiling_read2.argtypes = [vp, vp, i64, vp, vp]
    lib.sbd_ceiling_rewrite.argtypes = [vp, i64, vp]
    lib.sbd_ceiling_segments.argtypes = [vp, i64, vp, i64, vp]
    sp = vp(stream.cuda_stream)
    nbytes = old.numel() * 2
    sink = torch.zeros(4, dtype=torch.int32, device=old.device)

    def timed(fn):
        if fn() != 0:
            raise RuntimeError("ceiling kernel launch failed")
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    out = {}
    ms = timed(lambda: lib.sbd_ceiling_copy(old.data_ptr(), scratch.data_ptr(), nbytes, sp))
    out["copy"] = round(2 * nbytes / (ms * 1e-3) / 1e9, 1)
    ms = timed(lambda: lib.sbd_ceiling_read2(old.data_ptr(), new.data_ptr(), nbytes,
                                             sink.data_ptr(), sp))
    out["read2"] = round(2 * nbytes / (ms * 1e-3) / 1e9, 1)
    ms = timed(lambda: lib.sbd_ceiling_rewrite(snap.data_ptr(), nbytes, sp))
    out["rewrite_in_place"] = round(2 * nbytes / (ms * 1e-3) / 1e9, 1)
    if segs64 is not None and segs64.numel():
        # every listed segment lies inside the snapshot arena (checked here,
        # on the host, before the kernel indexes with them)
        if int(segs64[0]) < 0 or int(segs64[-1]) >= nbytes // 64:
            raise RuntimeError("segment list outside the snapshot")
        ms = timed(lambda: lib.sbd_ceiling_segments(snap.data_ptr(), nbytes, segs64.data_ptr(),
                                                    segs64.numel(), sp))
        out["segments_64B_rewrite"] = round(2 * 64 * segs64.numel() / (ms * 1e-3) / 1e9, 1)
        out["segments_64B_rewrite_ms"] = round(ms, 4)
    log(f"[bench] ceilings (GB/s moved): {out}")
    return out


def wire_run(args, props):
    """Encode the list's delta into the flush's positions block, decode it
    back, and hash positions and values; checked, then timed with HIP events."""
    import torch

    import sparse_bf16_delta_amd as sbd
    from sparse_bf16_delta_amd.plan import DiffPlan
    import workloads

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    cfg = workloads.CONFIGS[args.config]
    lr = args.lr if args.lr is not None else (1e-6 if cfg.key == "llama7b" else cfg.lrs[0])
    mode = args.mode or cfg.mode
    numels = cfg.numels
    n_model = sum(numels)
    offs, n_alloc = workloads.flat_layout(numels)
    old = torch.zeros(n_alloc, dtype=torch.bfloat16, device=dev)
    new = torch.zeros(n_alloc, dtype=torch.bfloat16, device=dev)
    for t, (o, n) in enumerate(zip(offs, numels)):
        workloads.fill_step_pair_(old[o:o + n], new[o:o + n], *workloads.seeds(cfg.seed_family, t),
                                  lr, mode)
    dplan = DiffPlan([old[o:o + n] for o, n in zip(offs, numels)],
                     [new[o:o + n] for o, n in zip(offs, numels)], n_model // 8 + 65536)
    dplan.run()
    nnz = dplan.changed()
    idx, val, offsets = dplan.idx[:nnz], dplan.val[:nnz], dplan.offsets
    pos, pos_off = sbd.wire_encode(idx, offsets, numels)
    back = sbd.wire_decode(pos, pos_off, offsets, numels)
    ok = torch.equal(back, idx)
    checksum = sbd.wire_checksum(pos, val)
    log(f"[bench] wire, {cfg.key}: {nnz:,} changed; positions block {pos.numel():,} bytes "
        f"({pos.numel() / max(nnz, 1):.3f} per entry); round trip identical: {ok}; "
        f"checksum {checksum:#x}")
    data = sbd.wire_encode_blocked(idx, offsets, numels)
    back_b = sbd.wire_decode_blocked(data, offsets, numels)
    ok_b = torch.equal(back_b, idx)
    log(f"[bench] blocked positions {data.numel():,} bytes ({data.numel() / max(nnz, 1):.3f} per "
        f"entry, {(data.numel() + 2 * nnz) / max(nnz, 1):.3f} per change with the values); "
        f"round trip identical: {ok_b}")
    if not (ok and ok_b):
        print("bench.py: wire decode does not invert encode", file=sys.stderr)
        sys.exit(1)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    from sparse_bf16_delta_amd import _abi
    import ctypes
    lib = _abi.load()
    k = len(numels)
    nums = (ctypes.c_int64 * k)(*numels)
    ws = torch.empty(lib.delta_workspace_size(0, k), dtype=torch.uint8, device=dev)
    po2 = torch.empty_like(pos_off)
    out = torch.empty_like(idx)
    hashes = torch.empty(2, dtype=torch.int64, device=dev)
    # decodes are timed as a receiver runs them on untrusted bytes: with the
    # violation count (and, for the blocked form, the table check) it implies
    viol = torch.zeros(1, dtype=torch.int64, device=dev)
    sh = ctypes.c_void_p(stream.cuda_stream)

    def enc():
        _abi.check(lib.delta_wire_encode(k, nums, idx.data_ptr(), offsets.data_ptr(), nnz,
                                         pos.data_ptr(), pos.numel(), po2.data_ptr(),
                                         ws.data_ptr(), ws.numel(), sh))

    def dec():
        _abi.check(lib.delta_wire_decode(k, nums, pos.data_ptr(), pos.numel(),
                                         pos_off.data_ptr(), offsets.data_ptr(), nnz,
                                         out.data_ptr(), viol.data_ptr(), ws.data_ptr(),
                                         ws.numel(), sh))

    data2 = torch.empty_like(data)

    def enc_b():
        _abi.check(lib.delta_wire_encode_blocked(k, nums, idx.data_ptr(), offsets.data_ptr(), nnz,
                                                 data2.data_ptr(), data2.numel(), ws.data_ptr(),
                                                 ws.numel(), sh))

    def dec_b():
        _abi.check(lib.delta_wire_decode_blocked(k, nums, data.data_ptr(), data.numel(),
                                                 offsets.data_ptr(), nnz, out.data_ptr(),
                                                 viol.data_ptr(), ws.data_ptr(), ws.numel(), sh))

    def hsh():
        _abi.check(lib.delta_wire_hash(pos.data_ptr(), pos.numel(), val.data_ptr(), nnz,
                                       hashes.data_ptr(), sh))

    rows = {}
    for name, fn, b in (("encode", enc, 4 * nnz + pos.numel()),
                        ("decode", dec, pos.numel() + 4 * nnz),
                        ("hash", hsh, pos.numel() + 2 * nnz),
                        ("encode_blocked", enc_b, 4 * nnz + data.numel()),
                        ("decode_blocked", dec_b, data.numel() + 4 * nnz)):
        ms = timed(fn)
        rows[name] = {"ms": round(ms, 4), "bytes": b,
                      "frac": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"[bench] {name:14s} {ms:8.3f} ms  {b / (ms * 1e-3) / 1e9:8.1f} GB/s "
            f"({100 * rows[name]['frac']:.1f} % of peak)")
    if int(viol.item()) != 0:
        print("bench.py: a timed decode found violations in well-formed bytes", file=sys.stderr)
        sys.exit(1)
    print(json.dumps({
        "metric": "wire encoding of the delta: encode, decode and hash times",
        "value": None, "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": False, "dtype": "u8", "data": "synthetic",
        "config": {"workload": f"{cfg.title}: {k} tensors, {n_model} elements, {mode} step lr "
                               f"{lr:g}"},
        "changed": nnz, "positions_bytes": pos.numel(), "blocked_positions_bytes": data.numel(),
        "bytes_per_change": {"per_parameter_width": round((pos.numel() + 2 * nnz) / max(nnz, 1), 4),
                             "blocked": round((data.numel() + 2 * nnz) / max(nnz, 1), 4)},
        "rows": rows,
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", None)},
    }), flush=True)


def receiver_run(args, props):
    """The receiver's side with its input in pinned host memory, as the
    network leaves it: the sparse delta (idx, val, offsets) and the XOR mask.
    Times, per mode: the host-to-device copy alone, copy then apply on one
    stream, the streamed pipeline (chunks of parameters or elements, copies
    overlapping applies), and for the delta the host-direct apply (the
    kernel reads the pinned delta itself).  Every variant's result is
    checked."""
    import torch

    import sparse_bf16_delta_amd as sbd
    from sparse_bf16_delta_amd.plan import ApplyPlan, DiffPlan, StreamedApplyPlan
    import workloads

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    cfg = workloads.CONFIGS[args.config]
    lr = args.lr if args.lr is not None else (1e-6 if cfg.key == "llama7b" else cfg.lrs[0])
    mode = args.mode or cfg.mode
    numels = cfg.numels
    n_model = sum(numels)
    offs, n_alloc = workloads.flat_layout(numels)
    old = torch.zeros(n_alloc, dtype=torch.bfloat16, device=dev)
    new = torch.zeros(n_alloc, dtype=torch.bfloat16, device=dev)
    for t, (o, n) in enumerate(zip(offs, numels)):
        workloads.fill_step_pair_(old[o:o + n], new[o:o + n], *workloads.seeds(cfg.seed_family, t),
                                  lr, mode)
    olds = [old[o:o + n] for o, n in zip(offs, numels)]
    news = [new[o:o + n] for o, n in zip(offs, numels)]
    snap = old.clone()
    snaps = [snap[o:o + n] for o, n in zip(offs, numels)]
    dplan = DiffPlan(olds, news, n_model // 8 + 65536)
    dplan.run()
    nnz = dplan.changed()
    t0 = time.perf_counter()
    h_idx = dplan.idx[:nnz].cpu().pin_memory()
    h_val = dplan.val[:nnz].cpu().pin_memory()
    h_off = dplan.offsets.cpu().pin_memory()
    mask = sbd.xor_mask(old, new)
    h_mask = mask.cpu().pin_memory()
    del mask
    log(f"[bench] receiver, {cfg.key}: {nnz:,} changed; delta {6 * nnz / 1e9:.3f} GB and mask "
        f"{2 * n_alloc / 1e9:.2f} GB pinned on the host in {time.perf_counter() - t0:.1f} s")
    k = len(numels)
    nchunks = max(1, min(args.chunks, k))
    bounds = sorted(set([round(i * k / nchunks) for i in range(nchunks + 1)]))
    d_idx = torch.empty_like(dplan.idx[:nnz])
    d_val = torch.empty_like(dplan.val[:nnz])
    d_off = torch.empty_like(dplan.offsets)
    d_mask = torch.empty(n_alloc, dtype=h_mask.dtype, device=dev)  # same dtype: a bit copy
    aplan = ApplyPlan(snaps)
    reps = max(args.steps, 5)

    def timed(fn, reset):
        """Median wall time of `reps` runs (each from the same start state):
        host-side copies and stream hand-offs make single runs noisy."""
        fn()
        torch.cuda.synchronize()
        samples = []
        for _ in range(reps):
            reset()
            torch.cuda.synchronize()
            t = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            samples.append(time.perf_counter() - t)
        return 1e3 * sorted(samples)[len(samples) // 2]

    def reset():
        snap.copy_(old)

    def copy_delta():
        d_idx.copy_(h_idx, non_blocking=True)
        d_val.copy_(h_val, non_blocking=True)
        d_off.copy_(h_off, non_blocking=True)

    def serial_sparse():
        copy_delta()
        aplan.run(d_idx, d_val, d_off, nnz)

    offs_h = h_off.tolist()
    splan = StreamedApplyPlan(snaps, bounds,
                              max(offs_h[hi] - offs_h[lo] for lo, hi in zip(bounds, bounds[1:])))

    def streamed_sparse():
        splan.run(h_idx, h_val, h_off)

    def host_direct_sparse():
        sbd.apply_many_host_(snaps, h_idx, h_val, h_off)

    def copy_mask():
        d_mask.copy_(h_mask, non_blocking=True)

    def serial_xor():
        copy_mask()
        sbd.xor_apply_(snap, d_mask)

    chunk = 1 << 27

    def streamed_xor():
        sbd.xor_apply_streamed_(snap, h_mask, chunk_elems=chunk)

    rows = {}
    for name, fn, check in (("sparse copy", copy_delta, None),
                            ("sparse copy+apply", serial_sparse, new),
                            ("sparse streamed", streamed_sparse, new),
                            ("sparse host-direct", host_direct_sparse, new),
                            ("xor copy", copy_mask, None),
                            ("xor copy+apply", serial_xor, new),
                            ("xor streamed", streamed_xor, new)):
        ms = timed(fn, reset)
        ok = True
        if check is not None:
            ok = torch.equal(snap.view(torch.int16), check.view(torch.int16))
        b = 6 * nnz if name.startswith("sparse") else 2 * n_alloc
        rows[name] = {"ms": round(ms, 3), "host_gbs": round(b / (ms * 1e-3) / 1e9, 2),
                      "identical": ok}
        log(f"[bench] {name:18s} {ms:9.3f} ms  {b / (ms * 1e-3) / 1e9:7.2f} GB/s from the host"
            f"{'' if ok else '  MISMATCH'}")
        if not ok:
            print("bench.py: receiver result mismatch", file=sys.stderr)
            sys.exit(1)
    print(json.dumps({
        "metric": "receiver with host-resident input: copy, copy+apply and streamed times "
                  "(median of steps runs)",
        "value": None, "unit": "ms", "n_gpus": 1, "steps": reps, "warmup": 1,
        "higher_is_better": False, "dtype": "u16", "data": "synthetic",
        "config": {"workload": f"{cfg.title}: {k} tensors, {n_model} elements, {mode} step lr "
                               f"{lr:g}; {len(bounds) - 1} parameter chunks, XOR chunks of "
                               f"{chunk} elements"},
        "changed": nnz, "rows": rows,
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", None)},
    }), flush=True)


def sharded_run(args, props):
    """Every rank of a W-way Shard(0) split of the list diffs its pieces with
    delta_diff_many_sharded (int64 global positions), one rank after another
    on this GPU; the ranks' deltas, concatenated per parameter in rank order,
    must equal the unsharded delta."""
    import torch

    import sparse_bf16_delta_amd as sbd
    from sparse_bf16_delta_amd.plan import DiffPlan
    import workloads

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    cfg = workloads.CONFIGS[args.config]
    lr = args.lr if args.lr is not None else (1e-6 if cfg.key == "llama7b" else cfg.lrs[0])
    mode = args.mode or cfg.mode
    numels = cfg.numels
    n_model = sum(numels)
    offs, n_alloc = workloads.flat_layout(numels)
    old = torch.zeros(n_alloc, dtype=torch.bfloat16, device=dev)
    new = torch.zeros(n_alloc, dtype=torch.bfloat16, device=dev)
    for t, (o, n) in enumerate(zip(offs, numels)):
        workloads.fill_step_pair_(old[o:o + n], new[o:o + n], *workloads.seeds(cfg.seed_family, t),
                                  lr, mode)
    shapes = [shape for _, shape in cfg.params]
    world = args.shards
    log(f"[bench] {cfg.key}: {len(shapes)} tensors, {n_model:,} elements, split over {world} "
        f"ranks by rows")

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    full = DiffPlan([old[o:o + n] for o, n in zip(offs, numels)],
                    [new[o:o + n] for o, n in zip(offs, numels)], n_model // 8 + 65536)
    t_full = timed(full.run)
    nnz_total = full.changed()
    f_off = full.offsets.cpu().tolist()
    rows, pieces = [], []
    for rank in range(world):
        lo, ln, fo, nel = [], [], [], []
        for (o, n), shape in zip(zip(offs, numels), shapes):
            first, count = sbd.shard0_piece(shape[0], world, rank)
            inner = n // shape[0]
            a, b = o + first * inner, o + (first + count) * inner
            lo.append(old[a:b])
            ln.append(new[a:b])
            fo.append(sbd.flat_offset(shape, first))
            nel.append(b - a)
        plan = DiffPlan(lo, ln, sum(nel) // 8 + 65536, flat_offsets=fo)
        t = timed(plan.run)
        k = plan.changed()
        rows.append({"rank": rank, "elements": sum(nel), "changed": k, "ms": round(t, 4),
                     "frac": round((4 * sum(nel) + 10 * k) / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
        pieces.append((plan.idx[:k].clone(), plan.val[:k].clone(), plan.offsets.cpu().tolist()))
        log(f"[bench] rank {rank}: {sum(nel):,} elements, {k:,} changed, {t:.3f} ms, "
            f"{100 * rows[-1]['frac']:.1f} % of peak (4n + 10 nnz)")
    # the ranks' deltas, in rank order per parameter, are the unsharded delta
    same = True
    for p in range(len(shapes)):
        gi = torch.cat([pi[pi_off[p]:pi_off[p + 1]] for pi, _, pi_off in pieces])
        gv = torch.cat([pv[pi_off[p]:pi_off[p + 1]] for _, pv, pi_off in pieces])
        fi = full.idx[f_off[p]:f_off[p + 1]].long()
        fv = full.val[f_off[p]:f_off[p + 1]]
        same &= torch.equal(gi, fi) and torch.equal(gv.view(torch.int16), fv.view(torch.int16))
    t_sum = sum(r["ms"] for r in rows)
    log(f"[bench] unsharded diff_many {t_full:.3f} ms; all ranks' sharded diffs {t_sum:.3f} ms; "
        f"concatenation identical: {same}")
    if not same:
        print("bench.py: sharded deltas do not concatenate to the unsharded delta", file=sys.stderr)
        sys.exit(1)
    print(json.dumps({
        "metric": "sharded diff: per-rank delta_diff_many_sharded time for a Shard(0) split",
        "value": None, "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": False, "dtype": "u16", "data": "synthetic",
        "config": {"workload": f"{cfg.title}: {len(shapes)} tensors, {n_model} elements, "
                               f"{mode} step lr {lr:g}, {world}-way Shard(0) split"},
        "unsharded_ms": round(t_full, 4), "sharded_sum_ms": round(t_sum, 4), "changed": nnz_total,
        "ranks": rows, "identical": same,
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", None)},
    }), flush=True)


def density_sweep(args, props):
    """Sparse path (diff + apply) and XOR path (xor_mask + xor_apply) on one
    flat 2^28-element tensor at each forced density, uniform and clustered:
    times, algorithmic bytes and the density where XOR becomes cheaper."""
    import torch

    import sparse_bf16_delta_amd as sbd
    from sparse_bf16_delta_amd.plan import ApplyPlan, DiffPlan
    import workloads

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    n = 1 << 28
    reps = max(args.steps, 1)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    rows = []
    log(f"[bench] density sweep, {n:,} elements, {reps} reps per op")
    log(f"[bench] {'pattern':9s} {'density':>8s} {'changed':>11s} {'diff ms':>8s} {'%pk':>5s} "
        f"{'apply ms':>9s} {'%pk':>5s} {'xor_mask':>9s} {'xor_apply':>10s} {'sparse/xor':>10s}")
    only = None
    if args.sweep_case:
        pat, _, dens = args.sweep_case.partition(":")
        only = (pat, float(dens))
        if pat not in ("uniform", "clustered") or only[1] not in workloads.DENSITIES:
            print(f"bench.py: --sweep-case {args.sweep_case}: pattern uniform or clustered, "
                  f"density one of {workloads.DENSITIES}", file=sys.stderr)
            sys.exit(2)
    for pattern in ("uniform", "clustered"):
        for di, frac in enumerate(workloads.DENSITIES):
            if only is not None and (pattern, frac) != only:
                continue
            old, new, k = workloads.density_case(n, frac, pattern, di, device=dev)
            snap = old.clone()
            mask = torch.empty(n, dtype=torch.int16, device=dev)
            cap = k + 65536
            dplan = DiffPlan([old], [new], cap)
            aplan = ApplyPlan([snap])
            t_diff = timed(dplan.run)
            got = dplan.changed()
            # the receiver knows the delta's entry count: the launch is sized to it
            t_apply = timed(lambda: aplan.run(dplan.idx, dplan.val, dplan.offsets, got))
            ok = got == k and torch.equal(snap.view(torch.int16), new.view(torch.int16))
            t_mask = timed(lambda: sbd.xor_mask(old, new, out=mask))
            t_xapp = timed(lambda: sbd.xor_apply_(snap, mask))
            back = old if (args.warmup + reps) % 2 else new  # xor_apply is self-inverse
            ok = ok and torch.equal(snap.view(torch.int16), back.view(torch.int16))
            pos = dplan.idx[:k].long()
            g128 = int(((pos >> 6)[1:] != (pos >> 6)[:-1]).sum().item()) + 1 if k else 0
            b_diff, b_apply, b_xor = 4 * n + 6 * k, 6 * k + 256 * g128, 6 * n
            f_diff = b_diff / (t_diff * 1e-3) / 1e9 / HBM_PEAK_GBS
            f_apply = b_apply / (t_apply * 1e-3) / 1e9 / HBM_PEAK_GBS
            ratio = (t_diff + t_apply) / (t_mask + t_xapp)
            rows.append({"pattern": pattern, "density": frac, "changed": k, "diff_ms": round(t_diff, 4),
                         "diff_frac": round(f_diff, 4), "apply_ms": round(t_apply, 4),
                         "apply_frac": round(f_apply, 4), "touched_lines_128B": g128,
                         "xor_mask_ms": round(t_mask, 4), "xor_apply_ms": round(t_xapp, 4),
                         "sparse_over_xor": round(ratio, 3), "identical": ok})
            log(f"[bench] {pattern:9s} {frac:8.3%} {k:11,d} {t_diff:8.3f} {100 * f_diff:5.1f} "
                f"{t_apply:9.3f} {100 * f_apply:5.1f} {t_mask:9.3f} {t_xapp:10.3f} {ratio:10.2f}"
                f"{'' if ok else '  MISMATCH'}")
            del old, new, snap, mask, dplan, aplan, pos
            if not ok:
                print("bench.py: density sweep result mismatch", file=sys.stderr)
                sys.exit(1)
    print(json.dumps({
        "metric": "density sweep: diff/apply and xor_mask/xor_apply times per density",
        "value": None, "unit": "ms", "n_gpus": 1, "steps": reps, "warmup": args.warmup,
        "higher_is_better": False, "dtype": "u16", "data": "synthetic",
        "config": {"workload": f"flat {n}-element bf16 tensor, forced subsets, uniform and "
                               f"clustered {workloads.CLUSTER_RUN}-element runs"},
        "sweep": rows,
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", None)},
    }), flush=True)


def layer_stream_run(args, props):
    """The 405B-shaped share (10 layers of 7 tensors, 64 GB per snapshot, old
    and new resident), streamed one layer at a time, each op in place on the
    resident `old`: xor_mask (old, new) into a one-layer mask, diff_many over
    the layer's tensors, apply_many into old (old becomes new), xor_apply of
    the mask (old comes back).  Per-op times are summed over the layers; a
    step is all ten layers."""
    import torch

    import sparse_bf16_delta_amd as sbd
    from sparse_bf16_delta_amd.plan import ApplyPlan, DiffPlan
    import workloads

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    cfg = workloads.CONFIGS["llama405b_share"]
    lr = args.lr if args.lr is not None else cfg.lrs[0]
    mode = args.mode or cfg.mode
    numels = cfg.numels
    n_model = sum(numels)
    offs, n_alloc = workloads.flat_layout(numels)
    per = 7
    layers = len(numels) // per
    log(f"[bench] device {props.name}, {props.total_memory / 2**30:.0f} GiB")
    log(f"[bench] workload {cfg.key}: {layers} layers x {per} tensors, {n_model:,} elements, "
        f"lr {lr:g}, {mode}")
    t0 = time.perf_counter()
    old = torch.zeros(n_alloc, dtype=torch.bfloat16, device=dev)
    new = torch.zeros(n_alloc, dtype=torch.bfloat16, device=dev)
    for t, (o, n) in enumerate(zip(offs, numels)):
        workloads.fill_step_pair_(old[o:o + n], new[o:o + n], *workloads.seeds(cfg.seed_family, t),
                                  lr, mode)
    torch.cuda.synchronize()
    log(f"[bench] generated inputs in {time.perf_counter() - t0:.1f} s")
    bounds = [offs[per * l] for l in range(layers)] + [n_alloc]
    region = max(bounds[l + 1] - bounds[l] for l in range(layers))
    mask = torch.empty(region, dtype=torch.int16, device=dev)
    L = []
    for l in range(layers):
        r0, r1 = bounds[l], bounds[l + 1]
        ts = range(per * l, per * l + per)
        lo = [old[offs[t]:offs[t] + numels[t]] for t in ts]
        ln = [new[offs[t]:offs[t] + numels[t]] for t in ts]
        n_l = sum(numels[t] for t in ts)
        cap = n_l // 8 + 65536
        dp = DiffPlan(lo, ln, cap)
        dp.run()
        k = dp.changed()
        if k > cap:
            cap = k + 65536
            dp = DiffPlan(lo, ln, cap)
            dp.run()
            k = dp.changed()
        poff = torch.tensor([offs[t] for t in ts], dtype=torch.int64, device=dev)
        pos = dp.idx[:k].long() + torch.repeat_interleave(poff, dp.nnz)
        g128 = int(((pos >> 6)[1:] != (pos >> 6)[:-1]).sum().item()) + 1 if k else 0
        del pos, poff
        # checksum of the delta: the restored `old` must give the same one again
        ck = (int(dp.idx[:k].to(torch.int64).sum().item()),
              int(dp.val[:k].view(torch.int16).to(torch.int64).sum().item()))
        L.append({"r0": r0, "r1": r1, "n": n_l, "nnz": k, "g128": g128, "dp": dp,
                  "ap": ApplyPlan(lo), "cap": cap, "ck": ck, "news": ln})
    nnz_total = sum(x["nnz"] for x in L)
    log(f"[bench] changed {nnz_total:,} of {n_model:,} ({nnz_total / n_model:.4%})")

    names = ["delta_diff_many", "delta_apply_many", "xor_mask", "xor_apply"]

    def layer_ops(x, ev=None):
        a, b = old[x["r0"]:x["r1"]], new[x["r0"]:x["r1"]]
        m = mask[:x["r1"] - x["r0"]]
        ops = (lambda: x["dp"].run(),
               lambda: x["ap"].run(x["dp"].idx, x["dp"].val, x["dp"].offsets, x["nnz"]),
               lambda: sbd.xor_mask(a, b, out=m),
               lambda: sbd.xor_apply_(a, m))
        # mask first (old, new), then diff, apply (old -> new), xor_apply (-> old)
        for i in (2, 0, 1, 3):
            if ev is not None:
                ev[2 * i].record(stream)
            ops[i]()
            if ev is not None:
                ev[2 * i + 1].record(stream)

    # one checked pass: after apply the layer equals new, after xor_apply old again
    for x in L:
        a, b = old[x["r0"]:x["r1"]], new[x["r0"]:x["r1"]]
        m = mask[:x["r1"] - x["r0"]]
        sbd.xor_mask(a, b, out=m)
        x["ap"].run(x["dp"].idx, x["dp"].val, x["dp"].offsets, x["nnz"])
        if not torch.equal(a.view(torch.int16), b.view(torch.int16)):
            print("bench.py: 405B-share apply check failed", file=sys.stderr)
            sys.exit(1)
        sbd.xor_apply_(a, m)
    for _ in range(args.warmup):
        for x in L:
            layer_ops(x)
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in L]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        for x, ev in zip(L, evs[k]):
            layer_ops(x, ev)
    torch.cuda.synchronize()
    ms_step = 1e3 * (time.perf_counter() - t_start) / args.steps
    op_ms = [sum(evs[k][l][2 * i].elapsed_time(evs[k][l][2 * i + 1])
                 for k in range(args.steps) for l in range(layers)) / args.steps
             for i in range(4)]
    for x in L:  # the restored old gives the same delta again
        x["dp"].run()
        ck = (int(x["dp"].idx[:x["nnz"]].to(torch.int64).sum().item()),
              int(x["dp"].val[:x["nnz"]].view(torch.int16).to(torch.int64).sum().item()))
        if x["dp"].changed() != x["nnz"] or ck != x["ck"]:
            print("bench.py: 405B-share timed steps changed the result", file=sys.stderr)
            sys.exit(1)
    g128 = sum(x["g128"] for x in L)
    alg = [4 * n_model + 6 * nnz_total, 6 * nnz_total + 256 * g128, 6 * n_alloc,
           2 * n_alloc + 256 * g128]
    traffic = measured_traffic(f"{cfg.key}:{mode}:{lr:g}")  # per launch, i.e. per layer
    kernels = []
    for name, ms, b in zip(names, op_ms, alg):
        gbs = b / (ms * 1e-3) / 1e9
        t = traffic.get(name) * layers if traffic.get(name) else None
        kernels.append({"kernel": name, "ms": round(ms, 3), "launches": layers, "alg_bytes": b,
                        "achieved_gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "traffic": t,
                        "moved_frac": round(t / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4) if t else None})
        log(f"[bench] {name:17s} {ms:9.3f} ms per step ({layers} launches)  {gbs:8.1f} GB/s "
            f"({100 * gbs / HBM_PEAK_GBS:.1f} % of peak)")
    # the step is the sparse-mode sync (diff + apply, as in the default run);
    # the XOR mode's two ops run interleaved per layer and are reported beside it
    dom = max(range(2), key=lambda i: op_ms[i])
    sync_ms = op_ms[0] + op_ms[1]
    xor_ms = op_ms[2] + op_ms[3]
    result = {
        "metric": METRIC,
        "value": round(2 * n_model / (sync_ms * 1e-3) / 1e9, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(sync_ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u16", "data": "synthetic",
        "config": {"workload": f"{cfg.title}: {len(numels)} tensors, {n_model} bf16 elements, "
                               f"{mode} step lr {lr:g}, streamed layer by layer",
                   "tensors": len(numels), "layers": layers, "elements": n_model,
                   "changed": nnz_total, "density": round(nnz_total / n_model, 6),
                   "touched_lines_128B": g128,
                   "step": "one sparse-mode sync, layer by layer: diff_many, then apply_many into "
                           "the resident old (which becomes new); value = one snapshot's bytes "
                           "per summed diff + apply time (HIP events)"},
        "roofline": {"bound": "hbm", "kernel": names[dom], "achieved": kernels[dom]["achieved_gbs"],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": kernels[dom]["frac"],
                     "traffic": kernels[dom]["traffic"]},
        "kernels": kernels,
        "xor_mode": {"ms_per_step": round(xor_ms, 3),
                     "weights_gbs": round(2 * n_model / (xor_ms * 1e-3) / 1e9, 2),
                     "step": "per layer, around the sync: xor_mask (old, new) into a one-layer "
                             "mask before it, xor_apply of the mask after it (old comes back)"},
        "wall_ms_per_step_all_ops": round(ms_step, 3),
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", None)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        x = L[0]
        result["cpu_baseline"] = cpu_baseline(args, cfg, old_views(old, offs, numels, 0, per),
                                              x["news"], x["dp"], x["nnz"])
    print(json.dumps(result), flush=True)


def old_views(old, offs, numels, layer, per):
    return [old[offs[t]:offs[t] + numels[t]] for t in range(per * layer, per * layer + per)]


def cpu_baseline(args, cfg, olds, news, dplan, nnz_total):
    """The CPU oracle, timed on this host on a bounded sample of the same
    workload: whole tensors in list order until the time budget is used.  The
    timed work per tensor is the bench's step, a sparse-mode sync (oracle
    diff, then oracle apply into a copy of old); the XOR mode's oracle pair is
    timed beside it.  The sample's GPU deltas are compared with the oracle's
    on the way."""
    import numpy as np
    import torch

    from oracle import oracle

    import workloads

    offs_dev = dplan.offsets.cpu().numpy()
    done_bytes, spent, xor_spent, tensors, elems, identical = 0, 0.0, 0.0, 0, 0, True
    for p, (o_t, n_t) in enumerate(zip(olds, news)):
        if spent + xor_spent >= args.cpu_seconds:
            break
        o = workloads.bits_numpy(o_t)
        x = workloads.bits_numpy(n_t)
        snap = o.copy()
        t0 = time.perf_counter()
        idx, val = oracle.diff(o, x)
        oracle.apply_(snap, idx, val)
        t1 = time.perf_counter()
        snap2 = o.copy()
        t2 = time.perf_counter()
        mask = oracle.xor_mask(o, x)
        oracle.xor_apply_(snap2, mask)
        t3 = time.perf_counter()
        spent += t1 - t0
        xor_spent += t3 - t2
        done_bytes += 2 * o.size
        tensors += 1
        elems += o.size
        identical &= bool(np.array_equal(snap, x) and np.array_equal(snap2, x))
        a, b = int(offs_dev[p]), int(offs_dev[p + 1])
        if b <= dplan.capacity:
            gi = dplan.idx[a:b].cpu().numpy()
            gv = dplan.val[a:b].view(torch.int16).cpu().numpy().view(np.uint16)
            identical &= bool(np.array_equal(gi, idx) and np.array_equal(gv, val))
    gbs = done_bytes / spent / 1e9 if spent > 0 else None
    xgbs = done_bytes / xor_spent / 1e9 if xor_spent > 0 else None
    log(f"[bench] cpu oracle: {tensors} tensors, {elems:,} elements, sparse sync {spent:.1f} s "
        f"({gbs:.3f} GB/s), XOR {xor_spent:.1f} s ({xgbs:.3f} GB/s), parity on sample: "
        f"{identical}")
    return {"value": round(gbs, 4) if gbs else None, "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"first {tensors} of {len(olds)} tensors ({elems} elements), one "
                      "sparse-mode sync per tensor (diff, then apply), single-threaded C",
            "xor_mode_value": round(xgbs, 4) if xgbs else None,
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model(),
            "sample_parity_identical": identical}


def cpu_torch_formulation(args, olds, news, dplan):
    """A second, labelled CPU point: the sources' own torch formulation (verl
    review, `shard_delta_indices`: an int16 view compare, nonzero and a
    gather; TRL article section 4.3: `snap[idx] = val`; XOR summary: mask and
    apply by XOR), with torch's intra-op threads on every host core, timed on
    whole tensors in list order until the budget is used.  Device-to-host
    copies are outside the timed region; the sample's deltas are compared with
    the GPU's."""
    import torch

    threads = torch.get_num_threads()
    offs_dev = dplan.offsets.cpu().tolist()
    done_bytes, spent, xor_spent, tensors, elems, identical = 0, 0.0, 0.0, 0, 0, True
    for p, (o_t, n_t) in enumerate(zip(olds, news)):
        if spent + xor_spent >= args.torch_cpu_seconds:
            break
        o = o_t.detach().reshape(-1).view(torch.int16).cpu()
        x = n_t.detach().reshape(-1).view(torch.int16).cpu()
        snap = o.clone()
        t0 = time.perf_counter()
        idx = (x != o).nonzero().squeeze(1)
        val = x[idx]
        snap[idx] = val
        t1 = time.perf_counter()
        snap2 = o.clone()
        t2 = time.perf_counter()
        mask = o ^ x
        snap2 ^= mask
        xor_spent += time.perf_counter() - t2
        spent += t1 - t0
        done_bytes += 2 * o.numel()
        tensors += 1
        elems += o.numel()
        a, b = offs_dev[p], offs_dev[p + 1]
        if b <= dplan.capacity:
            identical &= bool(torch.equal(dplan.idx[a:b].cpu().long(), idx) and
                              torch.equal(dplan.val[a:b].view(torch.int16).cpu(), val) and
                              torch.equal(snap, x) and torch.equal(snap2, x))
    gbs = done_bytes / spent / 1e9 if spent > 0 else None
    xgbs = done_bytes / xor_spent / 1e9 if xor_spent > 0 else None
    log(f"[bench] cpu torch formulation: {tensors} tensors, {elems:,} elements, sparse sync "
        f"{spent:.1f} s ({gbs:.3f} GB/s), XOR {xor_spent:.1f} s, {threads} threads, matches the "
        f"GPU on the sample: {identical}")
    return {"value": round(gbs, 4) if gbs else None, "unit": "GB/s", "threads": threads,
            "kind": "torch_cpu_formulation",
            "sample": f"first {tensors} of {len(olds)} tensors ({elems} elements), one "
                      "sparse-mode sync per tensor (int16-view compare + nonzero + gather, "
                      "index assignment)",
            "xor_mode_value": round(xgbs, 4) if xgbs else None,
            "sample_matches_gpu": identical}


if __name__ == "__main__":
    main()
