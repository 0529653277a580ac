"""Benchmark of the grouped materialise kernel on one MI355X.

One step = one st_materialize launch over every descriptor of a seeded synthetic checkpoint whose
blob is already resident in HBM (staging is measured separately).  Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--config 4] [--configs 2,3,4,5] [--all] [--no-cpu]

By default every benchmark family is timed in one run: the scaled-FP8 DiT checkpoint (c2), the
block-FP8 LLM checkpoint (c3), the NVFP4 checkpoint (c4) and the many-small-tensor blob (c5), each
with its own roofline fraction under "formats".  The headline ``value`` and ``roofline`` are the
NVFP4 checkpoint's, the largest of them (26.87 GB of traffic per launch).  ``--all`` adds the tiny
blob and the MXFP8 / MXFP4 checkpoints.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import tempfile
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
METRIC = "materialise GB/s (read+write) and % of HBM peak per checkpoint format"

WORKLOADS = {
    1: "tiny mixed blob: 2 bf16 [256,256], 2 fp32 [512], 2 e4m3fn [384,256] + fp32 scale, 2 fp16 [64,1000], unaligned",
    2: "scaled-FP8 DiT checkpoint: 57 blocks of e4m3fn [3072,3072]x4, [12288,3072], [3072,12288] with fp32 "
       "per-tensor scale_weight, 7 bf16 [3072] vectors per block",
    3: "block-FP8 LLM checkpoint: 28 layers, hidden 4096, e4m3fn q/k/v/o [4096,4096], gate/up [12288,4096], "
       "down [4096,12288] with fp32 128x128 weight_scale_inv grids, bf16 embedding [151936,4096] and norms",
    4: "NVFP4 checkpoint: 40 layers of [25600,5120] and [5120,25600] packed e2m1 with e4m3fn scale per 16 "
       "elements and fp32 global scale",
    5: "many-small-tensor stress blob: 20,000 tensors of 64 B - 64 KB, bf16/fp16/fp32/scaled-e4m3fn, unaligned",
    6: "MXFP8 LLM checkpoint: 28 layers, hidden 4096, e4m3fn q/k/v/o [4096,4096], gate/up [12288,4096], "
       "down [4096,12288] with an E8M0 scale per 32 elements along K, bf16 norms",
    7: "MXFP4 checkpoint: 40 layers of [25600,5120] and [5120,25600] packed e2m1 with an E8M0 scale per 32 "
       "elements along K",
}


ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ("device_checkpoint_dequantisation_amd/csrc/materialize.hip",
                  "device_checkpoint_dequantisation_amd/csrc/st_internal.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def profiled_traffic(k):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary
    (profiles/materialize_hbm_counters.md), or None when that summary does not cover config k or
    the kernel sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "materialize_hbm_counters.md")
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    sha, traffic = None, None
    for line in open(path):
        parts = line.split()
        if len(parts) == 2 and parts[0] == "kernel_sources_sha256":
            sha = parts[1]
        if len(parts) == 3 and parts[0] == "traffic_bytes" and parts[1] == f"c{k}":
            traffic = int(parts[2])
    return traffic if sha == h.hexdigest() else None


def pinned_to_device(device, nbytes, piece=1 << 30, reps=3):
    """Host-to-device copy rate on its own: ``nbytes`` copied from one pinned buffer (touched
    beforehand) into one device buffer of the same size, piece by piece, with hipMemcpyAsync on a
    side stream, timed with events on that stream.  The staged blob is left alone."""
    import torch
    n = min(piece, nbytes)
    host = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    host.fill_(0x3C)
    dst = torch.empty(n, dtype=torch.uint8, device=device)
    side = torch.cuda.Stream(device)
    side.wait_stream(torch.cuda.current_stream(device))
    best = None
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(side):
            a.record(side)
            for off in range(0, nbytes, n):
                m = min(n, nbytes - off)
                dst[:m].copy_(host[:m], non_blocking=True)
            b.record(side)
        side.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None else min(best, ms)
    del host, dst
    return nbytes / (best * 1e-3) / 1e9


def drop_page_cache(path):
    """Ask the kernel to evict the file's pages from the page cache (fsync, then
    POSIX_FADV_DONTNEED); True if the request was accepted.  The eviction is advisory."""
    try:
        fd = os.open(path, os.O_RDONLY)
        try:
            os.fsync(fd)
            os.posix_fadvise(fd, 0, 0, os.POSIX_FADV_DONTNEED)
        finally:
            os.close(fd)
        return True
    except (OSError, AttributeError):
        return False


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4, choices=sorted(WORKLOADS),
                    help="the headline workload (value, roofline, cpu_baseline)")
    ap.add_argument("--configs", default="2,3,4,5",
                    help="comma-separated families timed beside the headline (empty: the headline only)")
    ap.add_argument("--all", action="store_true", help="also measure the tiny blob and the MX families")
    ap.add_argument("--cold-stage", action=argparse.BooleanOptionalAction, default=True,
                    help="also stage the headline checkpoint after asking the kernel to drop it from the page cache")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU oracle sample budget")
    ap.add_argument("--unit-scale", type=int, default=0)
    ap.add_argument("--stream-chunk-mb", type=int, default=128, help="staging step of the overlapped load")
    ap.add_argument("--load-reps", type=int, default=2, help="repetitions of the end-to-end load comparison")
    ap.add_argument("--extras", action="store_true",
                    help="also measure, for the main config, the serial vs streamed end-to-end load, on-demand "
                         "per-layer loads and tensor-parallel shard decodes (they launch the kernel on other tables, "
                         "so a kernel-trace summary of the default command covers only the timed decode)")
    ap.add_argument("--shards", action="store_true",
                    help="also time the 8-way tensor-parallel shard decodes of the main config (part of --extras)")
    ap.add_argument("--out-types", action="store_true",
                    help="also time the fp16 and fp32 output types on the same checkpoint")
    ap.add_argument("--tmpdir", default=None)
    ap.add_argument("--keep", action="store_true", help="keep generated checkpoint files")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run one plain 1 GiB device copy (a known-size kernel that scales profiler byte counters)")
    ap.add_argument("--aligned-variant", action="store_true",
                    help="also time the scaled-FP8 checkpoint with every scale moved to the end (all weights 16-byte aligned)")
    return ap.parse_args()


def gen(k, d, overrides=None):
    import synth
    overrides = overrides or {}
    path = os.path.join(d, f"synthetic_c{k}{'_' + '_'.join(overrides) if overrides else ''}.safetensors")
    t0 = time.perf_counter()
    last = [t0]

    def progress(done, total):
        now = time.perf_counter()
        if now - last[0] > 10 or done == total:
            last[0] = now
            log(f"[bench] generating config {k}: {done}/{total} tensor groups, {now - t0:.0f}s")

    synth.write_config(k, path, progress=progress, **overrides)
    dt = time.perf_counter() - t0
    log(f"[bench] generated config {k}: {os.path.getsize(path) / 1e9:.3f} GB in {dt:.1f}s")
    return path, dt


def sampled_parity(path, ix, ck, rng, per_output=64, out_dtype="bf16"):
    """GPU outputs at random flat indices (plus first and last) against the oracle computed
    element by element on the same indices."""
    import torch
    import oracle
    mm = np.memmap(path, dtype=np.uint8, mode="r")
    h, outs = oracle.plan(mm)
    data = mm[h.data_offset:]
    checked = 0
    for o in outs:
        if o.numel == 0:
            continue
        idx = np.unique(np.concatenate([[0, o.numel - 1], rng.integers(0, o.numel, per_output)]))
        want = oracle.decode(o, data, idx, out_dtype)
        t = ck.tensors[o.name].reshape(-1)
        got = t[torch.from_numpy(idx).to(t.device)]
        got = (got.view(torch.int32).cpu().numpy().view(np.uint32) if out_dtype == "f32"
               else got.view(torch.int16).cpu().numpy().view(np.uint16))
        if not np.array_equal(got, want):
            return False, checked, o.name
        checked += len(idx)
    return True, checked, None


def cpu_baseline(path, budget_s, piece=1 << 20):
    """The oracle as it stands (single-threaded NumPy) decoding the checkpoint's outputs in file
    order, in calls of ``piece`` elements, until the time budget is spent; GB/s over the same
    algorithmic bytes as the kernel (each element's share of its output's read bytes + 2 bytes
    written).  Scale tensors count with the output they belong to."""
    import oracle
    mm = np.memmap(path, dtype=np.uint8, mode="r")
    h, outs = oracle.plan(mm)
    data = mm[h.data_offset:]
    nbytes = 0.0
    elems = 0
    done = 0
    t0 = time.perf_counter()
    with np.errstate(invalid="ignore", over="ignore"):
        for o in outs:
            read = (o.src.end - o.src.begin) + (o.scale.end - o.scale.begin if o.scale else 0) + \
                (o.scale2.end - o.scale2.begin if o.scale2 else 0)
            for a in range(0, o.numel, piece):
                b = min(o.numel, a + piece)
                oracle.decode(o, data, np.arange(a, b, dtype=np.int64))
                nbytes += read * (b - a) / o.numel + 2 * (b - a)
                elems += b - a
                if time.perf_counter() - t0 > budget_s:
                    break
            else:
                done += 1
                continue
            break
    dt = time.perf_counter() - t0
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "host_cpus": os.cpu_count(), "kind": "oracle",
            "sample": f"the first {elems:,} output elements in file order ({done} whole outputs of {len(outs)}, "
                      f"{nbytes / 1e9:.3f} GB of traffic) decoded by the single-threaded NumPy oracle in "
                      f"{piece:,}-element calls, {dt:.1f}s, on 1 of the host's {os.cpu_count()} CPUs"}


def measure(k, d, args, rng, overrides=None):
    import torch
    import device_checkpoint_dequantisation_amd as st
    path, gen_s = gen(k, d, overrides)
    t0 = time.perf_counter()
    ix = st.SafeTensorIndex.open(path, args.unit_scale)
    index_ms = (time.perf_counter() - t0) * 1e3
    dev = torch.device("cuda:0")
    ck = st.DeviceCheckpoint(ix, None, dev)
    pinned = torch.empty(512 << 20, dtype=torch.uint8, pin_memory=True)
    side = torch.cuda.Stream(dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    st.stage_file(path, ix, ck.blob, pinned, side)   # first staging: touches the new pinned pages
    side.synchronize()
    first_stage_s = time.perf_counter() - t0
    t0 = time.perf_counter()
    read_s = st.stage_file(path, ix, ck.blob, pinned, side)
    side.synchronize()
    stage_s = time.perf_counter() - t0
    h2d = pinned_to_device(dev, ix.data_size)   # the copy alone, from pinned pages already touched
    cold = None
    if k == args.config and args.cold_stage:
        if drop_page_cache(path):
            t0 = time.perf_counter()
            cold_read_s = st.stage_file(path, ix, ck.blob, pinned, side)
            side.synchronize()
            cold_s = time.perf_counter() - t0
            cold = {"file_to_pinned_GBps": round(ix.data_size / cold_read_s / 1e9, 2) if cold_read_s > 0 else None,
                    "file_to_device_GBps": round(ix.data_size / cold_s / 1e9, 2),
                    "page_cache": "dropped first (fsync + POSIX_FADV_DONTNEED, advisory)"}
            log(f"[bench] config {k}: staging after dropping the page cache {ix.data_size / cold_s / 1e9:.2f} GB/s")
        else:
            cold = {"page_cache": "could not be dropped on this host"}
        st.stage_file(path, ix, ck.blob, pinned, side)   # the blob as staged, for the timed decode
        side.synchronize()
    del pinned
    traffic = ix.traffic_bytes
    log(f"[bench] config {k}: {ix.num_outputs} outputs, traffic {traffic / 1e9:.3f} GB, index {index_ms:.1f} ms, "
        f"staged {ix.data_size / 1e9:.3f} GB in {stage_s:.2f}s (reads {read_s:.2f}s)")
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        ck.materialize(stream)
    torch.cuda.synchronize()
    ok, checked, bad = sampled_parity(path, ix, ck, rng)
    log(f"[bench] sampled parity vs oracle: {'ok' if ok else 'MISMATCH in ' + str(bad)} ({checked} elements)")
    shards = None
    if k == args.config and (args.extras or args.shards):
        shards = tp_shards(ix, ck, max(3, args.steps // 5))
        log(f"[bench] tensor-parallel shards: {shards}")
    # timed region: K back-to-back launches between one pair of HIP events on the launch stream, and
    # the wall clock; the mean launch duration is the events' interval over K (per-launch event pairs
    # would add a few microseconds to every interval, a tenth of a many-small launch)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        ck.materialize(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_ms = start.elapsed_time(end)
    # after the timed region: each launch between its own events, for the spread of single launches
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        ck.materialize(stream)
        b.record(stream)
    torch.cuda.synchronize()
    kms = np.array([a.elapsed_time(b) for a, b in evs])
    flushed = None
    if traffic < 2e9:   # cache-resident checkpoints: also time each launch after flushing the caches
        flushed = flushed_launch_ms(ck, stream, args.steps)
        log(f"[bench] config {k}: cold-cache launch {flushed['clean']['median']:.4f} ms clean, "
            f"{flushed['dirty']['median']:.4f} ms dirty (median) vs hot {float(np.median(kms)):.4f} ms")
    load = None
    if k == args.config and args.extras:
        load = end_to_end_loads(path, ix, ck, side, stream, args, rng)
    types = None
    if k == args.config and (args.extras or args.out_types):
        types = out_types(path, ck, args, rng)
        log(f"[bench] output types: {types}")
    res = {
        "k": k, "path": path, "traffic": traffic, "read": ix.data_size, "written": traffic - ix.data_size,
        "outputs": ix.num_outputs, "ms_per_step": wall * 1e3 / args.steps, "kernel_ms_mean": region_ms / args.steps,
        "kernel_ms_median": float(np.median(kms)), "kernel_ms_min": float(kms.min()), "index_ms": index_ms,
        "stage": dict({"file_to_pinned_GBps": round(ix.data_size / read_s / 1e9, 2) if read_s > 0 else None,
                       "pinned_to_device_GBps": round(h2d, 2),
                       "file_to_device_GBps": round(ix.data_size / stage_s / 1e9, 2),
                       "file_to_device_first_GBps": round(ix.data_size / first_stage_s / 1e9, 2),
                       "page_cache": "warm (file just written)",
                       "pinned_ring": "512 MiB; 'first' includes touching its freshly pinned pages",
                       "pinned_to_device": "1 GiB pinned buffer, touched, copied with hipMemcpyAsync on a side "
                                           "stream and timed with events there (best of 3)"},
                      **({"cold": cold} if cold else {}), **(load or {})),
        "gen_s": gen_s, "parity": "sampled-bit-exact" if ok else f"MISMATCH:{bad}", "parity_elements": checked,
        "shards": shards, "out_types": types, "flushed": flushed,
    }
    res["GBps"] = traffic / (res["ms_per_step"] * 1e-3) / 1e9
    res["kernel_GBps"] = traffic / (res["kernel_ms_mean"] * 1e-3) / 1e9
    del ck
    torch.cuda.empty_cache()
    return res


def flushed_launch_ms(ck, stream, steps):
    """Kernel time with cold caches, each launch timed on its own after a flush outside the timed
    events: "clean" writes a 1 GiB scratch buffer and then reads another 1 GiB buffer, so the L2 and
    the 256 MB Infinity Cache hold only clean lines of unrelated data; "dirty" only writes the 1 GiB
    buffer, so the launch also pays for writing back up to 256 MB of the scratch buffer's dirty lines
    as its own traffic evicts them (measured on MI355X: 37 us of fixed cost per launch against 7.6 us
    clean, while the per-copy cost of the many-small checkpoint is the same)."""
    import torch
    w = torch.empty(1 << 30, dtype=torch.uint8, device=ck.device)
    r = torch.empty(1 << 30, dtype=torch.uint8, device=ck.device)
    r.fill_(1)
    res = {}
    for mode in ("clean", "dirty"):
        ms = []
        for i in range(max(3, steps)):
            w.fill_(i & 0xFF)
            if mode == "clean":
                torch.sum(r, dtype=torch.int64)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            ck.materialize(stream)
            b.record(stream)
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        res[mode] = {"median": float(np.median(ms)), "min": float(np.min(ms))}
    del w, r
    return res


def out_types(path, ck, args, rng):
    """The same decode into fp16 and fp32 outputs: tables planned for each type, the blob copied
    from the bf16 checkpoint, sampled parity against the oracle's rounding to that type, and GB/s
    over that type's algorithmic bytes (bytes read + 2 or 4 bytes per element written)."""
    import torch
    import device_checkpoint_dequantisation_amd as st
    res = {}
    for dt in ("f16", "f32"):
        ix = st.SafeTensorIndex.open(path, args.unit_scale, dt)
        ck2 = st.DeviceCheckpoint(ix, None, ck.device)
        ck2.blob.copy_(ck.blob)
        stream = torch.cuda.current_stream(ck.device)
        for _ in range(args.warmup):
            ck2.materialize(stream)
        torch.cuda.synchronize()
        ok, checked, bad = sampled_parity(path, ix, ck2, rng, out_dtype=dt)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for a, b in evs:
            a.record(stream)
            ck2.materialize(stream)
            b.record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
        res[dt] = {"kernel_ms_mean": round(ms, 4), "traffic_bytes": ix.traffic_bytes,
                   "GBps": round(ix.traffic_bytes / (ms * 1e-3) / 1e9, 2),
                   "parity": "sampled-bit-exact" if ok else f"MISMATCH:{bad}", "parity_elements": checked}
        del ck2
        ix.close()
        torch.cuda.empty_cache()
    return res


def end_to_end_loads(path, ix, ck, side, stream, args, rng):
    """End-to-end load with a warm page cache: serial (stage everything, then one launch) against
    the overlapped pipeline (each staging step decoded while later steps are read and copied)."""
    import torch
    import device_checkpoint_dequantisation_amd as st
    pinned = torch.empty(512 << 20, dtype=torch.uint8, pin_memory=True)
    plan = st.StreamPlan(ix, args.stream_chunk_mb << 20)
    ck.stream(path, stream=stream, plan=plan)  # allocates the pinned ring once
    ck.synchronize()
    serial_s, stream_s, sstats = [], [], None
    for _ in range(args.load_reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        st.stage_file(path, ix, ck.blob, pinned, side)
        side.synchronize()
        ck.materialize(stream)
        torch.cuda.synchronize()
        serial_s.append(time.perf_counter() - t0)
        t0 = time.perf_counter()
        sstats = ck.stream(path, stream=stream, plan=plan)
        ck.synchronize()
        stream_s.append(time.perf_counter() - t0)
    del pinned
    sok, _, sbad = sampled_parity(path, ix, ck, rng)
    log(f"[bench] load: serial {min(serial_s):.3f}s, streamed {min(stream_s):.3f}s in {len(plan.steps)} steps "
        f"({sstats['launches']} launches); streamed parity {'ok' if sok else 'MISMATCH in ' + str(sbad)}")
    return {"serial_load_GBps": round(ix.data_size / min(serial_s) / 1e9, 2),
            "streamed_load_GBps": round(ix.data_size / min(stream_s) / 1e9, 2),
            "streamed_load_s": round(min(stream_s), 4), "serial_load_s": round(min(serial_s), 4),
            "stream_chunk_MiB": args.stream_chunk_mb, "stream_steps": len(plan.steps),
            "stream_launches": sstats["launches"], "streamed_parity": "sampled-bit-exact" if sok else f"MISMATCH:{sbad}",
            "streamed_first_decode_enqueued_ms": round(1e3 * sstats["seconds_first_launch"], 3),
            "first_outputs": "streamed: the first step's outputs are decoded as soon as its bytes land, "
                             "streamed_first_decode_enqueued_ms after the call starts; serial: no output "
                             "before the whole data section is staged (serial_load_s)"}


def cold_loads(path, args, rng):
    """The serial and the streamed end-to-end load once each after dropping the file's pages from
    the page cache (run last: reading the file back leaves its pages cached in another state than
    writing it did, which would change the warm figures measured after it), and the on-demand
    per-layer loads without a RAM tier the same way."""
    import re
    import torch
    import device_checkpoint_dequantisation_amd as st
    ix = st.SafeTensorIndex.open(path)
    dev = torch.device("cuda:0")
    ck = st.DeviceCheckpoint(ix, None, dev)
    pinned = torch.empty(512 << 20, dtype=torch.uint8, pin_memory=True)
    side = torch.cuda.Stream(dev)
    stream = torch.cuda.current_stream(dev)
    plan = st.StreamPlan(ix, args.stream_chunk_mb << 20)
    ck.stream(path, stream=stream, plan=plan)  # allocates the pinned ring once
    ck.synchronize()
    out = {}
    if not drop_page_cache(path):
        return {"page_cache": "could not be dropped on this host"}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    st.stage_file(path, ix, ck.blob, pinned, side)
    side.synchronize()
    ck.materialize(stream)
    torch.cuda.synchronize()
    out["serial_load_GBps"] = round(ix.data_size / (time.perf_counter() - t0) / 1e9, 2)
    drop_page_cache(path)
    ck.arena.view(torch.int16).fill_(0x7FBF)   # poison: the streamed load must write every output
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ck.stream(path, stream=stream, plan=plan)
    ck.synchronize()
    out["streamed_load_GBps"] = round(ix.data_size / (time.perf_counter() - t0) / 1e9, 2)
    ok, _, bad = sampled_parity(path, ix, ck, rng)
    out["streamed_parity"] = "sampled-bit-exact" if ok else f"MISMATCH:{bad}"
    del pinned, ck
    torch.cuda.empty_cache()
    # on-demand loads, one layer per load, no RAM tier (as lazy_loads' "file")
    sd = st.StreamStateDict(path, dev, index=ix)
    groups = {}
    for k in sd:
        m = re.match(r"^(.*?\.\d+)\.", k)
        groups.setdefault(m.group(1) if m else k.split(".")[0], []).append(k)
    src = sum(sd.meta(k).source_bytes for k in sd)
    drop_page_cache(path)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for keys in groups.values():
        got = sd.load(keys)
        torch.cuda.synchronize()
        del got
    out["lazy_per_layer_GBps"] = round(src / (time.perf_counter() - t0) / 1e9, 2)
    out["page_cache"] = "dropped before each load (fsync + POSIX_FADV_DONTNEED, advisory)"
    return out


SOURCE_BYTES = {"PASS_BF16": 2, "CAST_F16": 2, "CAST_F32": 4, "FP8_TENSOR": 1, "FP8_BLOCK128": 1,
                "NVFP4": 0.5 + 1 / 16, "MXFP8": 1 + 1 / 32, "MXFP4": 0.5 + 1 / 32}


def slice_traffic(ix, slices, out_bytes=2):
    """Algorithmic bytes of decoding `slices`: each element's source bytes (with its share of the
    NVFP4 / MX block scales) plus the output bytes; per-tensor and block-FP8 grid scales are
    counted per slice (4 bytes per scale the slice uses)."""
    outs = ix.outputs()
    total = 0.0
    for sl in slices:
        k = sl[0]
        r, c = ix.slice_shape(*sl)
        o = outs[k]
        total += r * c * (SOURCE_BYTES[o.kind] + out_bytes)
        if o.kind == "FP8_TENSOR":
            total += 4
        elif o.kind == "FP8_BLOCK128":
            total += 4 * -(-r // 128) * -(-c // 128)
        elif o.kind == "NVFP4":
            total += 4
    return int(total)


def tp_shards(ix, ck, steps, n=8):
    """Decode the whole checkpoint as n-way tensor-parallel shards of every 2-d output (row shards,
    then column shards; cuts on scale-block boundaries), one launch per layout, and check every
    shard against the unsharded decode on the GPU.  "col_shard_one" decodes one rank's column shard
    of every 2-d output (and every other output whole), as one GPU of an n-way tensor-parallel
    group would; its GB/s counts that table's own algorithmic bytes."""
    import torch
    import device_checkpoint_dequantisation_amd as st
    outs = ix.outputs()
    res = {}
    for label, axis in (("row_shards", 0), ("col_shards", 1), ("col_shard_one", 1)):
        slices = []
        for k, o in enumerate(outs):
            if len(o.shape) != 2:
                slices.append((k, None, None))
                continue
            dim = o.shape[axis]
            q = (128 if o.kind == "FP8_BLOCK128" else 16 if (o.kind == "NVFP4" and axis == 1)
                 else 32 if (o.kind in ("MXFP8", "MXFP4") and axis == 1) else 1)
            step = max(q, -(-dim // n // q) * q)
            for b in range(0, dim, step):
                part = (b, min(dim, b + step))
                slices.append((k, part, None) if axis == 0 else (k, None, part))
                if label == "col_shard_one":
                    break
        shapes = [ix.slice_shape(*sl) for sl in slices]
        offs, total = [], 0
        for r, c in shapes:
            offs.append(total)
            total += (2 * r * c + 255) // 256 * 256
        arena = torch.empty(max(total, 256) // 2, dtype=torch.bfloat16, device=ck.device)
        base = arena.data_ptr()
        ptrs = torch.tensor([base + o for o in offs], dtype=torch.int64).to(ck.device)
        raw, units = ix.table_slices(slices)
        nt = st.table_stream_stores(raw)
        strided = axis == 1  # column shards need the strided kernel; row shards are contiguous
        table = torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(ck.device)
        stream = torch.cuda.current_stream(ck.device)
        st.materialize(ck.blob, table, units, ptrs, stream, slices=strided, stream_stores=nt)
        torch.cuda.synchronize()
        ok = True
        for (k, rows, cols), (r, c), off in zip(slices, shapes, offs):
            got = arena[off // 2: off // 2 + r * c].view(r, c)
            whole = ck.tensors[outs[k].name]
            whole = whole.reshape(whole.shape[0], -1) if whole.dim() >= 2 else whole.reshape(-1, 1)
            r0, r1 = rows if rows else (0, whole.shape[0])
            c0, c1 = cols if cols else (0, whole.shape[1])
            ok &= torch.equal(got.view(torch.int16), whole[r0:r1, c0:c1].view(torch.int16))
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in evs:
            a.record(stream)
            st.materialize(ck.blob, table, units, ptrs, stream, slices=strided, stream_stores=nt)
            b.record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
        traffic = ix.traffic_bytes if label != "col_shard_one" else slice_traffic(ix, slices)
        res[label] = {"shards_per_output": n, "slices": len(slices), "kernel_ms_mean": round(ms, 4),
                      "kernel": "st_materialize_slices" if strided else "st_materialize",
                      "traffic_bytes": traffic, "GBps": round(traffic / (ms * 1e-3) / 1e9, 2),
                      "parity": "bit-exact vs whole decode" if ok else "MISMATCH"}
        del arena
    return res


def lazy_loads(path, dev):
    """On-demand loads through StreamStateDict, one layer (keys sharing their name up to the first
    numeric component) per load: without a RAM tier; filling a tier whose pinned memory is created as
    it fills; filling a tier preallocated when the mapping was created (its allocation timed on its
    own); and served from that tier."""
    import torch
    import device_checkpoint_dequantisation_amd as st
    import re
    probe = st.StreamStateDict(path, dev)
    groups = {}
    for k in probe:  # a layer: the name up to its first numeric component ("blocks.3", "model.layers.12")
        m = re.match(r"^(.*?\.\d+)\.", k)
        groups.setdefault(m.group(1) if m else k.split(".")[0], []).append(k)
    src = sum(probe.meta(k).source_bytes for k in probe)
    res = {"layers": len(groups), "source_bytes": src}
    for label, ram, pre in (("file", 0, False), ("file_into_new_ram", 1 << 40, False),
                            ("file_into_ram", 1 << 40, True), ("ram", None, None)):
        if ram is not None:
            sd = st.StreamStateDict(path, dev, ram_cache_bytes=ram, index=probe.index, ram_preallocate=pre)
            if pre:
                res["ram_preallocate"] = {"seconds": round(sd.ram_preallocate_seconds, 3),
                                          "bytes": sd.ram.arena.capacity,
                                          "GBps": round(sd.ram.arena.capacity / max(sd.ram_preallocate_seconds, 1e-9) / 1e9, 2)}
        before = dict(sd.stats)
        torch.cuda.synchronize()
        times = []
        for keys in groups.values():
            t0 = time.perf_counter()
            got = sd.load(keys)
            torch.cuda.synchronize()
            times.append(time.perf_counter() - t0)
            del got
        res[label] = {"GBps": round(src / sum(times) / 1e9, 2), "ms_per_layer_mean": round(1e3 * float(np.mean(times)), 3),
                      "ms_per_layer_max": round(1e3 * float(np.max(times)), 3),
                      "launches": int(sd.stats["launches"] - before.get("launches", 0)),
                      "ram_hits": int(sd.stats["ram_hits"] - before.get("ram_hits", 0))}
    return res


def family_line(k, v):
    """One family's figures for the "formats" object of the bench line."""
    tr = profiled_traffic(k)
    d = {"workload": WORKLOADS[k], "GBps": round(v["GBps"], 2), "hbm_peak_frac": round(v["GBps"] / HBM_PEAK_GBPS, 4),
         "roofline": {"bound": "hbm", "achieved": round(v["kernel_GBps"], 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                      "frac": round(v["kernel_GBps"] / HBM_PEAK_GBPS, 4), "traffic": tr,
                      "traffic_ratio": round(tr / v["traffic"], 4) if tr else None},
         "kernel_ms": {"mean": round(v["kernel_ms_mean"], 4), "single_launch_median": round(v["kernel_ms_median"], 4),
                       "single_launch_min": round(v["kernel_ms_min"], 4),
                       "how": "mean: HIP events around the K timed launches, over K; single launches: each "
                              "launch between its own events, after the timed region"},
         "traffic_bytes": v["traffic"], "read_bytes": v["read"], "written_bytes": v["written"], "outputs": v["outputs"],
         "parity": v["parity"], "parity_elements": v["parity_elements"], "staging": v["stage"]}
    if v.get("flushed"):
        for mode, label in (("clean", "flushed_cache"), ("dirty", "flushed_cache_dirty")):
            fl = v["flushed"][mode]
            d[label] = {"kernel_ms_median": round(fl["median"], 4),
                        "GBps": round(v["traffic"] / (fl["median"] * 1e-3) / 1e9, 2),
                        "hbm_peak_frac": round(v["traffic"] / (fl["median"] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                        "flush": ("1 GiB written, then another 1 GiB read: cold caches holding clean lines"
                                  if mode == "clean" else
                                  "1 GiB written: cold caches full of dirty lines that the launch writes back")}
    return d


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (each GPU decodes its own "
              f"outputs independently, and this library does not shard a checkpoint across GPUs)", file=sys.stderr)
        sys.exit(2)
    rng = np.random.default_rng(0)
    d = args.tmpdir or tempfile.mkdtemp(prefix="stmat_bench_")
    configs = [int(x) for x in args.configs.split(",") if x.strip()] if args.configs else []
    if args.all:
        configs += [k for k in sorted(WORKLOADS) if k not in configs]
    configs = [args.config] + [k for k in configs if k != args.config]
    results = {}
    cpu = None
    for k in configs:
        results[k] = measure(k, d, args, rng)
        r = results[k]
        log(f"[bench] config {k}: {r['GBps']:.1f} GB/s wall, {r['kernel_GBps']:.1f} GB/s by kernel events "
            f"({r['kernel_GBps'] / HBM_PEAK_GBPS:.3f} of HBM peak), parity {r['parity']}")
        if k == args.config and args.extras:
            results[k]["lazy"] = lazy_loads(results[k]["path"], "cuda:0")
            log(f"[bench] lazy per-layer loads: {results[k]['lazy']}")
        if k == args.config and not args.no_cpu:
            cpu = cpu_baseline(results[k]["path"], args.cpu_seconds)
            log(f"[bench] cpu oracle: {cpu['value']:.3f} GB/s ({cpu['sample']})")
        if k == args.config and args.extras:
            results[k]["cold_loads"] = cold_loads(results[k]["path"], args, rng)
            log(f"[bench] loads after dropping the page cache: {results[k]['cold_loads']}")
        if not args.keep:
            os.remove(results[k]["path"])
    aligned = None
    if args.aligned_variant:
        aligned = measure(2, d, args, rng, {"scales_last": True})
        if not args.keep:
            os.remove(aligned["path"])
    if args.copy_calibration:
        import torch
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
        b = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)   # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del a, b
    r = results[args.config]
    head = family_line(args.config, r)
    line = {
        "metric": METRIC, "value": round(r["GBps"], 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": WORKLOADS[args.config], "read_bytes": r["read"], "written_bytes": r["written"],
                   "outputs": r["outputs"], "hbm_peak_frac": round(r["GBps"] / HBM_PEAK_GBPS, 4),
                   "families_timed": [f"c{k}" for k in configs]},
        "roofline": {k: v for k, v in head["roofline"].items() if k != "traffic_ratio"},
        "cpu_baseline": cpu,
        "kernel_ms": head["kernel_ms"],
        "staging": r["stage"], "index_build_ms": round(r["index_ms"], 2), "parity": r["parity"],
        "formats": {f"c{k}": family_line(k, v) for k, v in results.items()},
    }
    if "lazy" in r:
        line["lazy_loads"] = r["lazy"]
    if "cold_loads" in r:
        line["loads_page_cache_dropped"] = r["cold_loads"]
    if r.get("shards"):
        line["tp_shards"] = r["shards"]
    if r.get("out_types"):
        line["output_types"] = r["out_types"]
    if aligned is not None:
        line["scaled_fp8_all_weights_16B_aligned"] = {"GBps": round(aligned["GBps"], 2),
                                                      "kernel_ms_mean": round(aligned["kernel_ms_mean"], 4),
                                                      "parity": aligned["parity"]}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
