"""Benchmark of the MLA decode hot path on one MI355X.

Workload: DeepSeek-V2 sized layer (128 heads, d_h^C 128, d_h^R 64, d_c 512,
bf16), batch 64, cached lengths uniform on [1024, 8192], 64-token pages in a
shuffled page table.  One step = append one new token per sequence (RoPE'd
key) + weight-absorbed decode over the attended lengths + 1 (q absorption,
split-KV attention, combine, W^UV), issued as one mla_decode_step call (the
append runs inside the first decode kernel).
Inputs are synthetic and seeded (mla_synth); the timed steps rotate over
several cache/weight replicas so that the 256 MB last-level cache cannot hold
the working set.

Prints one JSON line.  `value` is whole-step cached tokens per second with
every input resident in HBM; `roofline` describes the split-KV attention
kernel, timed with HIP events recorded on the launch stream around that
kernel; `cpu_baseline` times the fp64 oracle on a bounded sample of the same
workload on the host cores.
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

METRIC = "MLA decode cached-tokens/s + latent-cache GB/s, % of HBM/MFMA roofline"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
BYTES_PER_TOKEN = 1152          # one cached row: 576 bf16
FLOP_PER_TOKEN = 278528         # 2*128*576 (scores) + 2*128*512 (latent sum)
WARM_S = 1.0                    # untimed sustained-load warm-up per leg (--warm-seconds)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_splitkv_v2_b64_ragged_traffic.json")
KERNEL_SRCS = [os.path.join(ROOT, "mla_latent_kv_34_amd", "csrc", f)
               for f in ("decode_v2.hip", "splitkv_asm.h")]


def kernel_source_sha256() -> str:
    """Hash of the sources of the split-KV kernel (the traffic figures in
    TRAFFIC_FILE are only valid for the kernel they were counted on)."""
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def recorded_traffic(workload: str, workgroups: int, path: str = TRAFFIC_FILE):
    """HBM bytes per launch of decode_splitkv from the counter record, or None
    when the record does not describe this run: another workload, a
    non-default split-KV workgroup count (the counters were taken with one
    workgroup per compute unit), or kernel sources that changed since."""
    if workgroups != 0 or not os.path.exists(path):
        return None
    try:
        tf = json.load(open(path))
    except (OSError, ValueError):
        return None
    if tf.get("kernel_source_sha256") != kernel_source_sha256() or tf.get("workload") != workload:
        return None
    return tf.get("bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--warm-seconds", type=float, default=1.0,
                    help="untimed warm-up per leg after the --warmup steps, so that the timed steps "
                         "run at the clock a sustained decode loop settles at")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock budget of the oracle sample (cpu_baseline)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches only")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill measurement")
    ap.add_argument("--no-chunk", action="store_true", help="skip the chunked-prefill measurement")
    ap.add_argument("--no-hidden", action="store_true",
                    help="skip the decode-from-hidden-states measurement")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--batch", type=int, default=64,
                    help="batch of the ragged decode workload (64 is the headline configuration)")
    ap.add_argument("--workgroups", type=int, default=0,
                    help="split-KV workgroups of every decode call (0: one per compute unit, the "
                         "library's default)")
    ap.add_argument("--legs", default="tiny_decode,v2_b1_4k,v2_b4_128k",
                    help="comma-separated other decode workloads to time ('none' for none)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes (HBM counter calibration)")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="only write the traffic file from four rocprofv3 --pmc output folders "
                         "(FETCH_SIZE and WRITE_SIZE of this bench, then of --copy-bytes)")
    ap.add_argument("--traffic-command", default="", help="the profiling commands, recorded in the file")
    return ap.parse_args()


def copy_calibration(nbytes: int, reps: int = 3):
    """A plain device-to-device copy of known size, for scaling the HBM
    FETCH_SIZE / WRITE_SIZE counters of the profiled kernels."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": src.numel() * 4, "reps": reps}), flush=True)


def _pmc_rows(folder: str, counter: str):
    import csv
    path = os.path.join(folder, "run_counter_collection.csv")
    return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in csv.DictReader(open(path))
            if r["Counter_Name"] == counter]


def write_traffic(args):
    """Per-launch HBM traffic of decode_splitkv from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by what the same counter reads for a plain
    copy of known size (copy bytes / counted bytes of the largest dispatch)."""
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = args.traffic_from
    copy_bytes = 1 << 30

    def per_launch(folder, counter):
        v = [x for k, x in _pmc_rows(folder, counter) if "decode_splitkv" in k]
        return sum(v) / len(v), len(v)

    def copy_factor(folder, counter):
        counted = max(x for _, x in _pmc_rows(folder, counter)) * 1024.0
        return copy_bytes / counted

    f_kib, nf = per_launch(fetch_dir, "FETCH_SIZE")
    w_kib, nw = per_launch(write_dir, "WRITE_SIZE")
    ff, fw = copy_factor(cfetch_dir, "FETCH_SIZE"), copy_factor(cwrite_dir, "WRITE_SIZE")
    rec = {
        "kernel": "decode_splitkv", "workload": "v2_b64_ragged",
        "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib, "dispatches": [nf, nw],
        "copy_bytes": copy_bytes, "fetch_scale": ff, "write_scale": fw,
        "bytes_per_launch": f_kib * 1024.0 * ff + w_kib * 1024.0 * fw,
        "kernel_source_sha256": kernel_source_sha256(), "command": args.traffic_command,
    }
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec), flush=True)


def main():
    args = parse()
    if args.copy_bytes:
        copy_calibration(args.copy_bytes)
        return
    if args.traffic_from:
        write_traffic(args)
        return
    global WARM_S
    WARM_S = args.warm_seconds
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this build has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mla_latent_kv_34_amd as mla
    import mla_synth as syn

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    mla.load()  # fails loudly when the HIP library is not built
    dev = torch.device("cuda:0")
    d = syn.V2
    dims = mla.Dims(d.n_heads, d.d_nope, d.d_rope, d.d_latent, d.page_size, d.torch_dtype,
                    rope_base=d.rope_base)
    lens = syn.ragged_lengths(args.batch, 1024, 8192, seed=0)
    B = len(lens)
    attended = lens + 1
    tokens = int(attended.sum())

    print(f"[bench] building {args.replicas} replicas of batch {B}, {tokens} attended tokens",
          file=sys.stderr, flush=True)
    reps = []
    case0 = None
    for r in range(args.replicas):
        case = syn.decode_case(d, lens, append=True, seed=r, shuffle=True)
        if r == 0:
            case0 = case
        pool = torch.zeros((case.num_pages, d.page_size, d.row), dtype=d.torch_dtype, device=dev)
        table = torch.from_numpy(case.table).to(dev)
        zero = torch.zeros(1, dtype=torch.int32, device=dev)
        for b in range(B):  # fill the cached tokens (positions 0 .. lens[b]-1)
            c, kr = case.seq_rows(b)
            n = int(lens[b])
            mla.cache_append(dims, pool, table[b:b + 1].contiguous(), zero,
                             c[:n].unsqueeze(0).to(dev), kr[:n].unsqueeze(0).to(dev))
        new_c = torch.stack([case.seq_rows(b)[0][-1] for b in range(B)]).contiguous().to(dev)
        new_k = torch.stack([case.seq_rows(b)[1][-1] for b in range(B)]).contiguous().to(dev)
        seq_lens = torch.tensor(attended, dtype=torch.int32, device=dev)
        q_c, q_r = case.q_c.to(dev), case.q_r.to(dev)
        w_uk, w_uv = case.w_uk.to(dev), case.w_uv.to(dev)
        dec, out = mla.decode_step(dims, pool, table, seq_lens, new_c, new_k, q_c, q_r, w_uk, w_uv,
                                   n_workgroups=args.workgroups, prepare=True)
        reps.append(dict(dec=dec, out=out,
                         keep=(pool, table, seq_lens, new_c, new_k, q_c, q_r, w_uk, w_uv)))
        if r > 0:
            del case
    torch.cuda.synchronize()
    resident = sum(r["keep"][0].numel() * 2 for r in reps) / 1e9

    def step(i):
        reps[i % len(reps)]["dec"]()

    # ---- eager: whole-step time and per-launch attention-kernel time
    for i in range(args.warmup):
        step(i)
    warm_s = warm_clock(step, args.warm_seconds)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(args.steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    eager_ms = t0.elapsed_time(t1) / args.steps
    # attention kernel durations (events the library records around it), the
    # steps issued back to back as in the timed loop, one sync at the end
    kern_ms = back_to_back_kernel_ms(
        lambda i, ev: mla.decode_step(dims, *reps[i % len(reps)]["keep"][:9], out=reps[i % len(reps)]["out"],
                                      n_workgroups=args.workgroups, timing_events=ev, prepare=True)[0],
        args.steps,
        warm=lambda: warm_clock(step, args.warm_seconds))
    kern_pct = [round(float(v), 5) for v in np.percentile(kern_ms, [10, 50, 90])]
    kern_ms = float(np.mean(kern_ms))

    # ---- graph replay of the same steps
    graph_ms = None
    if not args.no_graph:
        graphs = []
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(len(reps)):  # warm the capture stream
                step(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        # one graph per step (for a step count that is not a multiple of the
        # replica count) and one graph holding a step on every replica in
        # turn, as a serving loop captures consecutive layers
        for i in range(len(reps)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i)
            graphs.append(g)
        R = len(reps)
        g_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_all):
            for i in range(R):
                step(i)

        def replay_steps(n):  # exactly n steps, replicas in turn from 0
            for _ in range(n // R):
                g_all.replay()
            for i in range(n % R):
                graphs[i].replay()

        replay_steps(args.warmup)
        warm_clock(lambda i: g_all.replay(), args.warm_seconds)  # capture left the GPU idle
        t0.record()
        replay_steps(args.steps)
        t1.record()
        torch.cuda.synchronize()
        graph_ms = t0.elapsed_time(t1) / args.steps

    ms = graph_ms if graph_ms is not None else eager_ms
    value = tokens / (ms * 1e-3)
    cache_bytes = tokens * BYTES_PER_TOKEN
    achieved = cache_bytes / (kern_ms * 1e-3) / 1e9
    kern_tflops = tokens * FLOP_PER_TOKEN / (kern_ms * 1e-3) / 1e12

    traffic = recorded_traffic(f"v2_b{B}_ragged", args.workgroups)

    pre = None
    if not args.no_prefill:
        pre = prefill_bench(mla, syn, dims, dev, args.prefill_steps)

    chk = None
    if not args.no_chunk:
        chk = chunk_bench(mla, syn, dims, dev, args.prefill_steps)

    hid = None
    n_reps = len(reps)
    if not args.no_hidden:
        hid = hidden_bench(mla, syn, dims, dev, lens, args.steps, args.warmup, args.replicas)

    legs = None
    names = [] if args.legs == "none" else [x for x in args.legs.split(",") if x]
    if names:
        legs = {name: decode_leg(mla, syn, dev, name, args.steps, args.warmup, not args.no_cpu,
                                 args.warm_seconds, args.workgroups) for name in names}

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(case0, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "cached tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"v2_b{B}_ragged: DeepSeek-V2 MLA layer (128 heads, d_h^C 128, d_h^R 64, d_c 512), "
                        f"batch {B}, cached 1024-8192 tokens (uniform), shuffled 64-token pages, "
                        "append 1 token + absorbed decode",
            "batch": B,
            "attended_tokens": tokens,
            "replicas": n_reps,
            "split_kv_workgroups": args.workgroups or "one per compute unit",
            "resident_cache_GB": round(resident, 3),
            "timing": "hip graph replay, one graph per %d consecutive steps" % n_reps if graph_ms is not None else "eager launches",
            "warmup": f"{args.warmup} steps, then {warm_s:.2f} s of untimed steps (sustained-load clock)",
        },
        "latent_cache_GBps": round(cache_bytes / (ms * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(cache_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "eager_ms_per_step": round(eager_ms, 5),
        "roofline": {
            "kernel": "decode_splitkv",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel_ms": round(kern_ms, 5),
            "kernel_ms_p10_p50_p90": kern_pct,
            "kernel_timing": "hip events (device-scope release) the library records around the kernel, steps issued back to back",
            "algorithmic_bytes": cache_bytes,
            "mfma": {"achieved": round(kern_tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(kern_tflops / MFMA_BF16_PEAK_TFLOPS, 4)},
        },
        "cpu_baseline": cpu,
        "decode_legs": legs,
        "prefill": pre,
        "prefill_chunk": chk,
        "decode_hidden": hid,
    }
    print(json.dumps(line), flush=True)


def warm_clock(step, seconds: float) -> float:
    """Untimed steps until `seconds` of wall time have passed (the GPU raises
    its clock over the first few hundred ms of sustained work; a short burst
    of steps would be timed at a lower clock than a serving loop runs at).
    Returns the seconds spent."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(32):
            step(i)
            i += 1
        torch.cuda.synchronize()
    return time.perf_counter() - t0


class DeviceEvent:
    """A HIP event created with hipEventReleaseToDevice: recording it makes a
    device-scope release instead of the default system-scope one, so its
    timestamp is not held back by writing the caches out for the host (the
    flag the HIP runtime provides for precise timing between events).  It
    has the .cuda_event handle the binding passes to the library, which
    records it on the launch stream."""
    _hip = None
    FLAGS = 0x40000000  # hipEventReleaseToDevice

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            import ctypes
            # the HIP runtime torch and the library use (one SONAME, loaded once)
            with open("/proc/self/maps") as fh:
                paths = sorted({ln.split()[-1] for ln in fh if "libamdhip64" in ln})
            if not paths:
                raise RuntimeError("the HIP runtime is not loaded")
            if len(paths) > 1:
                print(f"[bench] several HIP runtimes mapped: {paths}", file=sys.stderr, flush=True)
            cls._hip = ctypes.CDLL(paths[0])
        return cls._hip

    def __init__(self):
        import ctypes
        hip = self._runtime()
        h = ctypes.c_void_p()
        rc = hip.hipEventCreateWithFlags(ctypes.byref(h), ctypes.c_uint(self.FLAGS))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.cuda_event = h.value

    def elapsed_time(self, end) -> float:
        import ctypes
        ms = ctypes.c_float()
        rc = self._runtime().hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.cuda_event),
                                                 ctypes.c_void_p(end.cuda_event))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if self._hip is not None and getattr(self, "cuda_event", None):
            import ctypes
            self._hip.hipEventDestroy(ctypes.c_void_p(self.cuda_event))


def back_to_back_kernel_ms(make_call, n: int, warm=None):
    """Durations (ms) of the kernel that the library brackets with its two
    timing events, over n calls issued back to back on the current stream
    with a single synchronisation at the end (the regime of a decode loop).
    make_call(i, events) returns a prepared call that records into events.
    The calls are prepared first (host work that leaves the GPU idle, so its
    clock drops); warm(), when given, then brings the clock back to its
    sustained level right before the timed calls are issued."""
    import torch
    pairs = [(DeviceEvent(), DeviceEvent()) for _ in range(n)]
    calls = [make_call(i, pairs[i]) for i in range(n)]
    torch.cuda.synchronize()
    if warm is not None:
        warm()
    for c in calls:
        c()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in pairs]


def graph_replay_ms(calls, steps: int, warmup: int):
    """Mean ms per call when the calls (one per replica, in turn) are replayed
    from HIP graphs: one graph holding a call on every replica, plus one graph
    per replica for a step count that is not a multiple of the replica count."""
    import torch
    R = len(calls)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        for c in calls:
            c()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    g_all = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_all):
        for c in calls:
            c()
    singles = []
    for c in calls:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            c()
        singles.append(g)

    def replay(n):
        for _ in range(n // R):
            g_all.replay()
        for i in range(n % R):
            singles[i].replay()

    replay(warmup)
    warm_clock(lambda i: g_all.replay(), WARM_S)  # capture left the GPU idle
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    replay(steps)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


LEG_TEXT = {
    "tiny_decode": "tiny fp32 layer (n_h 4, d_h^C 16, d_h^R 8, d_c 32), batch 1, 64 cached tokens + 1 "
                   "appended, positions 0..64 (generic kernel family; latency only)",
    "v2_b1_4k": "DeepSeek-V2 layer, batch 1, 4096 cached tokens in contiguous 64-token pages, the query "
                "is the token at position 4095 (launch-bound latency)",
    "v2_b4_128k": "DeepSeek-V2 layer, batch 4 x 131072 cached tokens (151 MB of latent cache per "
                  "sequence), shuffled 64-token pages, split-KV over all compute units + combine",
}
LEG_REPLICAS = {"tiny_decode": 1, "v2_b1_4k": 8, "v2_b4_128k": 2}
LEG_ORACLE_HEADS = {"tiny_decode": None, "v2_b1_4k": None, "v2_b4_128k": 16}


def decode_leg(mla, syn, dev, name: str, steps: int, warmup: int, with_cpu: bool, warm_s: float,
               n_wg: int = 0):
    """One of the other decode workloads: step time by graph replay over
    cache/weight replicas (enough to exceed the 256 MB last-level cache where
    the working set is small), the split-KV kernel by back-to-back events, and
    the oracle timed on a sample of the same inputs."""
    import numpy as np
    import torch

    R = LEG_REPLICAS[name]
    print(f"[bench] decode leg {name}: {R} replicas", file=sys.stderr, flush=True)
    reps = []
    case0 = None
    for r in range(R):
        case = syn.config_case(name, seed=r)
        d = case.dims
        dims = mla.Dims(d.n_heads, d.d_nope, d.d_rope, d.d_latent, d.page_size, d.torch_dtype,
                        rope_base=d.rope_base)
        pool = torch.zeros((case.num_pages, d.page_size, d.row), dtype=d.torch_dtype, device=dev)
        table = torch.from_numpy(case.table).to(dev)
        zero = torch.zeros(1, dtype=torch.int32, device=dev)
        for b in range(case.batch):
            c, kr = case.seq_rows(b)
            n = int(case.cached[b])
            mla.cache_append(dims, pool, table[b:b + 1].contiguous(), zero,
                             c[:n].unsqueeze(0).to(dev), kr[:n].unsqueeze(0).to(dev))
        seq_lens = torch.tensor(case.attended, dtype=torch.int32, device=dev)
        q_c, q_r = case.q_c.to(dev), case.q_r.to(dev)
        w_uk, w_uv = case.w_uk.to(dev), case.w_uv.to(dev)
        if case.append:
            new_c = torch.stack([case.seq_rows(b)[0][-1] for b in range(case.batch)]).contiguous().to(dev)
            new_k = torch.stack([case.seq_rows(b)[1][-1] for b in range(case.batch)]).contiguous().to(dev)
            keep = (pool, table, seq_lens, new_c, new_k, q_c, q_r, w_uk, w_uv)
            fn = mla.decode_step
        else:
            keep = (pool, table, seq_lens, q_c, q_r, w_uk, w_uv)
            fn = mla.decode
        call, out = fn(dims, *keep, n_workgroups=n_wg, prepare=True)
        reps.append(dict(call=call, out=out, keep=keep, fn=fn, dims=dims))
        if r == 0:
            case0 = case
        else:
            del case
    torch.cuda.synchronize()
    tokens = int(case0.attended.sum())
    for i in range(warmup):
        reps[i % R]["call"]()
    warm_clock(lambda i: reps[i % R]["call"](), warm_s)
    ms = graph_replay_ms([r["call"] for r in reps], steps, warmup)
    kern = back_to_back_kernel_ms(
        lambda i, ev: reps[i % R]["fn"](reps[i % R]["dims"], *reps[i % R]["keep"], out=reps[i % R]["out"],
                                        n_workgroups=n_wg, timing_events=ev, prepare=True)[0], steps,
        warm=lambda: warm_clock(lambda i: reps[i % R]["call"](), warm_s))
    kern_pct = [round(float(v), 5) for v in np.percentile(kern, [10, 50, 90])]
    kern_ms = float(np.mean(kern))
    row_bytes = case0.dims.row * (2 if case0.dims.dtype == "bf16" else 4)
    cache_bytes = tokens * row_bytes
    flop = tokens * 2 * case0.dims.n_heads * (case0.dims.row + case0.dims.d_latent)
    achieved = cache_bytes / (kern_ms * 1e-3) / 1e9
    res = {
        "workload": f"{name}: {LEG_TEXT[name]}",
        "batch": int(case0.batch), "attended_tokens": tokens, "replicas": R,
        "split_kv_workgroups": n_wg or "one per compute unit",
        "us_per_step": round(ms * 1e3, 2),
        "value": round(tokens / (ms * 1e-3), 1), "unit": "cached tokens/s",
        "latent_cache_GBps": round(cache_bytes / (ms * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(cache_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "timing": f"hip graph replay over {R} replica(s)",
        "roofline": {
            "kernel": "decode_splitkv" if case0.dims.dtype == "bf16" else "generic decode",
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "kernel_ms": round(kern_ms, 5),
            "kernel_ms_p10_p50_p90": kern_pct, "algorithmic_bytes": cache_bytes,
            "kernel_timing": "hip events (device-scope release) the library records around the kernel, calls issued back to back",
            "mfma": {"achieved": round(flop / (kern_ms * 1e-3) / 1e12, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(flop / (kern_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
        },
    }
    del reps
    torch.cuda.synchronize()
    if with_cpu:
        res["cpu_oracle"] = leg_oracle(case0, LEG_ORACLE_HEADS[name])
    return res


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return len(os.sched_getaffinity(0))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def leg_oracle(case, heads):
    """The fp64 oracle on the leg's workload: every sequence, or the first
    `heads` heads of sequence 0 for the long-context leg; three runs on the
    host's BLAS threads and, for the small workloads, three on one thread."""
    import numpy as np
    from oracle import decode_ref

    f64 = lambda t: t.double().numpy()  # noqa: E731
    wk, wv = f64(case.w_uk), f64(case.w_uv)
    n_h = case.dims.n_heads
    sel = None if heads is None else list(range(heads))
    seqs = range(case.batch) if heads is None else [0]
    tokens = sum(int(case.attended[b]) for b in seqs)
    frac = 1.0 if heads is None else heads / n_h

    def one():
        t = time.perf_counter()
        for b in seqs:
            c, kr = case.seq_rows(b)
            decode_ref(f64(case.q_c[b]), f64(case.q_r[b]), f64(c), f64(kr), wk, wv,
                       base=case.dims.rope_base, heads=sel)
        return time.perf_counter() - t

    runs = [one() for _ in range(3 if heads is None else 1)]
    out = {"kind": "oracle", "unit": "cached tokens/s", "cores": _blas_threads(), "cpu_model": cpu_model(),
           "value": round(tokens * frac / min(runs), 1), "runs_s": [round(x, 3) for x in runs],
           "sample": ("the whole workload" if heads is None else
                      f"heads 0..{heads - 1} of sequence 0 ({tokens} attended tokens), tokens/s scaled "
                      f"by {heads}/{n_h}") + ", fp64 numpy"}
    if heads is None:
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(1):
                runs1 = [one() for _ in range(3)]
            out["one_thread"] = {"value": round(tokens / min(runs1), 1), "cores": 1,
                                 "runs_s": [round(x, 3) for x in runs1]}
        except ImportError:
            pass
    return out


def hidden_bench(mla, syn, dims, dev, lens, steps: int, warmup: int, replicas: int):
    """The same batch-64 decode step started from hidden states
    (mla_decode_hidden): the projections h -> [c^KV | k^R | c^Q] and
    c^Q -> [q^C | q^R] in front of the step.  Step time by graph replay over
    replicas (each with its own cache and weights); the projection kernels
    timed with the library's events, against HBM (their weights and
    activations are read or written once)."""
    import numpy as np
    import torch

    d = syn.V2
    B = len(lens)
    tokens = int((lens + 1).sum())
    print(f"[bench] decode from hidden states: {replicas} replicas", file=sys.stderr, flush=True)
    reps = []
    zero = torch.zeros(1, dtype=torch.int32, device=dev)
    for r in range(replicas):
        hc = syn.hidden_case(d, lens, seed=100 + r, shuffle=True)
        base = hc.base
        pool = torch.zeros((base.num_pages, d.page_size, d.row), dtype=d.torch_dtype, device=dev)
        table = torch.from_numpy(base.table).to(dev)
        for b in range(B):
            c, kr = base.seq_rows(b)
            n = int(lens[b])
            mla.cache_append(dims, pool, table[b:b + 1].contiguous(), zero,
                             c[:n].unsqueeze(0).to(dev), kr[:n].unsqueeze(0).to(dev))
        seq_lens = torch.tensor(base.attended, dtype=torch.int32, device=dev)
        args = [hc.h.to(dev)] + [w.to(dev) for w in hc.front] + [base.w_uk.to(dev), base.w_uv.to(dev)]
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        for e in ev:
            e.record()
        call, out = mla.decode_hidden(dims, pool, table, seq_lens, *args, prepare=True)
        call_t, _ = mla.decode_hidden(dims, pool, table, seq_lens, *args, out=out, timing_events=ev,
                                      prepare=True)
        w_o = syn.out_weight(d, 100 + r).to(dev)
        ev_l = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        for e in ev_l:
            e.record()
        ws = torch.empty(mla.decode_hidden_workspace_size(dims, B, d.d_model, d.d_cq), dtype=torch.uint8,
                         device=dev)
        call_l, u = mla.decode_layer(dims, pool, table, seq_lens, *args, w_o, workspace=ws, prepare=True)
        call_lt, _ = mla.decode_layer(dims, pool, table, seq_lens, *args, w_o, u=u, workspace=ws,
                                      timing_events=ev_l, prepare=True)
        w_uqk = mla.merge_query_weights(dims, args[4], args[6])

        def layer_merged(w_o, ws):
            w_ov = mla.merge_output_weights(dims, w_o, args[7])
            ev_v = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for e in ev_v:
                e.record()
            largs = args[:7] + [w_ov]                             # ..., W^UQ, W^QR, W^UK, W^OV
            c_v, u_v = mla.decode_layer_merged(dims, pool, table, seq_lens, *largs, workspace=ws, prepare=True)
            c_vt, _ = mla.decode_layer_merged(dims, pool, table, seq_lens, *largs, u=u_v, workspace=ws,
                                              timing_events=ev_v, prepare=True)
            return dict(call_v=c_v, call_vt=c_vt, ev_v=ev_v, keep_v=(w_ov, u_v))
        margs = args[:4] + [w_uqk, args[5], args[7]]             # h, W^DKV, W^KR, W^DQ, W^UQK, W^QR, W^UV
        ev_m = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        for e in ev_m:
            e.record()
        call_m, out_m = mla.decode_hidden_merged(dims, pool, table, seq_lens, *margs, workspace=ws,
                                                 prepare=True)
        call_mt, _ = mla.decode_hidden_merged(dims, pool, table, seq_lens, *margs, out=out_m, workspace=ws,
                                              timing_events=ev_m, prepare=True)
        reps.append(dict(call=call, call_t=call_t, ev=ev, call_l=call_l, call_lt=call_lt, ev_l=ev_l,
                         call_m=call_m, call_mt=call_mt, ev_m=ev_m, **layer_merged(w_o, ws),
                         keep=(pool, table, seq_lens, args, out, w_o, ws, u, w_uqk, out_m)))
        del hc, base
    torch.cuda.synchronize()
    R = len(reps)

    def measure(kc, kt, ke):
        """(mean event-bracketed ms, step ms by graph replay) of one call kind."""
        for i in range(warmup):
            reps[i % R][kc]()
        warm_clock(lambda i: reps[i % R][kc](), WARM_S / 2)
        evms = []
        for i in range(steps):
            r = reps[i % R]
            r[kt]()
            torch.cuda.synchronize()
            evms.append(r[ke][0].elapsed_time(r[ke][1]))
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            for r in reps:
                r[kc]()
        torch.cuda.current_stream().wait_stream(st)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in reps:
                r[kc]()
        singles = []
        for r in reps:
            gi = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gi):
                r[kc]()
            singles.append(gi)

        def replay(n):
            for _ in range(n // R):
                g.replay()
            for i in range(n % R):
                singles[i].replay()

        replay(warmup)
        warm_clock(lambda i: g.replay(), WARM_S / 2)  # capture left the GPU idle
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        replay(steps)
        t1.record()
        torch.cuda.synchronize()
        return float(np.mean(evms)), t0.elapsed_time(t1) / steps

    proj_ms, ms = measure("call", "call_t", "ev")
    wo_ms, layer_ms = measure("call_l", "call_lt", "ev_l")
    pm_ms, merged_ms = measure("call_m", "call_mt", "ev_m")
    wov_ms, layer_v_ms = measure("call_v", "call_vt", "ev_v")
    wov_bytes = 2 * (d.d_model * d.n_heads * d.d_latent + B * (d.n_heads * d.d_latent + d.d_model))
    wo_bytes = 2 * (d.d_model * d.n_heads * d.d_nope + B * (d.n_heads * d.d_nope + d.d_model))
    wo_gbps = wo_bytes / (wo_ms * 1e-3) / 1e9
    dm, dq = d.d_model, d.d_cq
    n1 = d.d_latent + d.d_rope + dq
    n2 = d.n_heads * (d.d_nope + d.d_rope)
    wbytes = 2 * (n1 * dm + n2 * dq)
    abytes = 2 * B * (dm + n1 + dq + n2)        # h in, stage-1 out, c^Q in, stage-2 out
    gbps = (wbytes + abytes) / (proj_ms * 1e-3) / 1e9
    n2m = d.n_heads * (d.d_latent + d.d_rope)
    mbytes = 2 * (n1 * dm + n2m * dq) + 2 * B * (dm + n1 + dq + n2m)
    return {"workload": "v2_b64_ragged from hidden states: h [64, 5120] -> c^KV, k^R, c^Q "
                        "(W^DKV, W^KR, W^DQ) -> q^C, q^R (W^UQ, W^QR), then the decode step",
            "value": round(tokens / (ms * 1e-3), 1), "unit": "cached tokens/s",
            "ms_per_step": round(ms, 5), "projections_ms": round(proj_ms, 5),
            "timing": "hip graph replay over %d replicas; projections by events, one step at a time" % R,
            "roofline": {"kernel": "proj_gemm (+ split-K reduce)", "bound": "hbm",
                         "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(gbps / HBM_PEAK_GBPS, 4), "algorithmic_bytes": wbytes + abytes},
            "merged": {"workload": "the same step with the pre-merged query weight W^UK_i^T W^UQ_i "
                                   "(mla_decode_hidden_merged): c^Q -> [q_lat | q^R] in place of c^Q -> q^C",
                       "value": round(tokens / (merged_ms * 1e-3), 1), "unit": "cached tokens/s",
                       "ms_per_step": round(merged_ms, 5), "projections_ms": round(pm_ms, 5),
                       "projection_bytes": mbytes,
                       "projections_GBps": round(mbytes / (pm_ms * 1e-3) / 1e9, 1)},
            "layer": {"workload": "the same step through W^O: u [64, 5120] = W^O [o_1..o_128] "
                                  "(mla_decode_layer)",
                      "value": round(tokens / (layer_ms * 1e-3), 1), "unit": "cached tokens/s",
                      "ms_per_step": round(layer_ms, 5), "w_o_ms": round(wo_ms, 5),
                      "roofline": {"kernel": "proj_gemm W^O (+ split-K reduce)", "bound": "hbm",
                                   "achieved": round(wo_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                   "frac": round(wo_gbps / HBM_PEAK_GBPS, 4),
                                   "algorithmic_bytes": wo_bytes}},
            "layer_merged": {"workload": "the layer with W^UV merged into W^O per head (mla_decode_layer_merged): "
                                         "u = W^OV [o_lat_1..o_lat_128]",
                             "value": round(tokens / (layer_v_ms * 1e-3), 1), "unit": "cached tokens/s",
                             "ms_per_step": round(layer_v_ms, 5), "w_ov_ms": round(wov_ms, 5),
                             "w_ov_bytes": wov_bytes,
                             "w_ov_GBps": round(wov_bytes / (wov_ms * 1e-3) / 1e9, 1)}}


def prefill_bench(mla, syn, dims, dev, steps: int):
    """Un-absorbed causal prefill of two 4096-token prompts (bulk append, K/V
    expansion, causal attention): prompt tokens/s and the MFMA fraction of the
    expansion + attention kernels (timed with the library's events)."""
    import numpy as np
    import torch

    print("[bench] prefill 2 x 4096", file=sys.stderr, flush=True)
    case = syn.config_case("v2_prefill_2x4k")
    B, T, H = case.batch, case.seq_len, case.dims.n_heads
    d = case.dims
    pool = torch.zeros((case.num_pages, d.page_size, d.row), dtype=d.torch_dtype, device=dev)
    table = torch.from_numpy(case.table).to(dev)
    args = [case.q_c.to(dev), case.q_r.to(dev), case.c_kv.to(dev), case.k_r.to(dev),
            case.w_uk.to(dev), case.w_uv.to(dev)]
    del case
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for e in ev:
        e.record()
    call, out = mla.prefill(dims, pool, table, *args, prepare=True)
    call_t, _ = mla.prefill(dims, pool, table, *args, out=out, timing_events=ev, prepare=True)
    for _ in range(3):
        call()
    warm_clock(lambda i: call(), WARM_S)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        call()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    kern = []
    for _ in range(steps):
        call_t()
        torch.cuda.synchronize()
        kern.append(ev[0].elapsed_time(ev[1]))
    kern_ms = float(np.mean(kern))
    pairs = B * H * T * (T + 1) // 2                       # causal (query, key) pairs
    flop = pairs * 2 * (d.d_nope + d.d_rope + d.d_nope)    # scores + weighted sum
    flop += 2 * B * T * d.d_latent * 2 * H * d.d_nope      # K^C and V^C expansion
    tflops = flop / (kern_ms * 1e-3) / 1e12
    return {"workload": "v2_prefill_2x4k: 2 prompts x 4096 tokens, causal, cache written",
            "value": round(B * T / (ms * 1e-3), 1), "unit": "prompt tokens/s",
            "ms_per_call": round(ms, 4), "kernels_ms": round(kern_ms, 4),
            "roofline": {"kernel": "expand + prefill_attn", "bound": "mfma",
                         "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "algorithmic_flop": flop}}


def chunk_bench(mla, syn, dims, dev, steps: int):
    """Chunked prefill: the last 512-token chunk of two 4096-token prompts,
    3584 positions already cached (append the chunk, expand K/V for all 4096
    positions, causal attention of the chunk's rows): chunk tokens/s and the
    MFMA fraction of the expansion + attention kernels."""
    import numpy as np
    import torch

    print("[bench] chunked prefill 2 x (3584 + 512)", file=sys.stderr, flush=True)
    P, T = 3584, 512
    case = syn.chunk_case(syn.V2, [P, P], T, seed=0)
    B, H, d = case.batch, case.dims.n_heads, case.dims
    ctx = P + T
    pool = torch.zeros((case.num_pages, d.page_size, d.row), dtype=d.torch_dtype, device=dev)
    table = torch.from_numpy(case.table).to(dev)
    mla.cache_append(dims, pool, table, torch.zeros(B, dtype=torch.int32, device=dev),
                     case.c_all[:, :P].contiguous().to(dev), case.k_all[:, :P].contiguous().to(dev))
    c_new, k_new = case.chunk_rows()
    start = torch.from_numpy(case.start.astype(np.int32)).to(dev)
    args = [case.q_c.to(dev), case.q_r.to(dev), c_new.contiguous().to(dev), k_new.contiguous().to(dev),
            case.w_uk.to(dev), case.w_uv.to(dev)]
    del case
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for e in ev:
        e.record()
    call, out = mla.prefill_chunk(dims, pool, table, start, *args, max_context=ctx, prepare=True)
    call_t, _ = mla.prefill_chunk(dims, pool, table, start, *args, max_context=ctx, out=out,
                                  timing_events=ev, prepare=True)
    for _ in range(3):
        call()
    warm_clock(lambda i: call(), WARM_S)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        call()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    kern = []
    for _ in range(steps):
        call_t()
        torch.cuda.synchronize()
        kern.append(ev[0].elapsed_time(ev[1]))
    kern_ms = float(np.mean(kern))
    pairs = B * H * (T * P + T * (T + 1) // 2)            # causal (query, key) pairs
    flop = pairs * 2 * (d.d_nope + d.d_rope + d.d_nope)    # scores + weighted sum
    flop += 2 * B * ctx * d.d_latent * 2 * H * d.d_nope    # K^C and V^C of every position
    tflops = flop / (kern_ms * 1e-3) / 1e12
    short = short_chunk_bench(mla, syn, dims, dev, steps)
    return {"workload": "v2_chunk_2x(3584+512): 2 sequences, 3584 cached + 512-token chunk, causal, "
                        "chunk rows written",
            "short_chunk": short,
            "value": round(B * T / (ms * 1e-3), 1), "unit": "chunk tokens/s",
            "ms_per_call": round(ms, 4), "kernels_ms": round(kern_ms, 4),
            "roofline": {"kernel": "expand + prefill_attn", "bound": "mfma",
                         "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "algorithmic_flop": flop}}


def short_chunk_bench(mla, syn, dims, dev, steps: int):
    """A 128-token chunk after 3968 cached positions (2 sequences), timed in
    both forms, expanded (every position's K/V) and absorbed (each chunk row a
    decode query), and with the library's automatic choice."""
    import numpy as np
    import torch

    P, T = 3968, 128
    case = syn.chunk_case(syn.V2, [P, P], T, seed=3)
    B, d = case.batch, case.dims
    pool = torch.zeros((case.num_pages, d.page_size, d.row), dtype=d.torch_dtype, device=dev)
    table = torch.from_numpy(case.table).to(dev)
    mla.cache_append(dims, pool, table, torch.zeros(B, dtype=torch.int32, device=dev),
                     case.c_all[:, :P].contiguous().to(dev), case.k_all[:, :P].contiguous().to(dev))
    c_new, k_new = case.chunk_rows()
    start = torch.from_numpy(case.start.astype(np.int32)).to(dev)
    args = [case.q_c.to(dev), case.q_r.to(dev), c_new.contiguous().to(dev), k_new.contiguous().to(dev),
            case.w_uk.to(dev), case.w_uv.to(dev)]
    res = {}
    for name, mode in (("expanded", mla.CHUNK_EXPAND), ("absorbed", mla.CHUNK_ABSORB),
                       ("auto", mla.CHUNK_AUTO)):
        call, _ = mla.prefill_chunk(dims, pool, table, start, *args, max_context=P + T, mode=mode,
                                    prepare=True)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            call()
        t1.record()
        torch.cuda.synchronize()
        res[name + "_ms"] = round(t0.elapsed_time(t1) / steps, 4)
    return {"workload": "v2_chunk_2x(3968+128): 2 sequences, 3968 cached + 128-token chunk",
            **res, "value": round(B * T / (res["auto_ms"] * 1e-3), 1),
            "unit": "chunk tokens/s (automatic choice)"}


def cpu_baseline(case, budget_s: float):
    """The fp64 oracle on whole sequences of replica 0 until the budget is spent."""
    import numpy as np
    from oracle import decode_ref

    threads = _blas_threads()
    f64 = lambda t: t.double().numpy()  # noqa: E731
    wk, wv = f64(case.w_uk), f64(case.w_uv)
    done_tok = 0
    seqs = 0
    t_start = time.perf_counter()
    for b in range(case.batch):
        c, kr = case.seq_rows(b)
        decode_ref(f64(case.q_c[b]), f64(case.q_r[b]), f64(c), f64(kr), wk, wv, base=case.dims.rope_base)
        done_tok += int(case.attended[b])
        seqs += 1
        if time.perf_counter() - t_start >= budget_s:
            break
    el = time.perf_counter() - t_start
    return {"value": round(done_tok / el, 1), "unit": "cached tokens/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{seqs} of {case.batch} sequences (all 128 heads, {done_tok} attended tokens) of the "
                      f"same workload, fp64 numpy, {el:.1f} s"}


if __name__ == "__main__":
    main()
