#!/usr/bin/env python3
"""Decode-step benchmark: paged FP8-E5M2 grouped-query decode attention.

Default workload: the ragged long batch (B=16, Hkv=4, Hq=32, head_dim 128,
page size 16, context lengths uniform in [2048, 33600], randomly permuted
pages in a 256K-token-per-sequence pool). A step is one xqa_decode call
(split kernel + combine kernel) over the whole batch, replayed from a HIP
graph; R input variants (different lengths, page tables, q and K/V bytes),
each with its own captured graph, are cycled so inputs change between
replays and the rotating footprint exceeds the on-package caches.

Order: generate -> upload -> CPU baseline leg (the float64 oracle timed on
the host cores; its output is also the correctness gate for variant 0) ->
graph gate (every variant's replay bitwise equal to its eager call) ->
independent warm-up of each arm -> timed replays of one graph holding R
consecutive steps (the headline; one-step-per-graph replays are reported too) ->
A/B/B/A eager vs graph blocks -> per-launch HIP-event timing of the split
kernel (the dominant one) and of the combine kernel on the stream they are
launched on -> single steps timed cold (caches flushed by reading 1 GiB
before each) and warm (the same input repeated) -> two query tokens per sequence (xqa_decode_multi), the same
workload as an E4M3 cache with per-tensor scales (xqa_decode_fp8), decode
over a quarter of each sequence's pages (xqa_decode_pages), and the KV
append (xqa_append_kv) per launch and in a graph of append + decode steps,
reported in detail. Prints one JSON line.
"""

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "us per decode step + achieved KV-read HBM GB/s (% of peak), B16 ragged ~17.8K"
HBM_PEAK_GBS = 8000.0

# HBM bytes per split-kernel launch on the ragged B16 workload, from
# rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE passes (KiB per dispatch, mean over
# the variants), scaled by what the same counters read for a plain 1 GiB copy
# (FETCH_SIZE x2.00, WRITE_SIZE x1.00). Valid only for the kernel sources
# whose hash is recorded; any change to them reports null until re-measured.
MEASURED_TRAFFIC = {
    "sources_sha256": "368f9555472a8e74562eee0e05082e8311a629f8d67d004b0804fb9ade9e6833",
    "fetch_kib": 133397.2, "fetch_scale": 2.0,
    "write_kib": 2328.0, "write_scale": 1.0,
}


def kernel_sources_sha256():
    """sha256 of the kernel sources' code: comments and blank lines removed,
    so that only a change to the code itself invalidates measured counters."""
    import hashlib
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "decode_attention_paged_e5m2_amd", "csrc")
    for f in ("xqa_kernels.hip", "xqa_internal.h"):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
        h.update("\n".join(ln for ln in lines if ln.strip()).encode())
    return h.hexdigest()


def measured_traffic_bytes(config):
    t = MEASURED_TRAFFIC
    if config != 4 or kernel_sources_sha256() != t["sources_sha256"]:
        return None
    return (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]) * 1024.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", type=int, default=4, help="workload 1..5 (4 = headline)")
    ap.add_argument("--variants", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=0, help="oracle repetitions (0 = auto, ~10-20 s)")
    ap.add_argument("--quick", action="store_true", help="skip A/B/B/A and warm-mode extras")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the floor, multi-token, E4M3 and KV-append legs and the clock "
                         "readings (profiling runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (5x), the reference "
                         "for scaling FETCH_SIZE / WRITE_SIZE counter readings")
    ap.add_argument("--calibrate-read", action="store_true",
                    help="run only a read of a 1 GiB buffer reduced to one value (5x): a second, "
                         "read-only reference for FETCH_SIZE")
    ap.add_argument("--abba-rounds", type=int, default=5, help="A/B/B/A rounds per arm pair")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class ClockSampler:
    """Samples GPU clocks and power in a background thread while timed work runs.

    Reads the amdgpu kernel driver's sysfs files (current shader / memory clock level and
    average power) every 20 ms; where they are not readable, rocm-smi (a
    child process) every 0.5 s. start()/stop() bracket the timed phases.
    """

    def __init__(self):
        import glob
        import threading
        self.samples = []
        self._stop = threading.Event()
        self._thread = None
        dev = None
        for d in sorted(glob.glob("/sys/class/drm/card*/device")):
            if os.path.exists(os.path.join(d, "pp_dpm_sclk")):
                dev = d
                break
        self.dev = dev
        self.hwmon = None
        if dev:
            hw = sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*")))
            for h in hw:
                for f in ("power1_average", "power1_input"):
                    if os.path.exists(os.path.join(h, f)):
                        self.hwmon = os.path.join(h, f)
                        break
        self.source = "sysfs" if dev else "rocm-smi"

    @staticmethod
    def _level(path):
        with open(path) as f:
            for line in f:
                if "*" in line:
                    return float(line.split(":", 1)[1].strip().rstrip("*").strip().lower()
                                 .replace("mhz", ""))
        return None

    def _read(self):
        if self.dev:
            rec = {"sclk_mhz": self._level(os.path.join(self.dev, "pp_dpm_sclk")),
                   "mclk_mhz": self._level(os.path.join(self.dev, "pp_dpm_mclk"))}
            if self.hwmon:
                with open(self.hwmon) as f:
                    rec["power_w"] = int(f.read().strip()) / 1e6
            return rec
        c = gpu_clocks() or {}
        rec = {}
        for k, v in c.items():
            digits = "".join(ch for ch in str(v) if ch.isdigit() or ch == ".")
            if "sclk" in k and "speed" in k and digits:
                rec["sclk_mhz"] = float(digits)
            elif "mclk" in k and "speed" in k and digits:
                rec["mclk_mhz"] = float(digits)
            elif "power" in k.lower() and digits:
                rec["power_w"] = float(digits)
        return rec

    def _run(self):
        period = 0.02 if self.dev else 0.5
        while not self._stop.is_set():
            try:
                self.samples.append(self._read())
            except Exception:
                pass
            self._stop.wait(period)

    def start(self):
        import threading
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()

    def stop(self):
        self._stop.set()
        if self._thread:
            self._thread.join(timeout=5)
        out = {"source": self.source, "samples": len(self.samples)}
        for key in ("sclk_mhz", "mclk_mhz", "power_w"):
            vals = [s[key] for s in self.samples if s.get(key) is not None]
            if vals:
                out[key] = {"min": min(vals), "median": statistics.median(vals), "max": max(vals)}
        return out


def under_profiler():
    """True when a profiler's library is preloaded into this process."""
    pre = os.environ.get("LD_PRELOAD", "") + os.environ.get("HSA_TOOLS_LIB", "")
    return "rocprof" in pre or any(k.startswith("ROCPROF") for k in os.environ)


def provenance(args, run_git=True):
    """Where the numbers come from: sources, build, toolchain, device, inputs.
    run_git: ask git for the commit (a child process); otherwise the build's
    record of it is used."""
    import hashlib
    import platform
    import subprocess
    import torch
    from decode_attention_paged_e5m2_amd import build as _build

    def sha(paths):
        h = hashlib.sha256()
        for pth in paths:
            with open(pth, "rb") as f:
                h.update(f.read())
        return h.hexdigest()

    pkg = os.path.join(ROOT, "decode_attention_paged_e5m2_amd")
    csrc = os.path.join(pkg, "csrc")
    srcs = sorted(os.path.join(csrc, f) for f in os.listdir(csrc))
    git = None
    if run_git:
        try:
            r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True,
                               text=True, timeout=10)
            if r.returncode == 0:
                git = r.stdout.strip()
        except Exception:
            pass
    info = {}
    bi = os.path.join(pkg, "_build_info.json")
    if os.path.exists(bi):
        with open(bi) as f:
            info = json.load(f)
    rocm = None
    for cand in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        if os.path.exists(cand):
            with open(cand) as f:
                rocm = f.read().strip()
            break
    props = torch.cuda.get_device_properties(0)
    lib = os.path.join(pkg, "libxqa.so")
    return {
        "git_sha": git or info.get("git_sha"),
        "git_sha_source": "git" if git else ("build info" if info.get("git_sha") else None),
        "sources_sha256": sha(srcs + [os.path.join(ROOT, "include", "xqa.h")]),
        "library_sha256": sha([lib]) if os.path.exists(lib) else None,
        "bench_sha256": sha([os.path.abspath(__file__)]),
        "build_flags": " ".join(_build.COMMON_FLAGS[:-2]),
        "build_info": info or None,
        "rocm_version": rocm,
        "hip_version": torch.version.hip,
        "torch_version": torch.__version__,
        "gpu_name": props.name,
        "gpu_arch": getattr(props, "gcnArchName", None),
        "gpu_compute_units": props.multi_processor_count,
        "host": platform.node(),
        "seeds": [[1000 + args.config, v] for v in range(args.variants)],
        "variants": args.variants,
    }


def abba(arms, pair, rounds, block):
    """A/B/B/A blocks of `block` steps: per arm median and IQR (us per step) and
    the paired B - A difference per round (B blocks' mean minus A blocks' mean)."""
    import numpy as np
    import torch
    a_name, b_name = pair
    res = {a_name: [], b_name: []}
    diffs = []
    for _ in range(rounds):
        got = {a_name: [], b_name: []}
        for arm in (a_name, b_name, b_name, a_name):
            torch.cuda.synchronize()
            t = time.perf_counter()
            arms[arm](block)
            torch.cuda.synchronize()
            got[arm].append((time.perf_counter() - t) / block * 1e6)
        res[a_name] += got[a_name]
        res[b_name] += got[b_name]
        diffs.append(statistics.mean(got[b_name]) - statistics.mean(got[a_name]))

    def summ(v):
        q1, med, q3 = np.percentile(v, [25, 50, 75])
        return {"median": float(med), "iqr": [float(q1), float(q3)], "n": len(v)}
    return {"A": a_name, "B": b_name, "rounds": rounds, "block_steps": block,
            a_name: summ(res[a_name]), b_name: summ(res[b_name]),
            "paired_B_minus_A": summ(diffs)}


def gpu_clocks():
    """Current GPU clocks and power as rocm-smi reports them (a child process), or None."""
    import subprocess
    try:
        res = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--json"],
                             capture_output=True, text=True, timeout=30)
        data = json.loads(res.stdout)
        card = next(iter(v for k, v in data.items() if k.startswith("card")))
        return {k: v for k, v in card.items() if "clock" in k.lower() or "power" in k.lower()}
    except Exception:
        return None


def host_cpu():
    """CPU model and BLAS library of the host, for the oracle baseline."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = "unknown", 1
    try:
        from threadpoolctl import threadpool_info
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if info:
            blas = f"{info[0].get('internal_api')} {info[0].get('version')}"
            threads = max(p.get("num_threads", 1) for p in info)
    except Exception:
        pass
    return model, blas, threads


def cpu_baseline_leg(w, gpu_out, reps_arg):
    """Time the float64 oracle on a full decode step; compare it with gpu_out."""
    import numpy as np
    import oracle
    model, blas, threads = host_cpu()
    kp, vp = w.pools()
    t = time.perf_counter()
    ref = oracle.decode_attention(w.q, kp, vp, w.block_table, w.context_lens, w.scale)
    one = time.perf_counter() - t
    reps = reps_arg or max(1, min(20, int(12.0 / max(one, 1e-3))))
    t = time.perf_counter()
    for _ in range(reps):
        oracle.decode_attention(w.q, kp, vp, w.block_table, w.context_lens, w.scale)
    cpu_s = (time.perf_counter() - t) / reps
    cpu = {"value": w.kv_bytes / cpu_s / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"full decode step of {w.name} (sum ctx={w.total_tokens}, {w.kv_bytes} KV bytes), "
                     f"{reps} repetitions, {cpu_s * 1e6:.0f} us/step; float64 numpy, "
                     f"BLAS {blas} with {threads} threads; CPU {model}"}
    log(f"cpu oracle: {cpu_s * 1e3:.1f} ms/step ({cpu['value']:.3f} GB/s) x{reps}")
    # tolerance: |gpu - ref| <= 2e-3 or <= 1e-2 |ref| per element; relative L2 <= 1e-3
    err = np.abs(gpu_out.astype(np.float64) - ref)
    ok_el = (err <= 2e-3) | (err <= 1e-2 * np.abs(ref))
    rel_l2 = float(np.sqrt((err ** 2).sum() / max((ref ** 2).sum(), 1e-300)))
    fails = int((~ok_el).sum()) + int((~np.isfinite(gpu_out)).sum())
    gate = {"ok": fails == 0 and rel_l2 <= 1e-3, "fails": fails, "max_abs": float(err.max()),
            "rel_l2": rel_l2}
    return cpu, gate


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode step shards by sequence or KV head with no exchange, see the design notes)",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    # Profiling runs (--no-extras, the calibrations, or any run under
    # rocprofv3, whose preloaded library would also load into a child and
    # initialise the GPU there) start no child process.
    read_clocks = not (args.no_extras or args.calibrate_copy or args.calibrate_read
                       or under_profiler())
    clocks_before = gpu_clocks() if read_clocks else None
    from decode_attention_paged_e5m2_amd import Xqa
    from workloads import make_config
    from workloads.device import to_device

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    if args.calibrate_copy:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n,
                          "dispatches": 5}))
        return 0
    if args.calibrate_read:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.int32, device=dev)
        res = torch.empty((), dtype=torch.int32, device=dev)
        for _ in range(5):
            torch.amax(src, dim=0, out=res)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device read (amax of a 1 GiB int32 buffer)",
                          "bytes_read": n, "bytes_written": 4, "dispatches": 5}))
        return 0

    t0 = time.time()
    works = [make_config(args.config, v) for v in range(args.variants)]
    devs = [to_device(w, dev) for w in works]
    w0 = works[0]
    log(f"generated+uploaded {len(works)} variants in {time.time() - t0:.1f}s; "
        f"Σctx={[w.total_tokens for w in works]}")
    kv_bytes = [w.kv_bytes for w in works]

    xqa = Xqa(max_batch=w0.batch, num_q_heads=w0.num_q_heads, num_kv_heads=w0.num_kv_heads,
              max_pages_per_seq=w0.max_pages_per_seq)
    info = xqa.info
    stream = torch.cuda.current_stream(dev)

    def call(d, out, fn=None):
        (fn or xqa.decode)(q=d.q, k_pages=d.k_pages, v_pages=d.v_pages, block_table=d.block_table,
                           context_lens=d.context_lens, scale=w0.scale, out=out)

    outs = [torch.empty_like(d.q) for d in devs]

    # ------------------------------------------- CPU oracle leg (and gate)
    # The float64 oracle is timed on the host cores as a reported baseline;
    # its output doubles as the correctness gate: no timing is admitted for a
    # GPU result that does not match it.
    call(devs[0], outs[0])
    torch.cuda.synchronize()
    gpu0 = outs[0].float().cpu().numpy()
    cpu = None
    if not args.no_cpu_baseline:
        cpu, gate = cpu_baseline_leg(w0, gpu0, args.cpu_reps)
        log(f"oracle gate: {gate}")
        if not gate["ok"]:
            print(json.dumps({"error": "parity gate failed", "stats": gate}))
            return 1

    eager = []
    for d, o in zip(devs, outs):
        call(d, o)
        eager.append(o.clone())
    torch.cuda.synchronize()

    graphs = []
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):      # warm the capture path off the timed stream
        for d, o in zip(devs, outs):
            call(d, o)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    for d, o in zip(devs, outs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call(d, o)
        graphs.append(g)
    torch.cuda.synchronize()
    for i, (g, o) in enumerate(zip(graphs, outs)):
        o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(o.view(torch.int16), eager[i].view(torch.int16)):
            print(json.dumps({"error": f"graph replay differs from eager (variant {i})"}))
            return 1
    log("graph == eager bitwise on all variants")

    R = len(graphs)

    # One graph holding R consecutive decode steps (one per input variant),
    # as a model's decode step holds one attention call per layer: the
    # graph-launch cost is paid once per R steps instead of once per step.
    multi = torch.cuda.CUDAGraph()
    with torch.cuda.graph(multi):
        for d, o in zip(devs, outs):
            call(d, o)
    torch.cuda.synchronize()
    for o in outs:
        o.fill_(float("nan"))
    multi.replay()
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        if not torch.equal(o.view(torch.int16), eager[i].view(torch.int16)):
            print(json.dumps({"error": f"multi-step graph differs from eager (variant {i})"}))
            return 1
    log(f"{R}-step graph == eager bitwise")

    def run_graph(n_steps, start=0):
        for s in range(n_steps):
            graphs[(start + s) % R].replay()

    def run_multi(n_steps):
        for _ in range(n_steps // R):
            multi.replay()

    def run_eager(n_steps, start=0):
        for s in range(n_steps):
            i = (start + s) % R
            call(devs[i], outs[i])

    # ---------------------------------------------------- headline timing
    # Steps are replays of the R-step graph; K is rounded up to a multiple
    # of R so every variant is stepped equally often.
    steps = -(-args.steps // R) * R
    run_eager(args.warmup)                 # each arm warms up on its own
    torch.cuda.synchronize()
    run_graph(args.warmup)
    torch.cuda.synchronize()
    run_multi(max(args.warmup, R))
    torch.cuda.synchronize()
    sampler = ClockSampler() if read_clocks else None
    if sampler:
        sampler.start()
    t_start = time.perf_counter()
    run_multi(steps)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    steps_bytes = sum(kv_bytes[s % R] for s in range(steps))
    gbs = steps_bytes / elapsed / 1e9
    us_step = elapsed / steps * 1e6
    log(f"{R}-step graph replay: {us_step:.2f} us/step, {gbs:.1f} GB/s KV "
        f"({100 * gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s)")

    torch.cuda.synchronize()
    t1 = time.perf_counter()
    run_graph(steps)
    torch.cuda.synchronize()
    us_1 = (time.perf_counter() - t1) / steps * 1e6
    log(f"1-step graph replay: {us_1:.2f} us/step")

    detail = {"us_per_step_graph_Rstep": us_step, "us_per_step_graph_1step": us_1,
              "kv_bytes_per_step_mean": statistics.mean(kv_bytes), "handle": info,
              "gpu_clocks_before": clocks_before}

    if not args.no_extras:
        # Floors. A replay of a graph costs the host ~15-20 us whatever the
        # graph holds, so a graph of a few near-empty steps measures the
        # host, not the GPU: the floors use graphs of FLOOR_STEPS steps, long
        # enough that the GPU's work per replay exceeds the host's launch.
        FLOOR_STEPS = 32
        floor_reps = max(steps // FLOOR_STEPS, 8)
        # Zero lengths: the decode graph's kernels with every context length 0
        # (launches, plan, zero rows), the fixed cost under each step.
        zero_lens = [torch.zeros_like(d.context_lens) for d in devs]
        zero_outs = [torch.empty_like(d.q) for d in devs]
        floor_g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(floor_g):
            for k in range(FLOOR_STEPS):
                d, z, o = devs[k % R], zero_lens[k % R], zero_outs[k % R]
                xqa.decode(q=d.q, k_pages=d.k_pages, v_pages=d.v_pages, block_table=d.block_table,
                           context_lens=z, scale=w0.scale, out=o)
        for _ in range(4):
            floor_g.replay()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(floor_reps):
            floor_g.replay()
        torch.cuda.synchronize()
        us_floor = (time.perf_counter() - t) / (floor_reps * FLOOR_STEPS) * 1e6
        if not all(bool((o == 0).all()) for o in zero_outs):
            print(json.dumps({"error": "zero-length step did not write zero rows"}))
            return 1
        log(f"floor (all lengths 0, graph of {FLOOR_STEPS} steps): {us_floor:.2f} us/step")
        detail["floor_us_per_step_zero_lengths"] = us_floor
        detail["floor_graph_steps"] = FLOOR_STEPS
        del floor_g
        # Launch floor: as many empty kernels (a zero-cycle spin, one
        # workgroup) per step as the decode step launches, same graph length.
        kernels_per_step = int(info.get("kernels_per_step", 2))
        empty_g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(empty_g):
            for _ in range(FLOOR_STEPS * kernels_per_step):
                torch.cuda._sleep(0)
        for _ in range(4):
            empty_g.replay()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(floor_reps):
            empty_g.replay()
        torch.cuda.synchronize()
        us_empty = (time.perf_counter() - t) / (floor_reps * FLOOR_STEPS) * 1e6
        log(f"launch floor ({kernels_per_step} empty kernels per step): {us_empty:.2f} us/step")
        detail["floor_us_per_step_empty_kernels"] = us_empty
        del empty_g
        # The same empty kernels, one step per graph replay: bounded by the
        # host's launch of a graph, the floor under the one-step-per-graph arm.
        empty1 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(empty1):
            for _ in range(kernels_per_step):
                torch.cuda._sleep(0)
        for _ in range(max(args.warmup, 2)):
            empty1.replay()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(steps):
            empty1.replay()
        torch.cuda.synchronize()
        detail["floor_us_per_step_empty_kernels_1step_graph"] = (time.perf_counter() - t) / steps * 1e6
        del empty1

    # ------------------------------------------------------ A/B/B/A blocks
    # Every arm warmed up on its own above; blocks of the same number of steps
    # run A B B A, `--abba-rounds` times, for the headline arm against eager
    # calls and against one step per graph replay. Reported per arm: median and
    # interquartile range of the blocks; per pair: the paired B - A difference.
    if not args.quick:
        blk = max(R, min(400, args.steps // 5) // R * R)
        arms = {"graph_Rstep": run_multi, "eager": run_eager, "graph_1step": run_graph}
        detail["abba_us_per_step"] = [
            abba(arms, ("graph_Rstep", "eager"), args.abba_rounds, blk),
            abba(arms, ("graph_Rstep", "graph_1step"), args.abba_rounds, blk)]
        for r in detail["abba_us_per_step"]:
            log(f"A/B/B/A {r['A']} {r[r['A']]['median']:.2f} vs {r['B']} {r[r['B']]['median']:.2f} us/step, "
                f"paired B-A {r['paired_B_minus_A']['median']:+.2f} us")
        # warm mode: the same variant back to back (may be cache resident)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(blk):
            graphs[0].replay()
        torch.cuda.synchronize()
        detail["warm_same_input_us_per_step"] = (time.perf_counter() - t) / blk * 1e6
    if sampler:
        detail["gpu_clocks_during_timing"] = sampler.stop()

    # --------------------------------------- per-launch timing of each kernel
    # HIP events recorded on the stream the kernels are launched on. A spin
    # kernel queued first keeps the GPU busy until every launch and event is
    # queued, so the host's argument checks never sit between an event and
    # the kernels it brackets.
    #  - split kernel: one event pair around n_ev back-to-back launches
    #    (variants in rotation); the mean launch duration is the pair's time
    #    over n_ev. It includes the short gaps between consecutive kernels,
    #    not the per-event overhead of the command processor.
    #  - per step: one pair around the split kernel and one around the
    #    combine kernel, for the split/combine breakdown in the details.
    n_ev = max(20, min(200, args.steps // 10))

    def queued_behind_spin(enqueue):
        spin_cycles = 20_000_000
        for _attempt in range(6):
            gate = torch.cuda.Event()
            torch.cuda._sleep(spin_cycles)
            gate.record(stream)
            enqueue()
            in_time = not gate.query()   # the spin outlasted the queueing
            torch.cuda.synchronize()
            if in_time:
                return True
            spin_cycles *= 4
        return False

    run_ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))

    def enqueue_split_run():
        run_ev[0].record(stream)
        for k in range(n_ev):
            i = k % R
            call(devs[i], outs[i], fn=xqa.split)
        run_ev[1].record(stream)

    ok_run = queued_behind_spin(enqueue_split_run)
    split_run_ms = run_ev[0].elapsed_time(run_ev[1])
    split_bytes = sum(kv_bytes[k % R] for k in range(n_ev))
    split_avg_us = split_run_ms * 1e3 / n_ev
    achieved = split_bytes / (split_run_ms * 1e-3) / 1e9

    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(n_ev)]

    def enqueue_pairs():
        for k in range(n_ev):
            i = k % R
            d = devs[i]
            ev[k][0].record(stream)
            call(d, outs[i], fn=xqa.split)
            ev[k][1].record(stream)
            xqa.combine(context_lens=d.context_lens, out=outs[i])
            ev[k][2].record(stream)

    ok_pairs = queued_behind_spin(enqueue_pairs)
    split_ms = [ev[k][0].elapsed_time(ev[k][1]) for k in range(n_ev)]
    comb_ms = [ev[k][1].elapsed_time(ev[k][2]) for k in range(n_ev)]
    detail["per_launch_timing_queued_behind_spin"] = ok_run and ok_pairs
    detail["split_kernel_us_mean"] = split_avg_us
    detail["split_kernel_launches_timed"] = n_ev
    detail["split_kernel_us_mean_event_pair_each"] = statistics.mean(split_ms) * 1e3
    detail["split_kernel_us_median_event_pair_each"] = statistics.median(split_ms) * 1e3
    detail["combine_kernel_us_mean_event_pair_each"] = statistics.mean(comb_ms) * 1e3
    log(f"split kernel: {split_avg_us:.2f} us mean per launch -> {achieved:.1f} GB/s "
        f"({100 * achieved / HBM_PEAK_GBS:.1f}% of peak); combine "
        f"{detail['combine_kernel_us_mean_event_pair_each']:.2f} us")

    # ------------------------------------------------- cold vs warm steps
    # One decode step per graph replay, bracketed by its own HIP event pair.
    # Cold: before each step a reduction reads a 1 GiB buffer (untimed,
    # outside the pair; it writes one byte, so no dirty lines are left to
    # write back), which streams through the L2 caches and the 256 MiB
    # on-package cache: the step reads its KV bytes from HBM even when they
    # would fit on package.
    # Warm: the same variant's step repeated with nothing in between.
    # Rotating: the variants in turn with nothing in between, as in the
    # headline graph but one step per replay. All three carry the same
    # event-pair overhead and the same per-replay graph launch, so cold minus
    # rotating is the cost of starting from flushed caches.
    if not args.quick:
        flush_buf = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        flush_out = torch.empty((), dtype=torch.uint8, device=dev)
        n_cold = max(20, min(100, args.steps // 20))

        def event_steps(flush, rotate):
            pairs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2))
                     for _ in range(n_cold)]

            def enqueue():
                for k in range(n_cold):
                    if flush:
                        torch.amax(flush_buf, dim=0, out=flush_out)
                    pairs[k][0].record(stream)
                    graphs[k % R if rotate else 0].replay()
                    pairs[k][1].record(stream)

            ok = queued_behind_spin(enqueue)
            return ok, statistics.median(a.elapsed_time(b) * 1e3 for a, b in pairs)

        ok_c, cold_us = event_steps(True, True)
        ok_r, rot_us = event_steps(False, True)
        ok_w, warm_us = event_steps(False, False)
        detail["cold_vs_warm_event_pair_us_per_step"] = {
            "cold_flushed_median": cold_us, "rotating_median": rot_us,
            "warm_same_input_median": warm_us, "steps": n_cold,
            "queued_behind_spin": ok_c and ok_r and ok_w}
        log(f"one step per event pair: cold (1 GiB read before each) {cold_us:.2f} us, "
            f"rotating variants {rot_us:.2f} us, warm (same input repeated) {warm_us:.2f} us")
        del flush_buf, flush_out

    # ------------------------------------------------- multi-token decode
    # Two new query tokens per sequence (causal between them): the G query
    # heads of a KV head times two tokens fill the 16-row matrix-core tile
    # that one token leaves half empty at G = 8; the KV bytes are the same.
    G = w0.num_q_heads // w0.num_kv_heads
    if 2 * G <= 16 and not args.no_extras:
        gen2 = torch.Generator().manual_seed(11)
        xqa2 = Xqa(max_batch=w0.batch, num_q_heads=w0.num_q_heads, num_kv_heads=w0.num_kv_heads,
                   max_pages_per_seq=w0.max_pages_per_seq, max_query_tokens=2)
        q2 = [torch.randn((w.batch, 2, w.num_q_heads, w.head_dim), generator=gen2).half().to(dev)
              for w in works]
        out2 = [torch.empty_like(x) for x in q2]

        def call2(i):
            d = devs[i]
            xqa2.decode(q=q2[i], k_pages=d.k_pages, v_pages=d.v_pages, block_table=d.block_table,
                        context_lens=d.context_lens, scale=w0.scale, out=out2[i])

        for i in range(R):
            call2(i)
        torch.cuda.synchronize()
        multi2 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(multi2):
            for i in range(R):
                call2(i)
        for _ in range(max(args.warmup // R, 2)):
            multi2.replay()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(steps // R):
            multi2.replay()
        torch.cuda.synchronize()
        us_m2 = (time.perf_counter() - t) / steps * 1e6
        detail["multi_token"] = {"tokens_per_sequence": 2, "us_per_step_graph_Rstep": us_m2,
                                 "ratio_to_one_token": us_m2 / us_step}
        log(f"two query tokens per sequence: {us_m2:.2f} us/step ({us_m2 / us_step:.3f}x one token)")
        xqa2.close()

    if not args.no_extras:
        # ------------------------------------------------------------ E4M3 cache
        # The same workload with its K/V quantised to E4M3 and per-tensor scales
        # (xqa_decode_fp8): same bytes per step, a different widening.
        works4 = [make_config(args.config, v, kv_format="e4m3") for v in range(R)]
        devs4 = [to_device(w, dev) for w in works4]
        out4 = [torch.empty_like(d.q) for d in devs4]

        def call4(i):
            d = devs4[i]
            xqa.decode(q=d.q, k_pages=d.k_pages, v_pages=d.v_pages, block_table=d.block_table,
                       context_lens=d.context_lens, scale=w0.scale, out=out4[i], kv_format="e4m3",
                       k_scale=0.5, v_scale=2.0)

        for i in range(R):
            call4(i)
        torch.cuda.synchronize()
        graph4 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph4):
            for i in range(R):
                call4(i)
        for _ in range(max(args.warmup // R, 2)):
            graph4.replay()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(steps // R):
            graph4.replay()
        torch.cuda.synchronize()
        us_e4 = (time.perf_counter() - t) / steps * 1e6
        bytes4 = statistics.mean(w.kv_bytes for w in works4)
        detail["e4m3_scaled"] = {"us_per_step_graph_Rstep": us_e4, "kv_gbs": bytes4 / us_e4 / 1e3,
                                 "ratio_to_e5m2": us_e4 / us_step}
        log(f"E4M3 cache with scales: {us_e4:.2f} us/step ({us_e4 / us_step:.3f}x E5M2)")
        del graph4, devs4, out4, works4
        torch.cuda.synchronize()

        # ---------------------------------------------------- page subsets
        # Decode over a quarter of each sequence's pages (every page drawn
        # with probability 1/4, the last page always), through
        # xqa_decode_pages: a selection kernel gathers the kept pages' ids,
        # then the same split and combine kernels run over them. KV bytes
        # count the kept tokens only.
        from workloads import make_selection
        xqa_p = Xqa(max_batch=w0.batch, num_q_heads=w0.num_q_heads, num_kv_heads=w0.num_kv_heads,
                    max_pages_per_seq=w0.max_pages_per_seq, max_selected_pages=w0.max_pages_per_seq)
        sels, kept_tokens = [], []
        for i, w in enumerate(works):
            sel, cnt = make_selection(w.context_lens, w.max_pages_per_seq, 0.25, [73, i])
            tok = 0
            for b in range(w.batch):
                n, c = int(w.context_lens[b]), int(cnt[b])
                if c > 0:   # ascending, in range, last page included
                    tok += w.page_size * (c - 1) + n - w.page_size * int(sel[b, c - 1])
            sels.append((torch.from_numpy(sel).to(dev), torch.from_numpy(cnt).to(dev)))
            kept_tokens.append(tok)
        outp = [torch.empty_like(d.q) for d in devs]

        def call_p(i):
            d = devs[i]
            xqa_p.decode_pages(q=d.q, k_pages=d.k_pages, v_pages=d.v_pages, block_table=d.block_table,
                               context_lens=d.context_lens, page_select=sels[i][0],
                               select_counts=sels[i][1], scale=w0.scale, out=outp[i])

        eager_p = []
        for i in range(R):
            call_p(i)
            eager_p.append(outp[i].clone())
        torch.cuda.synchronize()
        graph_p = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph_p):
            for i in range(R):
                call_p(i)
        graph_p.replay()
        torch.cuda.synchronize()
        if not all(torch.equal(outp[i].view(torch.int16), eager_p[i].view(torch.int16))
                   for i in range(R)):
            print(json.dumps({"error": "page-subset graph replay differs from eager"}))
            return 1
        for _ in range(max(args.warmup // R, 2)):
            graph_p.replay()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(steps // R):
            graph_p.replay()
        torch.cuda.synchronize()
        us_p = (time.perf_counter() - t) / steps * 1e6
        bytes_p = statistics.mean(kept_tokens) * w0.num_kv_heads * w0.head_dim * 2
        detail["page_subset"] = {"pages_drawn_with_probability": 0.25,
                                 "kept_tokens_per_step_mean": statistics.mean(kept_tokens),
                                 "us_per_step_graph_Rstep": us_p,
                                 "kv_gbs": bytes_p / us_p / 1e3}
        log(f"page subset (1/4 of the pages): {us_p:.2f} us/step, {bytes_p / us_p / 1e3:.1f} GB/s KV")
        xqa_p.close()
        del graph_p, outp, eager_p, sels
        torch.cuda.synchronize()

        # ------------------------------------------------------------ KV append
        # The step before decode in serving: each sequence's new token written
        # into its page slot as E5M2 (xqa_append_kv). Timed per launch with HIP
        # events on the launch stream, and inside one graph holding append +
        # decode for each of the R steps. It rewrites token n - 1 of every
        # sequence, so it runs after every decode measurement above.
        gen = torch.Generator().manual_seed(7)
        k_new = [torch.randn((w.batch, w.num_kv_heads, w.head_dim), generator=gen).half().to(dev)
                 for w in works]
        v_new = [torch.randn((w.batch, w.num_kv_heads, w.head_dim), generator=gen).half().to(dev)
                 for w in works]

        def append(i):
            d = devs[i]
            xqa.append_kv(k_new=k_new[i], v_new=v_new[i], block_table=d.block_table,
                          context_lens=d.context_lens, k_pages=d.k_pages, v_pages=d.v_pages)

        for i in range(R):
            append(i)
        torch.cuda.synchronize()
        ev_a = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(n_ev)]
        for k in range(n_ev):
            ev_a[k][0].record(stream)
            append(k % R)
            ev_a[k][1].record(stream)
        torch.cuda.synchronize()
        append_us = statistics.mean(ev_a[k][0].elapsed_time(ev_a[k][1]) for k in range(n_ev)) * 1e3
        full = torch.cuda.CUDAGraph()
        with torch.cuda.graph(full):
            for i in range(R):
                append(i)
                call(devs[i], outs[i])
        for _ in range(max(args.warmup // R, 2)):
            full.replay()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(steps // R):
            full.replay()
        torch.cuda.synchronize()
        us_full = (time.perf_counter() - t) / steps * 1e6
        # The same step with the append fused into the decode (xqa_decode_append).
        fused = torch.cuda.CUDAGraph()
        with torch.cuda.graph(fused):
            for i in range(R):
                d = devs[i]
                xqa.decode_append(q=d.q, k_new=k_new[i], v_new=v_new[i], k_pages=d.k_pages,
                                  v_pages=d.v_pages, block_table=d.block_table,
                                  context_lens=d.context_lens, scale=w0.scale, out=outs[i])
        for _ in range(max(args.warmup // R, 2)):
            fused.replay()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(steps // R):
            fused.replay()
        torch.cuda.synchronize()
        us_fused = (time.perf_counter() - t) / steps * 1e6
        detail["append_kv"] = {
            "us_per_launch_mean": append_us,
            "bytes_per_launch": w0.batch * w0.num_kv_heads * w0.head_dim * 2 * (2 + 1),
            "us_per_step_graph_Rstep_append_plus_decode": us_full,
            "us_per_step_graph_Rstep_fused_append_decode": us_fused,
        }
        log(f"KV append: {append_us:.2f} us per launch; append + decode graph {us_full:.2f} us/step; "
            f"fused {us_fused:.2f} us/step")

    detail["gpu_clocks_after"] = gpu_clocks() if read_clocks else None
    prov = provenance(args, run_git=read_clocks)
    line = {
        "metric": METRIC,
        "value": gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": us_step / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": w0.name.rsplit("_v", 1)[0],
            "batch": w0.batch, "num_kv_heads": w0.num_kv_heads, "num_q_heads": w0.num_q_heads,
            "head_dim": w0.head_dim, "page_size": w0.page_size, "kv_dtype": "fp8_e5m2",
            "context_lens": "variant-dependent; " + ",".join(str(w.total_tokens) for w in works) + " tokens",
            "variants": R,
            "timed_as": f"hipGraph replay, one graph of {R} consecutive decode steps (one per input variant)",
            "pct_of_hbm_peak": 100.0 * gbs / HBM_PEAK_GBS,
            "us_per_step": us_step,
        },
        "roofline": {"bound": "hbm", "kernel": "split_kernel", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "step_frac": gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic_bytes(args.config)},
        "cpu_baseline": cpu,
        "provenance": prov,
        "detail": detail,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
