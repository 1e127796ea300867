"""Per-layer decode latency and HBM bandwidth of the SketchSSM decode path.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c1] [--no-cpu]

K is rounded up to whole periods of the step loop (instances x 16 steps) so
that every window position and the flush weigh the same.

A step is one decode step of one layer: the read of every (b, h) item at the
current window position, plus the flush (apply the 16 buffered tokens, emit the
sketch) after every 16th read.  Steps rotate over several independent layer
instances (as a model's recurrent layers would) so that consecutive launches
touch different memory and the 256 MB Infinity Cache cannot serve them.  All
inputs are on the device before timing starts.

Prints one JSON line.  ``value`` is microseconds per layer decode step (lower is
better); the same line carries the achieved HBM GB/s, the read and flush kernel
times, the full-state-read baseline, a roofline entry for the read kernel and
the CPU oracle timed on a sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "per-layer decode µs + achieved HBM GB/s, Nano-9B layer, batch 256, mean rank 6"
HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "read_kernel_{}_traffic.md")  # per workload
READ_SOURCES = [os.path.join(ROOT, "rank_state_read_amd", "csrc", f)
                for f in ("read.hip", "device_common.h", "sketchssm_internal.h")]


def read_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in READ_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(config: str):
    """HBM bytes per read launch from the committed counter summary, if it was
    taken on this workload and on the read kernel as it is now (same source
    hash), else None."""
    try:
        text = open(TRAFFIC_FILE.format(config)).read()
    except OSError:
        return None
    keys = ("workload:", "source_hash:", "hbm_bytes_per_launch:")
    vals = dict(line.split(":", 1) for line in text.splitlines() if line.startswith(keys))
    if vals.get("workload", "").strip() != config:
        return None
    if vals.get("source_hash", "").strip() != read_source_hash():
        return None
    try:
        return int(float(vals["hbm_bytes_per_launch"].strip()))
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# algorithmic bytes (what the method has to move; no re-reads)
# ---------------------------------------------------------------------------
def _share(cfg) -> int:
    """Heads sharing one key/query head (1 unless keys and queries are grouped)."""
    return cfg.H // (cfg.kq_heads or cfg.H)


def token_bytes(cfg) -> float:
    """One token of the window per head: k (a shared key counted once per
    group), v, its decay (vector for KDA) and beta."""
    es = 2 if cfg.qkv == "bf16" else 4
    a = 4 * cfg.K if cfg.kind == "kda" else 4
    b = 4 if cfg.kind != "mamba2" else 0
    return cfg.K * es / _share(cfg) + cfg.V * es + a + b


def read_bytes(cfg, ranks, pos: int, dense_all: bool = False) -> int:
    """Bytes of one read launch at window position pos (0-based)."""
    es = 2 if cfg.qkv == "bf16" else 4
    tb = token_bytes(cfg)
    # q + (k,v,a,b in) + append + window + y
    per_item_common = cfg.K * es / _share(cfg) + tb + tb + pos * tb + cfg.V * 4
    total = 0
    frames_rows = set()
    for h in range(cfg.H):
        r = 0 if dense_all else int(ranks[h])
        state = cfg.K * cfg.V * 4 if r == 0 else r * cfg.V * 4
        total += cfg.B * (per_item_common + state)
    if not dense_all:
        # each distinct coefficient map is read once per launch
        frames_rows = {(int(h // (cfg.H // cfg.G)), int(ranks[h])) for h in range(cfg.H) if ranks[h] > 0}
        total += sum(r for _, r in frames_rows) * cfg.K * 4
    return total


def read_write_bytes(cfg) -> int:
    """The part of a read launch's bytes that it writes: y and the appended
    token of every item (the same at every window position)."""
    return int(cfg.B * cfg.H * (cfg.V * 4 + token_bytes(cfg)))


def flush_bytes(cfg, ranks, n_tokens: int, dense_all: bool = False) -> int:
    total = 0
    for h in range(cfg.H):
        r = 0 if dense_all else int(ranks[h])
        s = 2 * cfg.K * cfg.V * 4 if n_tokens > 0 else (cfg.K * cfg.V * 4 if r else 0)
        total += cfg.B * (s + n_tokens * token_bytes(cfg) + r * cfg.V * 4)
    if not dense_all:
        total += sum(int(r) for r in ranks) * cfg.K * 4  # basis rows, once per head
    return total


def rmw_bytes(cfg) -> int:
    """One standard per-token decode launch: the state read and written, the
    token (q, k, v, decay, beta) in and y out, for every item."""
    es = 2 if cfg.qkv == "bf16" else 4
    per_item = 2 * cfg.K * cfg.V * 4 + cfg.K * es / _share(cfg) + token_bytes(cfg) + cfg.V * 4
    return int(cfg.B * cfg.H * per_item)


def workload_name(cfg, ranks) -> str:
    nano = cfg.kind == "mamba2" and (cfg.H, cfg.K, cfg.V) == (128, 128, 80)
    layer = {"mamba2": "Nemotron-Nano-9B-v2-shaped Mamba-2" if nano else "Mamba-2",
             "gdn": "Gated-DeltaNet-style", "kda": "KDA-style"}[cfg.kind]
    shared = f", q/k shared by {_share(cfg)} heads" if _share(cfg) > 1 else ""
    return (f"{cfg.name}: {layer} layer, B={cfg.B} H={cfg.H} K={cfg.K} V={cfg.V} W={cfg.W}, "
            f"mean rank {cfg.mean_rank}, {int((ranks == 0).sum())} dense head(s), {cfg.qkv} q/k/v, fp32 state"
            f"{shared}")


def default_instances(cfg, ranks) -> int:
    """Layer instances to rotate over so that a launch cannot find its data in
    the 256 MB Infinity Cache: the launches between two of one instance read
    at least 1 GiB (at least 4 instances, as the Nano-shaped layer needs)."""
    per_launch = np.mean([read_bytes(cfg, ranks, p) for p in range(cfg.W)])
    return max(4, int(np.ceil((1 << 30) / per_launch)) + 1)


def step_bytes(cfg, ranks, dense_all=False) -> float:
    W = cfg.W
    rd = np.mean([read_bytes(cfg, ranks, p, dense_all) for p in range(W)])
    return rd + flush_bytes(cfg, ranks, W, dense_all) / W


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample
# ---------------------------------------------------------------------------
def cpu_baseline(cfg, wl, steps=None, n_items: int = 16384):
    from threadpoolctl import threadpool_limits

    from oracle import gather_items, items_oracle
    rng = np.random.default_rng(5)
    H = cfg.H
    per_head = max(1, min(cfg.B, n_items // H))
    items = [(int(b), h) for h in range(H) for b in rng.choice(cfg.B, per_head, replace=False)]
    if steps is None:
        steps = [wl.step(t) for t in range(cfg.W)]
    so = [gather_items(st, items) for st in steps]
    with threadpool_limits(limits=1):
        orc = items_oracle(wl, items)
        t0 = time.perf_counter()
        for s in so:
            orc.read(s["q"], s["k"], s["v"], s["a"], s["beta"])
        orc.flush()
        dt = time.perf_counter() - t0
    us_per_step = dt / cfg.W * 1e6 * (cfg.B * cfg.H) / len(items)
    return {"value": round(us_per_step, 1), "unit": "us per layer decode step", "cores": 1,
            "kind": "oracle",
            "sample": f"{len(items)} of {cfg.B * cfg.H} (b,h) items ({per_head} random sequences per head), "
                      f"one window of {cfg.W} reads + 1 flush, fp64 numpy, 1 thread, {dt:.1f} s; scaled to all items",
            "host_cpus_visible": len(os.sched_getaffinity(0)), "cpu_model": _cpu_model()}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------------------
# practical ceilings: the library's streaming probe over 1 GiB
# ---------------------------------------------------------------------------
STREAM_BYTES = 1 << 30
# the read kernel writes about one byte for every eight it reads (y and the
# appended token against the window, token, sketch and map reads: 10.9% of the
# c1 launch's algorithmic bytes), so its ceiling is the best 8:1 stream
MIX_READS_PER_WRITE = 8


def matched_probe(nbytes: int, wbytes: int):
    """The streaming-probe launch that stands for a kernel launch of nbytes, of
    which wbytes written: (bytes read, reads per write).  The mix is the
    nearest the probe offers (2, 4, 8 or 16 reads per write); the size is
    rounded to whole 64 KB chunks (either unroll) and capped at one probe
    source, since a 1 GiB launch already streams at the full rate."""
    reads = nbytes - wbytes
    m = min((2, 4, 8, 16), key=lambda x: abs(np.log2(x) - np.log2(max(reads, 1) / max(wbytes, 1))))
    chunk = 16 * 4096
    return min(STREAM_BYTES, max(chunk, int(round(reads / chunk)) * chunk)), m


def stream_ceilings(torch, Bnd, timed, dev, launches=()) -> dict:
    """Best rate (read + written bytes per second) of the streaming probe for
    an 8:1 read:write mix, for reads alone and for a 1:1 copy, each the best
    of a few launch shapes; and torch's device-to-device copy for reference.

    launches: (bytes, written bytes) of kernel launches to match.  For each,
    the probe also streams a launch of the same size at the nearest mix it
    offers (2, 4, 8 or 16 reads per write) and the result gives the time a
    plain stream of that size and mix takes for the launch's bytes: the fixed
    cost of filling and draining the chip is then in both times, so the ratio
    shows what the kernel loses beyond it.

    Like the decode kernels, which rotate over layer instances, the probe
    never finds its data in the 256 MB last-level cache: successive launches
    read the two 1 GiB sources in turn (a launch smaller than a source reads
    the next of its disjoint regions) and write successive parts of a 2 GiB
    destination pool (the 128 MB written by one 8:1 launch would otherwise
    stay in that cache from one launch to the next)."""
    srcs = [torch.ones(STREAM_BYTES // 4, dtype=torch.float32, device=dev) for _ in range(2)]
    pool = torch.empty(2 * STREAM_BYTES // 4, dtype=torch.float32, device=dev)
    turn = [0]

    def launch(write_bytes, unroll, blocks, nt, read_bytes=STREAM_BYTES):
        i = turn[0]
        turn[0] += 1
        regions = max(1, STREAM_BYTES // read_bytes)   # disjoint regions per source
        src = srcs[i % 2][(i // 2) % regions * (read_bytes // 4):]
        span = max(write_bytes, 4096 * max(blocks, 1))  # bytes this launch writes
        slot = i % max(1, pool.numel() * 4 // span)
        dst = pool[slot * span // 4:]
        Bnd.sketchssm_stream_probe(src, read_bytes, dst, write_bytes, unroll, blocks, nt)

    def rate(write_bytes, unroll, blocks, nt, read_bytes=STREAM_BYTES):
        f = lambda: launch(write_bytes, unroll, blocks, nt, read_bytes)  # noqa: E731
        f()
        us = timed(f, reps=6) * 1000.0
        return (read_bytes + write_bytes) / (us * 1e3)

    def best(write_bytes, shapes, read_bytes=STREAM_BYTES):
        return max((rate(write_bytes, u, b, nt, read_bytes), u, b, nt) for u, b in shapes for nt in (False, True))

    mix = best(STREAM_BYTES // MIX_READS_PER_WRITE, [(8, 0), (16, 0), (8, 2048), (16, 2048)])
    ro = best(0, [(4, 1024), (8, 1024), (8, 2048), (16, 1024), (16, 2048)])
    cp = best(STREAM_BYTES, [(4, 0), (8, 0), (8, 4096)])
    matched_us, matched_mix = [], []
    for nbytes, wbytes in launches:
        rd, m = matched_probe(nbytes, wbytes)
        shapes = [(16, 0)] + ([(8, 0)] if m <= 8 else [])
        r_best = best(rd // m, shapes, rd)
        matched_us.append(nbytes / (r_best[0] * 1e3))   # the launch's bytes at the probe's rate
        matched_mix.append(m)
    half = srcs[0][: STREAM_BYTES // 8]      # 512 MB, twice the Infinity Cache
    other = pool[: STREAM_BYTES // 8]
    other.copy_(half)
    tc_us = timed(lambda: other.copy_(half), reps=5) * 1000.0
    out = {"mix_GBps": round(mix[0], 1),
           "mix_desc": f"best {MIX_READS_PER_WRITE}:1 read:write stream of 1 GiB read, rotating buffers (streaming probe, "
                       f"unroll {mix[1]}, {'one block per chunk' if mix[2] == 0 else f'{mix[2]} blocks'}, "
                       f"{'non-temporal' if mix[3] else 'plain'} loads and stores)",
           "read_only_GBps": round(ro[0], 1), "copy_GBps": round(cp[0], 1),
           "torch_copy_GBps": round(2 * half.numel() * 4 / (tc_us * 1e3), 1),
           "matched_us": matched_us, "matched_mix": matched_mix}
    del srcs, pool, half, other
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=256)
    ap.add_argument("--config", default="c1")
    ap.add_argument("--instances", type=int, default=0,
                    help="independent layer instances the steps rotate over (default: enough that the other "
                         "instances' reads between two launches of one instance cover 1 GiB, at least 4)")
    ap.add_argument("--layers", type=int, default=0,
                    help="model decode loop over N recurrent layers (sets --instances N; e.g. 27 for the Nano model)")
    ap.add_argument("--calibration", default=None,
                    help="calibration file whose per-layer basis replaces the synthetic one (layer i uses basis i)")
    ap.add_argument("--kq-heads", type=int, default=0,
                    help="share q and k among H / N consecutive heads (grouped keys and queries)")
    ap.add_argument("--launch-order", default="bucket", choices=("bucket", "head", "low-first"),
                    help="launch order of the sketch heads: the planner's rank buckets from high to low "
                         "(default), head order, or buckets from low to high")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="only the warmup and timed decode steps (for counter runs)")
    ap.add_argument("--profile-dense", action="store_true",
                    help="as --profile, with the full-state-read baseline's steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="copy 1 GiB device to device three times (scales the HBM byte counters)")
    ap.add_argument("--quiet", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode path has no cross-GPU exchange and the "
              "benchmark runs on a single MI355X (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel() * 4, "copies": 3}), flush=True)
        return

    from rank_state_read_amd import binding as Bnd
    from rank_state_read_amd.layer import launch_order, layer_for_workload
    from workloads import CONFIGS, Workload

    def log(msg):
        if not args.quiet:
            print(msg, file=sys.stderr, flush=True)

    cfg = CONFIGS[args.config]
    if args.kq_heads:
        import dataclasses
        cfg = dataclasses.replace(cfg, kq_heads=args.kq_heads)
    W = cfg.W
    NI = args.layers or args.instances or default_instances(cfg, Workload(cfg).ranks)
    wl = Workload(cfg)
    cal = None
    if args.calibration:
        from rank_state_read_amd.calibration import load_calibration
        cal = load_calibration(args.calibration, K=cfg.K)
        if cal["groups"] != cfg.G or cal["rows"] < cfg.rank_cap:
            print(f"calibration basis {cal['omega'].shape} does not fit G={cfg.G}, rank cap {cfg.rank_cap}",
                  file=sys.stderr)
            sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # the planner's own order unless another is asked for
    order = None if args.launch_order == "bucket" else launch_order(wl.ranks, args.launch_order)
    t0 = time.time()
    lay0 = layer_for_workload(wl, device=dev, order=order)
    log(f"state generated ({time.time() - t0:.1f}s)")
    if cal is not None:
        lay0 = layer_for_workload(Workload(cfg, ranks=wl.ranks, basis=cal["omega"][0]), device=dev,
                                  S_init=lay0.S, order=order)
    lays = [lay0]
    for i in range(1, NI):
        wli = wl if cal is None else Workload(cfg, ranks=wl.ranks, basis=cal["omega"][i % len(cal["omega"])])
        lays.append(layer_for_workload(wli, device=dev, S_init=lay0.S, order=order))
    host_steps = [wl.step(t) for t in range(W)]
    inputs0 = [lay0.upload_step(st) for st in host_steps]

    def rolled(d, i):
        # instance i's own copy of a step's inputs: the batch rows rotated by
        # 37 i, so every launch reads token inputs no other launch has touched
        return {key: None if x is None else torch.roll(x, shifts=37 * i, dims=0).contiguous()
                for key, x in d.items()}

    inputs = [inputs0 if i == 0 else [rolled(d, i) for d in inputs0] for i in range(NI)]
    log(f"inputs generated ({time.time() - t0:.1f}s)")
    dense_plan = Bnd.Plan(lay0.shape, np.zeros(cfg.H, np.int32), wl.groups)
    for L in lays:
        L.flush(0)
    torch.cuda.synchronize()

    idx = {id(L): i for i, L in enumerate(lays)}

    def tok(L, pos):
        return inputs[idx[id(L)]][pos]

    def read(L, pos, y=None):
        d = tok(L, pos)
        return L.read(pos, d["q"], d["k"], d["v"], d["a"], d["beta"], y=y)

    def dense_read(L, pos):
        d = tok(L, pos)
        return L.dense_read(pos, d["q"], d["k"], d["v"], d["a"], d["beta"])

    def dense_flush(L, n):
        Bnd.sketchssm_flush(dense_plan, L.S, None, None, L.kbuf, L.vbuf, L.abuf, L.bbuf, n)

    def read_flush(L, dense=False):
        d = tok(L, W - 1)
        return L.read_flush(d["q"], d["k"], d["v"], d["a"], d["beta"], plan=dense_plan if dense else None)

    def run_steps(n, s0, dense=False, fused=True):
        """n layer steps starting at global step s0 (instance s % NI, position (s // NI) % W).
        fused: the window's last read and its flush in one call (the library fuses
        them where that pays), else the read and then the flush."""
        for s in range(s0, s0 + n):
            L = lays[s % NI]
            pos = (s // NI) % W
            if fused and pos == W - 1:
                read_flush(L, dense)
            elif dense:
                dense_read(L, pos)
                if pos == W - 1:
                    dense_flush(L, W)
            else:
                read(L, pos)
                if pos == W - 1:
                    L.flush(W)

    def timed(fn, reps=1):
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    # the timed steps cover whole periods (every layer instance through a whole
    # window), so that every window position and the flush weigh the same in the
    # mean: --steps is rounded up to a multiple of instances x W, and "steps" in
    # the output line is the number actually timed
    period = NI * W
    K = max(period, (args.steps + period - 1) // period * period)
    warm = max(0, args.warmup)
    # ---- whole decode steps (the headline) -----------------------------------
    # counter runs launch the read at every window position and the plain flush
    # (the fused last read is profiled by the kernel trace of a default run)
    if args.profile_dense:
        run_steps(warm, 0, dense=True, fused=False)
        ms = timed(lambda: run_steps(K, warm, dense=True, fused=False))
        print(json.dumps({"profile_run": "dense", "us_per_step": round(ms * 1000.0 / K, 3), "steps": K}),
              flush=True)
        return
    if args.profile:
        run_steps(warm, 0, fused=False)
        ms = timed(lambda: run_steps(K, warm, fused=False))
        print(json.dumps({"profile_run": True, "us_per_step": round(ms * 1000.0 / K, 3), "steps": K}),
              flush=True)
        return
    run_steps(warm, 0)
    torch.cuda.synchronize()
    ms = timed(lambda: run_steps(K, warm))
    us_step = ms * 1000.0 / K
    log(f"sketch path: {us_step:.2f} us/step over {K} steps")

    # ---- the read kernel alone, per window position ---------------------------
    per_pos = []
    for pos in range(W):
        def f(pos=pos):
            for i in range(NI):
                read(lays[i], pos)
        f()
        per_pos.append(timed(f, reps=8) * 1000.0 / NI)
    read_us = float(np.mean(per_pos))
    # ---- the flush alone (re-applies the same window; the time is what matters) --
    flush_us = timed(lambda: [L.flush(W) for L in lays], reps=4) * 1000.0 / NI
    init_us = timed(lambda: [L.flush(0) for L in lays], reps=4) * 1000.0 / NI
    read_flush_us = timed(lambda: [read_flush(L) for L in lays], reps=4) * 1000.0 / NI
    # the same steps with the last read and the flush as two calls
    run_steps(period, 0, fused=False)
    unfused_step_us = timed(lambda: run_steps(K, 0, fused=False)) * 1000.0 / K

    # ---- full-state-read baseline (every head dense) ----------------------------
    run_steps(period, 0, dense=True)
    ms_d = timed(lambda: run_steps(K, 0, dense=True))
    dense_step_us = ms_d * 1000.0 / K
    run_steps(period, 0, dense=True, fused=False)
    dense_unfused_step_us = timed(lambda: run_steps(K, 0, dense=True, fused=False)) * 1000.0 / K
    dense_pos = []
    for pos in (0, W // 2, W - 1):
        dense_pos.append(timed(lambda pos=pos: [dense_read(L, pos) for L in lays], reps=4) * 1000.0 / NI)
    dense_read_us = timed(lambda: [dense_read(L, p) for p in range(W) for L in lays], reps=2) * 1000.0 / (NI * W)
    dense_flush_us = timed(lambda: [dense_flush(L, W) for L in lays], reps=4) * 1000.0 / NI

    # ---- continuous batching: every sequence at its own window phase -----------
    # row b started at a random step, so it sits at window position
    # (phase_b + step) mod W; the rows whose window fills are flushed alone in
    # the same step
    phase = np.random.default_rng(11).integers(0, W, size=cfg.B)
    seq_tabs = []
    for k in range(W):
        pv = ((phase + k) % W).astype(np.int32)
        rows = np.nonzero(pv == W - 1)[0].astype(np.int32)
        seq_tabs.append((torch.from_numpy(pv).to(dev), torch.from_numpy(rows).to(dev),
                         torch.full((len(rows),), W, dtype=torch.int32, device=dev)))

    # with side=True each layer's row-list flush runs on a second stream (default
    # priority), ordered after that layer's read and before its next read, so
    # it can fill the CUs that the read's last blocks leave idle
    side_stream = torch.cuda.Stream()
    main_stream = torch.cuda.current_stream()
    flush_done = [None] * NI

    def seq_steps(n, s0, side=False):
        for s in range(s0, s0 + n):
            i = s % NI
            L = lays[i]
            k = (s // NI) % W
            pv, rows, cnt = seq_tabs[k]
            d = inputs[i][k]
            if flush_done[i] is not None:
                main_stream.wait_event(flush_done[i])
                flush_done[i] = None
            L.read_seq(pv, d["q"], d["k"], d["v"], d["a"], d["beta"])
            if rows.numel():
                if side:
                    ev = torch.cuda.Event()
                    ev.record(main_stream)
                    side_stream.wait_event(ev)
                    L.flush_seq(rows, cnt, stream=side_stream)
                    flush_done[i] = torch.cuda.Event()
                    flush_done[i].record(side_stream)
                else:
                    L.flush_seq(rows, cnt)
        for i in range(NI):
            if flush_done[i] is not None:
                main_stream.wait_event(flush_done[i])
                flush_done[i] = None

    seq_steps(period, 0)
    seq_step_us = timed(lambda: seq_steps(K, 0)) * 1000.0 / K
    seq_steps(period, 0, side=True)
    seq_side_us = timed(lambda: seq_steps(K, 0, side=True)) * 1000.0 / K

    # ---- standard per-token decode: every token reads and writes the state ------
    def rmw(L, pos):
        d = tok(L, pos)
        return L.rmw_step(d["q"], d["k"], d["v"], d["a"], d["beta"])

    [rmw(L, 0) for L in lays]
    rmw_us = timed(lambda: [rmw(L, p) for p in range(W) for L in lays], reps=2) * 1000.0 / (NI * W)

    # ---- practical HBM ceilings on this GPU, measured in the same run --------
    ranks = wl.ranks
    rb = [read_bytes(cfg, ranks, p) for p in range(W)]
    ceil = stream_ceilings(torch, Bnd, timed, dev, launches=[(b, read_write_bytes(cfg)) for b in rb])
    matched_us = float(np.mean(ceil["matched_us"]))
    read_GBps = float(np.mean([b / (t * 1e3) for b, t in zip(rb, per_pos)]))
    rb_avg = float(np.mean(rb))
    fb = flush_bytes(cfg, ranks, W)
    sb = step_bytes(cfg, ranks)
    achieved = rb_avg / (read_us * 1e3)
    out = {
        "metric": METRIC,
        "value": round(us_step, 3),
        "unit": "us per layer decode step",
        "n_gpus": 1,
        "steps": K,
        "steps_requested": args.steps,
        "warmup": warm,
        "ms_per_step": round(us_step / 1000.0, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "hbm_GBps": round(sb / (us_step * 1e3), 1),
        "config": {"workload": workload_name(cfg, ranks),
                   "global_batch": cfg.B, "layer_instances": NI, "parallelism": "none (1 GPU)",
                   **({"basis": f"calibration file, layers {cal['layer_ids'][:NI]}"} if cal is not None else {}),
                   **({"launch_order": args.launch_order} if order is not None else {})},
        "roofline": {"bound": "hbm", "kernel": "read_kernel (sketchssm_decode_read)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(cfg.name) if order is None else None,
                     "bytes_per_launch": int(rb_avg), "avg_launch_us": round(read_us, 3),
                     "ceiling_GBps": ceil["mix_GBps"], "ceiling": ceil["mix_desc"],
                     "frac_of_ceiling": round(achieved / ceil["mix_GBps"], 4),
                     "ceiling_matched_GBps": round(rb_avg / (matched_us * 1e3), 1),
                     "ceiling_matched": "streaming probe launches of each window position's read size and nearest "
                                        "read:write mix (2, 4, 8 or 16:1), rotating buffers",
                     "frac_of_matched_ceiling": round(matched_us / read_us, 4)},
        "detail": {
            "read_us_mean": round(read_us, 3),
            "read_us_per_pos": [round(x, 2) for x in per_pos],
            "read_GBps": round(read_GBps, 1),
            "stream_matched_us_per_pos": [round(x, 2) for x in ceil["matched_us"]],
            "stream_matched_mix_per_pos": ceil["matched_mix"],
            "flush_us": round(flush_us, 2),
            "flush_GBps": round(fb / (flush_us * 1e3), 1),
            "initial_sketch_us": round(init_us, 2),
            "read_flush_us": round(read_flush_us, 2),
            "layer_us_model": round((sum(per_pos[:-1]) + read_flush_us) / W, 3),
            "step_us_last_read_and_flush_apart": round(unfused_step_us, 3),
            "dense_step_us_last_read_and_flush_apart": round(dense_unfused_step_us, 3),
            "step_bytes": int(sb),
            "dense_step_us": round(dense_step_us, 3),
            "dense_read_us_mean": round(dense_read_us, 3),
            "dense_read_us_pos0_mid_last": [round(x, 2) for x in dense_pos],
            "dense_read_GBps": round(np.mean([read_bytes(cfg, ranks, p, True) for p in range(W)])
                                     / (dense_read_us * 1e3), 1),
            "dense_flush_us": round(dense_flush_us, 2),
            "read_ratio_dense_over_sketch": round(dense_read_us / read_us, 3),
            "layer_ratio_dense_over_sketch": round(dense_step_us / us_step, 3),
            "model_token_us_all_layers": round(us_step * NI, 2) if args.layers else None,
            "continuous_batching_step_us": round(seq_step_us, 3),
            "continuous_batching_step_us_flush_side_stream": round(seq_side_us, 3),
            "stream_read_only_GBps": ceil["read_only_GBps"],
            "stream_copy_GBps": ceil["copy_GBps"],
            "torch_copy_GBps": ceil["torch_copy_GBps"],
            "rmw_step_us": round(rmw_us, 2),
            "rmw_GBps": round(rmw_bytes(cfg) / (rmw_us * 1e3), 1),
            "ratio_rmw_over_sketch_step": round(rmw_us / us_step, 3),
        },
    }
    if not args.no_cpu:
        log("timing the CPU oracle on a sample ...")
        out["cpu_baseline"] = cpu_baseline(cfg, wl, host_steps)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
