#!/usr/bin/env python3
"""Benchmark of one routed MoE layer served from a shared expert-slot cache,
on one MI355X.

Default workload (one JSON line on stdout):
  decode, BF16: batch 1, 40 MoE layers, a sticky routing trace (keep p = 0.6),
  hidden 2048, 128 experts, top-8, SwiGLU intermediate 768, one LRU slot
  cache of 1894 slots (37% of the 40 x 128 pool) shared by all layers,
  B_P:B_H = 52.7:77.3.  One step = one decode token through all 40 layers;
  each layer call runs route -> cache decision -> fill copy -> grouped GEMV
  -> merge with the host partial.
  value = expert bytes evaluated on the GPU / (wall time - fill-copy time):
  the HBM-side throughput with every input resident; the PCIe fill time is
  measured with HIP events and reported separately (decode.* fields).  The
  events run in a first pass over the trace and the wall is taken from a
  second, event-free pass that makes the same cache decisions.
Also reported: the prefill chunk (8192 tokens, hidden 2048, 128 experts,
top-8, I 768, BF16) in TFLOP/s, and the CPU oracle timed on a bounded sample.

  python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense BF16 MFMA
PEAK_PCIE_GBPS = 63.0           # PCIe 5.0 x16, one direction: 32 GT/s x 16 lanes, 128b/130b
METRIC = "decode MoE-layer expert GB/s (%HBM peak); prefill MoE TFLOP/s (%MFMA peak)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
COPY_BYTES = 1 << 30


def forward_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in ("forward.hip", "common.h"):
        with open(os.path.join(ROOT, "routed_expert_cache_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(key, algorithmic_bytes=None):
    """HBM bytes per launch of `key` from the committed counter summary, or
    None when the kernels have changed since the counters were taken.  Where
    the counted run's launches moved a different algorithmic byte count (the
    decode trace sample differs), the counted traffic/algorithmic ratio is
    applied to this run's algorithmic bytes per launch."""
    try:
        with open(TRAFFIC_JSON) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != forward_source_hash() or key not in t.get("launches", {}):
        return None
    e = t["launches"][key]
    if algorithmic_bytes is not None and e.get("algorithmic_bytes"):
        return e["bytes"] / e["algorithmic_bytes"] * algorithmic_bytes
    return e["bytes"]


# kernels that make up one launch of each measured entry point (name prefixes);
# the BF16 counter run (--no-fp8) holds the first two, the FP8 one (--only-fp8)
# the others.  The FP8 decode launches of T = 1, 4 and 16 share a kernel name:
# they are told apart by order (the run does T = 1, 4, 16 in turn, the same
# number of launches each).
PMC_LAUNCHES = {
    "decode_bf16_forward": ["void moe::dec_fused_kernel<false"],
    "prefill_bf16_forward": ["moe::pf_count_kernel", "moe::pf_scan_kernel", "moe::pf_scatter_kernel",
                             "void moe::pf_gemm_kernel<false, true>", "void moe::pf_down_kernel<false>",
                             "moe::pf_combine_kernel"],
    "decode_fp8_forward": ["void moe::dec_fused_kernel<true"],
    "prefill_fp8_forward": ["moe::pf_count_kernel", "moe::pf_scan_kernel", "moe::pf_scatter_kernel",
                            "void moe::pf_gemm_kernel<true, true>", "void moe::pf_down_kernel<true>",
                            "moe::pf_combine_kernel"],
}
FP8_TS = (1, 4, 16)


def pmc_summary(fetch_dir, write_dir, bench_json):
    import csv
    import glob
    with open(bench_json) as fh:
        run = json.loads([ln for ln in fh.read().splitlines() if ln.startswith('{"metric"')][-1])
    fp8_run = "decode_fp8" in run and "roofline" not in run
    per = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        assert files, "no counter_collection.csv under %s" % d
        vals = {}
        rows = sorted((r for r in csv.DictReader(open(files[0])) if r["Counter_Name"] == counter),
                      key=lambda r: int(r["Dispatch_Id"]))
        seq = []   # (kernel, value) in dispatch order
        for r in rows:
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
            seq.append((r["Kernel_Name"], float(r["Counter_Value"])))
        # the calibration copy (a device-to-device copy of COPY_BYTES): the
        # copy kernel with the largest count
        copy = max((k for k in vals if "copybuffer" in k.lower()), key=lambda k: max(vals[k]))
        factor = max(vals[copy]) * 1024.0 / COPY_BYTES      # counter KiB per true KiB
        per[counter] = dict(vals=vals, seq=seq, factor=factor, copy_kernel=copy)
    # merge into the committed summary when it describes the same sources
    try:
        with open(TRAFFIC_JSON) as fh:
            out = json.load(fh)
        if out.get("source_sha256") != forward_source_hash():
            out = None
    except (OSError, ValueError):
        out = None
    if out is None:
        out = {"source_sha256": forward_source_hash(), "launches": {}, "counted_runs": {}}
    out.setdefault("calibration", {})
    out["calibration"]["fp8_run" if fp8_run else "bf16_run"] = {
        c: {"copy_kernel": per[c]["copy_kernel"], "copy_bytes": COPY_BYTES,
            "counter_kib_per_true_kib": round(per[c]["factor"], 4)} for c in per}

    def launch_bytes(prefixes, select=None):
        # the dispatches of each prefix in dispatch order, across every kernel
        # it matches (the FP8 decode forms of T = 1, 4, 16 are different kernels)
        tot, parts = 0.0, {}
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            for pre in prefixes:
                xs = [x for k, x in per[c]["seq"] if k.startswith(pre)]
                if not xs:
                    continue
                if select:
                    xs = select(xs)
                b = sum(xs) / len(xs) * 1024.0 / per[c]["factor"]   # bytes per dispatch
                parts["%s %s" % (pre.replace("void ", "").replace("moe::", ""), c)] = round(b)
                tot += b
        return tot, parts

    keys = ("decode_fp8_forward", "prefill_fp8_forward") if fp8_run else ("decode_bf16_forward", "prefill_bf16_forward")
    for key in keys:
        if key == "decode_fp8_forward":
            K = run["decode_fp8"]["steps"]
            for i, T in enumerate(FP8_TS):
                tot, parts = launch_bytes(PMC_LAUNCHES[key], lambda xs, i=i: xs[i * K:(i + 1) * K])
                byT = run["decode_fp8"]["by_T"]["T%d" % T]
                out["launches"]["decode_fp8_T%d_forward" % T] = {
                    "bytes": round(tot), "parts": parts,
                    "algorithmic_bytes": byT["experts_per_forward"] * byT["bytes_per_expert"]}
            continue
        select = None
        if key == "decode_bf16_forward":
            # the forward-only burst (n launches replaying the timed calls,
            # whose algorithmic bytes are known), which the split-form burst
            # (2 n launches, the last of this kernel in the run) follows
            n = run["roofline"]["launches"]

            def select(xs, n=n):
                assert len(xs) >= 3 * n, "fewer decode dispatches than the two bursts"
                return xs[len(xs) - 3 * n:len(xs) - 2 * n]
        tot, parts = launch_bytes(PMC_LAUNCHES[key], select)
        if parts:
            out["launches"][key] = {"bytes": round(tot), "parts": parts}
    if "decode_bf16_forward" in out["launches"] and not fp8_run:
        out["launches"]["decode_bf16_forward"]["algorithmic_bytes"] = run["roofline"]["bytes_per_launch"]
    out.setdefault("counted_runs", {})
    out["counted_runs"]["fp8_run" if fp8_run else "bf16_run"] = (
        {"fp8_steps": run["decode_fp8"]["steps"], "fp8_warmup": run["decode_fp8"]["warmup"]} if fp8_run
        else {"trace_steps": run["config"]["trace_steps"]})
    with open(TRAFFIC_JSON, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def assert_clean(what, cache=None, ws=None):
    """After a pass: the decode forward's hand-over word (first word of its
    workspace: non-zero when a bounded wait gave up and y is invalid) and the
    cache's device error word must both be clear, else the pass is not timed."""
    import torch
    torch.cuda.synchronize()
    if ws is not None:
        word = int(ws[:4].view(torch.int32).item())
        assert word == 0, "%s: the decode forward's hand-over timed out (ws word %d); y is invalid" % (what, word)
    if cache is not None:
        code = cache.error()
        assert code == 0, "%s: the cache kernels flagged bad data (error word %d)" % (what, code)


def calibrate_copy():
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("copy calibration: 4 copies of %d bytes" % COPY_BYTES)
    del src, dst
    torch.cuda.empty_cache()


class HipEvents:
    """Timing events created with hipEventDisableSystemFence: a record on a busy
    stream costs far less GPU time than torch's default events (no
    system-scope cache release), so the brackets disturb the path less."""

    def __init__(self, n):
        import ctypes
        import torch
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.lib.hipEventCreateWithFlags(ctypes.byref(e), 0x20000000) == 0
            self.ev.append(e)
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        self._f = ctypes.c_float()

    def record(self, i):
        self.lib.hipEventRecord(self.ev[i], self.stream)

    def ms(self, a, b):
        import ctypes
        assert self.lib.hipEventElapsedTime(ctypes.byref(self._f), self.ev[a], self.ev[b]) == 0
        return self._f.value

    def close(self):
        for e in self.ev:
            self.lib.hipEventDestroy(e)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=192)
    p.add_argument("--warmup", type=int, default=64)
    p.add_argument("--prefill-reps", type=int, default=10)
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--cpu-prefill", type=int, default=0, metavar="ROWS",
                   help="also time the oracle on ROWS tokens of the prefill BF16 chunk (about 40 s of host "
                        "work for weight generation and decoding besides the timed FFN)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-host-exec", action="store_true", help="skip the host executor (CPU) throughput run")
    p.add_argument("--no-host-branch", action="store_true",
                   help="skip decode passes 4 and 5 (the host branch on the CPU), e.g. under counter collection")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-resize", action="store_true", help="skip the safe-point resize timing")
    p.add_argument("--no-fp8", action="store_true", help="skip the FP8 decode and FP8 double-buffered prefill runs")
    p.add_argument("--fp8-steps", type=int, default=64)
    p.add_argument("--fp8-warmup", type=int, default=32)
    p.add_argument("--no-prefill-fp8", action="store_true", help="skip the FP8 double-buffered prefill run")
    p.add_argument("--only-fp8", action="store_true",
                   help="only the FP8 decode and FP8 prefill runs (the FP8 counter runs); no BF16 headline line")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="first run a plain 1 GiB device-to-device copy 4 times (counter calibration)")
    p.add_argument("--pmc-summary", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "BENCH_JSON"),
                   help="no GPU run: turn two rocprofv3 --pmc output folders (FETCH_SIZE, WRITE_SIZE) of "
                        "`bench.py --calibrate-copy ...` and that run's JSON line into profiles/traffic.json")
    return p.parse_args()


# ---------------------------------------------------------------- read ceiling
def read_ceiling(b, nbytes, reps=20):
    """Context for the decode roofline: the same number of bytes read from HBM
    (a 512 MB write before each rep evicts the caches), HIP-event timed like
    the forward, by (1) moe_stream_read, one launch of plain wide loads and
    nothing else: what a single launch streaming a working set this small
    reaches, start-up and tail included; (2) the same read kernel over a sweep
    of grid sizes and loads in flight per thread (moe_stream_read_cfg), the
    best median kept: the fastest single read-only launch of this many bytes
    found; (3) a library reduction (torch.sum over float32)."""
    import torch
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    flush = torch.empty((512 << 20) // 4, dtype=torch.float32, device="cuda")
    out = torch.empty((), dtype=torch.float32, device="cuda")
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    res = {"bytes": nbytes}

    def timed(fn):
        ev = HipEvents(2 * reps)
        for r in range(reps):
            flush.fill_(float(r))
            ev.record(2 * r)
            fn()
            ev.record(2 * r + 1)
        torch.cuda.synchronize()
        us = sorted(ev.ms(2 * r, 2 * r + 1) * 1e3 for r in range(reps))
        ev.close()
        med = us[len(us) // 2]
        return dict(median_us=med, best_us=us[0], GBps_median=nbytes / med / 1e3,
                    frac_median=nbytes / med / 1e3 / PEAK_HBM_GBPS)

    res["moe_stream_read"] = timed(lambda: b.stream_read(x, sink))
    sweep = []
    for n_wg in (256, 512, 1024, 2048, 4096, 8192):
        for unroll in (1, 2, 4, 8, 16):
            r = timed(lambda: b.stream_read_cfg(x, sink, n_wg, unroll))
            sweep.append(dict(n_wg=n_wg, unroll=unroll, median_us=r["median_us"]))
    best = min(sweep, key=lambda d: d["median_us"])
    res["stream_read_sweep_best"] = dict(best, GBps_median=nbytes / best["median_us"] / 1e3,
                                         frac_median=nbytes / best["median_us"] / 1e3 / PEAK_HBM_GBPS)
    res["stream_read_sweep"] = sweep
    res["torch_sum"] = timed(lambda: torch.sum(x, dim=0, out=out))
    return res


# ---------------------------------------------------------------- decode trace
def run_decode(b, K, W, host_GBps=None, host_branch=True):
    import torch
    from harness import gen, CONFIGS
    c = CONFIGS["decode_bf16"]
    L, E, k, H, I, C = c.L, c.E, c.k, c.H, c.I, c.C
    S = 3 * H * I * 2                                   # bytes of one BF16 expert
    n = W + K
    assert n <= c.steps, "warmup + steps must fit the %d-step trace" % c.steps
    log("decode: generating trace and weights")
    picks, logits = gen.decode_trace(c.cfg_id, L, n, E, k, c.p_keep)
    wg, wu, wd = gen.bank_bf16(c.cfg_id, E, H, I, c.w_std)
    host_banks = [t.cpu().pin_memory() for t in
                  b.pack_weights(b.W_BF16, *[torch.from_numpy(a).cuda() for a in (wg, wu, wd)])]
    host = b.HostPoolTables(host_banks, lambda i: gen.alias_base_expert(i // E, i % E, E, c.alias_stride), L * E)
    pool = b.SlotPool(C, H, I, b.W_BF16)
    x = torch.from_numpy(gen.activations_bf16(gen.np_rng(c.cfg_id, gen.S_ACT), n * L, H)).cuda().view(n, L, 1, H)
    lg = torch.from_numpy(logits).cuda()                # [n, L, 1, E]
    # host partial sums are inputs of the merge in passes 1-3; pass 4 computes them with the host executor
    yh = torch.randn((L, 1, H), dtype=torch.float32, device="cuda") * 0.01
    ids = torch.empty((1, k), dtype=torch.int32, device="cuda")
    w = torch.empty((1, k), dtype=torch.float32, device="cuda")
    out = b.StepOut(1, k, E)
    ws = b.forward_workspace(1, k, H, I, C, b.FWD_DECODE)
    y = torch.empty((L, 1, H), dtype=torch.float32, device="cuda")
    pick = out.pick_slot.view(1, k)

    rec_pick = torch.empty((K * L, 1, k), dtype=torch.int32, device="cuda")
    rec_w = torch.empty((K * L, 1, k), dtype=torch.float32, device="cuda")

    def layer_step(cache, s, l, ev=None, i=0, fill=True):
        if ev:
            ev.record(4 * i)
        cache.route_step(l, lg[s, l], ids, w, out, copy=False)      # router + cache step, one launch
        if ev:
            ev.record(4 * i + 1)
            rec_pick[i].copy_(pick)                                  # for the forward-only burst below
            rec_w[i].copy_(w)
            ev.record(4 * i + 2)
        if fill:
            cache.fill(out)                                          # PCIe: host pool -> filled slots
        if ev:
            ev.record(4 * i + 3)
        b.expert_forward_merge(pool.c, x[s, l], pick, w, b.FWD_DECODE, ws, yh[l], y_out=y[l])   # + merge
        if ev:
            ev.record(4 * i + 4)

    def run_trace(ev, fill=True):
        """Cold cache, W warm-up steps, then K timed steps; returns (wall s, counter deltas)."""
        cache = b.Cache(L, E, k, 1, pool, host, c.bp, c.bh)
        for s in range(W):
            for l in range(L):
                layer_step(cache, s, l, fill=fill)
        torch.cuda.synchronize()
        c0 = cache.read_state()[4].astype(np.int64)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        i = 0
        for s in range(W, W + K):
            for l in range(L):
                layer_step(cache, s, l, ev, i, fill=fill)
                i += 1
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        d = cache.read_state()[4].astype(np.int64) - c0    # calls, uniq, hits, misses, fills, host
        assert_clean("decode pass", cache, ws)
        cache.destroy()
        return wall, d

    # Three passes over the same trace from the same cold cache make the same
    # decisions (they do not depend on the copies).  Pass 1 brackets every
    # fill and forward with HIP events (fill time, forward time).  Pass 2 runs
    # the full path without events (each record costs GPU time): the
    # PCIe-inclusive wall.  Pass 3 leaves out the PCIe fill copies, the one
    # part that moves host memory: the filled slots then hold stale bytes but
    # the forward streams the same slots, so its wall is the path with every
    # input resident in HBM (`value`).
    log("decode: pass 1 (events): warmup %d steps, timing %d steps" % (W, K))
    ev = HipEvents(4 * K * L + 1)
    wall_ev, d = run_trace(ev)
    step_s = sum(ev.ms(4 * i, 4 * i + 1) for i in range(K * L)) / 1e3
    fill_s = sum(ev.ms(4 * i + 2, 4 * i + 3) for i in range(K * L)) / 1e3
    fwd_s = sum(ev.ms(4 * i + 3, 4 * i + 4) for i in range(K * L)) / 1e3
    ev.close()
    log("decode: pass 2 (no events)")
    wall, d2 = run_trace(None)
    assert np.array_equal(d, d2), "the two passes made different cache decisions"
    log("decode: pass 3 (no events, no PCIe fill copies)")
    y_eager_last = {}
    wall_res, d3 = run_trace(None, fill=False)
    assert np.array_equal(d, d3), "the passes made different cache decisions"
    y_eager_last["nofill"] = y.clone()

    # Pass 6: one hipGraph per 40-layer step.  The 40 layer calls (router +
    # decision with the layer read from a device scalar, fill, forward +
    # merge) are captured once; each step copies its logits and x into the
    # graph's input buffers and replays it.  With and without the fill copies.
    def run_graph(fill):
        cache = b.Cache(L, E, k, 1, pool, host, c.bp, c.bh)
        lg_s = torch.empty((L, 1, E), dtype=torch.float32, device="cuda")
        x_s = torch.empty((L, 1, H), dtype=torch.uint16, device="cuda")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for l in range(L):
                    cache.route_step(l, lg_s[l], ids, w, out, copy=False)
                    if fill:
                        cache.fill(out)
                    b.expert_forward_merge(pool.c, x_s[l], pick, w, b.FWD_DECODE, ws, yh[l], y_out=y[l])
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()

        def one(s):
            lg_s.copy_(lg[s])
            x_s.copy_(x[s])
            g.replay()

        for s in range(W):
            one(s)
        torch.cuda.synchronize()
        c0 = cache.read_state()[4].astype(np.int64)
        t0 = time.perf_counter()
        for s in range(W, W + K):
            one(s)
        torch.cuda.synchronize()
        wall_g = time.perf_counter() - t0
        dg = cache.read_state()[4].astype(np.int64) - c0
        assert_clean("decode graph pass", cache, ws)
        cache.destroy()
        del g
        return wall_g, dg

    log("decode: pass 6 (one captured graph per 40-layer step, replayed)")
    wall_g_nofill, dg1 = run_graph(False)
    assert np.array_equal(d, dg1), "the graph pass made different cache decisions"
    assert torch.equal(y.view(torch.int32), y_eager_last["nofill"].view(torch.int32)), \
        "the replayed graph's last step differs from the eager pass"
    wall_g_fill, dg2 = run_graph(True)
    assert np.array_equal(d, dg2), "the graph pass made different cache decisions"
    graph_info = dict(
        ms_per_step=wall_g_nofill / K * 1e3, ms_per_step_eager=wall_res / K * 1e3,
        ms_per_step_pcie_inclusive=wall_g_fill / K * 1e3, ms_per_step_pcie_inclusive_eager=wall / K * 1e3,
        GBps=int(d[2] + d[4]) * S / wall_g_nofill / 1e9,
        what="one hipGraph holding a whole 40-layer step (router + decision reading the layer from a device "
             "scalar, fill copy, forward + merge with the host partial), replayed once per token step after "
             "copying the step's logits and x into its input buffers; beside the same work launched eagerly "
             "(pass 3 without fills: `value`; pass 2 with fills); the replay's last y equals the eager pass's "
             "bit for bit")
    # Pass 4: the path as the pages run it, with the host branch.  Per layer
    # call: router + cache step; the logical ids, picks, gate weights and x
    # copied to pinned host buffers, then a pinned `ready` word written in
    # stream order; the host executor's dispatcher thread, waiting for that
    # word, evaluates the host set (moe_host_forward_signal) while the stream
    # runs the fill copies and the GPU evaluation of G; the merge waits for
    # the executor's `done` word and adds its y_host.  Reported beside pass 2
    # (the same path with the harness's y_host).
    wall_host, host_calls, host_s, calibrated, n_cores = None, 0, 0.0, None, len(os.sched_getaffinity(0))
    if host_branch:
        log("decode: pass 4 (with the host branch on the CPU)")
        n_cores = len(os.sched_getaffinity(0))
        n_thr = max(1, n_cores - 1)              # one core left to the thread launching GPU work
        # B_P and B_H of this machine at this expert shape (moe_calibrate_bandwidth):
        # the fill kernel and the DMA engines for B_P, the host executor with its
        # threads unpinned and pinned to physical cores for B_H
        log("decode: bandwidth calibration (fill kernel, DMA, host executor unpinned / pinned)")
        cal_scratch = b.SlotPool(16, H, I, b.W_BF16)
        cal_cache = b.Cache(L, E, k, 1, pool, host, c.bp, c.bh)
        cal_ids = list(range(16))                                    # layer 0: base experts 0..15
        ex_u = b.HostExec(n_thr)
        cal_unpinned = cal_cache.calibrate(cal_ids, cal_scratch, reps=5, host_exec=ex_u)
        ex_u.destroy()
        ex = b.HostExec(n_thr, pin=True)
        cal_pinned = cal_cache.calibrate(cal_ids, cal_scratch, reps=5, host_exec=ex)
        pin_cpus, pin_node = ex.cpus()
        assert_clean("calibration", cal_cache)
        cal_cache.destroy()
        del cal_scratch
        ids_log = torch.empty((1, k), dtype=torch.int32, device="cuda")
        h_ids = torch.empty((1, k), dtype=torch.int32).pin_memory()
        h_pick = torch.empty((1, k), dtype=torch.int32).pin_memory()
        h_w = torch.empty((1, k), dtype=torch.float32).pin_memory()
        h_x = torch.empty((1, H), dtype=torch.uint16).pin_memory()
        h_y = torch.empty((1, H), dtype=torch.float32).pin_memory()
        ready = torch.zeros(1, dtype=torch.int32).pin_memory()
        done = torch.zeros(1, dtype=torch.int32).pin_memory()
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        y_gpu = torch.empty((1, H), dtype=torch.float32, device="cuda")
        seq = [0]

        def layer_step_host(cache, s, l):
            seq[0] += 1
            cache.route_step(l, lg[s, l], ids, w, out, copy=False)
            torch.add(ids, l * E, out=ids_log)                           # logical ids index the host pool
            for hd, dd in ((h_ids, ids_log), (h_pick, pick), (h_w, w), (h_x, x[s, l])):
                hd.copy_(dd, non_blocking=True)
            b.host_signal(ready, seq[0])
            ex.forward_signal(host, b.W_BF16, H, I, h_x, h_ids, h_pick, h_w, h_y, ready, done, seq[0])
            cache.fill(out)
            b.expert_forward(pool.c, x[s, l], pick, w, b.FWD_DECODE, ws, y=y_gpu)
            b.merge_partial_after(y_gpu, h_y, done, seq[0], y_out=y[l], err=err)

        def run_host_trace(bp, bh):
            """Pass 4 (and 5): cold cache with this B_P:B_H, W warm-up and K timed steps."""
            cache4 = b.Cache(L, E, k, 1, pool, host, bp, bh)
            for s in range(W):
                for l in range(L):
                    layer_step_host(cache4, s, l)
            torch.cuda.synchronize()
            c0 = cache4.read_state()[4].astype(np.int64)
            t0 = time.perf_counter()
            for s in range(W, W + K):
                for l in range(L):
                    layer_step_host(cache4, s, l)
            torch.cuda.synchronize()
            wall_h = time.perf_counter() - t0
            dh = cache4.read_state()[4].astype(np.int64) - c0
            assert_clean("decode host-branch pass", cache4, ws)
            cache4.destroy()
            assert ex.status() == 0 and int(err.item()) == 0, "the host branch failed"
            return wall_h, dh

        wall_host, d4 = run_host_trace(c.bp, c.bh)
        assert np.array_equal(d, d4), "the passes made different cache decisions"
        host_calls, host_s = ex.stats()
        calibrated = None
        if True:
            # Pass 5: q* from this machine's rates as moe_calibrate_bandwidth
            # measured them (B_P: the fill kernel, B_H: the pinned executor)
            # instead of the quoted ratio; the same trace.
            bp_c, bh_c = cal_pinned["bp"], cal_pinned["bh"]                    # units of 0.1 GB/s
            log("decode: pass 5 (host branch, calibrated B_P:B_H %.1f:%.1f)" % (bp_c / 10, bh_c / 10))
            wall5, d5 = run_host_trace(bp_c, bh_c)
            calibrated = dict(B_P_GBps=bp_c / 10, B_H_GBps=bh_c / 10, wall_ms_per_step=wall5 / K * 1e3,
                              calibration=dict(
                                  pinned=cal_pinned, unpinned=cal_unpinned, cpus=pin_cpus, numa_node=pin_node,
                                  fill_events_GBps=(d[4] * S / fill_s / 1e9) if fill_s > 0 else None,
                                  what="moe_calibrate_bandwidth on 16 experts of the pool (9437184 B each), 5 "
                                       "reps: fill kernel and hipMemcpyAsync from pinned host memory, host "
                                       "executor on %d threads with decode-shaped calls; fill_events_GBps: "
                                       "pass 1's fill copies for comparison" % n_thr),
                              miss_rate=float(d5[3] / d5[1]), fills_per_layer_call=float(d5[4] / (K * L)),
                              host_experts_per_layer_call=float(d5[5] / (K * L)),
                              experts_on_gpu_per_layer_call=float((d5[2] + d5[4]) / (K * L)))
        ex.destroy()
    # Forward-only burst: the timed layer calls' forward launches again, back
    # to back with the same picks (the slots now hold other experts: the same
    # bytes), one event pair per step of 40 layers: the kernel's duration with
    # no event between its launches.
    log("decode: forward-only burst")
    evb = HipEvents(2 * K)
    for si in range(K):
        evb.record(2 * si)
        for l in range(L):
            i = si * L + l
            b.expert_forward_merge(pool.c, x[W + si, l], rec_pick[i], rec_w[i], b.FWD_DECODE, ws, yh[l], y_out=y[l])
        evb.record(2 * si + 1)
    torch.cuda.synchronize()
    burst_s = sum(evb.ms(2 * si, 2 * si + 1) for si in range(K)) / 1e3
    # the same burst in the split form (gate/up launch, then down launch: no
    # co-residency requirement), the price of the form that waits for nothing
    for si in range(K):
        evb.record(2 * si)
        for l in range(L):
            i = si * L + l
            b.expert_forward_merge(pool.c, x[W + si, l], rec_pick[i], rec_w[i], b.FWD_DECODE_SPLIT, ws, yh[l],
                                   y_out=y[l])
        evb.record(2 * si + 1)
    torch.cuda.synchronize()
    split_s = sum(evb.ms(2 * si, 2 * si + 1) for si in range(K)) / 1e3
    evb.close()
    assert_clean("decode forward-only burst", None, ws)
    n_g = int(d[2] + d[4])
    gpu_bytes = n_g * S
    res = dict(
        value=gpu_bytes / wall_res / 1e9,
        ms_per_step=wall_res / K * 1e3,
        roofline=dict(kernel="moe_expert_forward_merge decode (one kernel: gate/up, down, merge)",
                      bound="hbm", achieved=gpu_bytes / burst_s / 1e9, peak=PEAK_HBM_GBPS, unit="GB/s",
                      bytes_per_launch=gpu_bytes / (K * L), launches=K * L,
                      avg_launch_us=burst_s / (K * L) * 1e6,
                      timing="forward-only burst of the timed calls' launches, one HIP event pair per 40 launches",
                      avg_launch_us_in_trace=fwd_s / (K * L) * 1e6, traffic=None,
                      split_form_us_per_call=split_s / (K * L) * 1e6),
        detail=dict(
            wall_ms_per_step_pcie_inclusive=wall / K * 1e3,
            pcie_inclusive_GBps=gpu_bytes / wall / 1e9,
            wall_minus_fill_events_ms_per_step=(wall - fill_s) / K * 1e3,
            fill_ms_per_step=fill_s / K * 1e3,
            fill_GBps=(d[4] * S / fill_s / 1e9) if fill_s > 0 else None,
            fill_roofline=dict(bound="pcie", achieved=(d[4] * S / fill_s / 1e9) if fill_s > 0 else None,
                               peak=PEAK_PCIE_GBPS, unit="GB/s",
                               frac=(d[4] * S / fill_s / 1e9 / PEAK_PCIE_GBPS) if fill_s > 0 else None,
                               what="cache_fill_kernel: mapped pinned host memory -> slots, per fill event"),
            miss_rate=float(d[3] / d[1]),
            experts_on_gpu_per_layer_call=n_g / (K * L),
            fills_per_layer_call=float(d[4] / (K * L)),
            host_experts_per_layer_call=float(d[5] / (K * L)),
            host_branch=None if wall_host is None else dict(
                wall_ms_per_step=wall_host / K * 1e3,
                host_compute_us_per_call_with_host_picks=host_s / max(host_calls, 1) * 1e6,
                calls_with_host_picks=host_calls,
                calibrated_split=calibrated,
                note="pass 4: the full path with the host set evaluated by moe_host_forward on %d host threads, "
                     "handed over through pinned words while the GPU fills and evaluates G, beside "
                     "wall_ms_per_step_pcie_inclusive (pass 2: the harness's y_host)" % max(1, n_cores - 1)),
            layer_calls=int(d[0]),
            route_and_cache_step_us=step_s / (K * L) * 1e6,
            graph=graph_info,
        ),
    )
    res["roofline"]["frac"] = res["roofline"]["achieved"] / PEAK_HBM_GBPS
    res["roofline"]["traffic"] = measured_traffic("decode_bf16_forward", res["roofline"]["bytes_per_launch"])
    res["detail"]["wall_ms_per_step_with_events"] = wall_ev / K * 1e3
    res["roofline"]["read_ceiling"] = read_ceiling(b, int(res["roofline"]["bytes_per_launch"]) // 4096 * 4096)
    return res


# ---------------------------------------------------------------- prefill chunk
def run_prefill(b, reps):
    import torch
    from harness import gen, CONFIGS
    c = CONFIGS["prefill_bf16"]
    T, H, I, E, k = c.T, c.H, c.I, c.E, c.k
    log("prefill: generating weights and activations")
    wg, wu, wd = gen.bank_bf16(c.cfg_id, E, H, I, c.w_std)
    pool = b.SlotPool(E, H, I, b.W_BF16)
    b.pack_weights(b.W_BF16, *[torch.from_numpy(a).cuda() for a in (wg, wu, wd)], out_gu=pool.w_gu,
                   out_down=pool.w_down)
    xb = gen.activations_bf16(gen.np_rng(c.cfg_id, gen.S_ACT), T, H)
    wr = gen.router_matrix(gen.np_rng(c.cfg_id, gen.S_ROUTER), H, E, c.router_std)
    lg = torch.from_numpy(gen.router_logits(xb, wr)).cuda()
    x = torch.from_numpy(xb).cuda()
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = b.forward_workspace(T, k, H, I, E, b.FWD_PREFILL)
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    flops = 6.0 * H * I * T * k

    def run(ev=None, r=0):
        if ev:
            ev.record(3 * r)
        b.route_topk(lg, k, ids, w)
        if ev:
            ev.record(3 * r + 1)
        b.expert_forward(pool.c, x, ids, w, b.FWD_PREFILL, ws, y=y)
        if ev:
            ev.record(3 * r + 2)

    for _ in range(3):
        run()
    ev = HipEvents(3 * reps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r in range(reps):
        run(ev, r)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_s = sum(ev.ms(3 * r + 1, 3 * r + 2) for r in range(reps)) / 1e3 / reps
    layer_s = sum(ev.ms(3 * r, 3 * r + 2) for r in range(reps)) / 1e3 / reps
    ev.close()
    ach = flops / fwd_s / 1e12
    lib = library_gemm_reference(E, T * k // E, H, I, flops)
    return dict(
        workload="prefill_bf16: 8192 tokens, hidden 2048, 128 experts, top-8 of x.W_r, SwiGLU I 768, BF16, all experts resident",
        value=flops / layer_s / 1e12, unit="TFLOP/s", ms_per_layer=layer_s * 1e3, wall_ms_per_rep=wall / reps * 1e3,
        reps=reps, flops_per_layer=flops,
        roofline=dict(kernel="moe_expert_forward prefill (sort + gate/up GEMM + down GEMM + combine)",
                      bound="mfma", achieved=ach, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                      frac=ach / PEAK_BF16_TFLOPS, avg_launch_us=fwd_s * 1e6,
                      traffic=measured_traffic("prefill_bf16_forward"), library_gemm=lib),
    )


def library_gemm_reference(E, M, H, I, flops, reps=10):
    """Vendor-library reference for the prefill GEMMs: torch.bmm (hipBLASLt) in
    BF16 on the same per-expert shapes with every expert holding the mean M
    pairs (no sort, gather, ragged segments or combine), contiguous operands.
    A context figure beside the roofline, like the plain-read reference of
    the decode kernel; not the product path."""
    import torch
    out = {}
    tot = 0.0
    for name, N, K in (("gate_up", 2 * I, H), ("down", H, I)):
        a = torch.randn(E, M, K, device="cuda", dtype=torch.bfloat16)
        bm = torch.randn(E, K, N, device="cuda", dtype=torch.bfloat16).contiguous()
        c = torch.empty(E, M, N, device="cuda", dtype=torch.bfloat16)
        for _ in range(3):
            torch.bmm(a, bm, out=c)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            torch.bmm(a, bm, out=c)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tot += ms
        out[name] = dict(shape="%d x [%d x %d] . [%d x %d]" % (E, M, K, K, N), ms=ms,
                         TFLOPs=2.0 * E * M * N * K / ms / 1e9)
        del a, bm, c
    out["total_ms"] = tot
    out["TFLOPs_on_layer_flops"] = flops / tot / 1e9
    out["frac"] = out["TFLOPs_on_layer_flops"] / PEAK_BF16_TFLOPS
    return out


# ---------------------------------------------------------------- FP8 pools
def fp8_bank_packed(b, cfg_id, E, H, I, std, layer, out_gu, out_dp, out_s):
    """Draw E FP8 experts on the GPU, pack them, copy into the host tensors at rows [0, E)."""
    import torch
    from harness import gen
    for e in range(E):
        ex = gen.expert_fp8_torch(gen.torch_seed(cfg_id, gen.S_WEIGHTS, layer, e), H, I, std, device="cuda")
        gu, dp = b.pack_weights(b.W_FP8_B128, ex["gate"][None], ex["up"][None], ex["down"][None])
        out_gu[e].copy_(gu[0])
        out_dp[e].copy_(dp[0])
        for i, n in enumerate(("s_gate", "s_up", "s_down")):
            out_s[i][e].copy_(ex[n])
    torch.cuda.synchronize()


def run_decode_fp8(b, K, W, Ts=(1, 4, 16)):
    """Decode FP8 workload: 58-layer pool (layer 0 real, layers 1-57 metadata
    only), H 7168, E 256, top-8, I 2048, 1633 slots, 11.8:47.5; one step = the
    58 layer calls of one token step; the MALL is flushed before layer 0's GEMV."""
    import torch
    from harness import gen, CONFIGS
    c = CONFIGS["decode_fp8"]
    L, E, k, H, I, C = c.L, c.E, c.k, c.H, c.I, c.C
    S = 3 * H * I + 3 * (I // 128) * (H // 128) * 4
    log("decode fp8: drawing and packing layer 0 (%d experts)" % E)
    gu_h = torch.empty((E, 2 * I * H), dtype=torch.uint8, pin_memory=True)
    dp_h = torch.empty((E, H * I), dtype=torch.uint8, pin_memory=True)
    s_h = [torch.empty((E, I // 128, H // 128), dtype=torch.float32, pin_memory=True),
           torch.empty((E, I // 128, H // 128), dtype=torch.float32, pin_memory=True),
           torch.empty((E, H // 128, I // 128), dtype=torch.float32, pin_memory=True)]
    fp8_bank_packed(b, c.cfg_id, E, H, I, c.w_std, 0, gu_h, dp_h, s_h)
    host = b.HostPoolTables([gu_h, dp_h] + s_h, lambda i: i % E, L * E)   # layers >= 1 never copy
    pool = b.SlotPool(C, H, I, b.W_FP8_B128)
    flush = torch.empty((512 << 20) // 4, dtype=torch.float32, device="cuda")
    out_all = {}
    n = W + K
    for T in Ts:
        picks, logits = gen.decode_trace(c.cfg_id, L, n, E, k, c.p_keep, T=T, salt=T)
        lg = torch.from_numpy(logits).cuda()                        # [n, L, T, E]
        x = torch.from_numpy(gen.activations_bf16(gen.np_rng(c.cfg_id, gen.S_ACT, T), n * T, H)).cuda().view(n, T, H)
        cache = b.Cache(L, E, k, T, pool, host, c.bp, c.bh)
        out = b.StepOut(T, k, E)
        ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        ws = b.forward_workspace(T, k, H, I, C, b.FWD_DECODE)
        yh = torch.zeros((T, H), dtype=torch.float32, device="cuda")
        y = torch.empty((T, H), dtype=torch.float32, device="cuda")
        pick = out.pick_slot.view(T, k)
        ev = HipEvents(3 * K)
        fwd_counts = np.zeros(2, np.int64)

        def step(s, i=None):
            for l in range(L):
                cache.route_step(l, lg[s, l], ids, w, out, copy=False)
                if l == 0:
                    flush.add_(1.0)                                  # evict the MALL (512 MB read + write)
                    if i is not None:
                        ev.record(3 * i)
                    cache.fill(out)
                    if i is not None:
                        ev.record(3 * i + 1)
                    b.expert_forward_merge(pool.c, x[s], pick, w, b.FWD_DECODE, ws, yh, y_out=y)
                    if i is not None:
                        ev.record(3 * i + 2)
                    if i is not None:
                        cnt = out.counts                                # read after the run
                        fwd_counts_dev.append(cnt.clone())

        fwd_counts_dev = []
        for s in range(W):
            step(s)
        torch.cuda.synchronize()
        c0 = cache.read_state()[4].astype(np.int64)
        fwd_counts_dev.clear()
        t0 = time.perf_counter()
        for i, s in enumerate(range(W, n)):
            step(s, i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        c1 = cache.read_state()[4].astype(np.int64)
        assert_clean("decode fp8 T=%d" % T, cache, ws)
        cnts = torch.stack(fwd_counts_dev).cpu().numpy()
        n_g = int(cnts[:, 1].sum() + cnts[:, 4].sum())                  # layer-0 hits + fills
        fill_s = sum(ev.ms(3 * i, 3 * i + 1) for i in range(K)) / 1e3
        fwd_s = sum(ev.ms(3 * i + 1, 3 * i + 2) for i in range(K)) / 1e3
        ev.close()
        d = c1 - c0
        ach = n_g * S / fwd_s / 1e9
        tr = measured_traffic("decode_fp8_T%d_forward" % T, n_g * S / K)
        out_all["T%d" % T] = dict(
            traffic=tr, traffic_over_algorithmic=(tr / (n_g * S / K)) if tr else None,
            expert_GBps=ach, frac_hbm=ach / PEAK_HBM_GBPS, experts_per_forward=n_g / K,
            avg_forward_us=fwd_s / K * 1e6, bytes_per_expert=S,
            layer0_fill_GBps=(cnts[:, 4].sum() * S / fill_s / 1e9) if fill_s > 0 else None,
            miss_rate_all_layers=float(d[3] / d[1]), wall_ms_per_step=wall / K * 1e3)
        cache.destroy()
        del lg, x, ws
    return dict(workload="decode_fp8: 58-layer pool (layer 0 real, 1-57 metadata only), H 7168, E 256, top-8, "
                         "I 2048, FP8 E4M3 + 128x128 scales, 1633 slots (11%), B_P:B_H 11.8:47.5, sticky p 0.5",
                steps=K, warmup=W, by_T=out_all)


def run_prefill_fp8(b):
    """Prefill FP8 workload: 8192 tokens x 4 layers, H 7168, E 256, top-8,
    I 2048; all 4 x 256 experts in a pinned host pool; two full-layer buffers
    of the slot pool alternate; run once overlapped and once serial."""
    import torch
    from harness import gen, CONFIGS
    c = CONFIGS["prefill_fp8"]
    T, NL, H, I, E, k = c.T, c.layers, c.H, c.I, c.E, c.k
    log("prefill fp8: drawing and packing %d x %d experts" % (NL, E))
    gu_h = torch.empty((NL * E, 2 * I * H), dtype=torch.uint8, pin_memory=True)
    dp_h = torch.empty((NL * E, H * I), dtype=torch.uint8, pin_memory=True)
    s_h = [torch.empty((NL * E, I // 128, H // 128), dtype=torch.float32, pin_memory=True),
           torch.empty((NL * E, I // 128, H // 128), dtype=torch.float32, pin_memory=True),
           torch.empty((NL * E, H // 128, I // 128), dtype=torch.float32, pin_memory=True)]
    for l in range(NL):
        fp8_bank_packed(b, c.cfg_id, E, H, I, c.w_std, l, gu_h[l * E:(l + 1) * E], dp_h[l * E:(l + 1) * E],
                        [t[l * E:(l + 1) * E] for t in s_h])
    host = b.HostPoolTables([gu_h, dp_h] + s_h, lambda i: i, NL * E)
    pool = b.SlotPool(2 * E, H, I, b.W_FP8_B128)
    cache = b.Cache(NL, E, k, 1, pool, host, 118, 475)
    pf = b.PrefillPool(cache)
    log("prefill fp8: activations and router logits")
    xs, lgs = [], []
    for l in range(NL):
        xb = gen.activations_bf16(gen.np_rng(c.cfg_id, gen.S_ACT, l), T, H)
        wr = torch.from_numpy(gen.router_matrix(gen.np_rng(c.cfg_id, gen.S_ROUTER, l), H, E, c.router_std))
        xf = torch.from_numpy(xb).cuda().view(torch.bfloat16).to(torch.float64)
        lgs.append((xf @ wr.cuda().to(torch.float64)).to(torch.float32).contiguous())
        xs.append(torch.from_numpy(xb).cuda())
        del xf
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = b.forward_workspace(T, k, H, I, E, b.FWD_PREFILL)
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    flops = 6.0 * H * I * T * k
    layer_bytes = E * (3 * H * I + 3 * (I // 128) * (H // 128) * 4)
    compute = torch.cuda.current_stream()
    copy = torch.cuda.Stream()

    def run(serial, pf=pf, depth=2):
        """One pass over the NL layers through `depth` full-layer buffers
        (serial: each layer's copy waits for the previous layer's compute)."""
        ev = HipEvents(2 * NL)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for l in range(1 if serial else min(depth, NL)):
            pf.prefetch(l, copy)
        for l in range(NL):
            if serial and l > 0:
                copy.wait_stream(compute)
                pf.prefetch(l, copy)
            view = pf.acquire(l, compute)
            b.route_topk(lgs[l], k, ids, w)
            ev.record(2 * l)
            b.expert_forward(view, xs[l], ids, w, b.FWD_PREFILL, ws, y=y)
            ev.record(2 * l + 1)
            pf.release(l, compute)
            if not serial and l + depth < NL:
                pf.prefetch(l + depth, copy)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        fwd = [ev.ms(2 * l, 2 * l + 1) / 1e3 for l in range(NL)]
        ev.close()
        return wall, fwd

    run(False)                                                       # warm-up
    wall_o, fwd_o = run(False)
    wall_s, fwd_s = run(True)
    assert_clean("prefill fp8 double buffer", cache)
    # hand-over: the two buffers' layers become the decode cache's residents
    t0 = time.perf_counter()
    pf.finish()
    handover_ms = (time.perf_counter() - t0) * 1e3
    survivors = int((cache.read_state()[0] >= 0).sum())
    cache.destroy()
    del pool, cache, pf
    torch.cuda.empty_cache()
    from oracle import lru
    orc = lru.ExpertCache(NL, E, 2 * E, 118, 475)
    orc.reserve(0, 2 * E)
    t0 = time.perf_counter()
    orc.finish_prefill(0, 2, [(0, NL - 2), (1, NL - 1)])
    oracle_ho_ms = (time.perf_counter() - t0) * 1e3
    variants = dict(handover=dict(ms=handover_ms, survivors=survivors, cpu_oracle_ms=oracle_ho_ms,
                                  what="moe_prefill_finish after the 4-layer pass: 2 x 256 experts registered "
                                       "(tables only: a device sync, one kernel, the order rebuild)"))
    # a ring of three full-layer buffers
    log("prefill fp8: ring of three buffers")
    pool3 = b.SlotPool(3 * E, H, I, b.W_FP8_B128)
    cache3 = b.Cache(NL, E, k, 1, pool3, host, 118, 475)
    pf3 = b.PrefillPool(cache3, 3)
    run(False, pf3, 3)
    wall_r, fwd_r = run(False, pf3, 3)
    pf3.destroy()
    cache3.destroy()
    del pool3, cache3, pf3
    torch.cuda.empty_cache()
    variants["ring3"] = dict(ms_per_layer=wall_r / NL * 1e3, forward_ms_per_layer=sum(fwd_r) / NL * 1e3)
    # on-demand loading: a pool of 1.5 layers cannot hold two full-layer buffers
    log("prefill fp8: on-demand loading into %d slots" % (3 * E // 2))
    pool_d = b.SlotPool(3 * E // 2, H, I, b.W_FP8_B128)
    cache_d = b.Cache(NL, E, k, (E + k - 1) // k, pool_d, host, 118, 475)
    out_d = b.StepOut((E + k - 1) // k, k, E)
    ws_d = b.forward_workspace(T, k, H, I, pool_d.n_slots, b.FWD_PREFILL)
    pick_d = torch.empty((T, k), dtype=torch.int32, device="cuda")

    def run_on_demand():
        ev = HipEvents(3 * NL)
        fills, host_picks = 0, 0
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for l in range(NL):
            b.route_topk(lgs[l], k, ids, w)
            ev.record(3 * l)
            cache_d.prefill_load(l, ids, out_d, pick_slot=pick_d)
            ev.record(3 * l + 1)
            b.expert_forward(pool_d.c, xs[l], pick_d, w, b.FWD_PREFILL, ws_d, y=y)
            ev.record(3 * l + 2)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        load = [ev.ms(3 * l, 3 * l + 1) / 1e3 for l in range(NL)]
        fwd = [ev.ms(3 * l + 1, 3 * l + 2) / 1e3 for l in range(NL)]
        ev.close()
        return wall, load, fwd

    run_on_demand()                                                  # warm-up (the cache then holds layer 3)
    c0 = cache_d.read_state()[4].astype(np.int64)
    wall_d, load_d, fwd_d = run_on_demand()
    dd = cache_d.read_state()[4].astype(np.int64) - c0
    assert_clean("prefill fp8 on-demand loading", cache_d)
    host_left = int((pick_d < 0).sum())
    cache_d.destroy()
    del pool_d, cache_d
    torch.cuda.empty_cache()
    variants["on_demand"] = dict(
        slots=3 * E // 2, ms_per_layer=wall_d / NL * 1e3, load_ms_per_layer=sum(load_d) / NL * 1e3,
        forward_ms_per_layer=sum(fwd_d) / NL * 1e3, fills_per_layer=float(dd[4]) / NL,
        load_GBps=float(dd[4]) * (layer_bytes / E) / sum(load_d) / 1e9, host_picks_last_layer=host_left,
        roofline=dict(bound="pcie", achieved=float(dd[4]) * (layer_bytes / E) / sum(load_d) / 1e9,
                      peak=PEAK_PCIE_GBPS, unit="GB/s",
                      frac=float(dd[4]) * (layer_bytes / E) / sum(load_d) / 1e9 / PEAK_PCIE_GBPS,
                      what="the fill copies of moe_cache_prefill_load against PCIe 5.0 x16 (one direction)"),
        what="moe_cache_prefill_load (every miss filled by the fused fill kernel from mapped pinned memory) then "
             "the grouped GEMM over the whole pool; no overlap of load and compute")
    ach = flops / (sum(fwd_o) / NL) / 1e12
    return dict(workload="prefill_fp8: 8192 tokens x 4 layers, H 7168, E 256, top-8 of x.W_r, I 2048, FP8 E4M3 + "
                         "128x128 scales, pinned host pool, two full-layer slot buffers",
                ms_per_layer_overlapped=wall_o / NL * 1e3, ms_per_layer_serial=wall_s / NL * 1e3,
                overlap_gain=wall_s / wall_o, h2d_bytes_per_layer=layer_bytes,
                h2d_GBps_bound=layer_bytes / (wall_o / NL) / 1e9,
                forward_ms_per_layer=sum(fwd_o) / NL * 1e3, variants=variants,
                roofline=dict(kernel="moe_expert_forward prefill FP8 (sort + gate/up GEMM + down GEMM + combine)",
                              bound="mfma", achieved=ach, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                              frac=ach / PEAK_BF16_TFLOPS, traffic=measured_traffic("prefill_fp8_forward")))


def run_resize(b):
    """Cost of a safe-point resize at the decode BF16 shapes: a full cache of
    1894 slots (seeded so that its most recent half sits in the upper half of
    the slots: every kept expert has to move) shrinks in place to 947 slots,
    then grows into new banks of 1894 slots (every kept expert is copied)."""
    import torch
    from harness import gen, CONFIGS
    c = CONFIGS["decode_bf16"]
    L, E, k, H, I, C = c.L, c.E, c.k, c.H, c.I, c.C
    S = 3 * H * I * 2
    wg, wu, wd = gen.bank_bf16(c.cfg_id, E, H, I, c.w_std)
    host_banks = [t.cpu().pin_memory() for t in
                  b.pack_weights(b.W_BF16, *[torch.from_numpy(a).cuda() for a in (wg, wu, wd)])]
    host = b.HostPoolTables(host_banks, lambda i: gen.alias_base_expert(i // E, i % E, E, c.alias_stride), L * E)
    pool = b.SlotPool(C, H, I, b.W_BF16)
    cache = b.Cache(L, E, k, 1, pool, host, c.bp, c.bh)
    ids = np.random.default_rng(0).permutation(L * E)[:C]
    cache.seed([int(i) for i in ids], copy=True)
    torch.cuda.synchronize()
    half = C // 2
    t0 = time.perf_counter()
    cache.resize(pool.prefix(half))
    shrink_ms = (time.perf_counter() - t0) * 1e3
    moved = half                                             # the kept half all sat at slots >= C/2
    ok = int((cache.read_state()[0] >= 0).sum()) == half
    pool2 = b.SlotPool(C, H, I, b.W_BF16)
    t0 = time.perf_counter()
    cache.resize(pool2)
    grow_ms = (time.perf_counter() - t0) * 1e3
    cache.destroy()
    del pool, pool2, cache, host, host_banks
    torch.cuda.empty_cache()
    # the oracle's resize of the same table state (test infrastructure, timed beside)
    from oracle import lru
    orc = lru.ExpertCache(L, E, C, c.bp, c.bh)
    orc.seed([int(i) for i in ids])
    t0 = time.perf_counter()
    orc.resize(half)
    orc.resize(C)
    oracle_ms = (time.perf_counter() - t0) * 1e3
    hbm = 2 * moved * S / (shrink_ms / 1e3) / 1e9     # each moved byte read and written once
    return dict(workload="decode_bf16 cache: %d slots of %d B, full, shrink in place to %d then grow into new "
                         "banks of %d slots" % (C, S, half, C),
                shrink_ms=shrink_ms, shrink_moved_experts=moved, shrink_tables_ok=ok,
                shrink_copy_GBps=moved * S / (shrink_ms / 1e3) / 1e9,
                grow_ms=grow_ms, grow_copied_experts=half, grow_copy_GBps=half * S / (grow_ms / 1e3) / 1e9,
                roofline=dict(bound="hbm", achieved=hbm, peak=PEAK_HBM_GBPS, unit="GB/s", frac=hbm / PEAK_HBM_GBPS,
                              what="in-place shrink: moved expert bytes read + written over the call's wall time"),
                cpu_oracle_tables_ms=oracle_ms,
                note="wall of the synchronous call (tables kernel, order rebuild, bank copies); GB/s counts the "
                     "expert bytes copied (each read once and written once in HBM); cpu_oracle_tables_ms: the "
                     "oracle's shrink and grow of the same tables (no bytes)")


# ---------------------------------------------------------------- CPU oracle baseline
def cpu_prefill_oracle(rows):
    """The oracle on a sample of the prefill BF16 chunk: the exact float64
    FFN of `rows` tokens (each with its k picks), as oracle GFLOP/s (the
    weights are decoded to float64 before the timed part)."""
    from harness import gen, CONFIGS
    from oracle import route, ffn, numerics
    c = CONFIGS["prefill_bf16"]
    T, H, I, E, k = c.T, c.H, c.I, c.E, c.k
    wg, wu, wd = gen.bank_bf16(c.cfg_id, E, H, I, c.w_std)
    xb = gen.activations_bf16(gen.np_rng(c.cfg_id, gen.S_ACT), T, H)
    wr = gen.router_matrix(gen.np_rng(c.cfg_id, gen.S_ROUTER), H, E, c.router_std)
    lg = gen.router_logits(xb[:rows], wr)
    ids, w = route.topk_softmax(lg, k)
    cache = {}

    def expert(e):
        if e not in cache:
            cache[e] = (numerics.bf16_to_f64(wg[e]), numerics.bf16_to_f64(wu[e]), numerics.bf16_to_f64(wd[e]))
        return cache[e]
    for e in range(E):
        expert(e)                                           # decode the weights outside the timed part
    t0 = time.perf_counter()
    ffn.moe_output(numerics.bf16_to_f64(xb[:rows]), ids, w, expert)
    el = time.perf_counter() - t0
    fl = 6.0 * H * I * rows * k
    return dict(value=fl / el / 1e9, unit="GFLOP/s", rows=rows, seconds=el, us_per_token=el / rows * 1e6,
                sample="first %d tokens of the prefill BF16 chunk, float64 FFN of their %d picks" % (rows, k))


def cpu_baseline(budget_s):
    """The oracle, as it stands, on the decode trace: route, LRU cache step and
    the exact FFN of every pick, layer call after layer call from a cold cache,
    until `budget_s` of CPU time is spent."""
    from harness import gen, CONFIGS
    from oracle import route, lru, ffn, numerics
    c = CONFIGS["decode_bf16"]
    L, E, k, H, I = c.L, c.E, c.k, c.H, c.I
    S = 3 * H * I * 2
    n_steps = 8
    picks, logits = gen.decode_trace(c.cfg_id, L, n_steps, E, k, c.p_keep)
    wg, wu, wd = gen.bank_bf16(c.cfg_id, E, H, I, c.w_std)
    x = gen.activations_bf16(gen.np_rng(c.cfg_id, gen.S_ACT), n_steps * L, H).reshape(n_steps, L, 1, H)

    def expert(lid):
        be = gen.alias_base_expert(lid // E, lid % E, E, c.alias_stride)
        return numerics.bf16_to_f64(wg[be]), numerics.bf16_to_f64(wu[be]), numerics.bf16_to_f64(wd[be])

    cache = lru.ExpertCache(L, E, c.C, c.bp, c.bh)
    done, nbytes = 0, 0
    t0 = time.perf_counter()
    for s in range(n_steps):
        for l in range(L):
            ids, w = route.topk_softmax(logits[s, l], k)
            r = cache.step(l, ids)
            ffn.moe_partials(numerics.bf16_to_f64(x[s, l]), ids + l * E, w, expert, on_gpu=r.pick_slot >= 0)
            done += 1
            nbytes += len(r.uniq) * S
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    return dict(value=nbytes / el / 1e9, unit="GB/s", cores=int(threads), kind="oracle",
                sample="first %d layer calls of the decode BF16 trace from a cold cache (route + LRU step + "
                       "float64 FFN of every routed expert, GPU and host sets); bytes = distinct experts "
                       "evaluated x 9437184 B; %.1f s; host has %d cores available"
                       % (done, el, len(os.sched_getaffinity(0))))


def run_host_exec(b, seconds=3.0):
    """Throughput of the host executor (moe_host_forward) on this machine's cores:
    the B_H of the q* split.  Each call evaluates k = 8 host picks of one token,
    each a different expert, cycling through a pinned pool larger than the CPU
    caches, so the weights stream from host DRAM as the host set's do.  The
    weights are random values in the packed layout (the rate does not depend
    on them); parity is covered by the tests."""
    import torch
    threads = len(os.sched_getaffinity(0))
    ex = b.HostExec(threads)
    out = dict(threads=threads, simd=ex.simd(), picks_per_call=8)
    for name, wtype, H, I, n_pool in (("decode_bf16", b.W_BF16, 2048, 768, 64),
                                      ("decode_fp8", b.W_FP8_B128, 7168, 2048, 24)):
        el = 2 if wtype == b.W_BF16 else 1
        if wtype == b.W_BF16:
            gu = (torch.randn((n_pool, 2 * I * H)) * 0.02).to(torch.bfloat16).view(torch.uint16).pin_memory()
            dp = (torch.randn((n_pool, H * I)) * 0.02).to(torch.bfloat16).view(torch.uint16).pin_memory()
            banks = [gu, dp]
        else:
            gu = torch.randint(0, 0x7F, (n_pool, 2 * I * H), dtype=torch.uint8).pin_memory()   # no NaN codes
            dp = torch.randint(0, 0x7F, (n_pool, H * I), dtype=torch.uint8).pin_memory()
            sg = (torch.rand((n_pool, I // 128, H // 128)) * 1e-3).pin_memory()
            su = (torch.rand((n_pool, I // 128, H // 128)) * 1e-3).pin_memory()
            sd = (torch.rand((n_pool, H // 128, I // 128)) * 1e-3).pin_memory()
            banks = [gu, dp, sg, su, sd]
        pool = b.HostPoolTables(banks, lambda i: i, n_pool)
        expert_bytes = 3 * H * I * el + (3 * (I // 128) * (H // 128) * 4 if wtype != b.W_BF16 else 0)
        x = (torch.randn((1, H))).to(torch.bfloat16).view(torch.uint16)
        w = torch.full((1, 8), 0.125, dtype=torch.float32)
        pick = torch.full((1, 8), -1, dtype=torch.int32)
        y = torch.empty((1, H), dtype=torch.float32)
        call = 0

        def one(ids):
            ex.forward(pool, wtype, H, I, x, ids, pick, w, y)

        def ids_of(c):
            return torch.tensor([[(8 * c + j) % n_pool for j in range(8)]], dtype=torch.int32)

        for c in range(3):
            one(ids_of(c))
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < seconds:
            one(ids_of(call))
            call += 1
            n += 1
        dt = time.perf_counter() - t0
        one1 = torch.tensor([[call % n_pool] + [0] * 7], dtype=torch.int32)
        pick1 = torch.tensor([[-1] + [5] * 7], dtype=torch.int32)
        t1 = time.perf_counter()
        for r in range(10):
            one1[0, 0] = (call + 8 * r) % n_pool
            ex.forward(pool, wtype, H, I, x, one1, pick1, w, y)
        lat = (time.perf_counter() - t1) / 10
        out[name] = dict(expert_bytes=expert_bytes, calls=n, GBps=8 * n * expert_bytes / dt / 1e9,
                         ms_per_call_8_experts=dt / n * 1e3, ms_one_expert=lat * 1e3,
                         pool_GB=n_pool * expert_bytes / 1e9)
        del banks, pool, gu, dp
    ex.destroy()
    return out


def main():
    a = parse()
    if a.pmc_summary:
        pmc_summary(*a.pmc_summary)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the expert-slot cache path runs on a single MI355X "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import routed_expert_cache_amd.binding as b
    assert torch.cuda.is_available(), "needs a GPU"
    if a.calibrate_copy:
        calibrate_copy()
    if a.only_fp8:
        line = {"metric": METRIC, "value": None, "unit": "GB/s", "n_gpus": 1, "data": "synthetic",
                "note": "FP8 runs only (counter collection); not a headline line"}
        line["decode_fp8"] = run_decode_fp8(b, a.fp8_steps, a.fp8_warmup)
        torch.cuda.empty_cache()
        if not a.no_prefill_fp8:
            line["prefill_fp8"] = run_prefill_fp8(b)
        print(json.dumps(line), flush=True)
        return
    host_exec = None
    if not a.no_host_exec:
        log("host executor: expert GB/s on %d cores" % len(os.sched_getaffinity(0)))
        host_exec = run_host_exec(b)
    dec = run_decode(b, a.steps, a.warmup, host_exec["decode_bf16"]["GBps"] if host_exec else None,
                     host_branch=not a.no_host_branch)
    if host_exec:
        fr = dec["detail"].get("fill_GBps")
        if fr:
            host_exec["fill_GBps"] = fr
            host_exec["B_P_over_B_H_measured"] = {k: fr / host_exec[k]["GBps"] for k in ("decode_bf16", "decode_fp8")}
    line = {
        "metric": METRIC, "value": round(dec["value"], 2), "unit": "GB/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(dec["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_bf16: batch 1, 40 MoE layers x sticky trace (keep 0.6), hidden 2048, "
                               "128 experts, top-8, SwiGLU I 768, BF16, shared LRU cache 1894 slots (37%), "
                               "B_P:B_H 52.7:77.3; one step = one token through 40 layers",
                   "trace_steps": [a.warmup, a.warmup + a.steps]},
        "roofline": dec["roofline"],
        "decode": dec["detail"],
    }
    if not a.no_prefill:
        line["prefill"] = run_prefill(b, a.prefill_reps)
    if not a.no_fp8:
        line["decode_fp8"] = run_decode_fp8(b, a.fp8_steps, a.fp8_warmup)
        torch.cuda.empty_cache()
        if not a.no_prefill and not a.no_prefill_fp8:
            line["prefill_fp8"] = run_prefill_fp8(b)
            torch.cuda.empty_cache()
    if not a.no_resize:
        log("resize: shrink and grow of the decode cache")
        line["resize"] = run_resize(b)
    if host_exec:
        line["host_exec"] = host_exec
    if not a.no_cpu_baseline:
        log("cpu baseline: oracle for %.0f s" % a.cpu_seconds)
        line["cpu_baseline"] = cpu_baseline(a.cpu_seconds)
        if a.cpu_prefill:
            line["cpu_baseline"]["prefill_bf16"] = cpu_prefill_oracle(a.cpu_prefill)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
