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
  measured with HIP events and reported separately (decode.* fields).
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
METRIC = "decode MoE-layer expert GB/s (%HBM peak); prefill MoE TFLOP/s (%MFMA peak)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=192)
    p.add_argument("--warmup", type=int, default=64)
    p.add_argument("--prefill-reps", type=int, default=10)
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true")
    return p.parse_args()


# ---------------------------------------------------------------- decode trace
def run_decode(b, K, W):
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
    cache = b.Cache(L, E, k, 1, pool, host, c.bp, c.bh)
    x = torch.from_numpy(gen.activations_bf16(gen.np_rng(c.cfg_id, gen.S_ACT), n * L, H)).cuda().view(n, L, 1, H)
    lg = torch.from_numpy(logits).cuda()                # [n, L, 1, E]
    # host partial sums are inputs of the merge (the host branch is not on this path)
    yh = torch.randn((L, 1, H), dtype=torch.float32, device="cuda") * 0.01
    ids = torch.empty((1, k), dtype=torch.int32, device="cuda")
    w = torch.empty((1, k), dtype=torch.float32, device="cuda")
    out = b.StepOut(1, k, E)
    ws = b.forward_workspace(1, k, H, I, C, b.FWD_DECODE)
    yg = torch.empty((1, H), dtype=torch.float32, device="cuda")
    y = torch.empty((L, 1, H), dtype=torch.float32, device="cuda")
    pick = out.pick_slot.view(1, k)

    def layer_step(s, l, ev=None):
        b.route_topk(lg[s, l], k, ids, w)
        cache.step(l, ids, out, copy=False)
        if ev:
            ev[0].record()
        cache.fill(out)
        if ev:
            ev[1].record()
        b.expert_forward(pool.c, x[s, l], pick, w, b.FWD_DECODE, ws, y=yg)
        if ev:
            ev[2].record()
        b.merge_partial(yg, yh[l], y_out=y[l])

    log("decode: warmup %d steps" % W)
    for s in range(W):
        for l in range(L):
            layer_step(s, l)
    torch.cuda.synchronize()
    c0 = cache.read_state()[4].astype(np.int64)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K * L)]
    log("decode: timing %d steps" % K)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    for s in range(W, W + K):
        for l in range(L):
            layer_step(s, l, evs[i])
            i += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    c1 = cache.read_state()[4].astype(np.int64)
    d = c1 - c0                                          # calls, uniq, hits, misses, fills, host
    fill_s = sum(e[0].elapsed_time(e[1]) for e in evs) / 1e3
    fwd_s = sum(e[1].elapsed_time(e[2]) for e in evs) / 1e3
    n_g = int(d[2] + d[4])
    gpu_bytes = n_g * S
    hbm_s = wall - fill_s
    res = dict(
        value=gpu_bytes / hbm_s / 1e9,
        ms_per_step=hbm_s / K * 1e3,
        roofline=dict(kernel="moe_expert_forward decode (grouped GEMV: plan + gate/up + down launches)",
                      bound="hbm", achieved=gpu_bytes / fwd_s / 1e9, peak=PEAK_HBM_GBPS, unit="GB/s",
                      bytes_per_launch=gpu_bytes / (K * L), launches=K * L,
                      avg_launch_us=fwd_s / (K * L) * 1e6, traffic=None),
        detail=dict(
            wall_ms_per_step_pcie_inclusive=wall / K * 1e3,
            pcie_inclusive_GBps=gpu_bytes / wall / 1e9,
            fill_ms_per_step=fill_s / K * 1e3,
            fill_GBps=(d[4] * S / fill_s / 1e9) if fill_s > 0 else None,
            miss_rate=float(d[3] / d[1]),
            experts_on_gpu_per_layer_call=n_g / (K * L),
            fills_per_layer_call=float(d[4] / (K * L)),
            host_experts_per_layer_call=float(d[5] / (K * L)),
            layer_calls=int(d[0]),
        ),
    )
    res["roofline"]["frac"] = res["roofline"]["achieved"] / PEAK_HBM_GBPS
    cache.destroy()
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

    def run(ev=None):
        if ev:
            ev[0].record()
        b.route_topk(lg, k, ids, w)
        if ev:
            ev[1].record()
        b.expert_forward(pool.c, x, ids, w, b.FWD_PREFILL, ws, y=y)
        if ev:
            ev[2].record()

    for _ in range(3):
        run()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r in range(reps):
        run(evs[r])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_s = sum(e[1].elapsed_time(e[2]) for e in evs) / 1e3 / reps
    layer_s = sum(e[0].elapsed_time(e[2]) for e in evs) / 1e3 / reps
    ach = flops / fwd_s / 1e12
    return dict(
        workload="prefill_bf16: 8192 tokens, hidden 2048, 128 experts, top-8 of x.W_r, SwiGLU I 768, BF16, all experts resident",
        value=flops / layer_s / 1e12, unit="TFLOP/s", ms_per_layer=layer_s * 1e3, wall_ms_per_rep=wall / reps * 1e3,
        reps=reps, flops_per_layer=flops,
        roofline=dict(kernel="moe_expert_forward prefill (sort + gate/up GEMM + down GEMM + combine)",
                      bound="mfma", achieved=ach, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                      frac=ach / PEAK_BF16_TFLOPS, avg_launch_us=fwd_s * 1e6, traffic=None),
    )


# ---------------------------------------------------------------- CPU oracle baseline
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


def main():
    a = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the expert-slot cache path runs on a single MI355X "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import routed_expert_cache_amd.binding as b
    assert torch.cuda.is_available(), "needs a GPU"
    dec = run_decode(b, a.steps, a.warmup)
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
    if not a.no_cpu_baseline:
        log("cpu baseline: oracle for %.0f s" % a.cpu_seconds)
        line["cpu_baseline"] = cpu_baseline(a.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
