"""Full-shape parity along the workloads' own traces, in the launch
configuration the benchmark times: every step of the path runs through the C
ABI (router + cache decision in one launch, the fused fill copy of real
bytes, the grouped evaluation with the merge), and every layer output is
compared with the float64 oracle's on the same inputs.

* decode BF16 (40 layers, 128 experts, top-8, H 2048, I 768, 1894 slots,
  52.7:77.3): 3 trace steps x 40 layers from a cold cache, y on every call;
* decode FP8 (58-layer pool, 256 experts, H 7168, I 2048, 1633 slots,
  11.8:47.5) at T = 4 and 16: 2 trace steps, every token of layer 0's GPU
  partial sum;
* prefill FP8 (8192 tokens, 256 experts, H 7168, I 2048): one layer loaded
  through the full-layer double buffer (prefetch on a copy stream, acquire
  on the compute stream), the last 32 tokens checked.
"""
import numpy as np
import pytest
import torch

from harness import gen, CONFIGS
from oracle import route, lru, numerics, ffn
from tests.layer_setup import binding, dev, check_layer, pack_to_host, W_ABS

pytestmark = pytest.mark.gpu


def _fp8_expert_rowmajor(cfg_id, layer, e, H, I, std):
    """Row-major codes and scales of one FP8 expert, drawn on the GPU from its seed."""
    ex = gen.expert_fp8_torch(gen.torch_seed(cfg_id, gen.S_WEIGHTS, layer, e), H, I, std, device="cuda")
    return {n: v.cpu().numpy() for n, v in ex.items()}


def _fp8_expert64(ex):
    return (numerics.dequant_b128(ex["gate"], ex["s_gate"]), numerics.dequant_b128(ex["up"], ex["s_up"]),
            numerics.dequant_b128(ex["down"], ex["s_down"]))


def _fp8_host_bank(b, cfg_id, layer, experts, H, I, std):
    """Pinned packed banks holding `experts` (row r = experts[r]) of one layer."""
    n = len(experts)
    gu = torch.empty((n, 2 * I * H), dtype=torch.uint8, pin_memory=True)
    dp = torch.empty((n, H * I), dtype=torch.uint8, pin_memory=True)
    sc = [torch.empty((n, I // 128, H // 128), dtype=torch.float32, pin_memory=True),
          torch.empty((n, I // 128, H // 128), dtype=torch.float32, pin_memory=True),
          torch.empty((n, H // 128, I // 128), dtype=torch.float32, pin_memory=True)]
    for r, e in enumerate(experts):
        ex = gen.expert_fp8_torch(gen.torch_seed(cfg_id, gen.S_WEIGHTS, layer, e), H, I, std, device="cuda")
        g, d = b.pack_weights(b.W_FP8_B128, ex["gate"][None], ex["up"][None], ex["down"][None])
        gu[r].copy_(g[0])
        dp[r].copy_(d[0])
        for i, nm in enumerate(("s_gate", "s_up", "s_down")):
            sc[i][r].copy_(ex[nm])
    torch.cuda.synchronize()
    return [gu, dp] + sc


@pytest.mark.timeout(600)
def test_decode_bf16_trace_real_fills_every_layer_call():
    """The decode BF16 workload from a cold cache, 3 trace steps x 40 layers:
    fused router + cache step with the real PCIe fill copies, then the
    grouped evaluation merged with the host partial sum.  Router ids and
    weights, every decision and the tables against the oracle; y_gpu and
    y = y_gpu + y_host against the oracle's float64 partial sums on every one
    of the 120 layer calls; the forward's and the cache's error words clear."""
    b = binding()
    c = CONFIGS["decode_bf16"]
    L, E, k, H, I, C = c.L, c.E, c.k, c.H, c.I, c.C
    steps = 3
    picks, logits = gen.decode_trace(c.cfg_id, L, steps, E, k, c.p_keep)
    wg, wu, wd = gen.bank_bf16(c.cfg_id, E, H, I, c.w_std)
    host_banks = list(pack_to_host(0, *[torch.from_numpy(a) for a in (wg, wu, wd)]))
    base = lambda lid: gen.alias_base_expert(lid // E, lid % E, E, c.alias_stride)
    host = b.HostPoolTables(host_banks, base, L * E)
    pool = b.SlotPool(C, H, I, b.W_BF16)
    cache = b.Cache(L, E, k, 1, pool, host, c.bp, c.bh)
    orc = lru.ExpertCache(L, E, C, c.bp, c.bh)
    x = gen.activations_bf16(gen.np_rng(c.cfg_id, gen.S_ACT), steps * L, H).reshape(steps, L, 1, H)
    ws = b.forward_workspace(1, k, H, I, C, b.FWD_DECODE)
    out = b.StepOut(1, k, E)
    ids_d = torch.empty((1, k), dtype=torch.int32, device="cuda")
    w_d = torch.empty((1, k), dtype=torch.float32, device="cuda")
    yg_d = torch.empty((1, H), dtype=torch.float32, device="cuda")
    x64 = {}

    def expert64(lid):
        e = base(lid)
        if e not in x64:
            x64[e] = tuple(numerics.bf16_to_f64(a[e]) for a in (wg, wu, wd))
        return x64[e]

    fills = hosts = 0
    for s in range(steps):
        for l in range(L):
            cache.route_step(l, dev(logits[s, l]), ids_d, w_d, out, copy=True)
            rid, rw = route.topk_softmax(logits[s, l], k)
            r = orc.step(l, rid)
            assert np.array_equal(ids_d.cpu().numpy(), rid), (s, l)
            assert np.abs(w_d.cpu().numpy() - rw).max() <= W_ABS
            pick = out.pick_slot.view(1, k)
            assert np.array_equal(pick.cpu().numpy(), r.pick_slot), (s, l)
            fills += r.q
            hosts += len(r.misses) - r.q
            yg_ref, yh_ref = ffn.moe_partials(numerics.bf16_to_f64(x[s, l]), rid + l * E, rw, expert64,
                                              on_gpu=r.pick_slot >= 0)
            y = b.expert_forward_merge(pool.c, dev(x[s, l]), pick, w_d, b.FWD_DECODE, ws,
                                       dev(yh_ref.astype(np.float32)), y_gpu=yg_d)
            check_layer(yg_d.cpu().numpy(), yg_ref, "decode bf16 trace y_gpu step %d layer %d" % (s, l))
            check_layer(y.cpu().numpy(), yg_ref + yh_ref, "decode bf16 trace y step %d layer %d" % (s, l))
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 0
    assert cache.error() == 0
    slot_id, stamp, id_slot, tick, _ = cache.read_state()
    rs, rt, ri, rtick = orc.tables()
    assert np.array_equal(slot_id, rs) and np.array_equal(stamp, rt) and np.array_equal(id_slot, ri)
    assert tick == rtick
    assert fills > 0 and hosts > 0                         # both branches of the split ran
    cache.destroy()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", [4, 16])
def test_decode_fp8_trace_every_token(T):
    """The decode FP8 workload at T tokens: 2 steps of its sticky trace over
    the 58-layer pool (layer 0 with real weights and real fill copies,
    layers 1-57 metadata only), as the benchmark runs it.  Every token of
    layer 0's GPU partial sum is compared with the oracle's on both steps;
    decisions are bit-exact on every layer call."""
    b = binding()
    c = CONFIGS["decode_fp8"]
    L, E, k, H, I, C = c.L, c.E, c.k, c.H, c.I, c.C
    steps = 2
    picks, logits = gen.decode_trace(c.cfg_id, L, steps, E, k, c.p_keep, T=T, salt=T)
    # the oracle's decisions first: layer 0's G is made of experts that its own
    # calls filled, so only those need real bytes in the host pool
    orc = lru.ExpertCache(L, E, C, c.bp, c.bh)
    plan = []
    for s in range(steps):
        for l in range(L):
            rid, rw = route.topk_softmax(logits[s, l], k)
            r = orc.step(l, rid)
            plan.append((rid, rw, r))
    filled = sorted({int(f) for s in range(steps) for f in plan[s * L][2].fill_id})
    assert filled and all(f < E for f in filled)
    row_of = {e: i for i, e in enumerate(filled)}
    host_banks = _fp8_host_bank(b, c.cfg_id, 0, filled, H, I, c.w_std)
    # logical ids outside layer 0 never copy (metadata-only layers): row 0 stands in
    host = b.HostPoolTables(host_banks, lambda lid: row_of.get(lid, 0) if lid < E else 0, L * E)
    pool = b.SlotPool(C, H, I, b.W_FP8_B128)
    cache = b.Cache(L, E, k, T, pool, host, c.bp, c.bh)
    out = b.StepOut(T, k, E)
    ids_d = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w_d = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = b.forward_workspace(T, k, H, I, C, b.FWD_DECODE)
    x = gen.activations_bf16(gen.np_rng(c.cfg_id, gen.S_ACT, T), steps * T, H).reshape(steps, T, H)
    x64 = {}
    zero = (np.zeros((I, H)), np.zeros((I, H)), np.zeros((H, I)))
    for s in range(steps):
        for l in range(L):
            rid, rw, r = plan[s * L + l]
            cache.route_step(l, dev(logits[s, l]), ids_d, w_d, out, copy=(l == 0))
            pick = out.pick_slot.view(T, k)
            assert np.array_equal(ids_d.cpu().numpy(), rid), (s, l)
            assert np.array_equal(pick.cpu().numpy(), r.pick_slot), (s, l)
            if l != 0:
                continue
            y = b.expert_forward(pool.c, dev(x[s]), pick, w_d, b.FWD_DECODE, ws).cpu().numpy()
            on_gpu = r.pick_slot >= 0
            gpu_e = set(rid[on_gpu].tolist())
            for e in gpu_e - set(x64):
                x64[e] = _fp8_expert64(_fp8_expert_rowmajor(c.cfg_id, 0, e, H, I, c.w_std))
            # an expert is in G for all of its picks or for none; the host set's
            # partial sum is not compared here, so its experts stand in as zeros
            yg_ref, _ = ffn.moe_partials(numerics.bf16_to_f64(x[s]), rid, rw,
                                         lambda e: x64[e] if e in gpu_e else zero, on_gpu=on_gpu)
            for t in range(T):                             # every token, one by one
                check_layer(y[t:t + 1], yg_ref[t:t + 1], "decode fp8 T=%d step %d token %d" % (T, s, t))
            check_layer(y, yg_ref, "decode fp8 T=%d step %d" % (T, s))
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 0
    assert cache.error() == 0
    cache.destroy()


@pytest.mark.timeout(900)
def test_prefill_fp8_layer_through_double_buffer():
    """One prefill FP8 layer (8192 tokens, 256 experts, top-8 of x.W_r) read
    through the full-layer double buffer: the layer's 256 experts copied by
    moe_prefill_prefetch on a copy stream into the reserved slots, the
    compute stream acquiring the buffer's view, the grouped GEMM over it.
    The last 32 tokens are checked against the oracle: their pairs come last
    in the input order, so the counting sort places them at the ends of
    their experts' segments, in the ragged last M tiles; together they cover
    well over 64 experts.  Every output is finite."""
    b = binding()
    c = CONFIGS["prefill_fp8"]
    E, k, H, I, T = c.E, c.k, c.H, c.I, c.T
    host_banks = _fp8_host_bank(b, c.cfg_id, 0, list(range(E)), H, I, c.w_std)
    L = 2                                                  # layer 1 aliases layer 0's bytes
    host = b.HostPoolTables(host_banks, lambda lid: lid % E, L * E)
    pool = b.SlotPool(2 * E, H, I, b.W_FP8_B128)
    cache = b.Cache(L, E, k, 1, pool, host, 118, 475)
    pf = b.PrefillPool(cache)
    copy_stream = torch.cuda.Stream()
    x = gen.activations_bf16(gen.np_rng(c.cfg_id, gen.S_ACT), T, H)
    wr = gen.router_matrix(gen.np_rng(c.cfg_id, gen.S_ROUTER), H, E, c.router_std)
    lg = gen.router_logits(x, wr)
    ids_d, w_d = b.route_topk(dev(lg), k)
    rid, rw = route.topk_softmax(lg, k)
    assert np.array_equal(ids_d.cpu().numpy(), rid)
    ws = b.forward_workspace(T, k, H, I, E, b.FWD_PREFILL)
    x_d = dev(x)
    pf.prefetch(0, copy_stream)
    pf.prefetch(1, copy_stream)                            # the second buffer loads behind
    view = pf.acquire(0)
    y = b.expert_forward(view, x_d, ids_d, w_d, b.FWD_PREFILL, ws)
    pf.release(0)
    view1 = pf.acquire(1)
    y1 = b.expert_forward(view1, x_d, ids_d, w_d, b.FWD_PREFILL, ws)
    pf.release(1)
    torch.cuda.synchronize()
    y, y1 = y.cpu().numpy(), y1.cpu().numpy()
    assert np.all(np.isfinite(y))
    assert np.array_equal(y.view(np.uint32), y1.view(np.uint32))   # same bytes in the other buffer
    rows = np.arange(T - 32, T)
    assert len(set(rid[rows].reshape(-1).tolist())) >= 64
    cnt = np.bincount(rid.reshape(-1), minlength=E)
    assert np.count_nonzero(cnt[np.unique(rid[rows])] % 64) >= 32   # experts with a ragged last tile

    def expert64(e):
        return _fp8_expert64(_fp8_expert_rowmajor(c.cfg_id, 0, e, H, I, c.w_std))

    ref = ffn.moe_output(numerics.bf16_to_f64(x[rows]), rid[rows], rw[rows], expert64)
    check_layer(y[rows], ref, "prefill fp8 through the double buffer")
    for i, t in enumerate(rows):
        check_layer(y[t:t + 1], ref[i:i + 1], "prefill fp8 row %d" % t)
    pf.destroy()
    cache.destroy()
