"""GPU tests of the full-layer double buffer, hipGraph capture of a decode
step, and run-to-run determinism."""
import numpy as np
import pytest
import torch

from harness import gen
from oracle import route, lru, numerics, ffn
from tests.layer_setup import binding, dev, pinned, check_layer, oracle_partials, pack_to_host

pytestmark = pytest.mark.gpu


def _layer_banks(L, E, H, I, cfg_id=55):
    """Host pool of L layers x E experts (distinct draws) as pinned [L*E, ...]."""
    rng = gen.np_rng(cfg_id, gen.S_WEIGHTS)
    wg = np.empty((L * E, I, H), np.uint16)
    wu = np.empty((L * E, I, H), np.uint16)
    wd = np.empty((L * E, H, I), np.uint16)
    for i in range(L * E):
        wg[i], wu[i], wd[i] = gen.expert_bf16(rng, H, I, 0.02)
    packed = pack_to_host(0, *[torch.from_numpy(a) for a in (wg, wu, wd)])
    return (wg, wu, wd), list(packed)


def test_prefill_double_buffer_overlap():
    b = binding()
    L, E, H, I, T, k = 4, 8, 256, 128, 200, 2
    arrs, host_t = _layer_banks(L, E, H, I)
    expert64 = lambda lid: tuple(numerics.bf16_to_f64(a[lid]) for a in arrs)
    C = 2 * E + 3
    pool = b.SlotPool(C, H, I, b.W_BF16)
    host = b.HostPoolTables(host_t, lambda i: i, L * E)
    cache = b.Cache(L, E, k, 1, pool, host, 527, 773)
    pf = b.PrefillPool(cache)
    slot_id = cache.read_state()[0]
    assert np.all(slot_id[C - 2 * E:] == -2) and np.all(slot_id[:C - 2 * E] == -1)

    compute = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    rng = np.random.default_rng(0)
    xs = [gen.activations_bf16(rng, T, H) for _ in range(L)]
    routes = [route.topk_softmax(rng.standard_normal((T, E)).astype(np.float32), k) for _ in range(L)]
    ws = b.forward_workspace(T, k, H, I, E, b.FWD_PREFILL)
    big = torch.randn(2048, 2048, device="cuda")
    outs = []
    pf.prefetch(0, copy)
    pf.prefetch(1, copy)
    for l in range(L):
        view = pf.acquire(l, compute)
        for _ in range(20):                        # delay the compute stream
            big = torch.tanh(big @ big * 1e-3)
        ids, w = routes[l]
        y = b.expert_forward(view, dev(xs[l]), dev(ids.astype(np.int32)), dev(w.astype(np.float32)),
                             b.FWD_PREFILL, ws)
        outs.append(y)
        pf.release(l, compute)
        if l + 2 < L:
            pf.prefetch(l + 2, copy)
    torch.cuda.synchronize()
    for l in range(L):
        ids, w = routes[l]
        ref = ffn.moe_output(numerics.bf16_to_f64(xs[l]), ids + l * E, w, expert64)
        check_layer(outs[l].cpu().numpy(), ref, "layer %d" % l)
    # the buffers hold layers 2 and 3 byte for byte
    for l in (2, 3):
        v = pf.acquire(l, compute)
        base = C - 2 * E + (l % 2) * E
        for e in range(E):
            assert torch.equal(pool.w_gu[base + e].cpu(), host_t[0][l * E + e])
            assert torch.equal(pool.w_down[base + e].cpu(), host_t[1][l * E + e])
    pf.destroy()
    assert np.all(cache.read_state()[0][C - 2 * E:] == -1)
    cache.destroy()


def test_prefill_pool_errors():
    b = binding()
    H, I, E = 64, 32, 8
    arrs, host_t = _layer_banks(2, E, H, I, cfg_id=56)
    pool = b.SlotPool(2 * E - 1, H, I, b.W_BF16)
    cache = b.Cache(2, E, 2, 1, pool, b.HostPoolTables(host_t, lambda i: i, 2 * E), 527, 773)
    with pytest.raises(b.MoeError) as ei:
        b.PrefillPool(cache)
    assert ei.value.status == -3                  # MOE_ERR_NO_SPACE
    pool2 = b.SlotPool(2 * E, H, I, b.W_BF16)
    cache2 = b.Cache(2, E, 2, 1, pool2, b.HostPoolTables(host_t, lambda i: i, 2 * E), 527, 773)
    pf = b.PrefillPool(cache2)
    with pytest.raises(b.MoeError) as ei:
        pf.acquire(1)
    assert ei.value.status == -6                  # MOE_ERR_STATE
    # a buffer is overwritten only after the layer it holds was released
    copy = torch.cuda.Stream()
    pf.prefetch(0, copy)
    with pytest.raises(b.MoeError) as ei:
        pf.prefetch(0, copy)                      # layer 0 still holds buffer 0
    assert ei.value.status == -6
    pf.acquire(0)
    with pytest.raises(b.MoeError) as ei:
        pf.prefetch(0, copy)                      # acquired, not released
    assert ei.value.status == -6
    pf.release(0)
    pf.prefetch(0, copy)                          # released: the buffer may be loaded again
    pf.prefetch(1, copy)                          # the other buffer is empty
    with pytest.raises(b.MoeError) as ei:
        pf.prefetch(1, copy)
    assert ei.value.status == -6
    torch.cuda.synchronize()
    pf.destroy()


def _decode_setup(b, seed=1):
    L, E, k, H, I, C = 3, 16, 4, 256, 128, 10
    arrs, host_t = _layer_banks(L, E, H, I, cfg_id=57)
    pool = b.SlotPool(C, H, I, b.W_BF16)
    cache = b.Cache(L, E, k, 1, pool, b.HostPoolTables(host_t, lambda i: i, L * E), 527, 773)
    return dict(L=L, E=E, k=k, H=H, I=I, C=C, arrs=arrs, pool=pool, cache=cache, host_t=host_t)


def test_graph_capture_replays_equal_eager():
    """One decode layer step (route, cache step with fills, grouped GEMV,
    merge) captured once and replayed across steps equals eager execution."""
    b = binding()
    A = _decode_setup(b)
    B = _decode_setup(b)
    L, E, k, H = A["L"], A["E"], A["k"], A["H"]
    steps = 12
    rng = np.random.default_rng(3)
    picks = [np.stack([gen.sticky_trace(gen.np_rng(9, 3, l), steps, E, k, 0.5)[s] for l in range(L)]) for s in range(steps)]
    logits = np.zeros((steps, L, 1, E), np.float32)
    for s in range(steps):
        for l in range(L):
            logits[s, l] = gen.synth_logits(rng, picks[s][l][None], E)
    xs = rng.standard_normal((steps, L, 1, H)).astype(np.float32)
    xs = gen.to_bf16_bits(xs)
    yh = rng.standard_normal((steps, L, 1, H)).astype(np.float32)

    def make_bufs():
        return dict(lg=torch.zeros((1, E), dtype=torch.float32, device="cuda"),
                    x=torch.zeros((1, H), dtype=torch.uint16, device="cuda"),
                    yh=torch.zeros((1, H), dtype=torch.float32, device="cuda"),
                    ids=torch.zeros((1, k), dtype=torch.int32, device="cuda"),
                    w=torch.zeros((1, k), dtype=torch.float32, device="cuda"),
                    out=b.StepOut(1, k, E),
                    ws=b.forward_workspace(1, k, H, A["I"], A["C"], b.FWD_DECODE),
                    yg=torch.zeros((1, H), dtype=torch.float32, device="cuda"),
                    y=torch.zeros((1, H), dtype=torch.float32, device="cuda"))

    def layer_step(S, bufs, layer):
        b.route_topk(bufs["lg"], k, bufs["ids"], bufs["w"])
        S["cache"].step(layer, bufs["ids"], bufs["out"])
        b.expert_forward(S["pool"].c, bufs["x"], bufs["out"].pick_slot.view(1, k), bufs["w"], b.FWD_DECODE,
                         bufs["ws"], y=bufs["yg"])
        b.merge_partial(bufs["yg"], bufs["yh"], y_out=bufs["y"])

    ea = [make_bufs() for _ in range(L)]
    gb = [make_bufs() for _ in range(L)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graphs = []
    # warm-up outside capture is not needed by the library; capture one graph per layer
    with torch.cuda.stream(s):
        for l in range(L):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                layer_step(B, gb[l], l)
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    # capture must not have executed anything: B's cache is still empty
    assert np.all(B["cache"].read_state()[0] == -1)
    for st in range(steps):
        for l in range(L):
            for bufs in (ea[l], gb[l]):
                bufs["lg"].copy_(torch.from_numpy(logits[st, l]))
                bufs["x"].copy_(torch.from_numpy(xs[st, l]))
                bufs["yh"].copy_(torch.from_numpy(yh[st, l]))
            layer_step(A, ea[l], l)
            graphs[l].replay()
            torch.cuda.synchronize()
            for key in ("ids", "w", "yg", "y"):
                assert torch.equal(ea[l][key], gb[l][key]), (st, l, key)
            assert torch.equal(ea[l]["out"].pick_slot, gb[l]["out"].pick_slot)
            assert torch.equal(ea[l]["out"].counts, gb[l]["out"].counts)
    sa, sb = A["cache"].read_state(), B["cache"].read_state()
    for u, v in zip(sa[:3], sb[:3]):
        assert np.array_equal(u, v)
    assert torch.equal(A["pool"].w_gu, B["pool"].w_gu)


def test_forward_deterministic():
    b = binding()
    S = _decode_setup(b)
    pool = S["pool"]
    for s in range(pool.n_slots):
        for t in pool.banks():
            t[s].copy_(torch.randint(0, 1 << 14, t[s].shape, dtype=torch.int32).to(t.dtype))
    rng = np.random.default_rng(8)
    for mode, T in ((b.FWD_DECODE, 16), (b.FWD_PREFILL, 500)):
        x = dev(gen.activations_bf16(rng, T, S["H"]))
        ids = dev(np.stack([rng.choice(pool.n_slots, 4, replace=False) for _ in range(T)]).astype(np.int32))
        w = dev(rng.random((T, 4)).astype(np.float32))
        ws = b.forward_workspace(T, 4, S["H"], S["I"], pool.n_slots, mode)
        y1 = b.expert_forward(pool.c, x, ids, w, mode, ws).clone()
        y2 = b.expert_forward(pool.c, x, ids, w, mode, ws)
        assert torch.equal(y1, y2)


def test_one_graph_serves_every_layer():
    """The layer index is a device scalar, so ONE captured graph of a layer
    call (route + cache step with fills, grouped evaluation, merge) serves
    every layer: before each replay the layer scalar and the inputs are
    written, and the replays equal eager calls of the same layers bit for
    bit (ids, weights, picks, counts, y, tables and slot bytes).  Eager work
    and synchronisations run between the replays."""
    b = binding()
    A = _decode_setup(b)
    B = _decode_setup(b)
    L, E, k, H = A["L"], A["E"], A["k"], A["H"]
    steps = 10
    rng = np.random.default_rng(5)
    picks = [np.stack([gen.sticky_trace(gen.np_rng(9, 3, l), steps, E, k, 0.5)[s] for l in range(L)])
             for s in range(steps)]
    logits = np.zeros((steps, L, 1, E), np.float32)
    for s in range(steps):
        for l in range(L):
            logits[s, l] = gen.synth_logits(rng, picks[s][l][None], E)
    xs = gen.to_bf16_bits(rng.standard_normal((steps, L, 1, H)).astype(np.float32))
    yh = rng.standard_normal((steps, L, 1, H)).astype(np.float32)

    def make_bufs():
        return dict(layer=torch.zeros(1, dtype=torch.int32, device="cuda"),
                    lg=torch.zeros((1, E), dtype=torch.float32, device="cuda"),
                    x=torch.zeros((1, H), dtype=torch.uint16, device="cuda"),
                    yh=torch.zeros((1, H), dtype=torch.float32, device="cuda"),
                    ids=torch.zeros((1, k), dtype=torch.int32, device="cuda"),
                    w=torch.zeros((1, k), dtype=torch.float32, device="cuda"),
                    out=b.StepOut(1, k, E),
                    ws=b.forward_workspace(1, k, H, A["I"], A["C"], b.FWD_DECODE),
                    y=torch.zeros((1, H), dtype=torch.float32, device="cuda"))

    def layer_call(S, bufs):
        S["cache"].route_step(bufs["layer"], bufs["lg"], bufs["ids"], bufs["w"], bufs["out"], copy=True)
        b.expert_forward_merge(S["pool"].c, bufs["x"], bufs["out"].pick_slot.view(1, k), bufs["w"], b.FWD_DECODE,
                               bufs["ws"], bufs["yh"], y_out=bufs["y"])

    ea, gb = make_bufs(), make_bufs()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            layer_call(B, gb)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert np.all(B["cache"].read_state()[0] == -1)       # capture ran nothing
    for st in range(steps):
        for l in range(L):
            for bufs in (ea, gb):
                bufs["layer"].fill_(l)
                bufs["lg"].copy_(torch.from_numpy(logits[st, l]))
                bufs["x"].copy_(torch.from_numpy(xs[st, l]))
                bufs["yh"].copy_(torch.from_numpy(yh[st, l]))
            layer_call(A, ea)
            g.replay()
            torch.cuda.synchronize()
            for key in ("ids", "w", "y"):
                assert torch.equal(ea[key], gb[key]), (st, l, key)
            assert torch.equal(ea["out"].pick_slot, gb["out"].pick_slot)
            assert torch.equal(ea["out"].counts, gb["out"].counts)
            assert int(gb["out"].counts[6].item()) == l
    sa, sb = A["cache"].read_state(), B["cache"].read_state()
    for u, v in zip(sa[:3], sb[:3]):
        assert np.array_equal(u, v)
    assert sa[3] == sb[3] == 1 + steps * L
    assert torch.equal(A["pool"].w_gu, B["pool"].w_gu) and torch.equal(A["pool"].w_down, B["pool"].w_down)
    assert A["cache"].error() == 0 and B["cache"].error() == 0
