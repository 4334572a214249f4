"""The decode layer with its host branch: the cache step on the GPU, the host
set evaluated by the host executor on a side stream (moe_host_forward_enqueue)
while the GPU evaluates G, then the merge.  The layer output is checked
against the float64 oracle over a run of steps; a captured graph holding the
host function node replays to the eager bits."""
import numpy as np
import pytest
import torch

from oracle import ffn, numerics, route
from tests.layer_setup import binding, dev, check_layer, Bf16Bank
from harness import gen

pytestmark = pytest.mark.gpu


def _setup(b, E, H, I, k, T, C, cfg):
    bank = Bf16Bank(cfg, E, H, I)
    pool = b.SlotPool(C, H, I, b.W_BF16)
    host = b.HostPoolTables(bank.host, lambda i: i, E)
    cache = b.Cache(1, E, k, T, pool, host, 118, 475)   # B_P:B_H 11.8:47.5: most misses stay on the host
    return bank, pool, host, cache


def test_decode_steps_with_host_branch():
    b = binding()
    E, H, I, k, T, C, steps = 16, 256, 128, 4, 3, 6, 12
    bank, pool, host, cache = _setup(b, E, H, I, k, T, C, 81)
    ex = b.HostExec(4)
    out = b.StepOut(T, k, E)
    ws = b.forward_workspace(T, k, H, I, C, b.FWD_DECODE)
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    # pinned host copies the executor reads, and its output the merge reads
    h_ids = torch.empty((T, k), dtype=torch.int32).pin_memory()
    h_pick = torch.empty((T, k), dtype=torch.int32).pin_memory()
    h_w = torch.empty((T, k), dtype=torch.float32).pin_memory()
    h_x = torch.empty((T, H), dtype=torch.uint16).pin_memory()
    h_y = torch.empty((T, H), dtype=torch.float32).pin_memory()
    ids_d = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w_d = torch.empty((T, k), dtype=torch.float32, device="cuda")
    rng = np.random.default_rng(5)
    n_host = 0
    for s in range(steps):
        x = gen.activations_bf16(rng, T, H)
        lg = rng.standard_normal((T, E)).astype(np.float32)
        x_d, lg_d = dev(x), dev(lg)
        cache.route_step(0, lg_d, ids_d, w_d, out, copy=True)
        pick_d = out.pick_slot.view(T, k)
        for hd, d in ((h_ids, ids_d), (h_pick, pick_d), (h_w, w_d), (h_x, x_d)):
            hd.copy_(d, non_blocking=True)
        ev_in = torch.cuda.Event()
        ev_in.record(main)
        side.wait_event(ev_in)
        ex.enqueue(host, b.W_BF16, H, I, h_x, h_ids, h_pick, h_w, h_y, stream=side)
        ev_host = torch.cuda.Event()
        ev_host.record(side)
        y_gpu = b.expert_forward(pool.c, x_d, pick_d, w_d, b.FWD_DECODE, ws)   # overlaps the host branch
        main.wait_event(ev_host)
        y = b.merge_partial(y_gpu, h_y)
        torch.cuda.synchronize()
        assert ex.status() == 0
        ids, w = route.topk_softmax(lg, k)
        assert np.array_equal(ids_d.cpu().numpy(), ids)
        n_host += int((h_pick.numpy() < 0).sum())
        ref = ffn.moe_output(numerics.bf16_to_f64(x), ids, w, bank.expert64)
        check_layer(y.cpu().numpy(), ref, "step %d" % s)
    assert n_host > 0, "the run never left an expert to the host"
    ex.destroy()
    cache.destroy()


def test_host_node_in_captured_graph():
    b = binding()
    E, H, I, k, T = 8, 256, 128, 2, 4
    bank = Bf16Bank(82, E, H, I)
    host = b.HostPoolTables(bank.host, lambda i: i, E)
    ex = b.HostExec(3)
    rng = np.random.default_rng(6)
    x = gen.activations_bf16(rng, T, H)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    pick = np.full((T, k), -1, np.int32)
    h_in = [torch.from_numpy(a).pin_memory() for a in (x, ids, pick, w)]
    h_y = torch.zeros((T, H), dtype=torch.float32).pin_memory()
    y_d = torch.empty((T, H), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    ex.enqueue(host, b.W_BF16, H, I, *h_in, h_y, stream=s)
    s.synchronize()
    eager = h_y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ex.enqueue(host, b.W_BF16, H, I, *h_in, h_y, stream=s)
        y_d.copy_(h_y, non_blocking=True)
    for rep in range(3):
        h_y.zero_()
        y_d.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h_y.view(torch.int32), eager.view(torch.int32)), rep
        assert torch.equal(y_d.cpu().view(torch.int32), eager.view(torch.int32)), rep
    assert ex.status() == 0
    _, ref = ffn.moe_partials(numerics.bf16_to_f64(x), ids, w, bank.expert64, on_gpu=np.zeros((T, k), bool))
    check_layer(eager.numpy(), ref, "host branch")
    ex.destroy()


def test_decode_steps_with_signalled_host_branch():
    """The same decode steps with the host branch handed over through pinned
    words (moe_host_signal, moe_host_forward_signal, moe_merge_partial_after)
    instead of a stream host function."""
    b = binding()
    E, H, I, k, T, C, steps = 16, 256, 128, 4, 3, 6, 12
    bank, pool, host, cache = _setup(b, E, H, I, k, T, C, 83)
    ex = b.HostExec(4)
    out = b.StepOut(T, k, E)
    ws = b.forward_workspace(T, k, H, I, C, b.FWD_DECODE)
    h_ids = torch.empty((T, k), dtype=torch.int32).pin_memory()
    h_pick = torch.empty((T, k), dtype=torch.int32).pin_memory()
    h_w = torch.empty((T, k), dtype=torch.float32).pin_memory()
    h_x = torch.empty((T, H), dtype=torch.uint16).pin_memory()
    h_y = torch.empty((T, H), dtype=torch.float32).pin_memory()
    ready = torch.zeros(1, dtype=torch.int32).pin_memory()
    done = torch.zeros(1, dtype=torch.int32).pin_memory()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ids_d = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w_d = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y_gpu = torch.empty((T, H), dtype=torch.float32, device="cuda")
    rng = np.random.default_rng(7)
    xs, lgs, ys = [], [], []
    for s in range(steps):                       # launched back to back: one sync at the end
        x = gen.activations_bf16(rng, T, H)
        lg = rng.standard_normal((T, E)).astype(np.float32)
        xs.append(x)
        lgs.append(lg)
        x_d, lg_d = dev(x), dev(lg)
        cache.route_step(0, lg_d, ids_d, w_d, out, copy=True)
        pick_d = out.pick_slot.view(T, k)
        for hd, d in ((h_ids, ids_d), (h_pick, pick_d), (h_w, w_d), (h_x, x_d)):
            hd.copy_(d, non_blocking=True)
        b.host_signal(ready, s + 1)
        ex.forward_signal(host, b.W_BF16, H, I, h_x, h_ids, h_pick, h_w, h_y, ready, done, s + 1)
        b.expert_forward(pool.c, x_d, pick_d, w_d, b.FWD_DECODE, ws, y=y_gpu)
        ys.append(b.merge_partial_after(y_gpu, h_y, done, s + 1, err=err))
        del x_d, lg_d
    torch.cuda.synchronize()
    assert int(err.item()) == 0 and ex.status() == 0 and int(done[0]) == steps
    for s in range(steps):
        ids, w = route.topk_softmax(lgs[s], k)
        ref = ffn.moe_output(numerics.bf16_to_f64(xs[s]), ids, w, bank.expert64)
        check_layer(ys[s].cpu().numpy(), ref, "step %d" % s)
    ex.destroy()
    cache.destroy()
