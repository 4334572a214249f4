"""GPU tests of the prefill variants around the full-layer buffers: the
buffers' experts seeding the decode cache when prefill ends (moe_prefill_finish),
a ring of more than two buffers, the on-demand loading used when the pool
cannot hold two full layers (moe_cache_prefill_load), and every miss filled on
a decode step (MOE_STEP_FILL_ALL).  Tables, decisions and slot bytes are
compared bit for bit with the oracle cache; layer outputs with the float64
oracle."""
import numpy as np
import pytest
import torch

from harness import gen
from oracle import ffn, lru, numerics, route
from tests.layer_setup import binding, dev, check_layer
from tests.test_gpu_cache import Harness
from tests.test_gpu_pool import _layer_banks

pytestmark = pytest.mark.gpu


def _prefill_layers(pf, depth, L, compute, copy, work=None):
    """Run the layer loop of prefill over a ring of `depth` buffers: prefetch
    depth layers ahead, acquire, optional work on the buffer, release."""
    for l in range(min(depth, L)):
        pf.prefetch(l, copy)
    outs = []
    for l in range(L):
        view = pf.acquire(l, compute)
        if work is not None:
            outs.append(work(l, view))
        pf.release(l, compute)
        if l + depth < L:
            pf.prefetch(l + depth, copy)
    return outs


def _loaded(depth, L):
    """(buffer, layer) held at the end of the loop, least recently loaded first."""
    return [(l % depth, l) for l in range(max(0, L - depth), L)]


@pytest.mark.parametrize("depth,L,pre", [(2, 5, (35, 2, 9)), (3, 5, (27, 33, 14, 1)), (2, 1, (3,)), (4, 3, ())])
def test_finish_seeds_decode_tables(depth, L, pre):
    """Tables after the hand-over equal the oracle's, every resident slot
    holds its expert's bytes, and decode steps from there agree with the
    oracle (with the split, then with every miss filled)."""
    E, k, T_max = 8, 2, 4
    C = depth * E + 5
    h = Harness(L, E, C, T_max, k, 527, 773, seed_ids=pre, copy=True)
    first = C - depth * E
    pf = h.b.PrefillPool(h.cache, depth)
    h.orc.reserve(first, depth * E)
    h.compare_tables()
    compute, copy = torch.cuda.current_stream(), torch.cuda.Stream()
    _prefill_layers(pf, depth, L, compute, copy)
    pf.finish()
    h.orc.finish_prefill(first, depth, _loaded(depth, L))
    h.compare_tables()
    h.check_slot_bytes()
    rng = np.random.default_rng(depth * 10 + L)
    for s in range(40):
        layer = int(rng.integers(max(0, L - depth), L)) if s < 20 else int(rng.integers(0, L))
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(int(rng.integers(1, T_max + 1)))])
        h.step(layer, ids, fill_all=(s % 3 == 2))
    h.compare_tables()
    h.check_slot_bytes()
    assert h.cache.error() == 0
    h.cache.destroy()


def test_destroy_discards_the_buffers():
    E, L = 8, 3
    h = Harness(L, E, 2 * E + 2, 2, 2, 527, 773, seed_ids=(1, 20), copy=True)
    pf = h.b.PrefillPool(h.cache)
    _prefill_layers(pf, 2, L, torch.cuda.current_stream(), torch.cuda.Stream())
    pf.destroy()
    h.orc.reserve(2, 2 * E)
    h.orc.release(2, 2 * E)
    h.compare_tables()


def test_ring_depth_errors():
    E = 8
    h = Harness(2, E, 3 * E - 1, 2, 2, 527, 773)
    with pytest.raises(h.b.MoeError) as ei:
        h.b.PrefillPool(h.cache, 3)
    assert ei.value.status == -3                  # MOE_ERR_NO_SPACE
    with pytest.raises(h.b.MoeError) as ei:
        h.b.PrefillPool(h.cache, 1)
    assert ei.value.status == -2                  # MOE_ERR_SHAPE
    pf = h.b.PrefillPool(h.cache, 2)
    with pytest.raises(h.b.MoeError) as ei:
        h.b.PrefillPool(h.cache, 2)
    assert ei.value.status == -6                  # MOE_ERR_STATE
    pf.finish()


@pytest.mark.parametrize("C,T", [(10, 300), (13, 1000), (6, 1)])
def test_on_demand_load_decisions(C, T):
    """Batches far beyond T_max: the decisions of one step with every miss
    filled; picks of experts that found no slot go to the host."""
    L, E, k, T_max = 3, 16, 2, 8
    h = Harness(L, E, C, T_max, k, 118, 475, seed_ids=(5, 40), copy=True)
    rng = np.random.default_rng(C + T)
    for layer in (0, 1, 2, 1, 0, 2, 2):
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
        h.prefill_load(layer, ids)
    h.compare_tables()
    h.check_slot_bytes()
    assert h.cache.error() == 0
    h.cache.destroy()


def test_on_demand_load_errors():
    h = Harness(1, 16, 8, 7, 2, 118, 475)          # ceil(16/2) = 8 rows > T_max = 7
    ids = torch.zeros((20, 2), dtype=torch.int32, device="cuda")
    with pytest.raises(h.b.MoeError) as ei:
        h.cache.prefill_load(0, ids, h.out)
    assert ei.value.status == -2
    h2 = Harness(1, 16, 8, 8, 2, 118, 475)
    bad = dev(np.array([[0, 16], [3, -1]], np.int32))
    pick = h2.cache.prefill_load(0, bad, h2.out)
    assert h2.cache.error() != 0
    p = pick.cpu().numpy()
    assert p[0, 1] == -1 and p[1, 1] == -1 and p[0, 0] >= 0 and p[1, 0] >= 0


def test_prefill_then_decode_outputs():
    """Prefill through a ring of three buffers with the layer outputs checked,
    hand-over, then decode steps on the last layers hit the buffer slots and
    their outputs match the float64 oracle."""
    b = binding()
    L, E, H, I, T, k, depth = 4, 8, 256, 128, 150, 2, 3
    arrs, host_t = _layer_banks(L, E, H, I, cfg_id=58)
    expert64 = lambda lid: tuple(numerics.bf16_to_f64(a[lid]) for a in arrs)
    C = depth * E + 2
    pool = b.SlotPool(C, H, I, b.W_BF16)
    host = b.HostPoolTables(host_t, lambda i: i, L * E)
    cache = b.Cache(L, E, k, 1, pool, host, 527, 773)
    pf = b.PrefillPool(cache, depth)
    rng = np.random.default_rng(11)
    xs = [gen.activations_bf16(rng, T, H) for _ in range(L)]
    routes = [route.topk_softmax(rng.standard_normal((T, E)).astype(np.float32), k) for _ in range(L)]
    ws = b.forward_workspace(T, k, H, I, E, b.FWD_PREFILL)

    def work(l, view):
        ids, w = routes[l]
        return b.expert_forward(view, dev(xs[l]), dev(ids.astype(np.int32)), dev(w.astype(np.float32)),
                                b.FWD_PREFILL, ws).clone()

    outs = _prefill_layers(pf, depth, L, torch.cuda.current_stream(), torch.cuda.Stream(), work)
    torch.cuda.synchronize()
    for l in range(L):
        ids, w = routes[l]
        check_layer(outs[l].cpu().numpy(), ffn.moe_output(numerics.bf16_to_f64(xs[l]), ids + l * E, w, expert64),
                    "prefill layer %d" % l)
    pf.finish()
    slot_id = cache.read_state()[0]
    assert sorted(i for i in slot_id if i >= 0) == list(range((L - depth) * E, L * E))
    out = b.StepOut(1, k, E)
    wsd = b.forward_workspace(1, k, H, I, C, b.FWD_DECODE)
    for s in range(6):
        layer = L - 1 - (s % depth)
        x = gen.activations_bf16(rng, 1, H)
        ids, w = route.topk_softmax(rng.standard_normal((1, E)).astype(np.float32), k)
        cache.step(layer, dev(ids.astype(np.int32)), out)
        cnt = out.counts.cpu().numpy()
        assert cnt[1] == cnt[0], "a survivor of prefill missed"
        y = b.expert_forward(pool.c, dev(x), out.pick_slot.view(1, k), dev(w.astype(np.float32)), b.FWD_DECODE, wsd)
        check_layer(y.cpu().numpy(), ffn.moe_output(numerics.bf16_to_f64(x), ids + layer * E, w, expert64),
                    "decode step %d" % s)
    cache.destroy()


def test_on_demand_prefill_outputs():
    """Prefill without room for two full layers: on-demand loading per layer,
    the grouped GEMM over the whole slot pool for the experts that found a
    slot, the host executor for the rest; the sum matches the float64
    oracle, and the pool cannot take a double buffer."""
    b = binding()
    L, E, H, I, T, k = 2, 8, 256, 128, 180, 2
    arrs, host_t = _layer_banks(L, E, H, I, cfg_id=59)
    expert64 = lambda lid: tuple(numerics.bf16_to_f64(a[lid]) for a in arrs)
    C = 6                                           # fewer slots than one layer's experts
    pool = b.SlotPool(C, H, I, b.W_BF16)
    host = b.HostPoolTables(host_t, lambda i: i, L * E)
    cache = b.Cache(L, E, k, 4, pool, host, 527, 773)
    with pytest.raises(b.MoeError):
        b.PrefillPool(cache)
    ex = b.HostExec(4)
    out = b.StepOut(4, k, E)
    ws = b.forward_workspace(T, k, H, I, C, b.FWD_PREFILL)
    rng = np.random.default_rng(12)
    n_host = 0
    for l in (0, 1, 1, 0):
        x = gen.activations_bf16(rng, T, H)
        ids, w = route.topk_softmax(rng.standard_normal((T, E)).astype(np.float32), k)
        ids32 = ids.astype(np.int32)
        pick = cache.prefill_load(l, dev(ids32), out)
        y_gpu = b.expert_forward(pool.c, dev(x), pick, dev(w.astype(np.float32)), b.FWD_PREFILL, ws)
        pick_h = pick.cpu()
        n_host += int((pick_h < 0).sum())
        y_host = ex.forward(host, b.W_BF16, H, I, torch.from_numpy(x), torch.from_numpy(ids32 + l * E), pick_h,
                            torch.from_numpy(w.astype(np.float32)))
        y = y_gpu.cpu() + y_host
        check_layer(y.numpy(), ffn.moe_output(numerics.bf16_to_f64(x), ids + l * E, w, expert64), "layer %d" % l)
    assert n_host > 0
    assert cache.error() == 0
    ex.destroy()
    cache.destroy()


def test_on_demand_load_full_shape_decisions():
    """The on-demand loading of the FP8 prefill workload's shape (8192 tokens,
    256 experts, top-8, a 384-slot pool: no room for two full layers), four
    layers in a row: decisions, picks and tables bit-exact against the oracle
    (tiny weight rows: the decisions do not read them)."""
    L, E, k, T, C = 4, 256, 8, 8192, 384
    h = Harness(L, E, C, (E + k - 1) // k, k, 118, 475, copy=False)
    rng = np.random.default_rng(17)
    for layer in range(L):
        lg = rng.standard_normal((T, E)).astype(np.float32)
        ids, _ = route.topk_softmax(lg, k)
        r, _ = h.prefill_load(layer, ids)
        assert len(r.uniq) == E and r.q == min(len(r.misses), C - len(r.hits))
    h.compare_tables()
    assert h.cache.error() == 0
    h.cache.destroy()


def test_finish_full_shape_tables():
    """Hand-over at the FP8 prefill workload's shape: 4 layers of 256 experts
    through two full-layer buffers of a 1633-slot pool holding earlier decode
    residents; tables and slot bytes against the oracle afterwards."""
    L, E, k, C = 4, 256, 8, 1633
    rng = np.random.default_rng(18)
    pre = [int(i) for i in rng.choice(L * E, size=600, replace=False)]
    h = Harness(L, E, C, 1, k, 118, 475, seed_ids=pre, copy=True)
    first = C - 2 * E
    pf = h.b.PrefillPool(h.cache)
    h.orc.reserve(first, 2 * E)
    _prefill_layers(pf, 2, L, torch.cuda.current_stream(), torch.cuda.Stream())
    pf.finish()
    h.orc.finish_prefill(first, 2, _loaded(2, L))
    h.compare_tables()
    h.check_slot_bytes()
    h.cache.destroy()
