"""GPU tests of resizing the shared cache at a safe point (moe_cache_resize):
tables and slot bytes bit for bit against the oracle cache across shrinks and
growths, in place and into new memory, with decode steps between them; the
layer output (GPU part plus the host executor's part) stays the float64
oracle's MoE output before, across and after a resize."""
import numpy as np
import pytest
import torch

from harness import gen
from oracle import ffn, numerics, route
from tests.layer_setup import binding, dev, check_layer, Bf16Bank
from tests.test_gpu_cache import Harness

pytestmark = pytest.mark.gpu


def _steps(h, rng, n, fill_all):
    for _ in range(n):
        layer = int(rng.integers(0, h.L))
        T = int(rng.integers(1, h.T_max + 1))
        ids = np.stack([rng.choice(h.E, size=h.k, replace=False) for _ in range(T)])
        h.step(layer, ids, fill_all=fill_all)


def _resize(h, pool):
    h.cache.resize(pool)
    moves = h.orc.resize(pool.n_slots)
    h.pool = pool
    h.compare_tables()
    h.check_slot_bytes()
    return moves


@pytest.mark.parametrize("fill_all", [False, True])
def test_resize_sequence(fill_all):
    b = binding()
    h = Harness(3, 8, 12, 3, 2, 900, 475, seed_ids=(3, 17), copy=True)
    rng = np.random.default_rng(21 + fill_all)
    H, I = h.pool.H, h.pool.I
    _steps(h, rng, 30, fill_all)
    moves = _resize(h, h.pool.prefix(7))                 # shrink in place
    assert moves, "the shrink moved nothing: the case does not test moves"
    _steps(h, rng, 30, fill_all)
    _resize(h, b.SlotPool(15, H, I, b.W_BF16))           # grow into new memory
    _steps(h, rng, 30, fill_all)
    _resize(h, b.SlotPool(4, H, I, b.W_BF16))            # shrink into new memory
    _steps(h, rng, 20, fill_all)
    big = b.SlotPool(20, H, I, b.W_BF16)
    _resize(h, big.prefix(9))                            # grow into new memory ...
    _steps(h, rng, 20, fill_all)
    _resize(h, big)                                      # ... then in place
    _steps(h, rng, 30, fill_all)
    _resize(h, big.prefix(20))                           # same size: nothing changes
    h.compare_tables()
    assert h.cache.error() == 0
    h.cache.destroy()


def test_resize_to_one_slot_and_back():
    b = binding()
    h = Harness(2, 8, 6, 2, 2, 900, 475, copy=True)
    rng = np.random.default_rng(5)
    _steps(h, rng, 10, True)
    _resize(h, h.pool.prefix(1))
    _steps(h, rng, 10, True)
    _resize(h, b.SlotPool(9, h.pool.H, h.pool.I, b.W_BF16))
    _steps(h, rng, 10, True)
    h.cache.destroy()


def test_resize_errors():
    b = binding()
    h = Harness(2, 8, 2 * 8 + 2, 2, 2, 900, 475)
    H, I = h.pool.H, h.pool.I
    pf = b.PrefillPool(h.cache)
    with pytest.raises(b.MoeError) as ei:
        h.cache.resize(h.pool.prefix(4))
    assert ei.value.status == -6                          # MOE_ERR_STATE: prefill pool alive
    pf.destroy()
    with pytest.raises(b.MoeError) as ei:
        h.cache.resize(b.SlotPool(4, H + 32, I, b.W_BF16))
    assert ei.value.status == -1                          # MOE_ERR_ARG: other shape
    mixed = b.SlotPool(4, H, I, b.W_BF16)
    mixed.w_gu = h.pool.w_gu[:4]
    mixed.c = b.Slots(b.W_BF16, H, I, 4, mixed.w_gu.data_ptr(), mixed.w_down.data_ptr(), None, None, None)
    with pytest.raises(b.MoeError) as ei:
        h.cache.resize(mixed)
    assert ei.value.status == -1                          # MOE_ERR_ARG: one bank moved, one not
    h.compare_tables()                                    # a refused resize leaves the cache as it was
    h.cache.destroy()


def test_outputs_unchanged_across_resizes():
    """Decode steps with the host branch computing the host set: the layer
    output is the oracle's at every step while the cache shrinks to two
    slots and grows to fourteen."""
    b = binding()
    E, H, I, k, T = 16, 256, 128, 4, 3
    bank = Bf16Bank(84, E, H, I)
    pool = b.SlotPool(10, H, I, b.W_BF16)
    host = b.HostPoolTables(bank.host, lambda i: i, E)
    cache = b.Cache(1, E, k, T, pool, host, 527, 773)
    ex = b.HostExec(4)
    out = b.StepOut(T, k, E)
    ws = b.forward_workspace(T, k, H, I, 14, b.FWD_DECODE)
    rng = np.random.default_rng(9)
    ids_d = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w_d = torch.empty((T, k), dtype=torch.float32, device="cuda")
    big = b.SlotPool(14, H, I, b.W_BF16)
    plan = {8: pool.prefix(2), 16: big, 24: big.prefix(5)}
    n_host = 0
    for s in range(32):
        if s in plan:
            cache.resize(plan[s])
        x = gen.activations_bf16(rng, T, H)
        lg = rng.standard_normal((T, E)).astype(np.float32)
        cache.route_step(0, dev(lg), ids_d, w_d, out)
        pick = out.pick_slot.view(T, k)
        y_gpu = b.expert_forward(cache.slots.c, dev(x), pick, w_d, b.FWD_DECODE, ws)
        pick_h, ids_h, w_h = pick.cpu(), ids_d.cpu(), w_d.cpu()
        n_host += int((pick_h < 0).sum())
        y_host = ex.forward(host, b.W_BF16, H, I, torch.from_numpy(x), ids_h, pick_h, w_h)
        ids, w = route.topk_softmax(lg, k)
        ref = ffn.moe_output(numerics.bf16_to_f64(x), ids, w, bank.expert64)
        check_layer((y_gpu.cpu() + y_host).numpy(), ref, "step %d (C=%d)" % (s, cache.cfg.C))
    assert n_host > 0
    assert cache.error() == 0
    ex.destroy()
    cache.destroy()


def test_resize_fp8_pool_moves_every_bank():
    """FP8 slots carry five banks, the scale banks in 4-byte multiples that
    are not 16-byte multiples (128x128 blocks of a 256x128 expert: 8 bytes):
    after an in-place shrink and a grow into new banks every resident slot
    holds its expert's bytes in all five banks, and the tables match the
    oracle."""
    from oracle import lru
    from tests.layer_setup import Fp8Bank
    b = binding()
    E, H, I, k, C = 12, 256, 128, 2, 10
    bank = Fp8Bank(86, E, H, I)
    pool = b.SlotPool(C, H, I, b.W_FP8_B128)
    host = b.HostPoolTables(bank.host, lambda i: i, E)
    cache = b.Cache(1, E, k, 2, pool, host, 900, 475)
    orc = lru.ExpertCache(1, E, C, 900, 475)
    seeded = [int(i) for i in np.random.default_rng(3).permutation(E)[:C]]
    cache.seed(seeded, copy=True)
    orc.seed(seeded)
    host_rows = [bank.host[0], bank.host[1], bank.t["s_gate"], bank.t["s_up"], bank.t["s_down"]]

    def check(p):
        slot_id, stamp, id_slot, tick, _ = cache.read_state()
        rs, rt, ri, rtick = orc.tables()
        assert np.array_equal(slot_id, rs) and np.array_equal(stamp, rt) and np.array_equal(id_slot, ri)
        for s, lid in enumerate(slot_id):
            if lid >= 0:
                for dev_bank, hb in zip(p.banks(), host_rows):
                    assert torch.equal(dev_bank[s].cpu().reshape(-1).view(torch.uint8),
                                       hb[lid].reshape(-1).view(torch.uint8)), (s, lid)

    check(pool)
    small = pool.prefix(4)
    cache.resize(small)
    assert orc.resize(4), "nothing moved"
    check(small)
    grown = b.SlotPool(7, H, I, b.W_FP8_B128)
    cache.resize(grown)
    orc.resize(7)
    check(grown)
    assert cache.error() == 0
    cache.destroy()


def test_resize_full_shape_decode_cache():
    """The decode BF16 workload's cache (40 layers x 128 experts, top-8, 1894
    slots, 52.7:77.3) driven by its sticky trace, shrunk in place to 947
    slots and grown back into new banks of 1894, with trace steps between:
    tables against the oracle after every phase, slot bytes at the end (tiny
    weight rows: the tables and copies do not depend on their size)."""
    from harness import CONFIGS
    from oracle import route
    b = binding()
    c = CONFIGS["decode_bf16"]
    h = Harness(c.L, c.E, c.C, 1, c.k, c.bp, c.bh, copy=True)
    picks, logits = gen.decode_trace(c.cfg_id, c.L, 12, c.E, c.k, c.p_keep)

    def run(steps):
        for s in steps:
            for l in range(c.L):
                ids, _ = route.topk_softmax(logits[s, l], c.k)
                h.step(l, ids)

    run(range(0, 4))
    h.compare_tables()
    _resize(h, h.pool.prefix(c.C // 2))
    run(range(4, 8))
    h.compare_tables()
    _resize(h, b.SlotPool(c.C, h.pool.H, h.pool.I, b.W_BF16))
    run(range(8, 12))
    h.compare_tables()
    h.check_slot_bytes()
    assert h.cache.error() == 0
    h.cache.destroy()
