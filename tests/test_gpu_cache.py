"""GPU parity of the router, the cache decision kernel and the fill copy
against the oracle: bit-exact ids, dedup sets, hit flags, q*, victims, fill
and host lists, rewritten picks and the residency tables after every step."""
import numpy as np
import pytest
import torch

from harness import gen, CONFIGS
from oracle import route, lru, numerics
from tests.layer_setup import binding, pinned, dev, W_ABS

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------- E4M3 expansion
def test_e4m3_expansion_all_codes():
    b = binding()
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).repeat(3).cuda()
    codes = torch.cat([codes, codes[:5]])                 # ragged tail
    out = b.e4m3_to_bf16(codes).cpu().numpy().view(np.uint16)
    got = numerics.bf16_to_f64(out)
    ref = numerics.e4m3_to_f64(codes.cpu().numpy())
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))   # signed zero


# ---------------------------------------------------------------- router
@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (33, 8, 2), (64, 128, 8), (300, 256, 8), (17, 1000, 32), (5, 64, 32),
                                   (9, 100, 8), (40, 120, 4), (50, 512, 8)])
def test_route_topk(T, E, k):
    """Against the oracle router; the rows cover the threshold selection (a
    few candidates), its fallback (fewer groups of 16 than picks, or more than
    64 candidates when everything ties), ties and signed zeros."""
    b = binding()
    rng = np.random.default_rng(T * 1000 + E)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[:, ::7] = np.float32(0.5)                           # ties
    lg[0, :] = np.float32(1.0)                              # all tied
    if T > 2:
        lg[1, :E // 2] = np.float32(-0.0)
        lg[1, E // 2:] = np.float32(0.0)
    ids, w = b.route_topk(dev(lg), k)
    rid, rw = route.topk_softmax(lg, k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.abs(w.cpu().numpy() - rw).max() <= W_ABS


def test_route_topk_errors():
    b = binding()
    lg = torch.zeros((4, 8), dtype=torch.float32, device="cuda")
    with pytest.raises(b.MoeError):
        b.route_topk(lg, 9)


def test_route_tiny_config_logits():
    b = binding()
    c = CONFIGS["tiny"]
    x = gen.activations_bf16(gen.np_rng(c.cfg_id, gen.S_ACT), c.T, c.H)
    wr = gen.router_matrix(gen.np_rng(c.cfg_id, gen.S_ROUTER), c.H, c.E, c.router_std)
    lg = gen.router_logits(x, wr)
    ids, w = b.route_topk(dev(lg), c.k)
    rid, rw = route.topk_softmax(lg, c.k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.abs(w.cpu().numpy() - rw).max() <= W_ABS


# ---------------------------------------------------------------- cache decisions
class Harness:
    """A GPU cache and the oracle cache driven with the same steps."""

    def __init__(self, L, E, C, T_max, k, bp, bh, H=32, I=32, seed_ids=(), copy=False):
        b = binding()
        self.b, self.L, self.E, self.C, self.T_max, self.k = b, L, E, C, T_max, k
        self.pool = b.SlotPool(C, H, I, b.W_BF16)
        # host banks: one distinct row per logical id so copies are checkable
        rng = np.random.default_rng(L * 7 + E)
        n = L * E
        self.hb = [pinned(rng.integers(0, 1 << 16, size=(n, 2 * I * H), dtype=np.uint16)),
                   pinned(rng.integers(0, 1 << 16, size=(n, H * I), dtype=np.uint16))]
        self.host = b.HostPoolTables(self.hb, lambda i: i, n)
        self.cache = b.Cache(L, E, k, T_max, self.pool, self.host, bp, bh)
        self.out = b.StepOut(T_max, k, E)
        self.orc = lru.ExpertCache(L, E, C, bp, bh)
        if seed_ids:
            self.cache.seed(list(seed_ids), copy=copy)
            self.orc.seed(list(seed_ids))
        self.copy = copy

    def step(self, layer, ids, fill_all=False, oracle_layer=None):
        """layer: an int, or a device int32 scalar (then oracle_layer names it)."""
        T = ids.shape[0]
        self.cache.step(layer, dev(ids.astype(np.int32)), self.out, copy=self.copy, fill_all=fill_all)
        r = self.orc.step(layer if oracle_layer is None else oracle_layer, ids, fill_all=fill_all)
        self.compare(r, T)
        return r

    def prefill_load(self, layer, ids):
        """On-demand loading of a batch of any size: the same decisions as a
        step with every miss filled; the picks come back in their own array."""
        pick = self.cache.prefill_load(layer, dev(ids.astype(np.int32)), self.out, copy=self.copy)
        r = self.orc.step(layer, ids, fill_all=True)
        self.compare(r, 0)
        assert np.array_equal(pick.cpu().numpy(), r.pick_slot)
        return r, pick

    def route_step(self, layer, logits):
        """Router + step in one launch; checks ids and weights against the
        oracle router, then the step against the oracle cache."""
        T = logits.shape[0]
        ids = torch.empty((T, self.k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, self.k), dtype=torch.float32, device="cuda")
        self.cache.route_step(layer, dev(logits), ids, w, self.out, copy=self.copy)
        rid, rw = route.topk_softmax(logits, self.k)
        assert np.array_equal(ids.cpu().numpy(), rid)
        assert np.abs(w.cpu().numpy() - rw).max() <= W_ABS
        r = self.orc.step(layer, rid)
        self.compare(r, T)
        return ids, w

    def compare(self, r, T):
        b = self.b
        o = self.out
        cnt = o.counts.cpu().numpy()
        u, h, m = len(r.uniq), len(r.hits), len(r.misses)
        assert list(cnt[:6]) == [u, h, m, r.q_star, r.q, m - r.q], (cnt, r)
        U = o.U_max
        uniq = o.uniq.cpu().numpy()
        assert list(uniq[:u]) == r.uniq and np.all(uniq[u:] == -1)
        assert list(o.is_hit.cpu().numpy()[:u]) == r.is_hit
        q = r.q
        assert list(o.fill_id.cpu().numpy()[:q]) == r.fill_id
        assert list(o.fill_slot.cpu().numpy()[:q]) == r.fill_slot
        assert list(o.fill_evicted.cpu().numpy()[:q]) == r.fill_evicted
        assert np.all(o.fill_id.cpu().numpy()[q:U] == -1)
        assert list(o.host_id.cpu().numpy()[:m - q]) == r.host_id
        if T:
            assert np.array_equal(o.pick_slot.cpu().numpy()[:T * self.k], r.pick_slot.reshape(-1))

    def compare_tables(self):
        slot_id, stamp, id_slot, tick, counters = self.cache.read_state()
        rs, rt, ri, rtick = self.orc.tables()
        assert np.array_equal(slot_id, rs)
        assert np.array_equal(stamp, rt)
        assert np.array_equal(id_slot, ri)
        assert tick == rtick
        c = self.orc.counters
        assert list(counters) == [c["calls"], c["uniq"], c["hits"], c["misses"], c["fills"], c["host"]]

    def check_slot_bytes(self):
        slot_id = self.cache.read_state()[0]
        for s, lid in enumerate(slot_id):
            if lid >= 0:
                for k, bank in enumerate((self.pool.w_gu, self.pool.w_down)):
                    assert torch.equal(bank[s].cpu(), self.hb[k][lid]), (s, lid, k)


def test_tiny_config_one_step():
    """Tiny workload, one 32-token step: 4 seeded slots, all hit, q* = 1, no victim."""
    c = CONFIGS["tiny"]
    x = gen.activations_bf16(gen.np_rng(c.cfg_id, gen.S_ACT), c.T, c.H)
    wr = gen.router_matrix(gen.np_rng(c.cfg_id, gen.S_ROUTER), c.H, c.E, c.router_std)
    ids, _ = route.topk_softmax(gen.router_logits(x, wr), c.k)
    hz = Harness(c.L, c.E, c.C, c.T, c.k, c.bp, c.bh, seed_ids=c.seed_slots, copy=True)
    r = hz.step(0, ids)
    assert r.q_star == 1 and r.q == 0 and len(r.host_id) == 4
    hz.compare_tables()
    hz.check_slot_bytes()


def test_tiny_config_token_by_token():
    """The same tokens as 32 single-token steps: fills and victims happen."""
    c = CONFIGS["tiny"]
    x = gen.activations_bf16(gen.np_rng(c.cfg_id, gen.S_ACT), c.T, c.H)
    wr = gen.router_matrix(gen.np_rng(c.cfg_id, gen.S_ROUTER), c.H, c.E, c.router_std)
    ids, _ = route.topk_softmax(gen.router_logits(x, wr), c.k)
    hz = Harness(c.L, c.E, c.C, 1, c.k, c.bp, c.bh, seed_ids=c.seed_slots, copy=True)
    fills = 0
    for t in range(c.T):
        r = hz.step(0, ids[t:t + 1])
        fills += r.q
    assert fills > 0
    hz.compare_tables()
    hz.check_slot_bytes()


STRESS = [
    # L, E, C, T, k, bp, bh, steps
    (1, 8, 4, 1, 2, 118, 475, 80),
    (3, 8, 5, 2, 2, 118, 475, 120),
    (2, 16, 12, 4, 3, 527, 773, 120),
    (4, 32, 40, 16, 8, 118, 475, 60),
    (2, 256, 300, 16, 8, 900, 475, 40),     # all misses filled: q up to 128 (radix select)
    (3, 64, 70, 16, 8, 900, 475, 40),       # q clamped by free victims
    (40, 128, 1894, 1, 8, 527, 773, 100),   # decode BF16 shape
    (3, 64, 2500, 4, 8, 118, 475, 60),      # pool over two staging batches of the decision kernel
    (2, 3000, 4100, 16, 8, 900, 475, 30),   # layer row over two batches, pool over three
]


@pytest.mark.parametrize("case", STRESS)
def test_random_traces(case):
    L, E, C, T, k, bp, bh, steps = case
    rng = np.random.default_rng(sum(case))
    hz = Harness(L, E, C, T, k, bp, bh, copy=False)
    for s in range(steps):
        layer = int(rng.integers(0, L))
        Ts = int(rng.integers(1, T + 1))
        pool_e = int(rng.integers(k, E + 1))           # narrow expert range -> more hits/ties
        ids = np.stack([rng.choice(pool_e, size=k, replace=False) for _ in range(Ts)])
        hz.step(layer, ids)
    hz.compare_tables()


def test_sticky_decode_trace_short():
    """The decode BF16 workload's cache, 24 steps x 40 layers, metadata only."""
    c = CONFIGS["decode_bf16"]
    picks, logits = gen.decode_trace(c.cfg_id, c.L, 24, c.E, c.k, c.p_keep)
    hz = Harness(c.L, c.E, c.C, 1, c.k, c.bp, c.bh, copy=False)
    for s in range(24):
        for l in range(c.L):
            ids, _ = route.topk_softmax(logits[s, l], c.k)
            hz.step(l, ids)
            if s >= 10:
                hz.compare_tables()
    hz.compare_tables()


ROUTE_STEP = [
    # L, E, C, T, k, bp, bh, steps
    (4, 8, 5, 3, 2, 118, 475, 60),
    (40, 128, 1894, 1, 8, 527, 773, 80),    # decode BF16 shape
    (3, 256, 200, 16, 8, 118, 475, 40),     # decode FP8 layer width, 4 tokens per wave
    (2, 1000, 300, 5, 32, 900, 475, 20),    # 16 logits per lane
    (2, 60, 2500, 9, 4, 118, 475, 30),      # pool over two staging batches
    (3, 64, 150, 16, 8, 118, 475, 40),      # every wave routes a token
    (2, 128, 300, 12, 8, 527, 773, 30),     # decode BF16 layer width, 12 tokens
]


@pytest.mark.parametrize("case", ROUTE_STEP)
def test_route_step_fused(case):
    """moe_cache_route_step = moe_route_topk + moe_cache_step, bit for bit."""
    L, E, C, T, k, bp, bh, steps = case
    rng = np.random.default_rng(sum(case) + 5)
    hz = Harness(L, E, C, T, k, bp, bh, copy=False)
    b = hz.b
    for s in range(steps):
        layer = int(rng.integers(0, L))
        Ts = int(rng.integers(1, T + 1))
        lg = rng.standard_normal((Ts, E)).astype(np.float32)
        if s % 3 == 0:
            lg[:, ::5] = np.float32(0.25)          # ties across experts
        ids, w = hz.route_step(layer, lg)
        # the separate router gives the same bits
        ids2, w2 = b.route_topk(dev(lg), k)
        assert torch.equal(ids, ids2) and torch.equal(w, w2)
    hz.compare_tables()


@pytest.mark.parametrize("E,T", [(64, 16), (128, 1), (256, 1), (256, 3), (8, 32)])
def test_route_step_ties_and_signed_zeros(E, T):
    """Logits drawn from five values (+0 and -0 among them): most experts tie,
    so the pick order rests on the lower-index rule and the candidate count
    often passes 64 (the k-round fallback); the fused router against the
    oracle router and the separate router kernel."""
    b = binding()
    k = 8 if E >= 8 else 2
    hz = Harness(2, E, max(k, E // 2), T, k, 118, 475, copy=False)
    rng = np.random.default_rng(E * 100 + T)
    vals = np.array([-0.0, 0.0, 1.0, -1.0, 0.5], np.float32)
    for s in range(12):
        lg = vals[rng.integers(0, 5, size=(T, E))]
        if s == 0:
            lg[:] = np.float32(-0.0)               # every expert tied
        ids, w = hz.route_step(int(rng.integers(0, 2)), lg)
        ids2, w2 = b.route_topk(dev(lg), k)
        assert torch.equal(ids, ids2) and torch.equal(w, w2)
    hz.compare_tables()


def test_route_step_sticky_decode_trace():
    """The decode BF16 workload's logits through the fused router + step."""
    c = CONFIGS["decode_bf16"]
    picks, logits = gen.decode_trace(c.cfg_id, c.L, 12, c.E, c.k, c.p_keep)
    hz = Harness(c.L, c.E, c.C, 1, c.k, c.bp, c.bh, copy=False)
    for s in range(12):
        for l in range(c.L):
            hz.route_step(l, logits[s, l])
    hz.compare_tables()


def test_fill_copies_every_bank():
    hz = Harness(2, 8, 6, 2, 2, 900, 475, H=64, I=32, copy=True)
    rng = np.random.default_rng(3)
    for s in range(30):
        ids = np.stack([rng.choice(8, size=2, replace=False) for _ in range(2)])
        hz.step(int(rng.integers(0, 2)), ids)
    hz.compare_tables()
    hz.check_slot_bytes()


def test_separate_fill_call_equals_step_with_copy():
    hz = Harness(2, 8, 6, 2, 2, 900, 475, H=64, I=32, copy=False)
    rng = np.random.default_rng(4)
    for s in range(30):
        ids = np.stack([rng.choice(8, size=2, replace=False) for _ in range(2)])
        hz.step(int(rng.integers(0, 2)), ids)
        hz.cache.fill(hz.out)
    hz.compare_tables()
    hz.check_slot_bytes()


def test_bad_expert_id_sets_error_word():
    hz = Harness(1, 8, 4, 1, 2, 118, 475)
    ids = dev(np.array([[3, 11]], np.int32))
    hz.cache.step(0, ids, hz.out, copy=False)
    assert hz.cache.error() != 0
    ps = hz.out.pick_slot.cpu().numpy()
    assert ps[1] == -1
    assert hz.cache.error() == 0                          # cleared by the read


def test_argument_errors():
    b = binding()
    hz = Harness(1, 8, 4, 2, 2, 118, 475)
    with pytest.raises(b.MoeError):
        hz.cache.step(0, dev(np.zeros((3, 2), np.int32)), hz.out)        # T > T_max
    pageable = [torch.zeros((8, 2 * 32 * 32), dtype=torch.uint16), torch.zeros((8, 32 * 32), dtype=torch.uint16)]
    tabs = b.HostPoolTables.__new__(b.HostPoolTables)
    import ctypes
    arrs = [(ctypes.c_void_p * 8)(*[t.data_ptr()] * 8) for t in pageable]
    tabs._arrays = arrs
    tabs.c = b.HostPool(*[ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p)) for a in arrs], None, None, None)
    with pytest.raises(b.MoeError) as ei:
        b.Cache(1, 8, 2, 2, hz.pool, tabs, 118, 475)
    assert ei.value.status == -4                          # MOE_ERR_NOT_PINNED


@pytest.mark.parametrize("T", [1, 4, 16])
def test_route_step_fp8_decode_trace_full_shape(T):
    """The FP8 decode workload's cache: 58 layers x 256 experts, top-8, a
    1633-slot pool (11%), 118:475, its sticky trace at T tokens per step,
    through the fused router + step as the benchmark runs it: ids, weights,
    decisions and tables bit-exact against the oracle (metadata only)."""
    c = CONFIGS["decode_fp8"]
    C = c.C
    steps = 6 if T < 16 else 3
    picks, logits = gen.decode_trace(c.cfg_id, c.L, steps, c.E, c.k, c.p_keep, T=T, salt=T)
    hz = Harness(c.L, c.E, C, T, c.k, c.bp, c.bh, copy=False)
    for s in range(steps):
        for l in range(c.L):
            hz.route_step(l, logits[s, l])
    hz.compare_tables()


def test_device_layer_index():
    """The layer is a device scalar read by the kernel: the same call with the
    scalar changed in between serves two layers (what one captured graph of a
    layer call relies on); a layer outside [0, L) sets the device error word
    and decides nothing (tables unchanged, every pick to the host)."""
    b = binding()
    hz = Harness(3, 8, 5, 2, 2, 118, 475, copy=False)
    d_layer = torch.zeros(1, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(12)
    for s in range(12):
        layer = int(rng.integers(0, 3))
        d_layer.fill_(layer)
        ids = np.stack([rng.choice(8, size=2, replace=False) for _ in range(2)])
        hz.step(d_layer, ids, oracle_layer=layer)
    hz.compare_tables()
    before = hz.cache.read_state()
    for bad in (3, -1, 1 << 30):
        d_layer.fill_(bad)
        hz.cache.step(d_layer, dev(np.array([[0, 1], [2, 3]], np.int32)), hz.out, copy=False)
        assert np.all(hz.out.pick_slot.cpu().numpy() == -1)
        cnt = hz.out.counts.cpu().numpy()
        assert np.all(cnt[:6] == 0) and cnt[6] == bad
        assert hz.cache.error() != 0
        assert hz.cache.error() == 0                      # cleared by the read
    after = hz.cache.read_state()
    for u, v in zip(before[:3], after[:3]):
        assert np.array_equal(u, v)
    assert before[3] == after[3]
    hz.compare_tables()
