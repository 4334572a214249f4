"""GPU test of the bandwidth calibration that feeds q* ([FT] section "q* 策略":
B_P and B_H measured on the deployed machine at the deployed shapes)."""
import numpy as np
import pytest
import torch

from harness import gen
from oracle import lru, route
from tests.layer_setup import binding, dev, pack_to_host

pytestmark = pytest.mark.gpu


def test_calibrate_bandwidth_decode_shape():
    """At the decode BF16 expert shape (H 2048, I 768): the fill kernel, the
    DMA engines and the host executor give positive rates; bp and bh are
    those rates in 0.1 GB/s; the scratch slots hold the experts' bytes; the
    cache's tables are untouched; and a cache built with the measured bp:bh
    makes the oracle's decisions for those integers."""
    b = binding()
    L, E, k, H, I, C = 2, 16, 8, 2048, 768, 24
    wg, wu, wd = gen.bank_bf16(31, E, H, I, 0.02)
    host_t = list(pack_to_host(0, *[torch.from_numpy(a) for a in (wg, wu, wd)]))
    host = b.HostPoolTables(host_t, lambda i: i % E, L * E)
    pool = b.SlotPool(C, H, I, b.W_BF16)
    cache = b.Cache(L, E, k, 1, pool, host, 527, 773)
    scratch = b.SlotPool(8, H, I, b.W_BF16)
    ex = b.HostExec(4, pin=True)
    ids = [3, 17, 5, 30, 1, 12, 8, 21]
    r = cache.calibrate(ids, scratch, reps=4, host_exec=ex)
    ex.destroy()
    assert r["expert_bytes"] == 3 * H * I * 2
    for key in ("fill_GBps", "dma_GBps", "host_GBps"):
        assert 0.5 < r[key] < 1000, r
    assert r["bp"] == max(1, int(np.floor(r["fill_GBps"] * 10 + 0.5)))
    assert r["bh"] == max(1, int(np.floor(r["host_GBps"] * 10 + 0.5)))
    torch.cuda.synchronize()
    for i, lid in enumerate(ids):
        assert torch.equal(scratch.w_gu[i].cpu(), host_t[0][lid % E])
        assert torch.equal(scratch.w_down[i].cpu(), host_t[1][lid % E])
    assert np.all(cache.read_state()[0] == -1)           # the cache is still empty
    # without an executor only B_P is measured
    r2 = cache.calibrate(ids[:3], scratch, reps=2)
    assert r2["bh"] == 0 and r2["host_GBps"] == 0 and r2["bp"] >= 1
    cache.destroy()

    # the measured integers drive the split: decisions equal the oracle's
    bp, bh = r["bp"], r["bh"]
    cache = b.Cache(L, E, k, 1, pool, host, bp, bh)
    orc = lru.ExpertCache(L, E, C, bp, bh)
    out = b.StepOut(1, k, E)
    rng = np.random.default_rng(2)
    q_seen = set()
    for s in range(40):
        layer = int(rng.integers(0, L))
        ids_s = rng.choice(E, size=k, replace=False)[None]
        cache.step(layer, dev(ids_s.astype(np.int32)), out, copy=False)
        rr = orc.step(layer, ids_s)
        cnt = out.counts.cpu().numpy()
        assert list(cnt[:6]) == [len(rr.uniq), len(rr.hits), len(rr.misses), rr.q_star, rr.q,
                                 len(rr.misses) - rr.q]
        assert np.array_equal(out.pick_slot.cpu().numpy(), rr.pick_slot.reshape(-1))
        q_seen.add(rr.q_star)
    slot_id, stamp, id_slot, tick, _ = cache.read_state()
    rs, rt, ri, rtick = orc.tables()
    assert np.array_equal(slot_id, rs) and np.array_equal(stamp, rt) and tick == rtick
    cache.destroy()


def test_calibrate_argument_errors():
    b = binding()
    H, I, E = 64, 32, 4
    host_t = [torch.zeros((E, 2 * I * H), dtype=torch.uint16).pin_memory(),
              torch.zeros((E, H * I), dtype=torch.uint16).pin_memory()]
    pool = b.SlotPool(4, H, I, b.W_BF16)
    cache = b.Cache(1, E, 2, 1, pool, b.HostPoolTables(host_t, lambda i: i, E), 118, 475)
    small = b.SlotPool(1, H, I, b.W_BF16)
    with pytest.raises(b.MoeError) as ei:
        cache.calibrate([0, 1], small)                     # scratch too small
    assert ei.value.status == -2
    other = b.SlotPool(2, 2 * H, I, b.W_BF16)
    with pytest.raises(b.MoeError) as ei:
        cache.calibrate([0, 1], other)                     # another shape
    assert ei.value.status == -2
    with pytest.raises(b.MoeError) as ei:
        cache.calibrate([0, 9], pool)                      # id outside the pool
    assert ei.value.status == -1
    cache.destroy()
