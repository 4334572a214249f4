"""The host executor (moe_host_forward): the CPU side of the method, the
partial sum of the experts a cache step leaves to the host, computed from the
packed rows of the host pool.  Checked without a GPU against the float64
oracle's host partial sum, over both of its code paths and several thread
counts."""
import numpy as np
import pytest
import torch

from harness import gen
from oracle import ffn, numerics


def binding():
    return pytest.importorskip("routed_expert_cache_amd.binding")


# ---------------------------------------------------------------- brick packing (the documented layout)
def pack_rows(W, KB):
    """[N][K] -> bricks of 16 rows x KB columns, brick (t, kt) at (t*(K/KB) + kt),
    16-byte chunk 16 j + r holding W[16 t + r][KB kt + (KB/4) j + e]."""
    N, K = W.shape
    return W.reshape(N // 16, 16, K // KB, 4, KB // 4).transpose(0, 2, 3, 1, 4).reshape(-1)


def gate_up_rows(G, U):
    """Packed row 16 t + r = gate row 8 t + r (r < 8) or up row 8 t + r - 8."""
    I, H = G.shape
    return np.stack([G.reshape(I // 8, 8, H), U.reshape(I // 8, 8, H)], 1).reshape(2 * I, H)


def test_packer_matches_brick_format():
    rng = np.random.default_rng(0)
    for KB, dt in ((32, np.uint16), (64, np.uint8)):
        N, K = 48, 4 * KB
        W = rng.integers(0, 200, (N, K), dtype=dt)
        P = pack_rows(W, KB)
        per = KB // 4
        for row in range(N):
            for col in range(0, K, 3):
                t, r = row // 16, row % 16
                kt, j, e = col // KB, (col % KB) // per, col % per
                assert P[((t * (K // KB) + kt) * 64 + 16 * j + r) * per + e] == W[row, col]
    G = rng.integers(0, 100, (16, 4), dtype=np.uint16)
    U = rng.integers(100, 200, (16, 4), dtype=np.uint16)
    R = gate_up_rows(G, U)
    assert np.array_equal(R[8:16], U[0:8]) and np.array_equal(R[16:24], G[8:16])


# ---------------------------------------------------------------- banks
class BankBF16:
    def __init__(self, cfg, E, H, I):
        self.E, self.H, self.I = E, H, I
        self.wg, self.wu, self.wd = gen.bank_bf16(cfg, E, H, I, 0.05)
        gu = np.stack([pack_rows(gate_up_rows(self.wg[e], self.wu[e]), 32) for e in range(E)])
        dp = np.stack([pack_rows(self.wd[e], 32) for e in range(E)])
        self.banks = [torch.from_numpy(gu), torch.from_numpy(dp)]
        self.wtype = 0

    def expert64(self, e):
        return numerics.bf16_to_f64(self.wg[e]), numerics.bf16_to_f64(self.wu[e]), numerics.bf16_to_f64(self.wd[e])


class BankFP8:
    def __init__(self, cfg, E, H, I, special=False):
        self.E, self.H, self.I = E, H, I
        ex = [gen.expert_fp8_torch(gen.torch_seed(cfg, gen.S_WEIGHTS, 0, e), H, I, 0.05, device="cpu") for e in range(E)]
        self.t = {n: torch.stack([x[n] for x in ex]).contiguous() for n in ("gate", "up", "down", "s_gate", "s_up", "s_down")}
        if special:   # subnormal and signed-zero codes among the weights
            rng = np.random.default_rng(cfg)
            for n in ("gate", "up", "down"):
                a = self.t[n].numpy()
                mask = rng.random(a.shape) < 0.2
                a[mask] = rng.integers(0, 8, mask.sum()).astype(np.uint8) | (rng.integers(0, 2, mask.sum()).astype(np.uint8) << 7)
        g, u, d = (self.t[n].numpy() for n in ("gate", "up", "down"))
        gu = np.stack([pack_rows(gate_up_rows(g[e], u[e]), 64) for e in range(E)])
        dp = np.stack([pack_rows(d[e], 64) for e in range(E)])
        self.banks = [torch.from_numpy(gu), torch.from_numpy(dp), self.t["s_gate"], self.t["s_up"], self.t["s_down"]]
        self.wtype = 1

    def expert64(self, e):
        t = self.t
        return (numerics.dequant_b128(t["gate"][e].numpy(), t["s_gate"][e].numpy()),
                numerics.dequant_b128(t["up"][e].numpy(), t["s_up"][e].numpy()),
                numerics.dequant_b128(t["down"][e].numpy(), t["s_down"][e].numpy()))


def _case(bank, T, k, p_host, seed):
    rng = np.random.default_rng(seed)
    x = gen.activations_bf16(rng, T, bank.H)
    ids = np.stack([rng.choice(bank.E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    host = rng.random((T, k)) < p_host
    pick = np.where(host, -1, 7).astype(np.int32)   # only the sign is read
    return x, ids, w, host, pick


def _run(b, ex, bank, x, ids, pick, w):
    pool = b.HostPoolTables(bank.banks, lambda i: i, bank.E, pinned=False)
    return ex.forward(pool, bank.wtype, bank.H, bank.I, torch.from_numpy(x), torch.from_numpy(ids),
                      torch.from_numpy(pick), torch.from_numpy(w)).numpy()


def _check(y, bank, x, ids, w, host, rel_tol=2e-6):
    _, ref = ffn.moe_partials(numerics.bf16_to_f64(x), ids, w, bank.expert64, on_gpu=~host)
    assert np.all(y[~host.any(1)] == 0)           # tokens with no host pick
    scale = max(np.abs(ref).max(), 1e-30)
    rel = np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-30)
    assert rel <= rel_tol and np.abs(y - ref).max() <= 10 * rel_tol * scale, (rel, np.abs(y - ref).max() / scale)


@pytest.mark.parametrize("portable", [False, True])
@pytest.mark.parametrize("threads", [1, 4])
def test_host_forward_bf16(threads, portable):
    b = binding()
    bank = BankBF16(201, 6, 256, 96)
    x, ids, w, host, pick = _case(bank, 7, 3, 0.5, 1)
    host[0] = True                                   # a token with every pick on the host
    host[1] = False                                  # and one with none
    pick = np.where(host, -1, 7).astype(np.int32)
    ex = b.HostExec(threads, portable=portable)
    try:
        if not portable and ex.simd() != 512:
            pytest.skip("no AVX-512 on this CPU")
        _check(_run(b, ex, bank, x, ids, pick, w), bank, x, ids, w, host)
    finally:
        ex.destroy()


@pytest.mark.parametrize("portable", [False, True])
@pytest.mark.parametrize("special", [False, True])
def test_host_forward_fp8(special, portable):
    b = binding()
    bank = BankFP8(202 + special, 4, 256, 256, special=special)
    x, ids, w, host, pick = _case(bank, 5, 2, 0.6, 2)
    ex = b.HostExec(3, portable=portable)
    try:
        if not portable and ex.simd() != 512:
            pytest.skip("no AVX-512 on this CPU")
        _check(_run(b, ex, bank, x, ids, pick, w), bank, x, ids, w, host)
    finally:
        ex.destroy()


def test_same_bits_for_any_thread_count():
    b = binding()
    bank = BankBF16(203, 5, 128, 64)
    x, ids, w, host, pick = _case(bank, 9, 4, 0.5, 3)
    outs = []
    for n in (1, 2, 5, 8):
        ex = b.HostExec(n)
        outs.append(_run(b, ex, bank, x, ids, pick, w))
        outs.append(_run(b, ex, bank, x, ids, pick, w))   # and on a second call
        ex.destroy()
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))


def test_pinned_workers_same_bits_and_distinct_cores():
    """MOE_HOST_PIN: worker threads pinned to the allowed CPUs, one per
    physical core before any SMT sibling, and the results bit for bit those
    of an unpinned pool."""
    import os
    b = binding()
    bank = BankBF16(204, 5, 128, 64)
    x, ids, w, host, pick = _case(bank, 9, 4, 0.5, 3)
    allowed = sorted(os.sched_getaffinity(0))
    n = min(4, len(allowed))
    ref_ex, ex = b.HostExec(n), b.HostExec(n, pin=True)
    try:
        cpus, node = ex.cpus()
        assert all(c in allowed for c in cpus)
        cores = set()
        for c in allowed:
            with open("/sys/devices/system/cpu/cpu%d/topology/core_id" % c) as f1, \
                    open("/sys/devices/system/cpu/cpu%d/topology/physical_package_id" % c) as f2:
                cores.add((f2.read().strip(), f1.read().strip()))
        if len(cores) >= n:
            assert len(set(cpus)) == n                # distinct CPUs while cores last
        assert ref_ex.cpus()[0] == [-1] * n            # not pinned without the flag
        y1 = _run(b, ex, bank, x, ids, pick, w)
        y0 = _run(b, ref_ex, bank, x, ids, pick, w)
        assert np.array_equal(y1.view(np.uint32), y0.view(np.uint32))
    finally:
        ex.destroy()
        ref_ex.destroy()


def test_portable_and_simd_paths_agree():
    b = binding()
    bank = BankFP8(204, 3, 256, 128)
    x, ids, w, host, pick = _case(bank, 4, 2, 1.0, 4)
    ex_s, ex_p = b.HostExec(2), b.HostExec(2, portable=True)
    try:
        ys, yp = _run(b, ex_s, bank, x, ids, pick, w), _run(b, ex_p, bank, x, ids, pick, w)
        assert np.allclose(ys, yp, rtol=1e-5, atol=1e-6 * np.abs(yp).max())
    finally:
        ex_s.destroy()
        ex_p.destroy()


def test_no_host_pick_gives_zero_and_errors():
    b = binding()
    bank = BankBF16(205, 4, 64, 32)
    x, ids, w, host, _ = _case(bank, 3, 2, 0.0, 5)
    ex = b.HostExec(2)
    try:
        pick = np.zeros(ids.shape, np.int32)         # every pick on the GPU
        y = _run(b, ex, bank, x, ids, pick, w)
        assert np.all(y == 0)
        bad = ids.copy()
        bad[0, 0] = -3
        with pytest.raises(b.MoeError, match="MOE_ERR_ARG"):
            _run(b, ex, bank, x, bad, np.full(ids.shape, -1, np.int32), w)
        pool = b.HostPoolTables(bank.banks, lambda i: i, bank.E, pinned=False)
        with pytest.raises(b.MoeError, match="MOE_ERR_SHAPE"):
            ex.forward(pool, 0, 64, 40, torch.from_numpy(x), torch.from_numpy(ids), torch.from_numpy(pick),
                       torch.from_numpy(w))
    finally:
        ex.destroy()
    with pytest.raises(b.MoeError, match="MOE_ERR_ARG"):
        b.HostExec(0)


@pytest.mark.parametrize("portable", [False, True])
def test_fp8_nan_code_propagates(portable):
    """E4M3FN has NaN codes (0x7F, 0xFF) and no infinities: one NaN weight of
    an expert's gate matrix makes every output of the tokens that picked it
    NaN, and no other output."""
    b = binding()
    bank = BankFP8(206, 3, 128, 128)
    bank.t["gate"][1].view(-1)[5] = 0xFF              # repack with the NaN code
    g, u, d = (bank.t[n].numpy() for n in ("gate", "up", "down"))
    bank.banks[0] = torch.from_numpy(np.stack([pack_rows(gate_up_rows(g[e], u[e]), 64) for e in range(3)]))
    x = gen.activations_bf16(np.random.default_rng(7), 3, 128)
    ids = np.array([[1, 0], [2, 0], [0, 1]], np.int32)
    w = np.full((3, 2), 0.5, np.float32)
    pick = np.array([[-1, -1], [-1, -1], [-1, 5]], np.int32)   # token 2's pick of expert 1 is on the GPU
    ex = b.HostExec(2, portable=portable)
    try:
        y = _run(b, ex, bank, x, ids, pick, w)
    finally:
        ex.destroy()
    assert np.all(np.isnan(y[0])) and np.all(np.isfinite(y[1])) and np.all(np.isfinite(y[2]))


def test_signalled_calls_wait_for_ready_and_publish_done():
    """moe_host_forward_signal without a GPU: the ready word is written from
    the host.  Calls run in order once ready reaches their number, done is
    stored after y_host; a call whose ready never comes is skipped after the
    bounded wait, still publishes done, and leaves its failure in the status."""
    import time
    b = binding()
    bank = BankBF16(207, 4, 64, 32)
    pool = b.HostPoolTables(bank.banks, lambda i: i, bank.E, pinned=False)
    x, ids, w, host, pick = _case(bank, 2, 2, 1.0, 6)
    ready = torch.zeros(1, dtype=torch.int32)
    done = torch.zeros(1, dtype=torch.int32)
    ys = [torch.zeros((2, 64), dtype=torch.float32) for _ in range(2)]
    args = [torch.from_numpy(a) for a in (x, ids, pick, w)]
    ex = b.HostExec(2)
    try:
        ex.forward_signal(pool, 0, 64, 32, *args, ys[0], ready, done, 1)
        ex.forward_signal(pool, 0, 64, 32, *args, ys[1], ready, done, 2)
        time.sleep(0.05)
        assert int(done[0]) == 0 and np.all(ys[0].numpy() == 0)   # nothing runs before ready
        ready[0] = 2                                              # both calls' inputs are in
        t0 = time.time()
        while int(done[0]) != 2 and time.time() - t0 < 5:
            time.sleep(0.001)
        assert int(done[0]) == 2 and ex.status() == 0
        ref = _run(b, ex, bank, x, ids, pick, w)
        assert np.array_equal(ys[0].numpy(), ref) and np.array_equal(ys[1].numpy(), ref)
        ex.forward_signal(pool, 0, 64, 32, *args, ys[0], ready, done, 3)   # ready never reaches 3
        t0 = time.time()
        while int(done[0]) != 3 and time.time() - t0 < 10:
            time.sleep(0.01)
        assert int(done[0]) == 3 and time.time() - t0 >= 1.5
        assert ex.status() == -6                                  # MOE_ERR_STATE, then cleared
        assert ex.status() == 0
    finally:
        ex.destroy()
