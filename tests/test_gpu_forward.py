"""GPU parity of the grouped expert evaluation and the merge against the
float64 oracle: rel-L2 <= 5e-3 and max-abs <= 2e-2 max|ref| on the layer
outputs, at sizes spanning several tiles with ragged tails and at the
workloads' full shapes (sampled tokens where the oracle is slow)."""
import numpy as np
import pytest
import torch

from harness import gen, CONFIGS
from oracle import route, lru, numerics, ffn
from tests.layer_setup import binding, dev, pinned, check_layer, Bf16Bank, Fp8Bank, oracle_partials

pytestmark = pytest.mark.gpu


def _slots_identity(b, bank, wtype):
    pool = b.SlotPool(bank.E, bank.H, bank.I, wtype)
    bank.load_slots(pool, {e: e for e in range(bank.E)})
    return pool


def _run_forward(b, pool, x_bits, pick_slot, w, mode, T_max=None):
    T, k = pick_slot.shape
    ws = b.forward_workspace(T_max or T, k, pool.H, pool.I, pool.n_slots, mode)
    args = (pool.c, dev(x_bits), dev(pick_slot.astype(np.int32)), dev(w.astype(np.float32)), mode, ws)
    y = b.expert_forward(*args)
    torch.cuda.synchronize()
    out = y.cpu().numpy()
    if mode == b.FWD_DECODE:
        # the hand-over counters reset themselves: a second call on the same
        # workspace gives the same bits, and the error word stays clear
        y2 = b.expert_forward(*args)
        torch.cuda.synchronize()
        assert np.array_equal(y2.cpu().numpy().view(np.uint32), out.view(np.uint32))
        assert int(ws[:4].view(torch.int32).item()) == 0
    # forward + merge in one call: the same bits as the two calls
    yh = torch.randn((T, pool.H), dtype=torch.float32, device="cuda")
    yg = torch.full((T, pool.H), float("nan"), dtype=torch.float32, device="cuda")
    yb = torch.empty((T, pool.H), dtype=torch.uint16, device="cuda")
    yo = b.expert_forward_merge(*args[:5], ws, yh, y_gpu=yg, y_out_bf16=yb)
    ref_b = torch.empty_like(yb)
    ref_o = b.merge_partial(y, yh, y_out_bf16=ref_b)
    torch.cuda.synchronize()
    assert np.array_equal(yg.cpu().numpy().view(np.uint32), out.view(np.uint32))
    assert torch.equal(yo.view(torch.int32), ref_o.view(torch.int32))
    assert torch.equal(yb, ref_b)
    return out


# ---------------------------------------------------------------- decode, BF16
@pytest.mark.parametrize("T,E,k,H,I", [(1, 8, 2, 256, 128), (3, 8, 2, 256, 128), (16, 32, 4, 512, 256),
                                       (1, 128, 8, 2048, 768), (5, 24, 8, 1024, 384),
                                       (16, 24, 16, 256, 128),      # 256 picks, many shared slots
                                       (2, 8, 2, 96, 96),           # odd brick counts along H and I
                                       (16, 64, 8, 2048, 768)])     # several gate/up tasks per workgroup
def test_decode_bf16(T, E, k, H, I):
    b = binding()
    bank = Bf16Bank(90 + T, E, H, I)
    pool = _slots_identity(b, bank, b.W_BF16)
    rng = np.random.default_rng(T + E)
    x = gen.activations_bf16(rng, T, H)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = route.topk_softmax(lg, k)
    pick = ids.copy()
    on_gpu = rng.random(ids.shape) < 0.75
    pick[~on_gpu] = -1                                   # some picks to the host set
    y = _run_forward(b, pool, x, pick, w, b.FWD_DECODE)
    yg, _ = oracle_partials(x, ids, w, bank.expert64, on_gpu)
    check_layer(y, yg, "decode bf16")


@pytest.mark.parametrize("n_gpu", [1, 2])
def test_decode_few_groups_full_shape(n_gpu):
    """One or two groups at the decode shape (H 2048, I 768): most of the grid
    holds no gate/up task, and the down tasks start on workgroups that had
    none."""
    b = binding()
    T, E, k, H, I = 2, 16, 8, 2048, 768
    bank = Bf16Bank(70 + n_gpu, E, H, I)
    pool = _slots_identity(b, bank, b.W_BF16)
    rng = np.random.default_rng(40 + n_gpu)
    x = gen.activations_bf16(rng, T, H)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    ids[:, :n_gpu] = np.arange(n_gpu)                    # the GPU picks: the same n_gpu experts
    w = np.exp(rng.standard_normal((T, k)))
    w /= w.sum(1, keepdims=True)
    on_gpu = np.zeros(ids.shape, bool)
    on_gpu[:, :n_gpu] = True
    pick = np.where(on_gpu, ids, -1)
    y = _run_forward(b, pool, x, pick, w, b.FWD_DECODE)
    yg, _ = oracle_partials(x, ids, w, bank.expert64, on_gpu)
    check_layer(y, yg, "decode few groups")


def test_decode_more_down_tasks_than_workgroups():
    """H 16384: 1024 down tasks, more than the resident workgroups, so some
    workgroups hold two; each is started once per call, and two calls in a
    row on one workspace give the same bits with the error word clear."""
    b = binding()
    T, E, k, H, I = 2, 4, 2, 16384, 128
    bank = Bf16Bank(75, E, H, I)
    pool = _slots_identity(b, bank, b.W_BF16)
    rng = np.random.default_rng(75)
    x = gen.activations_bf16(rng, T, H)
    ids = np.array([[0, 1], [2, 1]])
    w = np.array([[0.6, 0.4], [0.3, 0.7]])
    y = _run_forward(b, pool, x, ids, w, b.FWD_DECODE)
    yg, _ = oracle_partials(x, ids, w, bank.expert64, np.ones(ids.shape, bool))
    check_layer(y, yg, "decode H 16384")


def test_decode_shared_slots_across_tokens():
    """Several tokens routed to the same slots: each slot streamed once."""
    b = binding()
    bank = Bf16Bank(77, 4, 256, 128)
    pool = _slots_identity(b, bank, b.W_BF16)
    T, k = 16, 2
    ids = np.array([[t % 4, (t + 1) % 4] for t in range(T)])
    w = np.full((T, k), 0.5)
    x = gen.activations_bf16(np.random.default_rng(0), T, 256)
    y = _run_forward(b, pool, x, ids, w, b.FWD_DECODE)
    yg, _ = oracle_partials(x, ids, w, bank.expert64, np.ones(ids.shape, bool))
    check_layer(y, yg)


def test_decode_pick_limit():
    b = binding()
    pool = b.SlotPool(4, 256, 128, b.W_BF16)
    ws = b.forward_workspace(16, 16, 256, 128, 4, b.FWD_DECODE)
    x = torch.zeros((16, 256), dtype=torch.uint16, device="cuda")
    with pytest.raises(b.MoeError) as ei:
        b.expert_forward(pool.c, x, torch.zeros((16, 17), dtype=torch.int32, device="cuda"),
                         torch.zeros((16, 17), device="cuda"), b.FWD_DECODE, ws)
    assert ei.value.status == -2                  # MOE_ERR_SHAPE: T*k > 256


def test_decode_all_host_gives_zero():
    b = binding()
    bank = Bf16Bank(78, 4, 256, 128)
    pool = _slots_identity(b, bank, b.W_BF16)
    x = gen.activations_bf16(np.random.default_rng(1), 2, 256)
    y = _run_forward(b, pool, x, np.full((2, 2), -1), np.full((2, 2), 0.5), b.FWD_DECODE)
    assert np.all(y == 0)


# ---------------------------------------------------------------- decode, FP8
@pytest.mark.parametrize("T,E,k,H,I", [(1, 8, 2, 256, 256), (4, 16, 4, 512, 384), (16, 24, 8, 1024, 256),
                                       (8, 16, 8, 512, 256),        # two brick rows per down task from T = 8
                                       (12, 40, 4, 768, 1024)])     # ... ragged T
def test_decode_fp8(T, E, k, H, I):
    b = binding()
    bank = Fp8Bank(60 + T, E, H, I)
    pool = _slots_identity(b, bank, b.W_FP8_B128)
    rng = np.random.default_rng(5 * T)
    x = gen.activations_bf16(rng, T, H)
    ids, w = route.topk_softmax(rng.standard_normal((T, E)).astype(np.float32), k)
    y = _run_forward(b, pool, x, ids, w, b.FWD_DECODE)
    yg, _ = oracle_partials(x, ids, w, bank.expert64, np.ones(ids.shape, bool))
    check_layer(y, yg, "decode fp8")


def test_decode_fp8_special_codes():
    """Subnormal, zero and sign codes in the weights decode exactly."""
    b = binding()
    bank = Fp8Bank(61, 2, 256, 128)
    rng = np.random.default_rng(9)
    for n in ("gate", "up", "down"):
        t = bank.t[n]
        mask = torch.from_numpy(rng.random(t.shape) < 0.2)
        sub = torch.from_numpy(rng.integers(0, 8, t.shape).astype(np.uint8) | (rng.integers(0, 2, t.shape).astype(np.uint8) << 7))
        t[mask] = sub[mask]
    bank.repack()
    pool = _slots_identity(b, bank, b.W_FP8_B128)
    x = gen.activations_bf16(rng, 3, 256)
    ids = np.array([[0, 1]] * 3)
    w = np.array([[0.7, 0.3]] * 3)
    y = _run_forward(b, pool, x, ids, w, b.FWD_DECODE)
    yg, _ = oracle_partials(x, ids, w, bank.expert64, np.ones(ids.shape, bool))
    check_layer(y, yg)


@pytest.mark.parametrize("T", [1, 4, 16])
def test_decode_fp8_full_shape(T):
    """Decode FP8 workload shape (H 7168, I 2048, top-8), sampled tokens."""
    b = binding()
    c = CONFIGS["decode_fp8"]
    E = min(c.E, T * c.k)                               # only the routed experts need slots
    bank = Fp8Bank(c.cfg_id, E, c.H, c.I, layer=T, device="cuda")
    pool = _slots_identity(b, bank, b.W_FP8_B128)
    rng = np.random.default_rng(100 + T)
    x = gen.activations_bf16(rng, T, c.H)
    ids = np.stack([rng.choice(E, size=c.k, replace=False) for _ in range(T)])
    w = np.exp(rng.standard_normal((T, c.k)))
    w /= w.sum(1, keepdims=True)
    y = _run_forward(b, pool, x, ids, w, b.FWD_DECODE)
    tok = [T - 1]                                       # last token (a ragged position)
    yg, _ = oracle_partials(x[tok], ids[tok], w[tok], bank.expert64, np.ones((len(tok), c.k), bool))
    check_layer(y[tok], yg, "decode fp8 full")


@pytest.mark.parametrize("T,n_gpu", [(1, 1), (1, 4), (2, 3), (2, 4)])
def test_decode_fp8_few_groups_full_shape(T, n_gpu):
    """Decode FP8 workload shape with one to four groups on the GPU (the rest
    of each token's picks on the host, as in most calls of the FP8 decode
    trace).  Every token is checked."""
    b = binding()
    c = CONFIGS["decode_fp8"]
    E, k = 8, c.k
    bank = Fp8Bank(c.cfg_id, E, c.H, c.I, layer=20 + 4 * T + n_gpu, device="cuda")
    pool = _slots_identity(b, bank, b.W_FP8_B128)
    rng = np.random.default_rng(200 + 10 * T + n_gpu)
    x = gen.activations_bf16(rng, T, c.H)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    on_gpu = ids < n_gpu                                  # experts 0 .. n_gpu-1 are the GPU set
    w = np.exp(rng.standard_normal((T, k)))
    w /= w.sum(1, keepdims=True)
    y = _run_forward(b, pool, x, np.where(on_gpu, ids, -1), w, b.FWD_DECODE)
    yg, _ = oracle_partials(x, ids, w, bank.expert64, on_gpu)
    check_layer(y, yg, "decode fp8 few groups")


# ---------------------------------------------------------------- decode, split launches
@pytest.mark.parametrize("wtype,T,E,k,H,I", [
    ("bf16", 1, 128, 8, 2048, 768),    # the decode BF16 shape: 8-row register-resident down tasks
    ("bf16", 4, 32, 8, 1024, 256),     # 16-row down tasks
    ("fp8", 1, 16, 8, 1024, 512),      # two brick rows per gate/up task, device-scope h loads
    ("fp8", 4, 16, 8, 1024, 512),      # two brick rows per down task (grids of 200 and 400: several rounds)
    ("fp8", 16, 32, 8, 1024, 512)])    # four brick rows per gate/up task
def test_decode_split_any_grid(wtype, T, E, k, H, I):
    """The split decode (gate/up launch, then down launch) waits for nothing,
    so it completes on any grid: one workgroup (which takes every task
    itself), a few, a few hundred (several rounds of gate/up tasks), and far
    more than the GPU holds at once (most workgroups start only after others
    end).  Every result matches the oracle, and on grids the GPU holds at
    once the single launch gives the same bits as the split pair.  The error
    word stays clear and the counters reset: calls run back to back on one
    workspace."""
    b = binding()
    bank = (Bf16Bank if wtype == "bf16" else Fp8Bank)(300 + T, E, H, I)
    pool = _slots_identity(b, bank, b.W_BF16 if wtype == "bf16" else b.W_FP8_B128)
    rng = np.random.default_rng(300 + T)
    x = gen.activations_bf16(rng, T, H)
    ids, w = route.topk_softmax(rng.standard_normal((T, E)).astype(np.float32), k)
    pick = np.where(rng.random(ids.shape) < 0.8, ids, -1)
    ws = b.forward_workspace(T, k, H, I, pool.n_slots, b.FWD_DECODE)
    args = (pool.c, dev(x), dev(pick.astype(np.int32)), dev(w.astype(np.float32)))
    yg, _ = oracle_partials(x, ids, w, bank.expert64, pick >= 0)
    try:
        for grid in (0, 1, 3, 200, 400, 4096):
            b.decode_grid_override(grid)
            print("split, grid", grid, flush=True)
            ys = b.expert_forward(*args, b.FWD_DECODE_SPLIT, ws).clone()
            torch.cuda.synchronize()
            assert int(ws[:4].view(torch.int32).item()) == 0, grid
            check_layer(ys.cpu().numpy(), yg, "decode split, grid %d" % grid)
            if grid <= 512:
                yf = b.expert_forward(*args, b.FWD_DECODE, ws)
                torch.cuda.synchronize()
                assert int(ws[:4].view(torch.int32).item()) == 0, grid
                assert torch.equal(yf.view(torch.int32), ys.view(torch.int32)), grid
    finally:
        b.decode_grid_override(0)


# ---------------------------------------------------------------- decode, the bounded wait's give-up path
@pytest.mark.parametrize("wtype,T,E,k,H,I", [
    ("bf16", 1, 128, 8, 2048, 768),    # 8-row register-resident down tasks (their own wait)
    ("bf16", 4, 32, 8, 1024, 256),     # 16-row down tasks
    ("fp8", 1, 16, 8, 1024, 512),      # device-scope h loads
    ("fp8", 4, 16, 8, 1024, 512)])     # two brick rows per down task
def test_decode_wait_gives_up(wtype, T, E, k, H, I):
    """The one-launch decode's down workgroups wait, bounded, for the start
    signal of the gate/up phase.  The wait test launches the down phase alone
    with those waits, so nothing raises the signal: every waiting workgroup
    gives up after `polls` polls, sets the workspace's error word and exits
    (the launch ends; no fault).  Zero-filled again, the same workspace then
    serves a normal call, which matches the oracle and leaves the word clear."""
    b = binding()
    bank = (Bf16Bank if wtype == "bf16" else Fp8Bank)(320 + T, E, H, I)
    pool = _slots_identity(b, bank, b.W_BF16 if wtype == "bf16" else b.W_FP8_B128)
    rng = np.random.default_rng(320 + T)
    x = gen.activations_bf16(rng, T, H)
    ids, w = route.topk_softmax(rng.standard_normal((T, E)).astype(np.float32), k)
    pick = np.where(rng.random(ids.shape) < 0.8, ids, -1)
    ws = b.forward_workspace(T, k, H, I, pool.n_slots, b.FWD_DECODE)
    args = (pool.c, dev(x), dev(pick.astype(np.int32)), dev(w.astype(np.float32)))
    yg, _ = oracle_partials(x, ids, w, bank.expert64, pick >= 0)
    for polls in (1, 64):
        print("wait test, polls", polls, flush=True)
        b.decode_wait_test(*args, ws, polls)
        torch.cuda.synchronize()
        assert int(ws[:4].view(torch.int32).item()) != 0, polls
        ws.zero_()
        y = b.expert_forward(*args, b.FWD_DECODE, ws)
        torch.cuda.synchronize()
        assert int(ws[:4].view(torch.int32).item()) == 0, polls
        check_layer(y.cpu().numpy(), yg, "decode after a wait test, polls %d" % polls)


# ---------------------------------------------------------------- prefill
@pytest.mark.parametrize("T,E,k,H,I", [(1, 8, 2, 256, 128), (300, 8, 2, 256, 128), (1000, 16, 4, 512, 192),
                                       (257, 8, 2, 128, 64)])   # two K steps in the down GEMM
def test_prefill_bf16(T, E, k, H, I):
    b = binding()
    bank = Bf16Bank(50 + E, E, H, I)
    pool = _slots_identity(b, bank, b.W_BF16)
    rng = np.random.default_rng(T)
    x = gen.activations_bf16(rng, T, H)
    ids, w = route.topk_softmax(rng.standard_normal((T, E)).astype(np.float32), k)
    y = _run_forward(b, pool, x, ids, w, b.FWD_PREFILL)
    ref = ffn.moe_output(numerics.bf16_to_f64(x), ids, w, bank.expert64)
    check_layer(y, ref, "prefill bf16")


def test_prefill_bf16_skewed_segments():
    """One expert gets most pairs (many tiles), one gets none."""
    b = binding()
    E, k, H, I, T = 6, 2, 256, 128, 700
    bank = Bf16Bank(41, E, H, I)
    pool = _slots_identity(b, bank, b.W_BF16)
    rng = np.random.default_rng(2)
    ids = np.stack([[0, 1 + (t % 4)] for t in range(T)])
    w = rng.random((T, k))
    x = gen.activations_bf16(rng, T, H)
    y = _run_forward(b, pool, x, ids, w, b.FWD_PREFILL)
    ref = ffn.moe_output(numerics.bf16_to_f64(x), ids, w, bank.expert64)
    check_layer(y, ref)


@pytest.mark.parametrize("T,E,k,H,I", [(130, 8, 2, 256, 128), (700, 16, 4, 512, 256)])
def test_prefill_fp8(T, E, k, H, I):
    b = binding()
    bank = Fp8Bank(70 + E, E, H, I)
    pool = _slots_identity(b, bank, b.W_FP8_B128)
    rng = np.random.default_rng(T + 1)
    x = gen.activations_bf16(rng, T, H)
    ids, w = route.topk_softmax(rng.standard_normal((T, E)).astype(np.float32), k)
    y = _run_forward(b, pool, x, ids, w, b.FWD_PREFILL)
    ref = ffn.moe_output(numerics.bf16_to_f64(x), ids, w, bank.expert64)
    check_layer(y, ref, "prefill fp8")


def test_prefill_bf16_full_shape_sampled():
    """Prefill BF16 workload (8192 tokens, H 2048, E 128, top-8, I 768), 64 sampled rows."""
    b = binding()
    c = CONFIGS["prefill_bf16"]
    bank = Bf16Bank(c.cfg_id, c.E, c.H, c.I)
    pool = _slots_identity(b, bank, b.W_BF16)
    x = gen.activations_bf16(gen.np_rng(c.cfg_id, gen.S_ACT), c.T, c.H)
    wr = gen.router_matrix(gen.np_rng(c.cfg_id, gen.S_ROUTER), c.H, c.E, c.router_std)
    lg = gen.router_logits(x, wr)
    ids_d, w_d = b.route_topk(dev(lg), c.k)
    ids, w = route.topk_softmax(lg, c.k)
    assert np.array_equal(ids_d.cpu().numpy(), ids)
    ws = b.forward_workspace(c.T, c.k, c.H, c.I, c.E, b.FWD_PREFILL)
    y = b.expert_forward(pool.c, dev(x), ids_d, w_d, b.FWD_PREFILL, ws).cpu().numpy()
    rows = np.random.default_rng(0).choice(c.T, 64, replace=False)
    ref = ffn.moe_output(numerics.bf16_to_f64(x[rows]), ids[rows], w[rows], bank.expert64)
    check_layer(y[rows], ref, "prefill bf16 full")


def test_prefill_fp8_full_shape_sampled():
    """Prefill FP8 workload layer (8192 tokens, H 7168, E 256, top-8 of x.W_r,
    I 2048, E4M3 with 128x128 scales), the first and the last token checked
    against the oracle, every output finite."""
    b = binding()
    c = CONFIGS["prefill_fp8"]
    bank = Fp8Bank(c.cfg_id, c.E, c.H, c.I, c.w_std, device="cuda", pin=False)
    pool = _slots_identity(b, bank, b.W_FP8_B128)
    x = gen.activations_bf16(gen.np_rng(c.cfg_id, gen.S_ACT), c.T, c.H)
    wr = gen.router_matrix(gen.np_rng(c.cfg_id, gen.S_ROUTER), c.H, c.E, c.router_std)
    lg = gen.router_logits(x, wr)
    ids_d, w_d = b.route_topk(dev(lg), c.k)
    ids, w = route.topk_softmax(lg, c.k)
    assert np.array_equal(ids_d.cpu().numpy(), ids)
    ws = b.forward_workspace(c.T, c.k, c.H, c.I, c.E, b.FWD_PREFILL)
    y = b.expert_forward(pool.c, dev(x), ids_d, w_d, b.FWD_PREFILL, ws).cpu().numpy()
    assert np.all(np.isfinite(y))
    rows = [0, c.T - 1]
    ref = ffn.moe_output(numerics.bf16_to_f64(x[rows]), ids[rows], w[rows], bank.expert64)
    check_layer(y[rows], ref, "prefill fp8 full")


def test_prefill_equals_decode_small_batch():
    b = binding()
    bank = Bf16Bank(43, 8, 256, 128)
    pool = _slots_identity(b, bank, b.W_BF16)
    rng = np.random.default_rng(4)
    x = gen.activations_bf16(rng, 8, 256)
    ids, w = route.topk_softmax(rng.standard_normal((8, 8)).astype(np.float32), 2)
    y1 = _run_forward(b, pool, x, ids, w, b.FWD_DECODE)
    y2 = _run_forward(b, pool, x, ids, w, b.FWD_PREFILL)
    ref = ffn.moe_output(numerics.bf16_to_f64(x), ids, w, bank.expert64)
    check_layer(y1, ref)
    check_layer(y2, ref)


# ---------------------------------------------------------------- merge
def test_merge_partial():
    b = binding()
    rng = np.random.default_rng(0)
    for T, H in [(1, 2048), (3, 7), (32, 256)]:
        yg = rng.standard_normal((T, H)).astype(np.float32)
        yh = rng.standard_normal((T, H)).astype(np.float32)
        yb = torch.empty((T, H), dtype=torch.uint16, device="cuda")
        out = b.merge_partial(dev(yg), dev(yh), y_out_bf16=yb).cpu().numpy()
        assert np.array_equal(out, yg + yh)                    # one float32 add: exact
        ref_b = torch.from_numpy(yg + yh).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(yb.cpu().numpy().view(np.uint16), ref_b)
    # host partial in pinned memory
    yh = pinned(np.ones((2, 64), np.float32))
    out = b.merge_partial(dev(np.zeros((2, 64), np.float32)), yh).cpu().numpy()
    assert np.all(out == 1)


# ---------------------------------------------------------------- the tiny workload end to end
def test_tiny_layer_end_to_end():
    """Route -> cache step (with fills) -> grouped evaluation -> merge with the
    host partial; compared to the oracle's exact layer output."""
    b = binding()
    c = CONFIGS["tiny"]
    bank = Bf16Bank(c.cfg_id, c.E, c.H, c.I)
    x = gen.activations_bf16(gen.np_rng(c.cfg_id, gen.S_ACT), c.T, c.H)
    wr = gen.router_matrix(gen.np_rng(c.cfg_id, gen.S_ROUTER), c.H, c.E, c.router_std)
    lg = gen.router_logits(x, wr)
    for T_step in (c.T, 1):                                # one 32-token step; 32 one-token steps
        pool = b.SlotPool(c.C, c.H, c.I, b.W_BF16)
        host = b.HostPoolTables(bank.host, lambda i: i, c.E)
        cache = b.Cache(c.L, c.E, c.k, T_step, pool, host, c.bp, c.bh)
        cache.seed(list(c.seed_slots))
        out = b.StepOut(T_step, c.k, c.E)
        orc = lru.ExpertCache(c.L, c.E, c.C, c.bp, c.bh)
        orc.seed(list(c.seed_slots))
        mode = b.FWD_DECODE if T_step <= 16 else b.FWD_PREFILL   # decode mode serves T <= 16
        ws = b.forward_workspace(T_step, c.k, c.H, c.I, c.C, mode)
        ys = []
        for t0 in range(0, c.T, T_step):
            lg_d = dev(lg[t0:t0 + T_step])
            ids_d, w_d = b.route_topk(lg_d, c.k)
            cache.step(0, ids_d, out)
            y_gpu = b.expert_forward(pool.c, dev(x[t0:t0 + T_step]), out.pick_slot.view(T_step, c.k), w_d,
                                     mode, ws)
            ids, w = route.topk_softmax(lg[t0:t0 + T_step], c.k)
            r = orc.step(0, ids)
            assert np.array_equal(out.pick_slot.cpu().numpy(), r.pick_slot.reshape(-1))
            yg_ref, yh_ref = oracle_partials(x[t0:t0 + T_step], ids, w, bank.expert64, r.pick_slot >= 0)
            check_layer(y_gpu.cpu().numpy(), yg_ref, "y_gpu")
            y = b.merge_partial(y_gpu, dev(yh_ref.astype(np.float32))).cpu().numpy()
            ys.append(y)
        y = np.concatenate(ys)
        ref = ffn.moe_output(numerics.bf16_to_f64(x), route.topk_softmax(lg, c.k)[0],
                             route.topk_softmax(lg, c.k)[1], bank.expert64)
        check_layer(y, ref, "tiny end to end")
        cache.destroy()


@pytest.mark.parametrize("wtype,H,I", [(0, 64, 32), (0, 256, 96), (1, 256, 128)])
def test_pack_matches_brick_format(wtype, H, I):
    """moe_pack_weights against the brick format stated in include/moe.h."""
    b = binding()
    rng = np.random.default_rng(H + I)
    dt = np.uint16 if wtype == 0 else np.uint8
    hi = 1 << 16 if wtype == 0 else 1 << 8
    n = 2
    wg = rng.integers(0, hi, (n, I, H), dtype=dt)
    wu = rng.integers(0, hi, (n, I, H), dtype=dt)
    wd = rng.integers(0, hi, (n, H, I), dtype=dt)
    gu, dp = b.pack_weights(wtype, dev(wg), dev(wu), dev(wd))
    gu, dp = gu.cpu().numpy(), dp.cpu().numpy()
    KB = 32 if wtype == 0 else 64
    per = KB // 4

    def brick_elem(N, K, t, kt, lane, e):
        return ((t * (K // KB) + kt) * 64 + lane) * per + e

    for ex in range(n):
        for row in range(0, 2 * I, 7):
            for col in range(0, H, 5):
                t, rr = row // 16, row % 16
                kt, j, e = col // KB, (col % KB) // per, col % per
                src = wg[ex, 8 * t + rr, col] if rr < 8 else wu[ex, 8 * t + rr - 8, col]
                assert gu[ex, brick_elem(2 * I, H, t, kt, 16 * j + rr, e)] == src
        for row in range(0, H, 3):
            for col in range(0, I, 7):
                t, rr = row // 16, row % 16
                kt, j, e = col // KB, (col % KB) // per, col % per
                assert dp[ex, brick_elem(H, I, t, kt, 16 * j + rr, e)] == wd[ex, row, col]


def test_stream_read_reads_every_word_once():
    """The measurement reference read folds every 32-bit word exactly once."""
    b = binding()
    for n16 in (1, 1000, 3 * 512 * 256 * 4 + 77):
        src = torch.randint(-2 ** 31, 2 ** 31 - 1, (n16 * 4,), dtype=torch.int32, device="cuda")
        sink = torch.zeros(256, dtype=torch.int32, device="cuda")
        b.stream_read(src, sink)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        ref = np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32))
        assert got == ref
