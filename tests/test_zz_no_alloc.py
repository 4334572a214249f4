"""The allocation-free decode entry point (moe_expert_forward_merge_static)
against the workspace entry point it shares its kernels with
(moe_expert_forward_merge): the same bits, on two calls in a row with the
second smaller, eagerly and replayed from a captured graph."""
import numpy as np
import pytest
import torch

from harness import gen
from oracle import route
from tests.layer_setup import binding, dev, Bf16Bank, Fp8Bank

pytestmark = pytest.mark.gpu


def _pool(b, bank, wtype):
    pool = b.SlotPool(bank.E, bank.H, bank.I, wtype)
    bank.load_slots(pool, {e: e for e in range(bank.E)})
    return pool


def _inputs(rng, T, E, k, H):
    x = dev(gen.activations_bf16(rng, T, H))
    ids, w = route.topk_softmax(rng.standard_normal((T, E)).astype(np.float32), k)
    pick = np.where(rng.random(ids.shape) < 0.8, ids, -1).astype(np.int32)
    yh = torch.randn((T, H), dtype=torch.float32, device="cuda")
    return x, dev(pick), dev(w.astype(np.float32)), yh


def _both(b, pool, x, pick, w, yh):
    T, k = pick.shape
    ws = b.forward_workspace(T, k, pool.H, pool.I, pool.n_slots, b.FWD_DECODE)
    ref_g = torch.empty((T, pool.H), dtype=torch.float32, device="cuda")
    ref_b = torch.empty((T, pool.H), dtype=torch.uint16, device="cuda")
    ref = b.expert_forward_merge(pool.c, x, pick, w, b.FWD_DECODE, ws, yh, y_gpu=ref_g, y_out_bf16=ref_b)
    got_g = torch.full((T, pool.H), float("nan"), dtype=torch.float32, device="cuda")
    got_b = torch.empty((T, pool.H), dtype=torch.uint16, device="cuda")
    got = b.expert_forward_merge_static(pool.c, x, pick, w, yh, y_gpu=got_g, y_out_bf16=got_b)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))
    assert torch.equal(got_g.view(torch.int32), ref_g.view(torch.int32))
    assert torch.equal(got_b, ref_b)
    assert int(ws[:4].view(torch.int32).item()) == 0


@pytest.mark.parametrize("wtype", [0, 1])
def test_static_scratch_equals_workspace_entry_point(wtype):
    """Two calls in a row on the static scratch, the second with fewer tokens
    and picks, each equal bit for bit to the workspace entry point."""
    b = binding()
    rng = np.random.default_rng(11 + wtype)
    if wtype == 0:
        E, H, I = 24, 2048, 768
        bank = Bf16Bank(95, E, H, I)
    else:
        E, H, I = 16, 512, 384
        bank = Fp8Bank(96, E, H, I)
    pool = _pool(b, bank, wtype)
    _both(b, pool, *_inputs(rng, 16, E, 8, H))              # the largest decode batch
    _both(b, pool, *_inputs(rng, 3, E, 4, H))               # then a smaller one
    _both(b, pool, *_inputs(rng, 1, E, 2, H))


def test_static_scratch_in_a_graph():
    """Captured once and replayed with new inputs, eager calls of both entry
    points and synchronisations in between: every replay equals the
    workspace entry point on the same inputs."""
    b = binding()
    E, H, I, T, k = 16, 1024, 256, 4, 4
    bank = Bf16Bank(97, E, H, I)
    pool = _pool(b, bank, 0)
    rng = np.random.default_rng(3)
    x, pick, w, yh = _inputs(rng, T, E, k, H)
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    b.expert_forward_merge_static(pool.c, x, pick, w, yh, y_out=y)   # first call on the device: outside capture
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            b.expert_forward_merge_static(pool.c, x, pick, w, yh, y_out=y)
    torch.cuda.current_stream().wait_stream(s)
    ws = b.forward_workspace(T, k, H, I, E, b.FWD_DECODE)
    for rep in range(4):
        x2, pick2, w2, yh2 = _inputs(rng, T, E, k, H)
        for dst, src in ((x, x2), (pick, pick2), (w, w2), (yh, yh2)):
            dst.copy_(src)
        _both(b, pool, *_inputs(rng, 2, E, k, H))             # other eager work on the same scratch
        g.replay()
        torch.cuda.synchronize()
        ref = b.expert_forward_merge(pool.c, x, pick, w, b.FWD_DECODE, ws, yh)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), ref.view(torch.int32)), rep


def test_static_scratch_size_limit():
    """A call whose h does not fit the 8 MiB scratch is refused on the host."""
    b = binding()
    E, H, I, T, k = 72, 128, 4096, 9, 8                   # h: 72 x 16 x 4096 BF16 = 9 MiB
    pool = b.SlotPool(E, H, I, b.W_BF16)
    x = torch.zeros((T, H), dtype=torch.uint16, device="cuda")
    pick = torch.arange(T * k, dtype=torch.int32, device="cuda").view(T, k)
    w = torch.full((T, k), 1.0 / k, device="cuda")
    yh = torch.zeros((T, H), dtype=torch.float32, device="cuda")
    with pytest.raises(b.MoeError) as ei:
        b.expert_forward_merge_static(pool.c, x, pick, w, yh)
    assert ei.value.status == -3                          # MOE_ERR_NO_SPACE
