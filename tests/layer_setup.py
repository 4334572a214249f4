"""Shared set-up for the GPU parity tests: inputs from harness/, expectations
from oracle/, results from the HIP library through its C ABI binding."""
import numpy as np
import torch

from harness import gen
from oracle import numerics, ffn

REL_L2 = 5e-3        # layer-output tolerances
MAX_ABS = 2e-2       # times max |ref|
W_ABS = 1e-6         # router weights


def binding():
    import routed_expert_cache_amd.binding as b
    return b


def pinned(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).pin_memory()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def check_layer(y, ref, what=""):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    mref = np.abs(ref).max()
    if mref == 0:
        assert np.abs(y).max() == 0, what
        return 0.0
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    mab = np.abs(y - ref).max() / mref
    assert rel <= REL_L2 and mab <= MAX_ABS, "%s rel_l2=%.3g max_abs/max=%.3g" % (what, rel, mab)
    return rel


def pack_to_host(wtype, wg, wu, wd, chunk=16, pin=True):
    """Pack row-major expert weights (torch, any device) into brick banks with
    the library's pack call; returns host tensors (pinned) [E, 2IH], [E, HI]."""
    b = binding()
    E, I, H = wg.shape
    gu = torch.empty((E, 2 * I * H), dtype=wg.dtype, pin_memory=pin)
    dp = torch.empty((E, H * I), dtype=wg.dtype, pin_memory=pin)
    for e0 in range(0, E, chunk):
        e1 = min(E, e0 + chunk)
        g_d, u_d, d_d = (t[e0:e1].cuda() for t in (wg, wu, wd))
        pg, pd = b.pack_weights(wtype, g_d, u_d, d_d)
        gu[e0:e1].copy_(pg)
        dp[e0:e1].copy_(pd)
    torch.cuda.synchronize()
    return gu, dp


class Bf16Bank:
    """E experts in BF16: row-major bits for the oracle, packed pinned banks for the library."""

    def __init__(self, cfg_id, E, H, I, std=0.02, layer=0):
        self.E, self.H, self.I = E, H, I
        self.wg, self.wu, self.wd = gen.bank_bf16(cfg_id, E, H, I, std, layer)
        t = [torch.from_numpy(a) for a in (self.wg, self.wu, self.wd)]
        self.host = list(pack_to_host(0, *t))
        self._cache = {}

    def expert64(self, e):
        if e not in self._cache:
            self._cache[e] = (numerics.bf16_to_f64(self.wg[e]), numerics.bf16_to_f64(self.wu[e]),
                              numerics.bf16_to_f64(self.wd[e]))
        return self._cache[e]

    def load_slots(self, pool, slot_of_expert):
        """Copy expert e's packed bytes into slot slot_of_expert[e] of a SlotPool."""
        for e, s in slot_of_expert.items():
            pool.w_gu[s].copy_(self.host[0][e])
            pool.w_down[s].copy_(self.host[1][e])


class Fp8Bank:
    """E FP8 experts (codes + 128x128 scales) drawn on `device`; row-major for the
    oracle, packed pinned banks (+ scales) for the library."""

    def __init__(self, cfg_id, E, H, I, std=0.02, layer=0, device="cpu", pin=True):
        self.E, self.H, self.I = E, H, I
        names = ("gate", "up", "down", "s_gate", "s_up", "s_down")
        shapes = [(E, I, H), (E, I, H), (E, H, I), (E, I // 128, H // 128), (E, I // 128, H // 128),
                  (E, H // 128, I // 128)]
        dts = [torch.uint8] * 3 + [torch.float32] * 3
        self.t = {n: torch.empty(s, dtype=d, pin_memory=pin) if pin else torch.empty(s, dtype=d)
                  for n, s, d in zip(names, shapes, dts)}
        for e in range(E):
            ex = gen.expert_fp8_torch(gen.torch_seed(cfg_id, gen.S_WEIGHTS, layer, e), H, I, std, device=device)
            for n in names:
                self.t[n][e].copy_(ex[n])
        self.repack(pin)
        self._cache = {}

    def repack(self, pin=True):
        gu, dp = pack_to_host(1, self.t["gate"], self.t["up"], self.t["down"], pin=pin)
        self.host = [gu, dp, self.t["s_gate"], self.t["s_up"], self.t["s_down"]]

    def expert64(self, e):
        if e not in self._cache:
            t = self.t
            self._cache[e] = (numerics.dequant_b128(t["gate"][e].numpy(), t["s_gate"][e].numpy()),
                              numerics.dequant_b128(t["up"][e].numpy(), t["s_up"][e].numpy()),
                              numerics.dequant_b128(t["down"][e].numpy(), t["s_down"][e].numpy()))
        return self._cache[e]

    def drop(self, e):
        self._cache.pop(e, None)

    def load_slots(self, pool, slot_of_expert):
        for e, s in slot_of_expert.items():
            pool.w_gu[s].copy_(self.host[0][e])
            pool.w_down[s].copy_(self.host[1][e])
            pool.s_gate[s].copy_(self.t["s_gate"][e])
            pool.s_up[s].copy_(self.t["s_up"][e])
            pool.s_down[s].copy_(self.t["s_down"][e])


def oracle_partials(x_bits, ids, w, expert64, on_gpu):
    return ffn.moe_partials(numerics.bf16_to_f64(x_bits), ids, w, expert64, on_gpu=on_gpu)
