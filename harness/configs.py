"""The five synthetic workloads, as data.

Bandwidths B_P (pinned-memory expert transfer) and B_H (host expert
processing) are integers in units of 0.1 GB/s, so 11.8:47.5 GB/s is 118:475.
The two ratios are the measured pairs quoted for a laptop and a server on the
FreeToken pages (the worked example of the q* policy, section "execution order
and engineering details").
"""
from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class TinyCfg:
    """Tiny layer: 32 tokens, hidden 256, 8 experts, top-2, intermediate 128."""
    name: str = "tiny"
    cfg_id: int = 1
    T: int = 32
    H: int = 256
    I: int = 128
    E: int = 8
    k: int = 2
    L: int = 1
    C: int = 4
    seed_slots: Tuple[int, ...] = (0, 1, 2, 3)
    bp: int = 118
    bh: int = 475
    w_std: float = 0.02
    router_std: float = 1.0 / 16.0          # 1/sqrt(H), read as a standard deviation


@dataclass(frozen=True)
class DecodeBF16Cfg:
    """Decode trace: batch 1, 40 layers x 512 steps, H 2048, E 128, top-8, I 768."""
    name: str = "decode_bf16"
    cfg_id: int = 2
    T: int = 1
    L: int = 40
    steps: int = 512
    H: int = 2048
    I: int = 768
    E: int = 128
    k: int = 8
    p_keep: float = 0.6
    capacity: float = 0.37
    bp: int = 527
    bh: int = 773
    w_std: float = 0.02
    alias_stride: int = 17                  # logical (l, e) -> base expert (e + 17 l) mod E

    @property
    def C(self) -> int:
        return int(self.capacity * self.L * self.E)   # floor(0.37 * 5120) = 1894


@dataclass(frozen=True)
class DecodeFP8Cfg:
    """Decode, FP8: T in {1,4,16}, H 7168, E 256, top-8, I 2048, 58-layer pool at 11%."""
    name: str = "decode_fp8"
    cfg_id: int = 3
    Ts: Tuple[int, ...] = (1, 4, 16)
    L: int = 58
    steps: int = 512
    H: int = 7168
    I: int = 2048
    E: int = 256
    k: int = 8
    p_keep: float = 0.5
    capacity: float = 0.11
    bp: int = 118
    bh: int = 475
    w_std: float = 0.02
    block: int = 128

    @property
    def C(self) -> int:
        return int(self.capacity * self.L * self.E)   # floor(0.11 * 14848) = 1633


@dataclass(frozen=True)
class PrefillBF16Cfg:
    """Prefill chunk: 8192 tokens, H 2048, E 128, top-8, I 768, all experts resident."""
    name: str = "prefill_bf16"
    cfg_id: int = 4
    T: int = 8192
    H: int = 2048
    I: int = 768
    E: int = 128
    k: int = 8
    w_std: float = 0.02

    @property
    def router_std(self) -> float:
        return self.H ** -0.5


@dataclass(frozen=True)
class PrefillFP8Cfg:
    """Prefill, FP8, double-buffered: 8192 tokens, 4 layers, H 7168, E 256, I 2048."""
    name: str = "prefill_fp8"
    cfg_id: int = 5
    T: int = 8192
    layers: int = 4
    H: int = 7168
    I: int = 2048
    E: int = 256
    k: int = 8
    w_std: float = 0.02
    block: int = 128

    @property
    def router_std(self) -> float:
        return self.H ** -0.5


CONFIGS = {
    "tiny": TinyCfg(),
    "decode_bf16": DecodeBF16Cfg(),
    "decode_fp8": DecodeFP8Cfg(),
    "prefill_bf16": PrefillBF16Cfg(),
    "prefill_fp8": PrefillFP8Cfg(),
}
