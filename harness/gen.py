"""Seeded generators of synthetic inputs (no method arithmetic lives here).

Random streams: ``np_rng(cfg_id, stream, *extra)`` is
``Generator(PCG64(SeedSequence([2026, cfg_id, stream, *extra])))`` with

    stream 0  expert weights        stream 3  sticky routing trace
    stream 1  activations           stream 4  gate logits of the trace
    stream 2  router matrix

Large banks (the FP8 workloads, 11 GB per layer) are drawn with torch's
generator on the device that will hold them, seeded from the same
SeedSequence; both the library under test and the oracle then read the very
same bytes.

Conventions:
* BF16 values are carried as uint16 bit patterns, rounded from float32 with
  round-to-nearest-even (torch's ``to(bfloat16)``).
* FP8 values are OCP E4M3FN codes (uint8) with one float32 scale per
  128 x 128 tile of the stored [out, in] matrix.  The quantiser below is an
  input generator: scale = amax(tile) / 448, code = RNE(clamp(w / scale)).
* Weight matrices are stored [out, in] row-major: W_gate, W_up are [I, H],
  W_down is [H, I].
"""
from __future__ import annotations

import numpy as np
import torch

S_WEIGHTS, S_ACT, S_ROUTER, S_TRACE, S_GATE = 0, 1, 2, 3, 4
E4M3_MAX = 448.0


def seed_words(cfg_id: int, stream: int, *extra: int) -> list:
    return [2026, int(cfg_id), int(stream), *[int(e) for e in extra]]


def np_rng(cfg_id: int, stream: int, *extra: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed_words(cfg_id, stream, *extra))))


def torch_seed(cfg_id: int, stream: int, *extra: int) -> int:
    ss = np.random.SeedSequence(seed_words(cfg_id, stream, *extra))
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


# ----------------------------------------------------------------- BF16 plumbing
def to_bf16_bits(a) -> np.ndarray:
    """float array -> uint16 BF16 bit patterns (float32 first, then RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float32)))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_as_f32(bits: np.ndarray) -> np.ndarray:
    """uint16 BF16 patterns -> float32 values (placing the 16 bits on top)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------- weights
def expert_bf16(rng: np.random.Generator, H: int, I: int, std: float):
    """One expert: (W_gate [I,H], W_up [I,H], W_down [H,I]) as BF16 bits. Draw order gate, up, down."""
    g = to_bf16_bits(rng.standard_normal((I, H), dtype=np.float32) * np.float32(std))
    u = to_bf16_bits(rng.standard_normal((I, H), dtype=np.float32) * np.float32(std))
    d = to_bf16_bits(rng.standard_normal((H, I), dtype=np.float32) * np.float32(std))
    return g, u, d


def bank_bf16(cfg_id: int, E: int, H: int, I: int, std: float, layer: int = 0):
    """E experts drawn one after another from stream 0 (extra word: layer)."""
    rng = np_rng(cfg_id, S_WEIGHTS, layer)
    wg = np.empty((E, I, H), np.uint16)
    wu = np.empty((E, I, H), np.uint16)
    wd = np.empty((E, H, I), np.uint16)
    for e in range(E):
        wg[e], wu[e], wd[e] = expert_bf16(rng, H, I, std)
    return wg, wu, wd


def quantize_e4m3_b128(w: torch.Tensor, block: int = 128):
    """float32 [R, Cc] -> (codes uint8 [R, Cc], scales float32 [R/b, Cc/b]).

    scale = amax(|tile|) / 448 (an all-zero tile gets scale 1); codes are the
    round-to-nearest-even E4M3FN encoding of clamp(w / scale, +-448)."""
    R, Cc = w.shape
    assert R % block == 0 and Cc % block == 0
    t = w.reshape(R // block, block, Cc // block, block)
    amax = t.abs().amax(dim=(1, 3)).to(torch.float32)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    q = (t / scale[:, None, :, None]).clamp_(-E4M3_MAX, E4M3_MAX)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(R, Cc)
    return codes, scale.contiguous()


def expert_fp8_torch(seed: int, H: int, I: int, std: float, device="cpu", block: int = 128):
    """One FP8 expert drawn with torch's generator on `device`.

    Returns dict of torch tensors: gate/up codes [I,H], down codes [H,I]
    (uint8) and their scales [I/128,H/128], [I/128,H/128], [H/128,I/128]."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = {}
    for name, shape in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        w = torch.empty(shape, dtype=torch.float32, device=device).normal_(0.0, std, generator=gen)
        out[name], out["s_" + name] = quantize_e4m3_b128(w, block)
        del w
    return out


def expert_fp8_np(rng: np.random.Generator, H: int, I: int, std: float, block: int = 128):
    """Small-shape FP8 expert from a numpy stream (CPU tests): same quantiser."""
    out = {}
    for name, shape in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        w = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))
        c, s = quantize_e4m3_b128(w, block)
        out[name], out["s_" + name] = c.numpy(), s.numpy()
    return out


# ----------------------------------------------------------------- activations / router
def activations_bf16(rng: np.random.Generator, T: int, H: int) -> np.ndarray:
    return to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))


def router_matrix(rng: np.random.Generator, H: int, E: int, std: float) -> np.ndarray:
    return (rng.standard_normal((H, E)) * std).astype(np.float32)


def router_logits(x_bits: np.ndarray, w_r: np.ndarray) -> np.ndarray:
    """logits = float32(x . W_r), the product formed in float64 and rounded once."""
    x = bf16_bits_as_f32(x_bits).astype(np.float64)
    return (x @ w_r.astype(np.float64)).astype(np.float32)


# ----------------------------------------------------------------- sticky routing traces
def sticky_trace(rng: np.random.Generator, steps: int, E: int, k: int, p: float) -> np.ndarray:
    """[steps, k] int32 expert picks of one sequence at one layer.

    Step 0: k distinct experts, uniform.  Step t: pick j keeps the previous
    step's expert with probability p (independently per pick); the picks not
    kept are redrawn in order j = 0..k-1, each uniformly among the experts not
    yet in this step's set (the dropped expert is eligible again)."""
    out = np.empty((steps, k), np.int32)
    out[0] = rng.choice(E, size=k, replace=False)
    for t in range(1, steps):
        keep = rng.random(k) < p
        cur = np.where(keep, out[t - 1], -1)
        used = set(int(v) for v in cur[keep])
        for j in range(k):
            if not keep[j]:
                r = int(rng.integers(0, E - len(used)))
                # the r-th expert (ascending) not in `used`
                for u in sorted(used):
                    if u <= r:
                        r += 1
                    else:
                        break
                cur[j] = r
                used.add(r)
        out[t] = cur
    return out


def synth_logits(rng: np.random.Generator, picks: np.ndarray, E: int) -> np.ndarray:
    """Router logits whose top-k are exactly `picks` ([n, k]).

    Picked experts get 16 + z (z ~ N(0,1)); all others get N(0,1) clipped to
    +-6.  Softmax over the picks then equals softmax(z) up to float32
    rounding of the logits."""
    n, k = picks.shape
    z = rng.standard_normal((n, k))
    lg = np.clip(rng.standard_normal((n, E)), -6.0, 6.0)
    rows = np.repeat(np.arange(n), k)
    lg[rows, picks.reshape(-1)] = 16.0 + z.reshape(-1)
    return lg.astype(np.float32)


def decode_trace(cfg_id: int, L: int, steps: int, E: int, k: int, p: float, T: int = 1, salt: int = 0):
    """Sticky traces for every (layer, sequence) and their logits.

    Returns picks [steps, L, T, k] int32 and logits [steps, L, T, E] float32."""
    picks = np.empty((steps, L, T, k), np.int32)
    for layer in range(L):
        for s in range(T):
            picks[:, layer, s, :] = sticky_trace(np_rng(cfg_id, S_TRACE, salt, layer, s), steps, E, k, p)
    logits = np.empty((steps, L, T, E), np.float32)
    for layer in range(L):
        rng = np_rng(cfg_id, S_GATE, salt, layer)
        logits[:, layer] = synth_logits(rng, picks[:, layer].reshape(steps * T, k), E).reshape(steps, T, E)
    return picks, logits


def alias_base_expert(layer: int, e: int, E: int, stride: int) -> int:
    """Host-bank aliasing of the decode BF16 pool: logical (l, e) -> base expert."""
    return (e + stride * layer) % E
