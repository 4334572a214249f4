"""Checks of the seeded input generators (no GPU)."""
import numpy as np
import torch

from harness import gen, CONFIGS
from oracle import route, numerics


def test_sticky_trace_statistics():
    E, k, p, steps = 128, 8, 0.6, 3000
    tr = gen.sticky_trace(gen.np_rng(2, gen.S_TRACE, 99), steps, E, k, p)
    assert tr.shape == (steps, k)
    for row in tr:
        assert len(set(row.tolist())) == k                  # no duplicate picks
    kept = (tr[1:] == tr[:-1]).mean()
    # a redrawn pick lands on its old expert with probability ~1/(E-k+1)
    expect = p + (1 - p) / (E - k)
    sigma = np.sqrt(expect * (1 - expect) / ((steps - 1) * k))
    assert abs(kept - expect) < 4 * sigma
    # redraws are uniform: every expert appears
    assert len(np.unique(tr)) == E
    # reproducible from the seed
    tr2 = gen.sticky_trace(gen.np_rng(2, gen.S_TRACE, 99), steps, E, k, p)
    assert np.array_equal(tr, tr2)


def test_synth_logits_route_to_picks():
    rng = gen.np_rng(2, gen.S_TRACE, 5)
    picks = gen.sticky_trace(rng, 200, 128, 8, 0.6)
    lg = gen.synth_logits(gen.np_rng(2, gen.S_GATE, 5), picks, 128)
    ids, w = route.topk_softmax(lg, 8)
    for t in range(200):
        assert sorted(ids[t].tolist()) == sorted(picks[t].tolist())


def test_quantiser_properties():
    rng = np.random.default_rng(0)
    w = torch.from_numpy(rng.standard_normal((256, 384), dtype=np.float32) * np.float32(0.02))
    codes, scales = gen.quantize_e4m3_b128(w)
    assert codes.dtype == torch.uint8 and scales.shape == (2, 3)
    c = codes.numpy()
    assert not np.any((c & 0x7F) == 0x7F)                   # never NaN
    deq = numerics.dequant_b128(c, scales.numpy())
    # each tile's amax maps to +-448 exactly (up to the scale's rounding)
    for bi in range(2):
        for bj in range(3):
            tile = np.abs(deq[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128])
            assert abs(tile.max() / float(scales[bi, bj]) - 448) < 1e-3
    rel = np.abs(deq - w.numpy().astype(np.float64)) / np.abs(w.numpy()).max()
    assert rel.max() < 2 ** -4


def test_bf16_rounding_is_rne():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5], np.float32)
    bits = gen.to_bf16_bits(vals)
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020]


def test_configs_shapes():
    assert CONFIGS["decode_bf16"].C == 1894
    assert CONFIGS["decode_fp8"].C == 1633
    assert CONFIGS["tiny"].C == 4


def test_router_logits_rounded_once():
    rng = gen.np_rng(1, gen.S_ACT)
    x = gen.activations_bf16(rng, 4, 256)
    wr = gen.router_matrix(gen.np_rng(1, gen.S_ROUTER), 256, 8, 1 / 16)
    lg = gen.router_logits(x, wr)
    ref = (numerics.bf16_to_f64(x) @ wr.astype(np.float64)).astype(np.float32)
    assert np.array_equal(lg, ref)
