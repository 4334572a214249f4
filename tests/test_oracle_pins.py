"""Pins of the CPU oracle to what the pages and mathematics fix (no GPU).

Each test names the passage or the mathematical fact it checks.  None of them
re-types the oracle's own formula as its expectation: expectations come from
values the pages print (tests/golden), exact rational arithmetic, closed
forms of special cases, independent library routines, or brute force.
"""
import math
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import numerics, route, qsplit, ffn
from tests.conftest import golden


# ---------------------------------------------------------------- q* split
def test_qstar_worked_examples_from_pages():
    g = golden("qstar_worked_examples.json")
    for c in g["cases"]:
        q = qsplit.q_star(c["m"], c["bp"], c["bh"])
        assert q == c["fills"], c["cite"]
        assert c["m"] - q == c["host"], c["cite"]
        # the printed approximate value of m*B_P/B_H
        assert abs(c["m"] * c["bp"] / c["bh"] - c["q_star_approx"]) < 0.05


@pytest.mark.parametrize("bp,bh", [(118, 475), (527, 773), (3, 10), (1, 1000)])
def test_qstar_balances_branch_times_exactly(bp, bh):
    """At q = m B_P / B_H the fill branch q S / B_P equals the host branch
    (m - q) S / (B_H - B_P) exactly (rational arithmetic), and the integer
    q* is within 1/2 of it unless the [1, m] clamp binds."""
    S = Fraction(44_050_944)
    for m in range(1, 130):
        q = Fraction(m * bp, bh)
        assert q * S / bp == (m - q) * S / (bh - bp)
        qi = qsplit.q_star(m, bp, bh)
        assert 1 <= qi <= m
        if 1 <= q <= m:
            assert abs(qi - q) <= Fraction(1, 2)
        elif q < 1:
            assert qi == 1          # at least one fill


def test_qstar_residual_zero_sends_all_to_transfer():
    """B_H <= B_P: residual max(B_H - B_P, 0) = 0, every miss is filled."""
    for m in range(0, 40):
        for bp, bh in [(773, 773), (900, 475), (475, 118)]:
            assert qsplit.q_star(m, bp, bh) == m


def test_qstar_special_values():
    assert qsplit.q_star(0, 118, 475) == 0
    assert qsplit.q_star(1, 118, 475) == 1          # rounds to 0, lifted to one fill
    assert qsplit.q_star(5, 0, 475) == 1            # no link bandwidth still keeps one fill
    with pytest.raises(ValueError):
        qsplit.q_star(3, 118, 0)


def test_qstar_table_by_exact_rounding():
    """Independent exact table: floor(m*bp/bh + 1/2) with Fraction, clamped."""
    expect = {
        (118, 475): {1: 1, 2: 1, 3: 1, 4: 1, 5: 1, 6: 1, 7: 2, 8: 2, 12: 3, 16: 4, 32: 8, 64: 16, 128: 32},
        (527, 773): {1: 1, 2: 1, 3: 2, 4: 3, 5: 3, 6: 4, 7: 5, 8: 5, 12: 8, 16: 11, 32: 22, 64: 44, 128: 87},
    }
    for (bp, bh), tab in expect.items():
        for m, q in tab.items():
            assert qsplit.q_star(m, bp, bh) == q, (bp, bh, m)
            assert math.floor(Fraction(m * bp, bh) + Fraction(1, 2)) in (q, 0)


# ---------------------------------------------------------------- E4M3 / BF16
def test_e4m3_all_codes_match_torch():
    """All 256 codes against torch.float8_e4m3fn -> float64 (library routine)."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = numerics.e4m3_to_f64(np.arange(256))
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


def test_e4m3_ocp_golden_values():
    g = golden("e4m3_ocp_values.json")["values"]
    for code, val in g.items():
        v = numerics.e4m3_to_f64(np.array([int(code, 16)]))[0]
        if val == "nan":
            assert np.isnan(v)
        else:
            assert v == val and np.signbit(v) == np.signbit(val), code


def test_e4m3_values_exact_in_bf16():
    """Every finite E4M3 value is exactly a BF16 value (so the expansion is unique)."""
    v = numerics.e4m3_to_f64(np.arange(256))
    v = v[~np.isnan(v)]
    bf = torch.from_numpy(v).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf, v)


def test_page_bias_trick_exact_on_normal_codes_only():
    """[OSDI] section 4.2: adding the exponent-bias difference 120 and
    zero-filling the mantissa gives the BF16 of a *normal* E4M3 code.  The
    literal trick is wrong for e = 0 codes (zero, subnormals) and the NaNs:
    18 codes in all."""
    wrong = []
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        bits = (s << 15) | ((e + 120) << 7) | (m << 4)
        val = numerics.bf16_to_f64(np.array([bits], np.uint16))[0]
        ref = numerics.e4m3_to_f64(np.array([c]))[0]
        if not (val == ref or (np.isnan(val) and np.isnan(ref))):
            wrong.append(c)
    assert len(wrong) == 18
    assert all(((c >> 3) & 15) == 0 or (c & 0x7F) == 0x7F for c in wrong)


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, 5000, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = numerics.bf16_to_f64(bits)
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok]) and np.array_equal(np.isnan(ref), np.isnan(got))


def test_dequant_tile_indexing():
    """The scale of element (r, c) is the one of tile (r // 128, c // 128):
    codes all 1.0 (0x38) with distinct scales reproduce the scale map."""
    R, Cc = 256, 384
    codes = np.full((R, Cc), 0x38, np.uint8)
    scales = (np.arange(6, dtype=np.float32).reshape(2, 3) + 1.0) * 0.5
    w = numerics.dequant_b128(codes, scales)
    assert w[0, 0] == 0.5 and w[127, 127] == 0.5 and w[0, 128] == 1.0
    assert w[128, 0] == 2.0 and w[255, 383] == 3.0 and w[200, 300] == 3.0


def test_post_scaling_identity_exact():
    """[OSDI] section 4.2: scale * sum(w x) == sum(scale * w * x) for a scale
    shared by the block, exactly in rational arithmetic."""
    rng = random.Random(5)
    for _ in range(20):
        scale = Fraction(rng.randint(1, 1 << 20), 1 << 30)
        codes = [rng.randrange(256) for _ in range(128)]
        codes = [c for c in codes if (c & 0x7F) != 0x7F]
        w = [Fraction(float(numerics.e4m3_to_f64(np.array([c]))[0])) for c in codes]
        x = [Fraction(rng.randint(-(1 << 8), 1 << 8), 1 << 7) for _ in codes]
        assert scale * sum(a * b for a, b in zip(w, x)) == sum(scale * a * b for a, b in zip(w, x))


# ---------------------------------------------------------------- routing
def _brute_topk(row, k):
    """Repeatedly take the largest remaining logit, lowest index on ties."""
    left = list(range(len(row)))
    out = []
    for _ in range(k):
        best = left[0]
        for e in left[1:]:
            if row[e] > row[best]:
                best = e
        out.append(best)
        left.remove(best)
    return out


def test_topk_matches_brute_force_with_ties():
    rng = np.random.default_rng(1)
    lg = rng.integers(-3, 4, size=(300, 16)).astype(np.float32)   # many ties
    ids, w = route.topk_softmax(lg, 5)
    for t in range(lg.shape[0]):
        assert list(ids[t]) == _brute_topk(lg[t], 5)


def test_topk_weights_are_renormalised_full_softmax():
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((200, 64)).astype(np.float32) * 3
    ids, w = route.topk_softmax(lg, 8)
    full = torch.softmax(torch.from_numpy(lg).double(), dim=1).numpy()
    sel = np.take_along_axis(full, ids, axis=1)
    ref = sel / sel.sum(axis=1, keepdims=True)
    assert np.allclose(w, ref, rtol=1e-12, atol=0)
    assert np.allclose(w.sum(1), 1.0, atol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 0)          # rank order = weight order


def test_topk_k_equals_E_and_k1():
    lg = np.array([[0.5, 2.0, 2.0, -1.0]], np.float32)
    ids, w = route.topk_softmax(lg, 1)
    assert ids.tolist() == [[1]] and w.tolist() == [[1.0]]
    ids, w = route.topk_softmax(lg, 4)
    assert ids.tolist() == [[1, 2, 0, 3]]
    assert w[0, 0] == w[0, 1]


# ---------------------------------------------------------------- FFN
def test_silu_closed_forms():
    a = np.linspace(-30, 30, 601)
    s = ffn.silu(a)
    assert ffn.silu(np.array([0.0]))[0] == 0.0
    assert np.allclose(s - ffn.silu(-a), a, rtol=0, atol=1e-12)   # silu(a) - silu(-a) = a
    assert abs(ffn.silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert np.allclose(torch.nn.functional.silu(torch.from_numpy(a)).numpy(), s, rtol=1e-15, atol=1e-300)


def test_ffn_hand_computed_scalar():
    """H = I = 1, x = 1, W_gate = 1, W_up = 2, W_down = 3:
    y = 3 * silu(1) * 2 = 6 / (1 + e^-1)."""
    y = ffn.expert_ffn(np.array([[1.0]]), np.array([[1.0]]), np.array([[2.0]]), np.array([[3.0]]))
    assert abs(y[0, 0] - 6.0 / (1.0 + math.exp(-1.0))) < 1e-15


def test_ffn_permutation_closed_form():
    """W_gate = P_g diag(a), W_up = P_u diag(b), W_down = P_d diag(c) with
    distinct permutations: y[P_d[i]] = c_i * silu(a_j x_j) * (b_l x_l) where the
    row i of h is (gate row i, up row i).  Catches transposed operands and
    swapped gate / up."""
    rng = np.random.default_rng(3)
    n = 7
    x = rng.standard_normal((1, n))
    a, b, c = rng.standard_normal(n), rng.standard_normal(n), rng.standard_normal(n)
    pg, pu, pd = rng.permutation(n), rng.permutation(n), rng.permutation(n)
    Wg = np.zeros((n, n)); Wu = np.zeros((n, n)); Wd = np.zeros((n, n))
    for i in range(n):
        Wg[i, pg[i]] = a[i]        # gate row i reads x[pg[i]]
        Wu[i, pu[i]] = b[i]        # up row i reads x[pu[i]]
        Wd[pd[i], i] = c[i]        # output pd[i] reads h[i]
    y = ffn.expert_ffn(x, Wg, Wu, Wd)[0]
    ref = np.zeros(n)
    for i in range(n):
        g = a[i] * x[0, pg[i]]
        u = b[i] * x[0, pu[i]]
        ref[pd[i]] = c[i] * (g / (1 + math.exp(-g))) * u
    assert np.allclose(y, ref, rtol=1e-14, atol=1e-15)


def test_ffn_rank_one_closed_form():
    """W_gate = p q^T, W_up = r s^T: h = silu(p (q.x)) * r (s.x); W_down = e_0 v^T."""
    rng = np.random.default_rng(4)
    H, I = 9, 5
    p, q, r, s, v = (rng.standard_normal(n) for n in (I, H, I, H, I))
    x = rng.standard_normal(H)
    Wd = np.zeros((H, I)); Wd[3] = v
    y = ffn.expert_ffn(x[None], np.outer(p, q), np.outer(r, s), Wd)[0]
    gq, us = float(q @ x), float(s @ x)
    h = [(p[i] * gq) / (1 + math.exp(-p[i] * gq)) * r[i] * us for i in range(I)]
    assert abs(y[3] - math.fsum(v[i] * h[i] for i in range(I))) < 1e-12
    assert np.all(y[np.arange(H) != 3] == 0)


def test_ffn_brute_force_loops():
    """Tiny random shapes: explicit fsum loops over the definition."""
    rng = np.random.default_rng(6)
    H, I, n = 6, 4, 3
    x = rng.standard_normal((n, H))
    Wg, Wu, Wd = rng.standard_normal((I, H)), rng.standard_normal((I, H)), rng.standard_normal((H, I))
    y = ffn.expert_ffn(x, Wg, Wu, Wd)
    for t in range(n):
        h = []
        for i in range(I):
            g = math.fsum(Wg[i, c] * x[t, c] for c in range(H))
            u = math.fsum(Wu[i, c] * x[t, c] for c in range(H))
            h.append(g / (1 + math.exp(-g)) * u)
        for o in range(H):
            assert abs(y[t, o] - math.fsum(Wd[o, i] * h[i] for i in range(I))) < 1e-12


def _tiny_layer(seed=7, T=6, H=8, I=4, E=5, k=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    Ws = {e: (rng.standard_normal((I, H)), rng.standard_normal((I, H)), rng.standard_normal((H, I)))
          for e in range(E)}
    ids, w = route.topk_softmax(rng.standard_normal((T, E)).astype(np.float32), k)
    return x, ids, w, Ws


def test_moe_output_special_cases():
    x, ids, w, Ws = _tiny_layer()
    # x = 0 -> y = 0
    assert np.all(ffn.moe_output(np.zeros_like(x), ids, w, lambda e: Ws[e]) == 0)
    # k = 1, w = 1 -> y = FFN of the single pick
    ids1 = ids[:, :1]
    y = ffn.moe_output(x, ids1, np.ones((x.shape[0], 1)), lambda e: Ws[e])
    for t in range(x.shape[0]):
        assert np.allclose(y[t], ffn.expert_ffn(x[t:t + 1], *Ws[int(ids1[t, 0])])[0], rtol=1e-14)
    # linear in the gate weights
    y1 = ffn.moe_output(x, ids, w, lambda e: Ws[e])
    y2 = ffn.moe_output(x, ids, 2 * w, lambda e: Ws[e])
    assert np.allclose(y2, 2 * y1, rtol=1e-14)


def test_partition_invariance():
    """[FT] q* policy: the GPU and host partial sums add up to the exact
    output whatever the split."""
    x, ids, w, Ws = _tiny_layer(T=10, E=6, k=3)
    y_all = ffn.moe_output(x, ids, w, lambda e: Ws[e])
    rng = np.random.default_rng(8)
    for _ in range(5):
        mask = rng.random(ids.shape) < 0.5
        yg, yh = ffn.moe_partials(x, ids, w, lambda e: Ws[e], on_gpu=mask)
        assert np.allclose(yg + yh, y_all, rtol=1e-12, atol=1e-13)
    yg, yh = ffn.moe_partials(x, ids, w, lambda e: Ws[e], on_gpu=np.zeros(ids.shape, bool))
    assert np.all(yg == 0)


def test_moe_partials_hand_worked_two_picks():
    """[FT] q* policy and [FT] "Graph 内的 CPU 执行分支": each pick carries its
    own gate weight and its own GPU/host route, and the gate weight scales
    that expert's output.  Two tokens x two picks of scalar experts
    (H = I = 1) with a gate weight of 100, so that for x > 0 silu(100 x) =
    100 x exactly in float64 (e^-100 x is below half an ulp) and
    FFN_e(x) = c_e * (100 x) * (b_e x) = 100 b_e c_e x^2 by hand:
      expert 0: b = 0.5, c = 0.01  ->  FFN_0(x) = 0.5 x^2
      expert 1: b = 2,   c = -0.03 ->  FFN_1(x) = -6 x^2
    Token 0 (x = 1): pick 0 = expert 1, w 0.75, on the GPU; pick 1 = expert
    0, w 0.25, on the host.  Token 1 (x = 2): pick 0 = expert 0, w 0.6, on
    the GPU; pick 1 = expert 1, w 0.4, on the host.  A weight or a route
    attached to the wrong pick (transposed, or taken from the other token)
    changes every one of the four values."""
    Ws = {0: (np.array([[100.0]]), np.array([[0.5]]), np.array([[0.01]])),
          1: (np.array([[100.0]]), np.array([[2.0]]), np.array([[-0.03]]))}
    x = np.array([[1.0], [2.0]])
    ids = np.array([[1, 0], [0, 1]])
    w = np.array([[0.75, 0.25], [0.6, 0.4]])
    on_gpu = np.array([[True, False], [True, False]])
    yg, yh = ffn.moe_partials(x, ids, w, lambda e: Ws[e], on_gpu=on_gpu)
    # by hand: 0.75 * -6 * 1, 0.25 * 0.5 * 1, 0.6 * 0.5 * 4, 0.4 * -6 * 4
    assert yg[0, 0] == pytest.approx(-4.5, rel=1e-15)
    assert yh[0, 0] == pytest.approx(0.125, rel=1e-15)
    assert yg[1, 0] == pytest.approx(1.2, rel=1e-15)
    assert yh[1, 0] == pytest.approx(-9.6, rel=1e-15)
    # the other split of the same picks: both of token 0 on the host, both of token 1 on the GPU
    yg2, yh2 = ffn.moe_partials(x, ids, w, lambda e: Ws[e], on_gpu=np.array([[False, False], [True, True]]))
    assert yg2[0, 0] == 0 and yh2[1, 0] == 0
    assert yh2[0, 0] == pytest.approx(-4.5 + 0.125, rel=1e-15)
    assert yg2[1, 0] == pytest.approx(1.2 - 9.6, rel=1e-15)
    # all on the GPU: the layer output
    y = ffn.moe_output(x, ids, w, lambda e: Ws[e])
    assert y[0, 0] == pytest.approx(-4.375, rel=1e-15) and y[1, 0] == pytest.approx(-8.4, rel=1e-15)


def test_moe_partials_hand_worked_vector_rows():
    """The same association with H = 2, I = 1 and the picks' order reversed
    in token 1, so the output rows are distinct vectors: expert e has gate
    row [100, 0], up row [b_e, 0] and down column [c_e, d_e]; for x = (s, t)
    with s > 0, FFN_e(x) = 100 b_e s^2 (c_e, d_e)."""
    Ws = {0: (np.array([[100.0, 0.0]]), np.array([[0.5, 0.0]]), np.array([[0.01], [0.02]])),
          1: (np.array([[100.0, 0.0]]), np.array([[2.0, 0.0]]), np.array([[-0.03], [0.01]])),
          2: (np.array([[100.0, 0.0]]), np.array([[1.0, 0.0]]), np.array([[0.0], [-0.01]]))}
    # 100 b c s^2 and 100 b d s^2 per expert at s = 1 and s = 2
    ffn0 = lambda s: np.array([0.5, 1.0]) * s * s
    ffn1 = lambda s: np.array([-6.0, 2.0]) * s * s
    ffn2 = lambda s: np.array([0.0, -1.0]) * s * s
    x = np.array([[1.0, 5.0], [2.0, -3.0]])
    ids = np.array([[2, 0, 1], [1, 2, 0]])
    w = np.array([[0.5, 0.3, 0.2], [0.1, 0.7, 0.2]])
    on_gpu = np.array([[True, False, True], [False, True, True]])
    yg, yh = ffn.moe_partials(x, ids, w, lambda e: Ws[e], on_gpu=on_gpu)
    exp_g0 = 0.5 * ffn2(1.0) + 0.2 * ffn1(1.0)
    exp_h0 = 0.3 * ffn0(1.0)
    exp_g1 = 0.7 * ffn2(2.0) + 0.2 * ffn0(2.0)
    exp_h1 = 0.1 * ffn1(2.0)
    np.testing.assert_allclose(yg[0], exp_g0, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(yh[0], exp_h0, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(yg[1], exp_g1, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(yh[1], exp_h1, rtol=1e-14, atol=1e-15)
