"""Pins of the CPU oracle against what the pages and mathematics fix.

None of these re-types the oracle's own formulas: expected values come from
the pages' worked examples, exact rational brute force (tests/brute.py),
closed forms on Hadamard inputs, invariances, and hand-built inputs whose
quantization is exact by construction.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import brute
import synth
from oracle import awq_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")
F16, F32, F64 = np.float16, np.float32, np.float64


def hadamard(n):
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


# --------------------------------------------------------------- step formula
def test_step_equation_worked_example():
    """Step-size equation of 'AWQ > Salient Weight Preservation' on a group
    whose values are all on the 1/16 grid (fixture derivation)."""
    g = json.load(open(os.path.join(GOLD, "step_equation_example.json")))
    u = np.array(g["u"], dtype=np.int64)
    w = (u / 16.0).astype(F16)[None, :]
    packed = O.pack(w, np.ones(128, F32))
    assert float(packed.step16[0, 0]) == g["expected_step"]
    assert float(packed.zero16[0, 0]) == g["expected_zero"]
    assert np.array_equal(packed.q[0].astype(np.int64), u + g["expected_code_offset"])
    # dequantization of exact codes returns the weights exactly
    wq = O.fake_quant(w, np.ones(128, F32), np.ones(128, F32))
    assert np.array_equal(wq.view(np.uint16), w.view(np.uint16))


def test_memory_arithmetic_13b():
    """Worked memory example of the modelrefs glossary page."""
    g = json.load(open(os.path.join(GOLD, "memory_13b.json")))
    b = O.packed_bytes(int(g["n_params"]), group=g["group_size"])
    assert b["fp16"] / 1e9 == pytest.approx(g["fp16_gb"], rel=1e-12)
    assert b["codes"] / 1e9 == pytest.approx(g["int4_gb"], rel=1e-12)
    assert b["steps"] / 1e9 == pytest.approx(g["scales_gb_approx"], rel=g["rel_tol_approx"])
    assert (b["codes"] + b["steps"]) / 1e9 == pytest.approx(g["total_gb_approx"],
                                                            rel=g["rel_tol_approx"])
    # zero points add the same again as the steps (not counted by the page)
    assert b["zeros"] == b["steps"]
    # the oracle's packed arrays have exactly these sizes
    rng = np.random.default_rng(0)
    W = rng.standard_normal((16, 256)).astype(F16)
    p = O.pack(W, np.ones(256, F32))
    bb = O.packed_bytes(W.size)
    assert p.qweight.nbytes == bb["codes"] and p.step16.nbytes == bb["steps"]
    assert p.zero16.nbytes == bb["zeros"]


# ------------------------------------------------ brute force on tiny inputs
def _tiny_case(seed, n=6, k=128, out=3):
    _, X, W = synth.make_custom(n, k, out, seed)
    return X, W


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_quantizer_matches_exact_rational_emulation(seed):
    X, W = _tiny_case(seed, k=256, out=4)
    sal = O.act_stats(X)
    s, inv_s = O.scale_table(sal)
    for i in (0, 7, 19):
        gq = O.quantize(O.scaled_weights(W, s[i]))
        wq = O.dequantize(gq, inv_s[i])
        s_fr = [Fraction(float(v)) for v in s[i]]
        for r in range(W.shape[0]):
            bw, bq = brute.fake_quant_row([Fraction(float(v)) for v in W[r]], s_fr)
            assert bq == gq.q[r].tolist()
            assert [Fraction(float(v)) for v in wq[r]] == bw


@pytest.mark.parametrize("seed", [3, 4])
def test_losses_match_exact_rationals(seed):
    X, W = _tiny_case(seed, n=5, k=128, out=3)
    sal = O.act_stats(X)
    res = O.search_layer(X, W, sal)
    Xf = [[Fraction(float(v)) for v in row] for row in X]
    Wf = [[Fraction(float(v)) for v in row] for row in W]
    for i in (0, 5, 13, 19):
        s_fr = [Fraction(float(v)) for v in res.s[i]]
        Wq = [brute.fake_quant_row(row, s_fr)[0] for row in Wf]
        exact = brute.mse_exact(Xf, Wf, Wq)
        assert res.losses[i] == pytest.approx(float(exact), rel=1e-12, abs=0)


QUANT_VARIANTS = [(32, 4, True), (64, 3, True), (128, 3, False), (64, 4, False), (32, 3, False)]


@pytest.mark.parametrize("group,w_bit,zp", QUANT_VARIANTS)
def test_quantizer_variants_match_exact_rationals(group, w_bit, zp):
    """Other group sizes, 3-bit codes and the symmetric variant, against the
    same exact-rational emulation."""
    X, W = _tiny_case(group + w_bit, k=256, out=3)
    s, inv_s = O.scale_table(O.act_stats(X))
    qmax = 2 ** w_bit - 1
    for i in (0, 11):
        gq = O.quantize(O.scaled_weights(W, s[i]), group, w_bit, zp)
        wq = O.dequantize(gq, inv_s[i], group)
        s_fr = [Fraction(float(v)) for v in s[i]]
        for r in range(W.shape[0]):
            bw, bq = brute.fake_quant_row([Fraction(float(v)) for v in W[r]], s_fr, group, qmax,
                                          not zp)
            assert bq == gq.q[r].tolist()
            assert [Fraction(float(v)) for v in wq[r]] == bw


@pytest.mark.parametrize("group,w_bit,zp", QUANT_VARIANTS[:3])
def test_variant_losses_match_exact_rationals(group, w_bit, zp):
    X, W = _tiny_case(7, n=4, k=128, out=2)
    res = O.search_layer(X, W, O.act_stats(X), group=group, w_bit=w_bit, zero_point=zp)
    Xf = [[Fraction(float(v)) for v in row] for row in X]
    Wf = [[Fraction(float(v)) for v in row] for row in W]
    for i in (0, 9):
        s_fr = [Fraction(float(v)) for v in res.s[i]]
        Wq = [brute.fake_quant_row(row, s_fr, group, 2 ** w_bit - 1, not zp)[0] for row in Wf]
        assert res.losses[i] == pytest.approx(float(brute.mse_exact(Xf, Wf, Wq)), rel=1e-12)


def test_symmetric_rtn_worked_group():
    """The round-to-nearest formula of the dev.to page on a group whose values
    are multiples of step = max|w| / 8 in [-8, 7] steps: every value is stored
    exactly (codes k + 8); a value of +8 steps would clamp to code 15."""
    k = np.array([(j % 16) - 8 for j in range(128)], dtype=np.int64)
    k[5] = -8                                     # max|w| = 8 steps, at a negative value
    w = (k / 64.0).astype(F16)[None, :]           # step = 8/64 / 8 = 1/64
    p = O.pack(w, np.ones(128, F32), zero_point=False)
    assert float(p.step16[0, 0]) == 1 / 64 and float(p.zero16[0, 0]) == 8
    assert np.array_equal(p.q[0].astype(np.int64), k + 8)
    assert np.array_equal(O.dequant_packed(p.qweight, p.step16, p.zero16)[0], w[0].astype(F64))
    w2 = w.copy()
    w2[0, 7] = F16(8 / 64.0)                      # +8 steps: outside the signed 4-bit range
    p2 = O.pack(w2, np.ones(128, F32), zero_point=False)
    assert p2.q[0, 7] == 15 and float(p2.step16[0, 0]) == 1 / 64


def test_three_bit_grid_group():
    """Step-size equation with 2^3 - 1 levels: a group spanning 7 steps is
    stored exactly."""
    u = np.array([(j % 8) - 3 for j in range(128)], dtype=np.int64)
    w = (u / 32.0).astype(F16)[None, :]
    p = O.pack(w, np.ones(128, F32), w_bit=3)
    assert float(p.step16[0, 0]) == 1 / 32 and float(p.zero16[0, 0]) == 3
    assert int(p.q.max()) == 7
    assert np.array_equal(O.dequant_packed(p.qweight, p.step16, p.zero16)[0], w[0].astype(F64))


def test_tile_squared_error_matches_exact_rationals():
    """The per-block squared error that full-size parity samples: each block
    equals the exact rational sum over that block, and the blocks of a
    partition add up to the layer loss times its element count."""
    X, W = _tiny_case(5, n=7, k=256, out=5)
    sal = O.act_stats(X)
    res = O.search_layer(X, W, sal)
    Xf = [[Fraction(float(v)) for v in row] for row in X]
    Wf = [[Fraction(float(v)) for v in row] for row in W]
    rows_parts = [slice(0, 3), slice(3, 7)]
    cols_parts = [slice(0, 2), slice(2, 5)]
    for i in (0, 11, 19):
        s_fr = [Fraction(float(v)) for v in res.s[i]]
        Wq = [brute.fake_quant_row(row, s_fr)[0] for row in Wf]
        total = 0.0
        for rs in rows_parts:
            for cs in cols_parts:
                got = O.tile_sq_error(X, W, res.s[i], res.inv_s[i], rs, cs)
                n_el = (rs.stop - rs.start) * (cs.stop - cs.start)
                exact = brute.mse_exact(Xf[rs], Wf[cs], Wq[cs]) * n_el
                assert got == pytest.approx(float(exact), rel=1e-12, abs=0)
                total += got
        assert total == pytest.approx(res.losses[i] * X.shape[0] * W.shape[0], rel=1e-12)


def test_stats_exact_mean_then_two_roundings():
    rng = np.random.default_rng(7)
    X = (rng.standard_normal((37, 64)) * 50).astype(F16)
    X[0, :4] = [F16(65504.0), F16(-65504.0), F16(2.0 ** -24), F16(-(2.0 ** -20))]
    X[1, 4] = F16(0.0)
    sal = O.act_stats(X)
    for k in range(X.shape[1]):
        m = brute.mean_abs_exact([Fraction(float(v)) for v in X[:, k]])
        want = brute.round_rne(brute.round_rne(m, brute.BINARY64), brute.BINARY32)
        assert Fraction(float(sal[k])) == want


def test_stats_statistical_sanity():
    """Non-outlier channels of N(0,1) activations: E|x| = sqrt(2/pi)."""
    spec, X, _ = synth.make_layer(1)
    sal = O.act_stats(X)
    med = float(np.median(sal))
    assert med == pytest.approx(math.sqrt(2 / math.pi), abs=0.03)
    # the outlier channels are exactly the large ones
    assert int((sal > 5).sum()) == spec.n_outliers


def test_scale_table_against_high_precision_pow():
    rng = np.random.default_rng(11)
    sal = np.concatenate([rng.uniform(1e-6, 120, 24), [0.0, 1e-4, 1.0, 2.0]]).astype(F32)
    s, inv_s = O.scale_table(sal)
    floor = Fraction(float(F32(1e-4)))
    for k, v in enumerate(sal):
        base = max(Fraction(float(v)), floor)
        for i in range(20):
            exact = brute.pow_decimal(base, Fraction(i, 20))
            want = brute.round_rne(brute.round_rne(exact, brute.BINARY64), brute.BINARY32)
            assert Fraction(float(s[i, k])) == want, (k, i)
            assert Fraction(float(inv_s[i, k])) == brute.round_rne(1 / want)
    assert np.all(s[0] == 1) and np.all(inv_s[0] == 1)


# ------------------------------------------------------ special cases / RTN
def test_alpha_zero_is_plain_rtn():
    """alpha = 0 means no scaling (search_scale listing), so grid point 0 must be
    plain round-to-nearest group quantization of W, brute-forced without s."""
    X, W = _tiny_case(5, n=4, k=256, out=3)
    res = O.search_layer(X, W, O.act_stats(X))
    assert np.all(res.s[0] == 1)
    gq = O.quantize(O.scaled_weights(W, res.s[0]))
    Xf = [[Fraction(float(v)) for v in row] for row in X]
    Wf = [[Fraction(float(v)) for v in row] for row in W]
    Wq_rtn = []
    for r, row in enumerate(Wf):
        codes, deq = [], []
        for g0 in range(0, 256, 128):
            step, zero, q = brute.quantize_group(row[g0:g0 + 128])
            codes += q
            deq += [brute.round_rne(brute.round_rne((qq - zero) * step), brute.BINARY16) for qq in q]
        assert codes == gq.q[r].tolist()
        Wq_rtn.append(deq)
    assert res.losses[0] == pytest.approx(float(brute.mse_exact(Xf, Wf, Wq_rtn)), rel=1e-12)


def _grid_layer(rows, k, rng, s_pow2):
    """W whose scaled groups lie exactly on their own quantization grid."""
    W = np.empty((rows, k), dtype=F64)
    codes = np.empty((rows, k), dtype=np.int64)
    for r in range(rows):
        for g0 in range(0, k, 128):
            c = rng.integers(0, 16, 128)
            c[rng.integers(0, 128)] = 0
            c[(rng.integers(0, 127) + 1 + np.argmin(c)) % 128] = 15
            z = int(rng.integers(1, 15))
            step = 2.0 ** -int(rng.integers(6, 10))
            ws = (c - z) * step
            W[r, g0:g0 + 128] = ws / s_pow2[g0:g0 + 128]
            codes[r, g0:g0 + 128] = c
    Wh = W.astype(F16)
    assert np.array_equal(Wh.astype(F64), W)          # exactly representable
    return Wh, codes


def test_scaling_identity_is_exact_when_rounding_is_exact():
    """Scaling identity of 'AWQ > Salient Weight Preservation': scaling a
    column by s and dividing it back cancels exactly; with power-of-two s and
    groups on their grid nothing rounds, so the codes are the construction,
    the dequantized weight is W bit for bit and the loss is zero."""
    rng = np.random.default_rng(3)
    k = 256
    s = (2.0 ** rng.integers(-2, 3, k)).astype(F32)
    W, codes = _grid_layer(4, k, rng, s.astype(F64))
    p = O.pack(W, s)
    assert np.array_equal(p.q.astype(np.int64), codes)
    wq = O.fake_quant(W, s, (F32(1) / s).astype(F32))
    assert np.array_equal(wq.view(np.uint16), W.view(np.uint16))
    X = (rng.standard_normal((8, k))).astype(F16)
    assert O.output_mse(X, W, wq) == 0.0


def test_zero_range_group():
    W = np.zeros((2, 128), F16)
    W[1] = F16(0.375)
    p = O.pack(W, np.ones(128, F32))
    assert np.all(p.step16 == 1)
    assert p.zero16[0, 0] == 0 and not np.signbit(p.zero16[0, 0])
    wq = O.fake_quant(W, np.ones(128, F32), np.ones(128, F32))
    assert np.array_equal(wq[0], W[0])


# ------------------------------------------------ closed form: single outlier
def _single_outlier_case(out=4):
    n = k = 128
    j = 37
    X = hadamard(n)
    X[:, j] *= 2.0
    X = X.astype(F16)
    base = np.tile(np.array([-5, 10] + [0] * 126, dtype=F64) / 16.0, (out, 1))
    rng = np.random.default_rng(1)
    base[:, 2:] = rng.integers(-5, 11, (out, 126)) / 16.0
    base[:, j] = 0.0
    u0 = np.array([129, 130, 131, 132][:out], dtype=F64) / 256.0
    W = base.copy()
    W[:, j] = u0 / 16.0
    return X, W.astype(F16), u0, j


def test_single_outlier_loss_closed_form_and_monotone():
    """Hadamard activations with one channel doubled: X^T X is diagonal, the
    loss separates per weight, and only the outlier weight has error.  Scaling
    it by 2^alpha shrinks that error ('How does AWQ protect channels', the
    1/s argument), so the loss decreases strictly along the grid and follows
    (2^-alpha - u0)^2 / 64 per row."""
    X, W, u0, j = _single_outlier_case()
    sal = O.act_stats(X)
    assert sal[j] == 2 and np.all(np.delete(sal, j) == 1)
    res = O.search_layer(X, W, sal)
    assert np.all(np.diff(res.losses) < 0)
    assert res.best == 19
    for i, a in enumerate(O.alphas()):
        e = (2.0 ** -a - u0) / 16.0                 # exact outlier weight error
        delta = 2.0 ** -16                          # fp16 half-ulp on [1/32, 1/16)
        closed = np.mean(4 * e * e)
        bound = np.mean(4 * (2 * np.abs(e) * delta + delta * delta))
        assert abs(res.losses[i] - closed) <= bound + 1e-15
    assert res.losses[0] == pytest.approx(np.mean((1 - u0) ** 2 / 64), rel=1e-9)


def test_all_equal_saliency_ties_choose_first():
    """|x| = 1 everywhere gives s = 1 for every alpha: identical losses, and the
    strict comparison of the search keeps the first grid point."""
    X = hadamard(128).astype(F16)
    rng = np.random.default_rng(2)
    W = (rng.standard_normal((3, 128)) * 0.02).astype(F16)
    res = O.search_layer(X, W, O.act_stats(X))
    assert np.all(res.losses == res.losses[0]) and res.best == 0


def test_argmin_rules():
    assert O.argmin_first([3.0, 1.0, 1.0, 2.0]) == 1
    assert O.argmin_first([np.nan, 2.0, np.inf, 2.0]) == 1
    assert O.argmin_first([np.inf, np.nan, 5.0]) == 2
    with pytest.raises(O.NonFiniteLosses):
        O.argmin_first([np.nan, np.inf, np.nan])


# --------------------------------------------------------------- invariances
def test_weight_power_of_two_scaling():
    X, W = _tiny_case(8, n=16, k=256, out=8)
    sal = O.act_stats(X)
    a = O.search_layer(X, W, sal)
    W4 = (W.astype(F32) * 4).astype(F16)
    b = O.search_layer(X, W4, sal)
    assert np.allclose(b.losses, a.losses * 16, rtol=1e-12, atol=0)
    pa, pb = O.pack(W, a.s_best), O.pack(W4, a.s_best)
    assert np.array_equal(pa.q, pb.q) and np.array_equal(pa.zero16, pb.zero16)
    assert np.array_equal(pb.step16.astype(F32), pa.step16.astype(F32) * 4)


def test_activation_power_of_two_scaling():
    X, W = _tiny_case(9, n=16, k=256, out=8)
    a = O.search_layer(X, W, O.act_stats(X))
    X2 = (X.astype(F32) * 2).astype(F16)
    b = O.search_layer(X2, W, O.act_stats(X2))
    # s changes by 2^alpha per grid point (a common factor per group), so only
    # codes within rounding of a tie can move
    assert np.allclose(b.losses, a.losses * 4, rtol=2e-3)


def test_permutations():
    X, W = _tiny_case(10, n=16, k=256, out=8)
    sal = O.act_stats(X)
    a = O.search_layer(X, W, sal)
    # output rows
    perm = np.random.default_rng(0).permutation(W.shape[0])
    b = O.search_layer(X, W[perm], sal)
    assert np.allclose(b.losses, a.losses, rtol=1e-12, atol=0)
    pa, pb = O.pack(W, a.s_best), O.pack(W[perm], a.s_best)
    assert np.array_equal(pa.qweight[perm], pb.qweight)
    # tokens: saliency is an exact sum, hence bit-identical
    tp = np.random.default_rng(1).permutation(X.shape[0])
    assert np.array_equal(O.act_stats(X[tp]).view(np.uint32), sal.view(np.uint32))
    c = O.search_layer(X[tp], W, sal)
    assert np.allclose(c.losses, a.losses, rtol=1e-12, atol=0)
    # whole groups of 128 columns
    cols = np.concatenate([np.arange(128, 256), np.arange(0, 128)])
    d = O.search_layer(X[:, cols], W[:, cols], sal[cols])
    assert np.allclose(d.losses, a.losses, rtol=1e-12, atol=0)
    pd = O.pack(W[:, cols], a.s_best[cols])
    assert np.array_equal(pd.q, pa.q[:, cols])


# ------------------------------------------------------------- error bounds
def test_rounding_error_bound_and_zero_range():
    """Max rounding error is half a step (dev.to 'Why does naive 4-bit
    quantization...' and 'Salient Weight Preservation'); the zero point lies
    in [0, 15] whenever the group straddles 0."""
    _, X, W = synth.make_layer(1)
    sal = O.act_stats(X)
    s, _ = O.scale_table(sal)
    for i in (0, 10, 19):
        ws = O.scaled_weights(W, s[i])
        gq = O.quantize(ws)
        step = np.repeat(gq.step, 128, axis=1).astype(F64)
        zero = np.repeat(gq.zero, 128, axis=1).astype(F64)
        err = np.abs((gq.q.astype(F64) - zero) * step - ws.astype(F64))
        x = ws.astype(F64) / step + zero
        clamped = (x < -0.5) | (x > 15.5)
        assert np.all(err[~clamped] <= step[~clamped] * (0.5 + 2.0 ** -18))
        assert np.all(err <= step * (1 + 2.0 ** -18))
        g = ws.reshape(ws.shape[0], -1, 128)
        straddle = (g.min(axis=2) <= 0) & (g.max(axis=2) >= 0)
        assert np.all((gq.zero[straddle] >= 0) & (gq.zero[straddle] <= 15))
        # the group minimum always lands on code 0
        amin = g.argmin(axis=2)
        qg = gq.q.reshape(g.shape)
        assert np.all(np.take_along_axis(qg, amin[:, :, None], 2) == 0)


def test_pack_layout_and_roundtrip():
    q = np.array([[1, 2, 3, 4, 5, 6, 7, 8, 15, 15, 15, 15, 15, 15, 15, 15]], dtype=np.uint8)
    w = O.pack_codes(q)
    assert w.dtype == np.int32 and w.shape == (1, 2)
    assert w.view(np.uint32)[0, 0] == 0x87654321
    assert w[0, 1] == -1
    rng = np.random.default_rng(4)
    qq = rng.integers(0, 16, (5, 256)).astype(np.uint8)
    assert np.array_equal(O.unpack_codes(O.pack_codes(qq)), qq)


# ------------------------------------------------- W4A16 product (decode)
def _random_packed(rng, rows, k):
    words = rng.integers(0, 2 ** 32, (rows, k // 8), dtype=np.uint64).astype(np.uint32)
    step = rng.uniform(1e-3, 0.1, (rows, k // 128)).astype(F16)
    zero = rng.integers(0, 16, (rows, k // 128)).astype(F16)
    return words.view(np.int32), step, zero


def test_w4a16_matches_exact_rationals():
    """The W4A16 product against exact rational arithmetic on tiny inputs,
    with the nibbles read from each 32-bit word by plain integer shifts
    (column 8w + j in bits 4j..4j+3)."""
    rng = np.random.default_rng(11)
    rows, k, m = 3, 256, 2
    qw, st, zr = _random_packed(rng, rows, k)
    x = rng.standard_normal((m, k)).astype(F16)
    y = O.w4a16_matmul(x, qw, st, zr)
    for t in range(m):
        for o in range(rows):
            acc = Fraction(0)
            for col in range(k):
                word = int(qw.view(np.uint32)[o, col // 8])
                code = (word >> (4 * (col % 8))) & 0xF
                g = col // 128
                acc += Fraction(float(x[t, col])) * (code - Fraction(float(zr[o, g]))) \
                    * Fraction(float(st[o, g]))
            assert y[t, o] == pytest.approx(float(acc), rel=1e-12, abs=1e-300)


def test_w4a16_on_grid_weights_reproduce_the_layer():
    """Weights on their group's grid (power-of-two steps) survive pack and the
    W4A16 dequantization exactly, so the product equals x W^T."""
    rng = np.random.default_rng(12)
    k = 384
    W, _ = _grid_layer(5, k, rng, np.ones(k))
    p = O.pack(W, np.ones(k, F32))
    assert np.array_equal(O.dequant_packed(p.qweight, p.step16, p.zero16), W.astype(F64))
    x = rng.standard_normal((4, k)).astype(F16)
    want = x.astype(F64) @ W.astype(F64).T
    assert np.allclose(O.w4a16_matmul(x, p.qweight, p.step16, p.zero16), want, rtol=1e-14,
                       atol=1e-14)


# ------------------------------------------- folding 1/s into the producer
def _rmsnorm64(h, gamma):
    h = h.astype(F64)
    return h / np.sqrt(np.mean(h * h, axis=1, keepdims=True) + 1e-6) * gamma.astype(F64)


def test_fold_matches_exact_rationals():
    rng = np.random.default_rng(31)
    src = (rng.standard_normal((40, 3)) * rng.choice([1e-4, 1.0, 300.0], (40, 1))).astype(F16)
    s = rng.uniform(0.05, 40.0, 40).astype(F32)
    got = O.fold_inverse_scale(src, s)
    for j in range(40):
        for c in range(3):
            q = Fraction(float(src[j, c])) / Fraction(float(s[j]))
            want = brute.round_rne(brute.round_rne(q, brute.BINARY32), brute.BINARY16)
            assert Fraction(float(got[j, c])) == want
    big = O.fold_inverse_scale(np.array([60000.0, -60000.0], F16), np.array([0.5, 0.5], F32))
    assert np.isposinf(big[0]) and np.isneginf(big[1])


def test_fold_into_rmsnorm_preserves_the_layer():
    """Salient Weight Preservation page: the norm's gain times 1/s cancels the
    column scaling of W, so the scaled pair computes the same outputs; with
    power-of-two s nothing rounds and the outputs agree exactly."""
    rng = np.random.default_rng(32)
    n, out = 256, 24
    h = rng.standard_normal((6, n)).astype(F16)
    gamma = rng.uniform(0.5, 1.5, n).astype(F16)
    W = (rng.standard_normal((out, n)) * 0.05).astype(F16)
    y = _rmsnorm64(h, gamma) @ W.astype(F64).T
    s2 = (2.0 ** rng.integers(-3, 4, n)).astype(F32)
    g2 = O.fold_inverse_scale(gamma, s2)
    y2 = _rmsnorm64(h, g2) @ (W.astype(F64) * s2.astype(F64)[None, :]).T
    assert np.array_equal(y2, y) or np.allclose(y2, y, rtol=1e-15, atol=0)
    s = rng.uniform(0.1, 30.0, n).astype(F32)
    g = O.fold_inverse_scale(gamma, s)
    yf = _rmsnorm64(h, g) @ (W.astype(F64) * s.astype(F64)[None, :]).T
    bound = (np.abs(_rmsnorm64(h, gamma)) @ np.abs(W.astype(F64)).T) * (2.0 ** -11 + 2.0 ** -23)
    assert np.all(np.abs(yf - y) <= bound)


def test_fold_into_previous_linear_preserves_the_layer():
    """A preceding linear (weight rows and bias) absorbs 1/s the same way."""
    rng = np.random.default_rng(33)
    n, k, out = 128, 64, 16
    h = rng.standard_normal((5, k)).astype(F16)
    Wp = (rng.standard_normal((n, k)) * 0.1).astype(F16)
    bp = rng.standard_normal(n).astype(F16)
    W = (rng.standard_normal((out, n)) * 0.05).astype(F16)
    s = rng.uniform(0.1, 30.0, n).astype(F32)
    z = h.astype(F64) @ Wp.astype(F64).T + bp.astype(F64)
    y = z @ W.astype(F64).T
    zf = h.astype(F64) @ O.fold_inverse_scale(Wp, s).astype(F64).T \
        + O.fold_inverse_scale(bp, s).astype(F64)
    yf = zf @ (W.astype(F64) * s.astype(F64)[None, :]).T
    zabs = np.abs(h.astype(F64)) @ np.abs(Wp.astype(F64)).T + np.abs(bp.astype(F64))
    bound = (zabs @ np.abs(W.astype(F64)).T) * (2.0 ** -11 + 2.0 ** -23)
    assert np.all(np.abs(yf - y) <= bound)


# ------------------------------------------------------- saliency ablations
def test_weight_saliency_is_the_column_mean_of_abs_w():
    rng = np.random.default_rng(41)
    W = (rng.standard_normal((9, 16)) * 0.02).astype(F16)
    got = O.weight_saliency(W)
    for k in range(16):
        m = brute.mean_abs_exact([Fraction(float(v)) for v in W[:, k]])
        assert Fraction(float(got[k])) == brute.round_rne(brute.round_rne(m, brute.BINARY64),
                                                          brute.BINARY32)


@pytest.mark.parametrize("n_keep", [0, 1, 3, 7, 12])
def test_select_top_channels_brute_force(n_keep):
    sal = np.array([0.5, 2.0, 2.0, 0.1, 7.0, 2.0, 0.5, 0.0, 3.0, 2.0, 1e-5, 7.0], F32)
    got = O.select_top_channels(sal, n_keep)
    ranked = sorted(range(len(sal)), key=lambda k: (-float(sal[k]), k))[:n_keep]
    for k in range(len(sal)):
        assert got[k] == (sal[k] if k in ranked else F32(1.0))
    # kept channels scale, the others have s = 1 at every grid point
    s, _ = O.scale_table(got)
    for k in range(len(sal)):
        if k not in ranked:
            assert np.all(s[:, k] == 1.0)


def test_literal_division_changes_loss_negligibly():
    """Folding s back by multiplying with fp32(1/s) instead of dividing by s
    moves the dequantized weight by at most one fp16 rounding step."""
    _, X, W = synth.make_layer(1)
    sal = O.act_stats(X)
    s, inv_s = O.scale_table(sal)
    for i in (5, 15):
        gq = O.quantize(O.scaled_weights(W, s[i]))
        a = O.output_mse(X, W, O.dequantize(gq, inv_s[i]))
        b = O.output_mse(X, W, O.dequantize(gq, inv_s[i], literal_div=s[i]))
        assert abs(a - b) <= 1e-5 * a


# ------------------------------------------------ the .5-tie flags of codes
def _f32_steps(x, n):
    """x moved by n binary32 ulps (n < 0: towards -inf)."""
    v = np.float32(x)
    d = np.float32(np.inf if n > 0 else -np.inf)
    for _ in range(abs(n)):
        v = np.nextafter(v, d)
    return v


NEAR_HALF_CASES = [
    # (value, within one ulp of x of a half-integer?)
    (2.5, True), (_f32_steps(2.5, 1), True), (_f32_steps(2.5, -1), True),
    (_f32_steps(2.5, 2), False), (_f32_steps(2.5, -2), False),
    (3.0, False), (2.0, False), (0.0, False), (0.5, True), (_f32_steps(0.5, 3), False),
    (-2.5, True), (_f32_steps(-2.5, 1), True), (_f32_steps(-2.5, -1), True),
    (-3.25, False), (14.5, True), (_f32_steps(14.5, -1), True), (_f32_steps(14.5, 2), False),
    # ulp 0.25 in [2^21, 2^22): an integer is two ulps from a half-integer, a
    # quarter one ulp; ulp 0.5 in [2^22, 2^23): every value is a tie or one ulp from one
    (2097152.0, False), (2097152.25, True), (2097153.75, True),
    (4194304.5, True), (4194305.0, True), (4194306.0, True),
    # every binary32 value at or beyond 2^23 is an integer, 0.5 from a half-integer, ulp >= 1
    (8388609.0, True), (-16777218.0, True),
]


@pytest.mark.parametrize("x,want", NEAR_HALF_CASES)
def test_near_half_hand_values(x, want):
    """The tie flag counts the codes whose pre-round binary32 quotient lies
    within one binary32 ulp of a half-integer (round-half-to-even, dev.to "Why
    does naive 4-bit quantization wreck LLM accuracy?" round-to-nearest; the
    quotient of the step-size equation of "AWQ > Salient Weight Preservation").
    Expected values from the binary32 spacing at each value, worked by hand."""
    got = O._near_half(np.array([x], dtype=F32))[0]
    assert bool(got) == want, (float(x), float(np.spacing(np.float32(abs(x)))))


def test_tie_flags_mark_codes_that_an_ulp_can_flip():
    """On random groups, a code flagged as near a tie is exactly one whose
    rounding changes when its quotient moves by one ulp either way (computed
    with exact rationals), or whose group's zero point does; unflagged codes
    never change."""
    rng = np.random.default_rng(21)
    ws = (rng.standard_normal((64, 256)) * 0.05).astype(F32)
    # plant exact and near ties: groups whose quotient lands on x.5 by construction
    ws[:8, :128] = ((np.arange(128) % 16 - 7.5) / 16).astype(F32)
    gq = O.quantize(ws)
    for r in range(ws.shape[0]):
        for g in range(ws.shape[1] // 128):
            step = Fraction(float(gq.step[r, g]))
            for j in range(128):
                x = brute.round_rne(Fraction(float(ws[r, 128 * g + j])) / step)
                xf = np.float32(float(x))
                ulp = Fraction(float(np.spacing(np.float32(abs(xf)))))
                flips = {brute.rint_even(x - ulp), brute.rint_even(x), brute.rint_even(x + ulp)}
                code_flag = bool(O._near_half(np.array([xf]))[0])
                if len(flips) > 1:
                    assert code_flag, (r, g, j, float(x))
                if not (code_flag or gq.zero_tie[r, g]):
                    assert not gq.tie[r, 128 * g + j]
                assert gq.tie[r, 128 * g + j] == (code_flag or gq.zero_tie[r, g])
    assert gq.tie[:8, :128].all()  # planted exact ties


# ------------------------------------------------- non-finite activations
def test_stats_non_finite_columns():
    """A channel whose tokens hold a NaN has saliency NaN, one holding an
    infinity (and no NaN) +inf (IEEE sums of |x|); the other channels keep
    their exact mean, checked against exact rationals."""
    rng = np.random.default_rng(22)
    X = rng.standard_normal((37, 24)).astype(F16)
    X[3, 1] = np.nan
    X[5, 2] = np.inf
    X[6, 3] = -np.inf
    X[7, 4] = np.nan
    X[8, 4] = np.inf
    sal = O.act_stats(X)
    assert np.isnan(sal[1]) and np.isnan(sal[4])
    assert sal[2] == np.inf and sal[3] == np.inf
    for k in [0] + list(range(5, 24)):
        exact = brute.mean_abs_exact([Fraction(float(v)) for v in X[:, k]])
        assert sal[k] == np.float32(float(brute.round_rne(brute.round_rne(exact, brute.BINARY64))))


# --------------------------------------- the W4A16 error-bound scale
def test_w4a16_abs_matmul_matches_exact_rationals_and_bounds_the_product():
    """sum_k |x| (q + |z|) |step| against exact rationals with an independent
    bit-level unpack, and as a bound of |x (q - z) step| (triangle inequality)
    that is attained when x >= 0 and the zeros are <= 0."""
    rng = np.random.default_rng(23)
    rows, k, m = 3, 256, 2
    qw, st, zr = _random_packed(rng, rows, k)
    zr[1, 0] = F16(-7.0)
    st[2, 1] = F16(-0.03125)
    x = rng.standard_normal((m, k)).astype(F16)
    b = O.w4a16_abs_matmul(x, qw, st, zr)
    for t in range(m):
        for o in range(rows):
            acc = Fraction(0)
            for col in range(k):
                word = int(qw.view(np.uint32)[o, col // 8])
                code = (word >> (4 * (col % 8))) & 0xF
                g = col // 128
                acc += abs(Fraction(float(x[t, col]))) * (code + abs(Fraction(float(zr[o, g])))) \
                    * abs(Fraction(float(st[o, g])))
            assert b[t, o] == pytest.approx(float(acc), rel=1e-12, abs=1e-300)
    y = O.w4a16_matmul(x, qw, st, zr)
    assert np.all(np.abs(y) <= b * (1 + 1e-12))
    xp = np.abs(x)
    zn = -np.abs(zr)
    stp = np.abs(st)
    assert np.allclose(O.w4a16_matmul(xp, qw, stp, zn), O.w4a16_abs_matmul(xp, qw, stp, zn),
                       rtol=1e-12, atol=0)


# ------------------------------------------- planted mistakes must be caught
@pytest.mark.parametrize("mutation", ["floor_round", "symmetric_step", "grid_to_one",
                                      "no_zero_canon", "nibble_order", "fold_multiplies",
                                      "abs_bound_drops_zero", "tie_exact_only",
                                      "stats_nan_ignored", "no_unscale", "loss_over_tokens_only",
                                      "argmin_last", "stats_over_features", "no_floor",
                                      "pow_in_binary32"])
@pytest.mark.filterwarnings("ignore:divide by zero encountered:RuntimeWarning")
def test_planted_mistakes_fail_a_pin(mutation, monkeypatch):
    """Each plausible slip in the oracle trips at least one pin above."""
    if mutation == "no_unscale":
        # the quantized scaled weight is not divided by s again
        orig = O.dequantize
        monkeypatch.setattr(O, "dequantize", lambda gq, inv_s_row, group=128, literal_div=None:
                            orig(gq, np.ones_like(np.asarray(inv_s_row, F32)), group, literal_div))
        with pytest.raises(AssertionError):
            test_scaling_identity_is_exact_when_rounding_is_exact()
    elif mutation == "loss_over_tokens_only":
        # the squared error averaged over tokens but summed over outputs
        orig = O.search_layer

        def per_token(X, W, sal, *a, **kw):
            r = orig(X, W, sal, *a, **kw)
            r.losses = r.losses * np.asarray(W).shape[0]
            return r
        monkeypatch.setattr(O, "search_layer", per_token)
        with pytest.raises(AssertionError):
            test_losses_match_exact_rationals(3)
    elif mutation == "argmin_last":
        def last(losses):
            best, best_i = np.inf, -1
            for i, v in enumerate(np.asarray(losses, dtype=F64)):
                if v <= best:
                    best, best_i = v, i
            if best_i < 0:
                raise O.NonFiniteLosses("no finite loss on the grid")
            return best_i
        monkeypatch.setattr(O, "argmin_first", last)
        with pytest.raises(AssertionError):
            test_argmin_rules()
    elif mutation == "stats_over_features":
        # the mean taken along the wrong axis (per token instead of per channel)
        orig = O.act_stats
        monkeypatch.setattr(O, "act_stats", lambda X: orig(np.ascontiguousarray(np.asarray(X).T)))
        with pytest.raises((AssertionError, IndexError)):
            test_stats_exact_mean_then_two_roundings()
    elif mutation == "no_floor":
        orig = O.scale_table
        monkeypatch.setattr(O, "scale_table", lambda sal, n_grid=20, floor=None:
                            orig(sal, n_grid, 0.0))
        with pytest.raises(AssertionError):
            test_scale_table_against_high_precision_pow()
    elif mutation == "pow_in_binary32":
        def pow32(sal, n_grid=20, floor=O.SAL_FLOOR):
            base = np.maximum(np.asarray(sal, F32), F32(floor))
            s = np.power(base[None, :], O.alphas(n_grid).astype(F32)[:, None]).astype(F32)
            return s, (F32(1.0) / s).astype(F32)
        monkeypatch.setattr(O, "scale_table", pow32)
        with pytest.raises(AssertionError):
            test_scale_table_against_high_precision_pow()
    elif mutation == "floor_round":
        monkeypatch.setattr(O.np, "rint", np.floor)
        with pytest.raises(AssertionError):
            test_quantizer_matches_exact_rational_emulation(0)
    elif mutation == "symmetric_step":
        orig = O.quantize

        def sym(ws, group=128, w_bit=4, zero_point=True):
            gq = orig(ws, group, w_bit, zero_point)
            g = ws.reshape(ws.shape[0], -1, group)
            gq.step = (np.abs(g).max(axis=2) / F32(8)).astype(F32)
            return gq
        monkeypatch.setattr(O, "quantize", sym)
        with pytest.raises(AssertionError):
            test_step_equation_worked_example()
    elif mutation == "grid_to_one":
        monkeypatch.setattr(O, "alphas", lambda n=20: np.arange(n, dtype=F64) / (n - 1))
        with pytest.raises(AssertionError):
            test_single_outlier_loss_closed_form_and_monotone()
    elif mutation == "nibble_order":
        orig = O.unpack_codes

        def reversed_nibbles(qweight):
            u = orig(qweight)
            r, k = u.shape
            return u.reshape(r, k // 8, 8)[:, :, ::-1].reshape(r, k)
        monkeypatch.setattr(O, "unpack_codes", reversed_nibbles)
        with pytest.raises(AssertionError):
            test_w4a16_matches_exact_rationals()
    elif mutation == "fold_multiplies":
        monkeypatch.setattr(O, "fold_inverse_scale",
                            lambda src, s: (np.asarray(src, F16).astype(F32)
                                            * np.asarray(s, F32).reshape((-1,) + (1,) * (np.asarray(src).ndim - 1))
                                            ).astype(F16))
        with pytest.raises(AssertionError):
            test_fold_into_rmsnorm_preserves_the_layer()
    elif mutation == "abs_bound_drops_zero":
        def no_zero(x, qweight, step16, zero16, group=128):
            q = O.unpack_codes(qweight).astype(F64)
            st = np.abs(np.repeat(np.asarray(step16, F16).astype(F64), group, axis=1))
            return np.abs(np.asarray(x, F16).astype(F64)) @ (q * st).T
        monkeypatch.setattr(O, "w4a16_abs_matmul", no_zero)
        with pytest.raises(AssertionError):
            test_w4a16_abs_matmul_matches_exact_rationals_and_bounds_the_product()
    elif mutation == "tie_exact_only":
        monkeypatch.setattr(O, "_near_half", lambda x: np.abs(
            x.astype(F64) - (np.floor(x.astype(F64)) + 0.5)) == 0)
        with pytest.raises(AssertionError):
            test_near_half_hand_values(_f32_steps(2.5, 1), True)
    elif mutation == "stats_nan_ignored":
        orig = O.act_stats
        monkeypatch.setattr(O, "act_stats", lambda X: orig(np.where(np.isnan(X), F16(0), X)))
        with pytest.raises(AssertionError):
            test_stats_non_finite_columns()
    elif mutation == "no_zero_canon":
        orig = O.quantize

        def negz(ws, group=128, w_bit=4, zero_point=True):
            gq = orig(ws, group, w_bit, zero_point)
            gq.zero = np.where(gq.zero == 0, F32(-0.0), gq.zero)
            return gq
        monkeypatch.setattr(O, "quantize", negz)
        with pytest.raises(AssertionError):
            test_zero_range_group()


# ------------------------------------------------------ regression fixtures
def test_input_generator_manifest():
    """The seeded inputs are frozen: every configured layer's leading cut hashes
    to the recorded digest (tests/golden/make_golden.py wrote them)."""
    g = json.load(open(os.path.join(GOLD, "input_manifest.json")))
    for key, cfg in synth.CONFIGS.items():
        for li, spec in enumerate(cfg.layers):
            _, X, W = synth.make_layer(key, li, **g["cut"])
            assert synth.digest(X, W) == g["digests"][f"{key}:{spec.name}"], (key, spec.name)


def test_oracle_config1_regression():
    g = json.load(open(os.path.join(GOLD, "oracle_config1.json")))
    _, X, W = synth.make_layer(1, 0)
    sal = O.act_stats(X)
    assert synth.digest(sal) == g["sal_digest"]
    res = O.search_layer(X, W, sal)
    # binary64 contractions: equal up to the BLAS's summation order
    assert res.losses == pytest.approx(np.array(g["losses"]), rel=1e-12, abs=0)
    assert res.best == g["best"]
