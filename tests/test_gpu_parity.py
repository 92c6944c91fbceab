"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars (element by element, same seeded inputs on both sides):
  * saliency: bit-exact (both sides sum exactly);
  * packed codes, steps, zero points: bit-exact (both divide exactly);
  * per-grid-point losses: within 1e-3 relative (observed far tighter);
  * chosen index: identical unless the oracle's two best losses lie within
    1e-3 relative of each other; s_best bit-exact against the oracle's s row;
  * packed codes and zero points: a difference is allowed only where the
    oracle flags the pre-round value as within one binary32 ulp of a .5 tie,
    at most 1e-6 of the elements (none occurs: the kernel divides exactly);
  * full-size layers of every configuration: all 20 losses within 1e-3 of the
    oracle's committed whole-layer losses, the chosen index by the rule above,
    per-tile partial sums of sampled tiles within 1e-3 of the oracle's block
    sums, and the pack at the chosen alpha.
"""
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
from oracle import awq_oracle as O

pytestmark = pytest.mark.gpu

LOSS_RTOL = 1e-3


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def awq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import post_bit_weight_awq_amd as m
    m.load()
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def run_layer(awq, X, W, n_grid=20):
    Xd, Wd = dev(X), dev(W)
    sal = awq.awq_act_stats(Xd)
    res = awq.awq_search_layer(Xd, Wd, sal, awq.default_config(n_grid=n_grid))
    torch.cuda.synchronize()
    return Xd, Wd, sal, res


def check_best(gpu_best, ref_losses):
    order = np.argsort(ref_losses, kind="stable")
    best = O.argmin_first(ref_losses)
    if gpu_best == best:
        return
    second = ref_losses[order[1]]
    assert abs(second - ref_losses[best]) <= LOSS_RTOL * ref_losses[best], (gpu_best, best)
    assert gpu_best in order[:2]


def check_pack(qw, st, zr, ref, label=""):
    """Packed codes, zero points and words against the oracle's pack under the
    rule for codes decided at a .5 tie: steps bit-exact; a code or zero point
    may differ only where the oracle flags its pre-round binary32 value as
    within one ulp of a half-integer, and such differences must stay at or
    below 1e-6 of the elements.  The pack kernel divides exactly, so none
    differs at all; the counts are printed."""
    assert np.array_equal(st.view(np.uint16), ref.step16.view(np.uint16)), "steps"
    q = O.unpack_codes(qw)
    code_diff = q != ref.q
    zero_diff = zr.view(np.uint16) != ref.zero16.view(np.uint16)
    n = code_diff.size
    n_tie, n_code, n_zero = int(ref.tie.sum()), int(code_diff.sum()), int(zero_diff.sum())
    _say(f"  pack {label}: {n_tie} of {n} codes near a .5 tie ({n_tie / n:.1e}); "
         f"{n_code} codes and {n_zero} zero points differ")
    assert not (code_diff & ~ref.tie).any(), "a code away from any tie differs"
    assert not (zero_diff & ~ref.zero_tie).any(), "a zero point away from any tie differs"
    assert n_code <= 1e-6 * n and n_zero <= 1e-6 * zero_diff.size
    # packed words: equal wherever all eight nibbles agree
    words_diff = (qw.view(np.uint32) != ref.qweight.view(np.uint32))
    assert not (words_diff & ~code_diff.reshape(code_diff.shape[0], -1, 8).any(axis=2)).any()
    assert n_code == 0 and n_zero == 0, "exact division: no code may differ"


# ------------------------------------------------------------------ stats
STATS_CASES = [(1, 0), (2, 0), (3, 0), (4, 0), (4, 1), (5, 0), (5, 3)]


@pytest.mark.parametrize("cfg,layer", STATS_CASES)
def test_stats_bitexact_configs(awq, cfg, layer):
    _say(f"stats config {cfg} layer {layer}")
    _, X, _ = synth.make_layer(cfg, layer, out_features=1)
    sal = host(awq.awq_act_stats(dev(X)))
    ref = O.act_stats(X)
    assert np.array_equal(sal.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("n,k", [(1, 8), (37, 520), (3, 4096), (1000, 136), (8192, 512), (9000, 64)])
def test_stats_edge_shapes(awq, n, k):
    _say(f"stats edge {n}x{k}")
    rng = np.random.default_rng(n * 7 + k)
    X = (rng.standard_normal((n, k)) * rng.choice([1e-6, 1.0, 3e3], size=k)).astype(np.float16)
    X[0, 0] = np.float16(65504.0)
    if k > 1:
        X[0, 1] = np.float16(2.0 ** -24)
    sal = host(awq.awq_act_stats(dev(X)))
    assert np.array_equal(sal.view(np.uint32), O.act_stats(X).view(np.uint32))


# -------------------------------------------------------------------- pack
PACK_CASES = [(1, 0), (2, 0), (3, 0), (4, 1), (5, 2)]


@pytest.mark.parametrize("cfg,layer", PACK_CASES)
def test_pack_bitexact_configs(awq, cfg, layer):
    _say(f"pack config {cfg} layer {layer}")
    spec, X, W = synth.make_layer(cfg, layer, n_tokens=64)
    sal = O.act_stats(X)
    s, _ = O.scale_table(sal)
    s_row = s[13]
    qw, st, zr = awq.awq_pack(dev(W), dev(s_row))
    ref = O.pack(W, s_row)
    check_pack(host(qw), host(st), host(zr), ref, f"config {cfg} layer {layer}")


def test_pack_edge_groups(awq):
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((5, 384)) * 0.02).astype(np.float16)
    W[0, :128] = 0                              # zero range: step 1
    W[1, 128:256] = np.float16(0.25)            # constant group
    W[2, 256:] = np.abs(W[2, 256:]) + np.float16(0.01)   # all-positive group
    W[3, :128] = (np.arange(128) % 16 - 5) / 16  # on the grid: integer quotients
    W[4, :128] = (np.arange(128) % 16 - 7.5) / 16  # half-integer quotients and zero: exact ties
    s = rng.uniform(0.25, 4.0, 384).astype(np.float32)
    s[:128] = 1.0
    qw, st, zr = (host(t) for t in awq.awq_pack(dev(W), dev(s)))
    ref = O.pack(W, s)
    assert ref.tie[4, :128].all() and ref.zero_tie[4, 0]  # exact .5 ties, rounded to even
    check_pack(qw, st, zr, ref, "edge groups")


# The pack kernel's sweep mapping: one group per row, a group count per row
# that is odd or coprime to the teams per wavefront, single and ragged
# sweeps, and the three group sizes (teams of 1, 2 and 4 lanes).
PACK_SWEEP = [(1, 128, 128), (3, 10368, 128), (77, 384, 32), (1000, 640, 64), (2, 13824, 128),
              (513, 1280, 32)]


@pytest.mark.parametrize("o,k,group", PACK_SWEEP)
def test_pack_sweep_shapes(awq, o, k, group):
    _say(f"pack sweep shape {o}x{k} group {group}")
    rng = np.random.default_rng(7 * o + k)
    W = (rng.standard_normal((o, k)) * 0.02).astype(np.float16)
    s = rng.uniform(0.25, 4.0, k).astype(np.float32)
    cfg = awq.default_config(group_size=group)
    qw, st, zr = (host(t) for t in awq.awq_pack(dev(W), dev(s), cfg))
    check_pack(qw, st, zr, O.pack(W, s, group), f"{o}x{k} group {group}")


@pytest.mark.parametrize("zp", [True, False])
def test_pack_groups_far_from_zero(awq, zp):
    """Narrow groups far from zero (zero points of a few hundred to about ten
    thousand, on both sides of the |z| <= 2048 bound under which the kernel
    moves the zero point out of the clamp), and near zero."""
    _say(f"pack groups far from zero, zero_point {zp}")
    rng = np.random.default_rng(11)
    k = 1024
    rows = [off + rng.uniform(-hw, hw, (8, k))
            for off, hw in ((40.0, 0.04), (100.0, 0.35), (-3.0, 0.03), (1000.0, 0.25),
                            (-2000.0, 0.5), (0.0, 0.02))]
    W = np.concatenate(rows).astype(np.float16)
    s = np.ones(k, dtype=np.float32)
    cfg = awq.default_config(zero_point=zp)
    qw, st, zr = (host(t) for t in awq.awq_pack(dev(W), dev(s), cfg))
    ref = O.pack(W, s, zero_point=zp)
    if zp:
        z = np.abs(ref.zero16.astype(np.float64))
        assert (z > 2048).any() and ((z > 16) & (z <= 2048)).any()
    check_pack(qw, st, zr, ref, f"far from zero, zero_point {zp}")


# ----------------------------------------------- search: oracle-sized cases
SEARCH_SMALL = [
    ("cfg1", dict(config=1)),
    ("cfg2", dict(config=2)),
    ("cfg3_cut", dict(config=3, n_tokens=200, out_features=300)),
    ("cfg4_up_cut", dict(config=4, layer=0, n_tokens=130, out_features=260)),
    ("cfg4_down_cut", dict(config=4, layer=1, n_tokens=96, out_features=200)),
    ("cfg5_qkv_cut", dict(config=5, layer=0, n_tokens=160, out_features=256)),
    ("cfg5_down_cut", dict(config=5, layer=3, n_tokens=64, out_features=136)),
]


@pytest.mark.parametrize("name,kw", SEARCH_SMALL, ids=[c[0] for c in SEARCH_SMALL])
def test_search_matches_oracle(awq, name, kw):
    config = kw.pop("config")
    layer = kw.pop("layer", 0)
    _say(f"search {name}")
    spec, X, W = synth.make_layer(config, layer, **kw)
    Xd, Wd, sal, res = run_layer(awq, X, W)
    sal_h = host(sal)
    ref = O.search_layer(X, W, sal_h)
    losses = host(res.losses)
    rel = np.abs(losses - ref.losses) / ref.losses
    _say(f"  max rel loss diff {rel.max():.3e}; best gpu {int(host(res.best_idx)[0])} "
         f"oracle {ref.best}")
    assert np.all(rel <= LOSS_RTOL)
    best = int(host(res.best_idx)[0])
    check_best(best, ref.losses)
    assert np.array_equal(host(res.s_best).view(np.uint32), ref.s[best].view(np.uint32))
    # then pack at the GPU's choice, against the oracle at the same s
    qw, st, zr = (host(t) for t in awq.awq_pack(Wd, res.s_best))
    check_pack(qw, st, zr, O.pack(W, ref.s[best]), name)


@pytest.mark.parametrize("n,k,o", [(64, 1024, 300), (16, 384, 77)])
def test_group_params_bit_exact(awq, n, k, o):
    """The per-group quantizer parameters the preparation stage leaves in the
    workspace (binary32 step, 1/step, -zero, 15 - zero for every grid point,
    column group and output row) equal the oracle's quantizer applied to
    fp32(W diag(s_i)), bit for bit.  Offsets: the workspace holds the partial
    sums, the scale table, the reciprocal table and the parameters, in that
    order, each region starting on a 256-byte boundary."""
    _say(f"group params {n}x{k}->{o}")
    _, X, W = synth.make_custom(n, k, o, seed=n + k)
    Xd, Wd = dev(X), dev(W)
    sal = awq.awq_act_stats(Xd)
    res = awq.awq_search_layer(Xd, Wd, sal, stages=awq._lib.STAGE_PREPARE)
    torch.cuda.synchronize()
    n_grid, ng = 20, k // 128
    a256 = lambda v: (v + 255) // 256 * 256
    off_inv = a256(res.plan.scales_offset + 4 * n_grid * k)
    off_prm = a256(off_inv + 4 * n_grid * k)
    prm = host(res.workspace[off_prm:off_prm + 16 * n_grid * ng * o].view(torch.float32))
    prm = prm.reshape(n_grid, ng, o, 4)
    s_tab, _ = O.scale_table(host(sal))
    for i in range(n_grid):
        gq = O.quantize(O.scaled_weights(W, s_tab[i]))
        step = gq.step.T  # [ng, o]
        zero = gq.zero.T
        got = prm[i]
        assert np.array_equal(got[..., 0].view(np.uint32), step.view(np.uint32)), i
        inv = (np.float32(1) / step).astype(np.float32)
        assert np.array_equal(got[..., 1].view(np.uint32), inv.view(np.uint32)), i
        assert np.array_equal(got[..., 2], -zero), i
        assert np.array_equal(got[..., 3], np.float32(15) - zero), i


@pytest.mark.parametrize("n_tokens", [256, 1100])
def test_search_is_deterministic(awq, n_tokens):
    """Three runs of the whole path are bitwise identical (a race check as
    well): saliency, all losses, the choice, s_best and the packed layer, on
    the fused path (256 tokens) and the contraction path (1100 tokens)."""
    _, X, W = synth.make_layer(3, n_tokens=n_tokens, out_features=512)
    Xd, Wd = dev(X), dev(W)
    runs = []
    for _ in range(3):
        sal = awq.awq_act_stats(Xd)
        res = awq.awq_search_layer(Xd, Wd, sal)
        qw, st, zr = awq.awq_pack(Wd, res.s_best)
        runs.append([host(t) for t in (sal, res.losses, res.best_idx, res.s_best, qw, st, zr)])
    for other in runs[1:]:
        for x, y in zip(runs[0], other):
            assert x.tobytes() == y.tobytes()


def test_search_on_side_stream(awq):
    _, X, W = synth.make_layer(1)
    Xd, Wd = dev(X), dev(W)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        sal = awq.awq_act_stats(Xd)
        r = awq.awq_search_layer(Xd, Wd, sal)
    s.synchronize()
    ref = O.search_layer(X, W, O.act_stats(X))
    assert np.allclose(r.losses.cpu().numpy(), ref.losses, rtol=LOSS_RTOL)


# ------------------------------------------------------------- edge cases
@pytest.mark.parametrize("n,k,o,n_grid", [(1, 128, 1, 20), (5, 128, 3, 1), (33, 256, 129, 64),
                                          (129, 384, 257, 7)])
def test_search_edge_shapes(awq, n, k, o, n_grid):
    _say(f"search edge {n}x{k}->{o} grid {n_grid}")
    _, X, W = synth.make_custom(n, k, o, seed=n + k + o)
    Xd, Wd, sal, res = run_layer(awq, X, W, n_grid=n_grid)
    ref = O.search_layer(X, W, host(sal), n_grid=n_grid)
    losses = host(res.losses)
    assert losses.shape == (n_grid,)
    assert np.all(np.abs(losses - ref.losses) <= LOSS_RTOL * ref.losses)
    check_best(int(host(res.best_idx)[0]), ref.losses)


@pytest.mark.parametrize("n,k,o", [(700, 256, 2048), (300, 256, 2048), (700, 256, 2000),
                                   (700, 1024, 2048), (760, 384, 1970)])
def test_search_split_last_round(awq, n, k, o):
    """Shapes whose work units fill the chip 2.5 times: the last half round runs
    as half-height tiles, with ragged token tiles (the second half of the last
    one can be empty), ragged last output tiles (2000 = 15 x 128 + 80,
    1970 = 15 x 128 + 50) and one to eight column groups."""
    _say(f"search split last round {n}x{k}->{o}")
    _, X, W = synth.make_custom(n, k, o, seed=n + o)
    Xd, Wd, sal, res = run_layer(awq, X, W)
    assert res.plan.tile_out == 128  # the fused kernels (at most four 256-token tiles)
    ref = O.search_layer(X, W, host(sal))
    losses = host(res.losses)
    rel = np.abs(losses - ref.losses) / ref.losses
    _say(f"  max rel loss diff {rel.max():.3e}")
    assert np.all(rel <= LOSS_RTOL)
    check_best(int(host(res.best_idx)[0]), ref.losses)


def test_search_grid_stage_repeated(awq):
    """The grid and select stages run again on the same workspace, with no new
    preparation, give bitwise the same losses (and the oracle's): the stages keep
    no state between launches beyond the prepared tables, and the partial sums
    of a search (including its split last round) add in a fixed order."""
    n, k, o = 700, 1024, 2048
    _say(f"search grid stage repeated {n}x{k}->{o}")
    _, X, W = synth.make_custom(n, k, o, seed=7)
    Xd, Wd, sal, res = run_layer(awq, X, W)
    assert res.plan.tile_tokens == 512
    first = host(res.losses).copy()
    ref = O.search_layer(X, W, host(sal))
    assert np.all(np.abs(first - ref.losses) <= LOSS_RTOL * ref.losses)
    for _ in range(3):
        again = awq.awq_search_layer(Xd, Wd, sal, workspace=res.workspace,
                                     stages=awq._lib.STAGE_GRID | awq._lib.STAGE_SELECT)
        torch.cuda.synchronize()
        assert np.array_equal(host(again.losses).view(np.uint64), first.view(np.uint64))


@pytest.mark.filterwarnings("ignore:invalid value encountered:RuntimeWarning")
def test_search_degenerate_inputs(awq):
    # all-zero activations: saliency 0 is floored, every loss is 0, the first wins
    X = np.zeros((16, 256), np.float16)
    W = (np.random.default_rng(0).standard_normal((8, 256)) * 0.02).astype(np.float16)
    _, _, sal, res = run_layer(awq, X, W)
    assert np.all(host(res.losses) == 0) and int(host(res.best_idx)[0]) == 0
    # Hadamard activations: |x| = 1 gives s = 1 for every alpha, equal losses, index 0
    h = np.array([[1.0]])
    while h.shape[0] < 128:
        h = np.block([[h, h], [h, -h]])
    X = h.astype(np.float16)
    _, _, sal, res = run_layer(awq, X, W[:, :128].copy())
    losses = host(res.losses)
    assert np.all(losses == losses[0]) and int(host(res.best_idx)[0]) == 0
    # a NaN weight makes every loss NaN: no choice, s_best all NaN
    Wn = W.copy()
    Wn[0, 0] = np.float16(np.nan)
    _, _, sal, res = run_layer(awq, np.ones((4, 256), np.float16), Wn)
    assert int(host(res.best_idx)[0]) == -1
    assert np.all(np.isnan(host(res.s_best)))
    with pytest.raises(awq.AwqError) as err:
        res.best()
    assert err.value.code == awq._lib.AWQ_ERR_NONFINITE


@pytest.mark.filterwarnings("ignore:invalid value encountered:RuntimeWarning")
def test_search_degenerate_inputs_contraction_path(awq):
    """The same degenerate inputs on the contraction path (1100 tokens): all-zero
    activations give zero losses and index 0; a NaN weight makes every grid
    point's weight error NaN in its group, so no loss is finite: index -1 and
    s_best all NaN."""
    rng = np.random.default_rng(1)
    W = (rng.standard_normal((40, 256)) * 0.02).astype(np.float16)
    _, _, sal, res = run_layer(awq, np.zeros((1100, 256), np.float16), W)
    assert res.plan.tile_out == 256
    assert np.all(host(res.losses) == 0) and int(host(res.best_idx)[0]) == 0
    Wn = W.copy()
    Wn[7, 130] = np.float16(np.nan)
    X = (rng.standard_normal((1100, 256))).astype(np.float16)
    _, _, sal, res = run_layer(awq, X, Wn)
    assert res.plan.tile_out == 256
    assert np.all(np.isnan(host(res.losses)))
    assert int(host(res.best_idx)[0]) == -1
    assert np.all(np.isnan(host(res.s_best)))


@pytest.mark.parametrize("n,k", [(64, 512), (9000, 64), (4096, 2048)])
def test_stats_non_finite(awq, n, k):
    """NaN and infinities in X: a channel holding a NaN gets saliency NaN, one
    holding an infinity (and no NaN) +inf, the rest their exact mean, on the
    one-launch path (64 x 512) and the two-pass path (9000 x 64: more than
    8192 rows; 4096 x 2048: more than 4M elements)."""
    rng = np.random.default_rng(n + k)
    X = rng.standard_normal((n, k)).astype(np.float16)
    X[n // 2, 1] = np.nan
    X[n - 1, 2] = np.inf
    X[0, 3] = -np.inf
    X[1, 4] = np.nan
    X[n - 1, 4] = np.inf
    sal = host(awq.awq_act_stats(dev(X)))
    ref = O.act_stats(X)
    assert np.isnan(ref[1]) and np.isnan(ref[4]) and ref[2] == np.inf and ref[3] == np.inf
    assert np.array_equal(np.isnan(sal), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(sal[fin].view(np.uint32), ref[fin].view(np.uint32))


@pytest.mark.filterwarnings("ignore:invalid value encountered:RuntimeWarning")
@pytest.mark.parametrize("n_tokens", [64, 1100])
@pytest.mark.parametrize("kind", ["nan", "inf", "both"])
def test_search_non_finite_saliency(awq, n_tokens, kind):
    """A NaN and/or an infinite saliency (finite X), on the fused path (64
    tokens) and the contraction path (1100 tokens): the scale table follows
    the oracle's floor-then-power (alpha = 0 still gives s = 1, other grid
    points NaN or inf), bit for bit; every grid point above 0 has a NaN loss
    on both sides, and the search keeps alpha = 0."""
    _, X, W = synth.make_layer(1, 0, n_tokens=n_tokens, out_features=64)
    _say(f"non-finite saliency {kind}, {n_tokens} tokens")
    sal_h = O.act_stats(X).copy()
    if kind in ("nan", "both"):
        sal_h[3] = np.nan
    if kind in ("inf", "both"):
        sal_h[200] = np.inf
    res = awq.awq_search_layer(dev(X), dev(W), dev(sal_h))
    torch.cuda.synchronize()
    ref = O.search_layer(X, W, sal_h)
    losses = host(res.losses)
    assert np.array_equal(np.isnan(losses), np.isnan(ref.losses))
    fin = np.isfinite(ref.losses)
    assert fin[0] and not fin[1:].any()
    assert abs(losses[0] - ref.losses[0]) <= LOSS_RTOL * ref.losses[0]
    assert int(host(res.best_idx)[0]) == ref.best == 0
    k = X.shape[1]
    st = host(res.workspace[res.plan.scales_offset:res.plan.scales_offset + 4 * 20 * k]
              .view(torch.float32)).reshape(20, k)
    assert np.array_equal(np.isnan(st), np.isnan(ref.s))
    ok = ~np.isnan(ref.s)
    assert np.array_equal(st[ok].view(np.uint32), ref.s[ok].view(np.uint32))
    assert np.array_equal(host(res.s_best), np.ones(k, np.float32))


def test_explicit_stream_argument(awq):
    """Calls given stream= rather than run under torch.cuda.stream(): the
    binding allocates their workspaces and outputs on that stream, so memory
    the current stream allocates and fills while they run never aliases them
    (the two-pass statistics path, whose workspace is dropped on return)."""
    _, X, W = synth.make_layer(3, n_tokens=2048, out_features=384)
    Xd, Wd = dev(X), dev(W)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    sal = awq.awq_act_stats(Xd, stream=side)
    res = awq.awq_search_layer(Xd, Wd, sal, stream=side)
    qw, st, zr = awq.awq_pack(Wd, res.s_best, stream=side)
    for _ in range(8):  # churn on the current stream meanwhile
        junk = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
        junk.fill_(0xAB)
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    sal_h = host(sal)
    assert np.array_equal(sal_h.view(np.uint32), O.act_stats(X).view(np.uint32))
    ref = O.search_layer(X, W, sal_h)
    assert np.all(np.abs(host(res.losses) - ref.losses) <= LOSS_RTOL * ref.losses)
    best = int(host(res.best_idx)[0])
    check_best(best, ref.losses)
    check_pack(host(qw), host(st), host(zr), O.pack(W, ref.s[best]), "explicit stream")


# ------------------------- layers of many token tiles: the contraction path
# At least five 256-token tiles: the preparation stage writes every grid
# point's weight error dW_i = fp16(Wq_i - W) once and the grid stage contracts
# it (tiles of 256 tokens x 256 outputs; groups of 4 pairs, runs of up to 8
# token tiles).
GEMM_CASES = [
    ("ragged", dict(n=2000, k=384, o=300)),     # last token tile 208 rows, last output tile 44
    ("exact", dict(n=2048, k=256, o=512)),
    ("nine_tiles", dict(n=2100, k=256, o=700)),  # a second run of one token tile
    ("five_tiles", dict(n=1100, k=512, o=1300)),  # one run of five tiles; last group of 3 pairs
    ("wide_k", dict(n=1800, k=11008, o=257)),   # 86 column groups of 128; ragged outputs
]


@pytest.mark.parametrize("name,shape", GEMM_CASES, ids=[c[0] for c in GEMM_CASES])
def test_search_contraction_path_matches_oracle(awq, name, shape):
    n, k, o = shape["n"], shape["k"], shape["o"]
    _say(f"contraction path {name}: {n}x{k}->{o}")
    _, X, W = synth.make_custom(n, k, o, seed=n + k + o, token_scale=True)
    Xd, Wd, sal, res = run_layer(awq, X, W)
    assert (res.plan.tile_tokens, res.plan.tile_out) == (256, 256)
    sal_h = host(sal)
    ref = O.search_layer(X, W, sal_h)
    losses = host(res.losses)
    rel = np.abs(losses - ref.losses) / ref.losses
    best = int(host(res.best_idx)[0])
    _say(f"  max rel loss diff {rel.max():.3e}; best gpu {best} oracle {ref.best}")
    assert np.all(rel <= LOSS_RTOL)
    check_best(best, ref.losses)
    assert np.array_equal(host(res.s_best).view(np.uint32), ref.s[best].view(np.uint32))


@pytest.mark.parametrize("n,k,o,n_grid", [(1025, 128, 1, 20), (1300, 128, 3, 1),
                                          (1100, 256, 129, 64), (4097, 128, 2, 3)])
def test_search_contraction_path_edge_shapes(awq, n, k, o, n_grid):
    """The contraction path at its edges: one output row, two 64-column K
    steps, a last token tile of one row (1025 and 4097 tokens), 1 and 64 grid
    points (the weight error of every grid point in the workspace)."""
    _say(f"contraction edge {n}x{k}->{o} grid {n_grid}")
    _, X, W = synth.make_custom(n, k, o, seed=n + k + o + n_grid)
    Xd, Wd, sal, res = run_layer(awq, X, W, n_grid=n_grid)
    assert (res.plan.tile_tokens, res.plan.tile_out) == (256, 256)
    ref = O.search_layer(X, W, host(sal), n_grid=n_grid)
    losses = host(res.losses)
    rel = np.abs(losses - ref.losses) / ref.losses
    _say(f"  max rel loss diff {rel.max():.3e}")
    assert np.all(rel <= LOSS_RTOL)
    check_best(int(host(res.best_idx)[0]), ref.losses)


@pytest.mark.parametrize("group,w_bit,zp", [(64, 4, True), (32, 4, True), (128, 3, True),
                                            (128, 4, False), (32, 3, False)])
def test_search_contraction_path_quantizer_variants(awq, group, w_bit, zp):
    n, k, o = 2061, 512, 260
    _say(f"contraction path variant g{group} b{w_bit} zp{zp}")
    _, X, W = synth.make_custom(n, k, o, seed=group + w_bit, token_scale=True)
    Xd, Wd = dev(X), dev(W)
    sal = awq.awq_act_stats(Xd)
    cfg = awq.default_config(group_size=group, w_bit=w_bit, zero_point=zp)
    res = awq.awq_search_layer(Xd, Wd, sal, cfg)
    torch.cuda.synchronize()
    assert res.plan.tile_tokens == 256
    ref = O.search_layer(X, W, host(sal), group=group, w_bit=w_bit, zero_point=zp)
    losses = host(res.losses)
    assert np.all(np.abs(losses - ref.losses) <= LOSS_RTOL * ref.losses)
    check_best(int(host(res.best_idx)[0]), ref.losses)


@pytest.mark.parametrize("group,w_bit,zp", [(128, 4, True), (32, 3, False)])
def test_contraction_weight_error_matches_oracle(awq, group, w_bit, zp):
    """The weight error the preparation stage writes for every grid point,
    dW_i = fp16(Wq_i - W), bit for bit against the oracle's fake-quantized
    weight minus W (the fp16 difference of two fp16 values, one rounding).
    The kernel takes the exact quotient wherever its reciprocal product lies
    near a tie, so its codes are the oracle's; the rule for codes decided at
    a .5 tie would still admit differences only there (at most 1e-6 of the
    elements, each one code), and none occurs."""
    n, k, o = 2048, 384, 300
    _say(f"contraction weight error {n}x{k}->{o} g{group} b{w_bit} zp{zp}")
    _, X, W = synth.make_custom(n, k, o, seed=5, token_scale=True)
    Xd, Wd = dev(X), dev(W)
    sal = awq.awq_act_stats(Xd)
    cfg = awq.default_config(group_size=group, w_bit=w_bit, zero_point=zp)
    res = awq.awq_search_layer(Xd, Wd, sal, cfg, stages=awq._lib.STAGE_PREPARE)
    torch.cuda.synchronize()
    n_grid = 20
    a256 = lambda v: (v + 255) // 256 * 256
    off_inv = a256(res.plan.scales_offset + 4 * n_grid * k)
    off_dw = a256(off_inv + 4 * n_grid * k)
    dw = host(res.workspace[off_dw:off_dw + 2 * n_grid * o * k].view(torch.float16))
    dw = dw.reshape(n_grid, o, k)
    s_tab, inv_s = O.scale_table(host(sal))
    diff = ties = 0
    for i in range(n_grid):
        gq = O.quantize(O.scaled_weights(W, s_tab[i]), group, w_bit, zp)
        wq = O.dequantize(gq, inv_s[i], group)
        want = (wq.astype(np.float64) - W.astype(np.float64)).astype(np.float16)
        bad = want.view(np.uint16) != dw[i].view(np.uint16)
        assert not (bad & ~gq.tie).any(), i  # a difference only at a near-tie code
        diff += int(bad.sum())
        ties += int(gq.tie.sum())
    _say(f"  {diff} of {n_grid * o * k} weight-error elements differ ({ties} near a tie)")
    assert diff <= 1e-6 * n_grid * o * k
    assert diff == 0, "the producer takes the exact quotient near ties"


def test_contraction_grid_stage_repeated(awq):
    """Grid and select stages rerun on one prepared workspace give bitwise the
    same losses (fixed per-tile partial slots, fixed-order sums)."""
    n, k, o = 2100, 512, 600
    _, X, W = synth.make_custom(n, k, o, seed=9)
    Xd, Wd, sal, res = run_layer(awq, X, W)
    assert res.plan.tile_tokens == 256
    first = host(res.losses).copy()
    for _ in range(3):
        again = awq.awq_search_layer(Xd, Wd, sal, workspace=res.workspace,
                                     stages=awq._lib.STAGE_GRID | awq._lib.STAGE_SELECT)
        torch.cuda.synchronize()
        assert np.array_equal(host(again.losses).view(np.uint64), first.view(np.uint64))


def test_contraction_path_replays_in_a_hip_graph(awq):
    """Statistics, the contraction-path search and pack captured in one HIP
    graph and replayed with eager work between replays: every replay equals
    the eager run bit for bit."""
    _, X, W = synth.make_custom(2048, 512, 512, seed=13)
    Xd, Wd = dev(X), dev(W)

    def run():
        sal = awq.awq_act_stats(Xd)
        res = awq.awq_search_layer(Xd, Wd, sal)
        q, st, z = awq.awq_pack(Wd, res.s_best)
        return sal, res.losses, res.best_idx, res.s_best, q, st, z

    ref = [t.clone() for t in run()]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = run()
    for rep in range(3):
        junk = torch.randn(1 << 20, device="cuda")
        junk.mul_(2.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), f"replay {rep}"


# ----------------------------------- full-size layers against the oracle
GOLD_FULL = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                         "oracle_full_layers.json")
FULL = [(2, 0), (3, 0), (4, 0), (4, 1), (5, 0), (5, 1), (5, 2), (5, 3)]


@pytest.mark.parametrize("cfg,layer", FULL)
def test_full_size_layer_matches_oracle(awq, cfg, layer):
    """Every full-size configured layer, in the launch configuration the
    benchmark times: the saliency bit-exact against the oracle; all 20
    per-grid-point losses within 1e-3 relative of the oracle's whole-layer
    losses (tests/golden/oracle_full_layers.json, written by
    tests/golden/make_golden.py from the oracle alone, for inputs whose
    digests it records); the chosen index by the first-minimum rule; s_best
    bit-exact; the per-tile partial sums of sampled tiles against the
    oracle's block sums; and the codes packed at the chosen alpha against the
    oracle's pack of the whole layer."""
    import json
    gold = json.load(open(GOLD_FULL))["layers"][f"{cfg}:{layer}"]
    spec, X, W = synth.make_layer(cfg, layer)
    _say(f"full-size config {cfg} layer {spec.name}: {spec.n_tokens}x{spec.in_features}"
         f"->{spec.out_features}")
    assert [spec.n_tokens, spec.in_features, spec.out_features] == gold["shape"]
    assert synth.digest(X) == gold["x_digest"] and synth.digest(W) == gold["w_digest"]
    Xd, Wd, sal, res = run_layer(awq, X, W)
    sal_h = host(sal)
    assert synth.digest(sal_h) == gold["sal_digest"]
    assert np.array_equal(sal_h.view(np.uint32), O.act_stats(X).view(np.uint32))
    ref_losses = np.array(gold["losses"])
    losses = host(res.losses)
    rel = np.abs(losses - ref_losses) / ref_losses
    best = int(host(res.best_idx)[0])
    _say(f"  max rel loss diff over 20 grid points {rel.max():.3e}; best gpu {best} "
         f"oracle {gold['best']}")
    assert np.all(rel <= LOSS_RTOL)
    check_best(best, ref_losses)
    s_tab, inv_s = O.scale_table(sal_h)
    assert np.array_equal(host(res.s_best).view(np.uint32), s_tab[best].view(np.uint32))
    # per-tile partial sums of a few tiles (the last, ragged, and random ones)
    plan = res.plan
    ws = res.workspace
    n_grid = 20
    nt, no = plan.n_token_tiles, plan.n_out_tiles
    part = host(ws[plan.partials_offset:plan.partials_offset + 16 * n_grid * nt * no]
                .view(torch.float64)).reshape(n_grid, nt, no, 2).sum(axis=3)
    count = float(spec.n_tokens) * spec.out_features
    assert np.allclose(losses, part.reshape(n_grid, -1).sum(axis=1) / count, rtol=1e-12)
    rng = np.random.default_rng(cfg * 10 + layer)
    tm, tn = plan.tile_tokens, plan.tile_out
    tiles = [(nt - 1, no - 1)] + [(int(rng.integers(nt)), int(rng.integers(no))) for _ in range(2)]
    for (ti, oi) in tiles:
        rows = slice(ti * tm, min((ti + 1) * tm, spec.n_tokens))
        cols = slice(oi * tn, min((oi + 1) * tn, spec.out_features))
        for i in (0, best, n_grid - 1):
            want = O.tile_sq_error(X, W, s_tab[i], inv_s[i], rows, cols)
            got = part[i, ti, oi]
            assert abs(got - want) <= LOSS_RTOL * want, (ti, oi, i, got, want)
    del Xd
    # pack at the chosen alpha, the whole layer
    qw, st, zr = (host(t) for t in awq.awq_pack(Wd, res.s_best))
    del Wd, res
    check_pack(qw, st, zr, O.pack(W, s_tab[best]), f"config {cfg} {spec.name}")


# ------------------------------------------- W4A16 product with packed weights
def _w4a16_check(awq, x, qw, st, zr):
    y = host(awq.awq_w4a16_matmul(dev(x), dev(qw), dev(st), dev(zr)))
    want = O.w4a16_matmul(x, qw, st, zr)
    scale = O.w4a16_abs_matmul(x, qw, st, zr)
    k = x.shape[1]
    # binary32 accumulation of exact fp16 products: per group (<= 128 terms),
    # two roundings for step * (sum x q - z sum x), then the groups and the
    # 16 per-wavefront partials; bound with margin for the MFMA's summation order
    tol = (k / 128 + 160) * 2.0 ** -22 * scale
    err = np.abs(y.astype(np.float64) - want)
    assert np.all(err <= tol + 1e-30), float((err / np.maximum(scale, 1e-30)).max())
    return y, want


# The streaming kernel (up to 4 tokens) takes SL = ceil(K / 2048) 16-byte code
# loads per lane and row; the cases reach every SL from 2 to 8:
#   SL 2: K <= 4096; SL 3: (1, 5120, 15360) the 13B qkv decode shape, (4, 5120,
#   300); SL 4: (1, 8192, 512), (3, 7680, 77) (three tokens staged as four in
#   60.5 KiB of LDS); SL 5: (1, 9216, 700), (2, 10240, 129); SL 6: (1, 11008,
#   4096); SL 7: (1, 12416, 4100), 388 slices per row so the seventh load per
#   lane covers 4 lanes, 4100 rows at three rows per wavefront and pass with the
#   last pass ragged, and (1, 13824, 64); SL 8: (1, 16384, 300), (2, 15360, 129).
# (1, 128, 20000) and (2, 512, 40000): more rows than one round of four-row
# passes holds, so each wavefront runs several passes.  (3, 8192, 40): three
# tokens at K = 8192 need 68 KiB staged, so the MFMA kernel takes them.
W4_CASES = [(1, 4096, 4096), (3, 384, 17), (16, 128, 16), (17, 256, 33), (40, 5120, 300),
            (1, 13824, 64), (1, 12416, 4100), (1, 128, 20000), (2, 512, 40000), (2, 128, 1),
            (16, 256, 12300), (33, 384, 4100), (16, 256, 8200), (16, 384, 24600),
            (1, 9216, 700), (2, 10240, 129), (1, 5120, 15360), (4, 5120, 300), (1, 8192, 512),
            (3, 7680, 77), (1, 11008, 4096), (1, 16384, 300), (2, 15360, 129), (3, 8192, 40)]


@pytest.mark.parametrize("m,k,o", W4_CASES)
def test_w4a16_matches_oracle(awq, m, k, o):
    _say(f"w4a16 {m}x{k} -> {o}")
    _, X, W = synth.make_custom(max(m, 4), k, o, seed=m + k + o)
    x = X[:m].copy()
    sal = O.act_stats(X)
    s, _ = O.scale_table(sal)
    p = O.pack(W, s[9])
    _w4a16_check(awq, x, p.qweight, p.step16, p.zero16)


def test_w4a16_any_codes_and_zero_points(awq):
    """Random codes and zero points far outside 0..15 (all-positive or
    all-negative groups store such zeros): the zero enters once per group."""
    rng = np.random.default_rng(21)
    o, k, m = 48, 640, 5
    qw = rng.integers(0, 2 ** 32, (o, k // 8), dtype=np.uint64).astype(np.uint32).view(np.int32)
    st = rng.uniform(1e-4, 0.05, (o, k // 128)).astype(np.float16)
    zr = rng.choice([-2000.0, -37.0, 0.0, 7.0, 15.0, 300.0, 4096.0], (o, k // 128)).astype(np.float16)
    x = rng.standard_normal((m, k)).astype(np.float16)
    _w4a16_check(awq, x, qw, st, zr)


def test_w4a16_after_gpu_pack(awq):
    """The decode product consumes awq_pack's own output (search -> pack -> use)."""
    _, X, W = synth.make_layer(3, n_tokens=64, out_features=256)
    Xd, Wd, sal, res = run_layer(awq, X, W)
    qw, st, zr = awq.awq_pack(Wd, res.s_best)
    x = (X[:2].astype(np.float32) / host(res.s_best)[None, :]).astype(np.float16)
    _w4a16_check(awq, x, host(qw), host(st), host(zr))


# ------------------------------------------------------ folding 1/s upstream
@pytest.mark.parametrize("rows,cols", [(5120, 1), (4096, 4096), (37, 13), (64, 8), (3, 1000)])
def test_fold_bitexact(awq, rows, cols):
    _say(f"fold {rows}x{cols}")
    rng = np.random.default_rng(rows + cols)
    src = (rng.standard_normal((rows, cols)) * rng.choice([1e-5, 1.0, 2e3], (rows, 1))).astype(np.float16)
    s = rng.uniform(1.6e-4, 50.0, rows).astype(np.float32)
    s[0] = 1.6e-4                                   # overflow to infinity in fp16
    src[0, 0] = np.float16(30000.0)
    want = O.fold_inverse_scale(src if cols > 1 else src[:, 0], s)
    got = host(awq.awq_fold_inverse_scale(dev(src if cols > 1 else src[:, 0]), dev(s)))
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def test_fold_in_place_and_unaligned(awq):
    rng = np.random.default_rng(3)
    src = rng.standard_normal((17, 24)).astype(np.float16)
    s = rng.uniform(0.5, 4.0, 17).astype(np.float32)
    want = O.fold_inverse_scale(src, s)
    t = dev(src)
    awq.awq_fold_inverse_scale(t, dev(s), out=t)       # in place, vector path
    assert np.array_equal(host(t).view(np.uint16), want.view(np.uint16))
    flat = dev(np.concatenate([np.zeros(1, np.float16), src.ravel()]))
    view = flat[1:].view(17, 24)                        # 2-byte offset: one element per thread
    out = torch.empty_like(view)
    awq.awq_fold_inverse_scale(view, dev(s), out=out)
    assert np.array_equal(host(out).view(np.uint16), want.view(np.uint16))


# ------------------------------------------------------- saliency ablations
def test_weight_saliency_bitexact(awq):
    _, _, W = synth.make_layer(2, n_tokens=8, out_features=700)
    got = host(awq.awq_weight_saliency(dev(W)))
    assert np.array_equal(got.view(np.uint32), O.weight_saliency(W).view(np.uint32))


@pytest.mark.parametrize("n,n_keep", [(4096, 41), (5120, 51), (13824, 138), (100, 0),
                                      (100, 100), (3000, 1), (2049, 2048), (1, 1)])
def test_select_top_matches_oracle(awq, n, n_keep):
    rng = np.random.default_rng(n + n_keep)
    sal = rng.choice(np.array([0.0, 0.25, 0.5, 3.0, 3.0, 17.0], np.float32), n) \
        * rng.choice([1.0, 1.0, 1.0, 0.5], n).astype(np.float32)     # many ties
    sal[rng.integers(0, n, max(1, n // 50))] = rng.uniform(1, 100, max(1, n // 50)).astype(np.float32)
    got = host(awq.awq_select_top_channels(dev(sal), n_keep))
    want = O.select_top_channels(sal, n_keep)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_select_top_in_place(awq):
    _, X, _ = synth.make_layer(2, n_tokens=64, out_features=1)
    sal = O.act_stats(X)
    t = dev(sal)
    awq.awq_select_top_channels(t, 41, out=t)
    assert np.array_equal(host(t).view(np.uint32), O.select_top_channels(sal, 41).view(np.uint32))


# ------------------------- quantizer variants: group size, bit width, symmetric
GPU_VARIANTS = [(64, 4, True), (32, 4, True), (128, 3, True), (64, 3, False), (128, 4, False),
                (32, 3, False)]


@pytest.mark.parametrize("group,w_bit,zp", GPU_VARIANTS)
def test_variant_search_and_pack_match_oracle(awq, group, w_bit, zp):
    _say(f"variant group {group} w_bit {w_bit} zero_point {zp}")
    spec, X, W = synth.make_layer(2, n_tokens=300, out_features=200)
    cfg = awq.default_config(group_size=group, w_bit=w_bit, zero_point=zp)
    Xd, Wd = dev(X), dev(W)
    sal = awq.awq_act_stats(Xd)
    res = awq.awq_search_layer(Xd, Wd, sal, cfg)
    ref = O.search_layer(X, W, host(sal), group=group, w_bit=w_bit, zero_point=zp)
    losses = host(res.losses)
    rel = np.abs(losses - ref.losses) / ref.losses
    _say(f"  max rel loss diff {rel.max():.3e}")
    assert np.all(rel <= LOSS_RTOL)
    best = int(host(res.best_idx)[0])
    check_best(best, ref.losses)
    qw, st, zr = (host(t) for t in awq.awq_pack(Wd, res.s_best, cfg))
    pref = O.pack(W, ref.s[best], group, w_bit, zp)
    assert np.array_equal(qw, pref.qweight)
    assert np.array_equal(st.view(np.uint16), pref.step16.view(np.uint16))
    assert np.array_equal(zr.view(np.uint16), pref.zero16.view(np.uint16))


@pytest.mark.parametrize("n,k,o,group,w_bit,zp", [(700, 1024, 2048, 64, 4, True),
                                                  (700, 1024, 2000, 32, 4, True),
                                                  (760, 640, 1970, 32, 3, False)])
def test_variant_split_last_round(awq, n, k, o, group, w_bit, zp):
    """Groups of 64 and 32 columns on the 512-token tile with the partial last
    round on the 256-token tile (ragged token tiles and last output tiles): all
    losses against the oracle."""
    _say(f"variant split last round {n}x{k}->{o} group {group} w_bit {w_bit} zp {zp}")
    _, X, W = synth.make_custom(n, k, o, seed=n + o + group)
    cfg = awq.default_config(group_size=group, w_bit=w_bit, zero_point=zp)
    Xd, Wd = dev(X), dev(W)
    sal = awq.awq_act_stats(Xd)
    res = awq.awq_search_layer(Xd, Wd, sal, cfg)
    torch.cuda.synchronize()
    assert res.plan.tile_tokens == 512
    ref = O.search_layer(X, W, host(sal), group=group, w_bit=w_bit, zero_point=zp)
    losses = host(res.losses)
    rel = np.abs(losses - ref.losses) / ref.losses
    _say(f"  max rel loss diff {rel.max():.3e}")
    assert np.all(rel <= LOSS_RTOL)
    check_best(int(host(res.best_idx)[0]), ref.losses)


@pytest.mark.parametrize("cfg_layer", [(2, 0), (5, 1)])
@pytest.mark.parametrize("group,w_bit,zp", [(64, 3, True), (32, 4, False)])
def test_variant_full_size_sampled_tiles(awq, group, w_bit, zp, cfg_layer):
    """Quantizer variants on a full-size layer of each grid path: the 7B q_proj
    (512 tokens, fused kernels) and the 13B o_proj (4096 tokens, weight error
    produced and contracted); per-tile partial sums of sampled tiles against
    the oracle's."""
    spec, X, W = synth.make_layer(*cfg_layer)
    _say(f"variant full size {spec.name} group {group} w_bit {w_bit} zero_point {zp}")
    cfg = awq.default_config(group_size=group, w_bit=w_bit, zero_point=zp)
    Xd, Wd = dev(X), dev(W)
    sal = awq.awq_act_stats(Xd)
    res = awq.awq_search_layer(Xd, Wd, sal, cfg)
    plan = res.plan
    nt, no = plan.n_token_tiles, plan.n_out_tiles
    part = host(res.workspace[plan.partials_offset:plan.partials_offset + 16 * 20 * nt * no]
                .view(torch.float64)).reshape(20, nt, no, 2).sum(axis=3)
    s_tab, inv_s = O.scale_table(host(sal))
    rng = np.random.default_rng(group + w_bit)
    tm, tn = plan.tile_tokens, plan.tile_out
    for (ti, oi) in [(nt - 1, no - 1), (0, int(rng.integers(no)))]:
        rows = slice(ti * tm, min((ti + 1) * tm, spec.n_tokens))
        cols = slice(oi * tn, min((oi + 1) * tn, spec.out_features))
        for i in (0, 7, 19):
            want = O.tile_sq_error(X, W, s_tab[i], inv_s[i], rows, cols, group, w_bit, zp)
            assert abs(part[i, ti, oi] - want) <= LOSS_RTOL * want, (ti, oi, i)


@pytest.mark.gpu
def test_hot_path_replays_in_a_hip_graph(awq):
    # stats, the search (both grid launches of the 512-token layer), pack and
    # both W4A16 kernels captured once and replayed with eager work between the
    # replays: every replay equals the eager result bit for bit
    _say("hip graph: stats + search + pack + w4a16, 512x4096 -> 4096")
    _, X, W = synth.make_custom(512, 4096, 4096, seed=11)
    Xd = torch.from_numpy(X).cuda()
    Wd = torch.from_numpy(W).cuda()
    xq = Xd[:16].contiguous()

    def run():
        sal = awq.awq_act_stats(Xd)
        res = awq.awq_search_layer(Xd, Wd, sal)
        q, st, z = awq.awq_pack(Wd, res.s_best)
        y1 = awq.awq_w4a16_matmul(xq[:1], q, st, z)
        y16 = awq.awq_w4a16_matmul(xq, q, st, z)
        return sal, res.losses, res.best_idx, res.s_best, q, st, z, y1, y16

    ref = [t.clone() for t in run()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = run()
    for rep in range(3):
        junk = torch.randn(1 << 20, device="cuda")
        junk.mul_(2.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), f"replay {rep}"
    assert int(ref[2].item()) >= 0
