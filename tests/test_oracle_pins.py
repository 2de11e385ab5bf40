"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test fixes the oracle to something outside itself: a value the pages
print (tests/golden), a closed form, a library routine (torch's
scaled_dot_product_attention in float64), an exact construction with a
known answer, or an independent per-token brute force written with Python
loops. ``test_planted_mistakes`` then plants plausible mistakes in copies of
oracle functions and shows that these pins catch each one.
"""
import collections
import json
import math
import os

import numpy as np
import pytest

from oracle import vsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ----------------------------------------------------------------------------
# geometry
# ----------------------------------------------------------------------------

def test_wan_routing_log_line():
    g = _golden("wan_routing_log.json")
    geo = O.geometry(g["dit_seq_shape"], g["block_size"])
    s = O.routing_summary(geo, g["topk"])
    assert s["seq_len"] == g["seq_len"]
    assert s["num_blocks"] == g["num_blocks"]
    assert s["keep_ratio"] == g["keep_ratio"]
    assert list(s["dit_seq_shape"]) == g["dit_seq_shape"]
    assert geo.cube_volume == _golden("block_shapes.json")["wan_block_tokens"]


def test_fastbsa_sparsity_keeps_one_sixteenth():
    g = _golden("block_shapes.json")
    geo = O.geometry((16, 46, 80), g["fastbsa_chunk"])
    assert geo.cube_volume == g["h3_block_tokens"]
    keep = geo.num_blocks * (1.0 - g["fastbsa_sparsity"])
    assert keep == 60.0 and geo.num_blocks == 960


@pytest.mark.parametrize("latent,cube,prefix", [
    ((31, 22, 40), (4, 8, 8), 0), ((16, 46, 80), (4, 4, 4), 0),
    ((21, 30, 52), (4, 4, 4), 512), ((5, 6, 7), (2, 4, 4), 0),
    ((3, 5, 7), (4, 8, 8), 0), ((4, 4, 4), (2, 2, 2), 20), ((1, 1, 1), (1, 1, 1), 0),
])
def test_block_counts_closed_form(latent, cube, prefix):
    geo = O.geometry(latent, cube, prefix)
    V = int(np.prod(cube))
    counts = geo.counts
    assert counts.sum() == geo.seq_len == prefix + int(np.prod(latent))
    # prefix blocks: V tokens each, the last one holds the remainder
    for p in range(geo.num_prefix_blocks):
        assert counts[p] == min(V, prefix - p * V)
    # video cubes: product over axes of min(cube, grid - start)
    nT, nH, nW = geo.nblk
    for bt in range(nT):
        for bh in range(nH):
            for bw in range(nW):
                c = geo.num_prefix_blocks + (bt * nH + bh) * nW + bw
                want = 1
                for L, cs, b in zip(latent, cube, (bt, bh, bw)):
                    want *= min(cs, L - b * cs)
                assert counts[c] == want


def test_valid_count_histograms():
    h = lambda g, lo: dict(collections.Counter(g.counts[lo:].tolist()))
    assert h(O.geometry((31, 22, 40), (4, 8, 8)), 0) == {256: 70, 192: 45, 144: 5}
    assert h(O.geometry((16, 46, 80), (4, 4, 4)), 0) == {64: 880, 32: 80}
    g5 = O.geometry((21, 30, 52), (4, 4, 4), 512)
    assert (g5.num_blocks, g5.num_prefix_blocks) == (624, 8)
    assert h(g5, 8) == {64: 455, 32: 65, 16: 91, 8: 13}


def test_block_map_by_enumeration():
    """Every token is in exactly one block; membership matches a direct walk
    over the cube grid."""
    latent, cube, P = (5, 6, 7), (2, 4, 4), 11
    geo = O.geometry(latent, cube, P)
    T, H, W = latent
    seen = np.zeros(geo.seq_len, dtype=int)
    for m in geo.members:
        seen[m] += 1
    assert np.all(seen == 1)
    c = 0
    for bt in range(0, T, cube[0]):
        for bh in range(0, H, cube[1]):
            for bw in range(0, W, cube[2]):
                toks = sorted(P + (t * H + hh) * W + w
                              for t in range(bt, min(T, bt + cube[0]))
                              for hh in range(bh, min(H, bh + cube[1]))
                              for w in range(bw, min(W, bw + cube[2])))
                assert list(geo.members[geo.num_prefix_blocks + c]) == toks
                c += 1
    assert c == geo.num_blocks


# ----------------------------------------------------------------------------
# pool
# ----------------------------------------------------------------------------

def _coord_features(latent, prefix, D=8):
    T, H, W = latent
    x = np.zeros((prefix + T * H * W, D))
    x[:prefix, 3] = np.arange(prefix)
    t, hh, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    x[prefix:, 0] = t.ravel()
    x[prefix:, 1] = hh.ravel()
    x[prefix:, 2] = w.ravel()
    return x


@pytest.mark.parametrize("latent,cube,prefix", [
    ((31, 22, 40), (4, 8, 8), 0), ((21, 30, 52), (4, 4, 4), 512), ((5, 6, 7), (2, 4, 4), 20),
])
def test_pool_centroid(latent, cube, prefix):
    """Pooling the coordinates gives the centroid of each block's valid
    region: the midpoint of each clipped axis range."""
    geo = O.geometry(latent, cube, prefix)
    pooled = O.pool(_coord_features(latent, prefix), geo)
    V = geo.cube_volume
    for p in range(geo.num_prefix_blocks):
        lo, hi = p * V, min(prefix, (p + 1) * V) - 1
        assert pooled[p, 3] == pytest.approx((lo + hi) / 2, abs=1e-12)
    nT, nH, nW = geo.nblk
    for bt in range(nT):
        for bh in range(nH):
            for bw in range(nW):
                c = geo.num_prefix_blocks + (bt * nH + bh) * nW + bw
                for a, b in enumerate((bt, bh, bw)):
                    lo = b * cube[a]
                    hi = min(latent[a], lo + cube[a]) - 1
                    assert pooled[c, a] == pytest.approx((lo + hi) / 2, abs=1e-12)


def test_pool_centroid_wan_last_cube_by_hand():
    geo = O.geometry((31, 22, 40), (4, 8, 8))
    pooled = O.pool(_coord_features((31, 22, 40), 0), geo)
    # last cube: t in 28..30, h in 16..21, w in 32..39
    assert tuple(pooled[-1, :3]) == (29.0, 18.5, 35.5)


def test_pool_constant_and_linear():
    geo = O.geometry((5, 6, 7), (2, 4, 4), 9)
    x = np.full((geo.seq_len, 4), 3.25)
    assert np.all(O.pool(x, geo) == 3.25)
    y = _rand((geo.seq_len, 4), 0)
    np.testing.assert_allclose(O.pool(2 * x - y, geo), 2 * O.pool(x, geo) - O.pool(y, geo),
                               atol=1e-13)


# ----------------------------------------------------------------------------
# score + select
# ----------------------------------------------------------------------------

def test_select_known_order_construction():
    """q = e0 everywhere and k = r_cube * e0: cube scores are r_j / sqrt(D),
    so the kept set is the topk largest r."""
    latent, cube, D = (5, 6, 7), (2, 4, 4), 16
    geo = O.geometry(latent, cube)
    r = np.random.default_rng(3).permutation(geo.num_blocks).astype(float) - 4.0
    q = np.zeros((geo.seq_len, D)); q[:, 0] = 1.0
    k = np.zeros((geo.seq_len, D)); k[:, 0] = r[geo.block_of_token]
    s = O.block_scores(O.pool(q, geo), O.pool(k, geo, video_only=True), D)
    np.testing.assert_allclose(s, np.broadcast_to(r / 4.0, s.shape), atol=1e-14)
    for topk in (1, 3, geo.num_blocks):
        sel = O.select_topk(s, topk)
        want = np.sort(np.argsort(-r)[:topk])
        assert np.all(sel == want)


def test_select_matches_full_sort():
    s = _rand((7, 50), 11)
    for topk in (1, 5, 49, 50):
        sel = O.select_topk(s, topk)
        for i in range(7):
            want = sorted(sorted(range(50), key=lambda j: (-s[i, j], j))[:topk])
            assert list(sel[i]) == want


def test_select_ties_go_to_lower_index():
    s = np.array([[1.0, 2.0, 2.0, 0.5, 2.0, 2.0]])
    assert list(O.select_topk(s, 2)[0]) == [1, 2]
    assert list(O.select_topk(s, 3)[0]) == [1, 2, 4]
    assert list(O.select_topk(np.zeros((1, 5)), 2)[0]) == [0, 1]


@pytest.mark.parametrize("topk", [0, -1, 13])
def test_select_rejects_bad_topk(topk):
    with pytest.raises(ValueError):
        O.select_topk(np.zeros((2, 12)), topk)


def test_check_selection_band():
    s = np.array([[0.5, 0.3, 0.3 + 5e-7, 0.1]])
    ok = O.check_selection(np.array([[0, 1]]), s, 2)
    assert ok["mismatch_rows"] == [] and ok["band_rows"] == 1
    ok2 = O.check_selection(np.array([[0, 2]]), s, 2)
    assert ok2["mismatch_rows"] == []
    bad = O.check_selection(np.array([[1, 2]]), s, 2)
    assert bad["mismatch_rows"] == [0]
    assert O.check_selection(np.array([[2, 0]]), s, 2)["mismatch_rows"] == [0]


# ----------------------------------------------------------------------------
# attend
# ----------------------------------------------------------------------------

def _sdpa64(q, k, v):
    import torch
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v))[0, 0].numpy()


@pytest.mark.parametrize("latent,cube,prefix,D", [
    ((8, 8, 8), (4, 4, 4), 0, 64), ((5, 6, 7), (2, 4, 4), 0, 32),
    ((3, 5, 7), (4, 8, 8), 0, 16), ((4, 4, 4), (2, 2, 2), 20, 16),
])
def test_all_blocks_equals_dense_sdpa(latent, cube, prefix, D):
    geo = O.geometry(latent, cube, prefix)
    q, k, v = (_rand((geo.seq_len, D), s) for s in (1, 2, 3))
    _, sel, out = O.forward_head(q, k, v, geo, geo.num_blocks)
    np.testing.assert_allclose(out, _sdpa64(q, k, v), rtol=0, atol=1e-12)


def test_softmax_rows_sum_to_one_and_convex_hull():
    geo = O.geometry((5, 6, 7), (2, 4, 4), 9)
    D = 16
    q, k, v = (_rand((geo.seq_len, D), s) for s in (4, 5, 6))
    s = O.block_scores(O.pool(q, geo), O.pool(k, geo, video_only=True), D)
    sel = O.select_topk(s, 3)
    out, rs = O.attend_dense_masked(q, k, v, sel, geo, return_rowsums=True)
    assert np.max(np.abs(rs - 1.0)) < 1e-12
    for i in range(geo.num_q_blocks):
        keep = np.isin(geo.block_of_token, O.kept_blocks(sel[i], geo))
        rows = geo.members[i]
        assert np.all(out[rows] <= v[keep].max(0) + 1e-12)
        assert np.all(out[rows] >= v[keep].min(0) - 1e-12)
    ones = O.attend_dense_masked(q, k, np.ones_like(v), sel, geo)
    assert np.max(np.abs(ones - 1.0)) < 1e-12
    scaled = O.attend_dense_masked(q, k, -2.5 * v, sel, geo)
    np.testing.assert_allclose(scaled, -2.5 * out, rtol=0, atol=1e-12)


def test_equal_keys_give_mean_of_kept_values():
    geo = O.geometry((5, 6, 7), (2, 4, 4), 5)
    D = 8
    q = _rand((geo.seq_len, D), 1)
    k = np.tile(_rand((1, D), 2), (geo.seq_len, 1))
    v = _rand((geo.seq_len, D), 3)
    sel = O.select_topk(_rand((geo.num_q_blocks, geo.num_blocks), 4), 4)
    out = O.attend_dense_masked(q, k, v, sel, geo)
    for i in range(geo.num_q_blocks):
        keep = np.isin(geo.block_of_token, O.kept_blocks(sel[i], geo))
        np.testing.assert_allclose(out[geo.members[i]],
                                   np.broadcast_to(v[keep].mean(0), (geo.members[i].size, D)),
                                   atol=1e-12)


BRUTE_CASES = [
    ((8, 8, 8), (4, 4, 4), 0, 4, 16),      # the tiny workload's grid
    ((5, 6, 7), (2, 4, 4), 0, 5, 8),       # partial cubes on every axis
    ((3, 5, 7), (4, 8, 8), 0, 1, 8),       # one cube larger than the grid
    ((4, 4, 4), (2, 2, 2), 20, 3, 8),      # prefix with a partial prefix block
]


@pytest.mark.parametrize("latent,cube,prefix,topk,D", BRUTE_CASES)
def test_brute_force_per_token(latent, cube, prefix, topk, D):
    geo = O.geometry(latent, cube, prefix)
    q, k, v = (_rand((geo.seq_len, D), s) for s in (7, 8, 9))
    _, _, out = O.forward_head(q, k, v, geo, topk)
    ql, kl, vl = q.tolist(), k.tolist(), v.tolist()
    toks = np.random.default_rng(0).choice(geo.seq_len, size=min(12, geo.seq_len), replace=False)
    toks = sorted(set(toks.tolist()) | {0, geo.seq_len - 1})
    for n in toks:
        bf = O.brute_force_token(ql, kl, vl, latent, cube, prefix, topk, n)
        np.testing.assert_allclose(out[n], bf, rtol=0, atol=1e-12)


# q and k/v on different grids (fastbsa "Use": separate latent and chunk
# shapes for q and k; R20): (latent_q, cube_q, latent_k, cube_k, prefix, topk, D)
CROSS_CASES = [
    ((4, 6, 5), (2, 2, 3), (3, 5, 7), (2, 4, 4), 0, 3, 8),    # partial cubes on both sides
    ((2, 4, 4), (1, 2, 2), (4, 4, 4), (2, 2, 2), 6, 2, 8),    # prefix: 2 query, 1 key prefix blocks
    ((3, 3, 3), (1, 1, 1), (3, 3, 3), (3, 3, 3), 0, 1, 8),    # one-token query blocks, one key cube
]


@pytest.mark.parametrize("lq,cq,lk,ck,prefix,topk,D", CROSS_CASES)
def test_brute_force_cross_grids(lq, cq, lk, ck, prefix, topk, D):
    gq, gk = O.geometry(lq, cq, prefix), O.geometry(lk, ck, prefix)
    q = _rand((gq.seq_len, D), 17)
    k, v = _rand((gk.seq_len, D), 18), _rand((gk.seq_len, D), 19)
    _, sel, out = O.forward_head(q, k, v, gq, topk, gk=gk)
    assert sel.shape == (gq.num_q_blocks, topk) and sel.max() < gk.num_blocks
    ql, kl, vl = q.tolist(), k.tolist(), v.tolist()
    for n in sorted(set(range(0, gq.seq_len, 5)) | {gq.seq_len - 1}):
        bf = O.brute_force_token(ql, kl, vl, lq, cq, prefix, topk, n, latent_k=lk, cube_k=ck)
        np.testing.assert_allclose(out[n], bf, rtol=0, atol=1e-12)


def test_cross_grid_all_blocks_equals_dense_sdpa():
    """Every key cube kept: dense attention of Nq queries over Nk keys."""
    gq, gk = O.geometry((3, 4, 6), (2, 2, 4), 5), O.geometry((5, 3, 6), (4, 2, 2), 5)
    D = 16
    q = _rand((gq.seq_len, D), 21)
    k, v = _rand((gk.seq_len, D), 22), _rand((gk.seq_len, D), 23)
    _, _, out = O.forward_head(q, k, v, gq, gk.num_blocks, gk=gk)
    np.testing.assert_allclose(out, _sdpa64(q, k, v), rtol=0, atol=1e-12)


def test_one_token_query_blocks_score_each_token():
    """Query cubes of one token: the pooled query is the token itself, so a
    token's kept cubes are the top-k of q_n . kbar_j (closed form)."""
    gq, gk = O.geometry((2, 3, 4), (1, 1, 1)), O.geometry((2, 3, 4), (1, 3, 2))
    D = 8
    q, k = _rand((gq.seq_len, D), 24), _rand((gk.seq_len, D), 25)
    kbar = np.stack([k[m].mean(axis=0) for m in gk.members])
    s, sel, _ = O.forward_head(q, k, k, gq, 2, gk=gk)
    np.testing.assert_allclose(s, q @ kbar.T / math.sqrt(D), rtol=0, atol=1e-12)
    want = np.sort(np.argsort(-(q @ kbar.T), axis=1, kind="stable")[:, :2], axis=1)
    assert np.array_equal(sel, want)


def test_topk_for_sparsity():
    """fastbsa "Use" passes sparsity 0.9375: 1/16 of the cubes are kept
    (R21: floor(nb * (1 - s)), at least one, at most all)."""
    g = _golden("block_shapes.json")
    assert O.topk_for_sparsity(960, g["fastbsa_sparsity"]) == 60     # the page's 1/16 of 960
    assert O.topk_for_sparsity(624, 0.9375) == 39
    assert O.topk_for_sparsity(120, 0.9375) == 7        # 7.5: the kept fraction stays <= 1/16
    assert O.topk_for_sparsity(1320, 0.9375) == 82      # 82.5
    assert O.topk_for_sparsity(120, 0.9) == 12          # 120 * (1 - 0.9) = 11.999999999999998 in binary
    assert O.topk_for_sparsity(120, 0.0) == 120
    assert O.topk_for_sparsity(120, 0.999) == 1         # 0.12 -> at least one
    assert O.topk_for_sparsity(7, 0.5) == 3             # 3.5
    for bad in (-0.1, 1.0, float("nan")):
        with pytest.raises(ValueError):
            O.topk_for_sparsity(120, bad)


def test_topk_for_sparsity_exact_rationals():
    """Against exact rational arithmetic: for every block count up to 4096
    and the sparsities a/16 (exact in binary) and a/100 (decimal, inexact in
    binary), the kept count is max(1, floor(nb * (1 - s))) computed with
    fractions.Fraction."""
    from fractions import Fraction
    for den, nums in ((16, range(16)), (100, (0, 1, 10, 25, 50, 75, 80, 90, 95, 99))):
        for a in nums:
            s = Fraction(a, den)
            for nb in list(range(1, 257)) + [600, 624, 960, 1000, 1320, 2048, 4095, 4096]:
                want = max(1, int(nb * (1 - s)))        # int() of a positive Fraction is floor
                assert O.topk_for_sparsity(nb, a / den) == want, (nb, a, den)


def test_shift_of_all_keys_changes_nothing():
    """Adding one vector b to every key adds q.b to a whole row of logits and
    qbar_i.b to a whole row of block scores: selection and output stay."""
    geo = O.geometry((5, 6, 7), (2, 4, 4), 7)
    D = 16
    q, k, v = (_rand((geo.seq_len, D), s) for s in (1, 2, 3))
    b = 3.0 * _rand((1, D), 4)
    s1, sel1, o1 = O.forward_head(q, k, v, geo, 4)
    s2, sel2, o2 = O.forward_head(q, k + b, v, geo, 4)
    assert np.all(sel1 == sel2)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(s2 - s1, np.broadcast_to((O.pool(q, geo) @ b.T) / 4.0, s1.shape),
                               atol=1e-12)


def test_decode_bf16_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x4049, 0x7F7F, 0x0001], dtype=np.uint16)
    want = [1.0, -1.0, 0.0, -0.0, 3.140625, 3.3895313892515355e38, 2.0 ** -133]
    assert O.decode_bf16(bits).tolist() == want


def test_decode_f16_exact():
    """Closed forms of IEEE binary16: one, a negative power of two, the
    largest finite value (2 - 2^-10) * 2^15, the smallest normal 2^-14, the
    smallest subnormal 2^-24, the largest subnormal (1 - 2^-10) * 2^-14,
    1/3 rounded to 11 significant bits, signed zero and infinity."""
    bits = np.array([0x3C00, 0xC000, 0x7BFF, 0x0400, 0x0001, 0x03FF, 0x3555, 0x8000, 0x7C00, 0xFC00],
                    dtype=np.uint16)
    want = [1.0, -2.0, 65504.0, 2.0 ** -14, 2.0 ** -24, (1 - 2.0 ** -10) * 2.0 ** -14,
            1365.0 / 4096.0, -0.0, np.inf, -np.inf]
    got = O.decode_f16(bits)
    assert got.tolist() == want
    assert np.signbit(got[7])
    assert np.isnan(O.decode_f16(np.array([0x7E00, 0xFC01], dtype=np.uint16))).all()


def test_decode_f16_matches_numpy_on_every_pattern():
    """All 65536 patterns against numpy's own binary16 type (NaNs aside)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = O.decode_f16(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


# ----------------------------------------------------------------------------
# comparison helpers (fastbsa "How it works": outputs are validated against
# dense-masked attention; these norms make that call)
# ----------------------------------------------------------------------------

def test_error_norms_closed_forms():
    rng = np.random.default_rng(41)
    ref = rng.standard_normal((37, 16))
    # out = ref + d * e_i: max_abs is exactly |d|, rel_l2 is |d| / ||ref||
    for d in (0.25, -0.125):
        out = ref.copy()
        out[5, 3] += d
        e = O.error_norms(out, ref)
        assert e["max_abs"] == abs(d)
        assert e["rel_l2"] == pytest.approx(abs(d) / math.sqrt(float(np.sum(ref * ref))), rel=1e-12)
    # out = 2 ref: rel_l2 1 (normalised by the reference, not by out)
    assert O.error_norms(2.0 * ref, ref)["rel_l2"] == pytest.approx(1.0, rel=1e-14)
    # out = -ref: rel_l2 2; out = ref: zeros
    assert O.error_norms(-ref, ref)["rel_l2"] == pytest.approx(2.0, rel=1e-14)
    assert O.error_norms(ref, ref) == {"max_abs": 0.0, "rel_l2": 0.0}
    # a zero reference is guarded: 0 for a zero output, infinity otherwise
    z = np.zeros((3, 4))
    assert O.error_norms(z, z) == {"max_abs": 0.0, "rel_l2": 0.0}
    assert O.error_norms(z + 1.0, z)["rel_l2"] == math.inf
    assert O.error_norms(np.zeros((0, 4)), np.zeros((0, 4))) == {"max_abs": 0.0, "rel_l2": 0.0}
    with pytest.raises(ValueError):
        O.error_norms(z, np.zeros((4, 3)))


def test_error_norms_by_block_localises_an_error():
    """An error confined to one block shows up in that block's own norms at
    full size while the whole-tensor relative L2 stays small."""
    g = O.geometry((5, 6, 7), (2, 4, 4), 7)
    ref = np.random.default_rng(43).standard_normal((g.seq_len, 8))
    out = ref.copy()
    bad = 5
    out[g.members[bad]] *= 1.5
    per = O.error_norms_by_block(out, ref, g)
    assert set(per) == set(range(g.num_q_blocks))
    assert per[bad]["rel_l2"] == pytest.approx(0.5, rel=1e-12)
    assert all(per[i]["rel_l2"] == 0.0 for i in per if i != bad)
    assert O.error_norms(out, ref)["rel_l2"] < 0.5
    assert O.error_norms_by_block(out, ref, g, blocks=[bad, 0]).keys() == {bad, 0}


# ----------------------------------------------------------------------------
# planted mistakes: each must be caught by one of the pins above
# ----------------------------------------------------------------------------

def _pool_zero_padded(x, g, video_only=False):
    first = g.num_prefix_blocks if video_only else 0
    out = np.empty(x.shape[:-2] + (g.num_q_blocks - first, x.shape[-1]))
    for i in range(first, g.num_q_blocks):
        out[..., i - first, :] = x[..., g.members[i], :].sum(axis=-2) / g.cube_volume
    return out


def _select_ties_high(scores, topk):
    order = np.argsort(-scores[..., ::-1], axis=-1, kind="stable")[..., :topk]
    return np.sort(scores.shape[-1] - 1 - order, axis=-1)


def _kept_no_prefix(sel_row, g):
    return np.array([g.num_prefix_blocks + int(j) for j in sel_row])


def _scores_swapped(qbar, kbar, D):
    # operands swapped: s[i, j] = kbar_i . qbar_j (square when nq == nb)
    return np.swapaxes(np.matmul(qbar, np.swapaxes(kbar, -1, -2)), -1, -2) * D ** -0.5


def _attend_wrong_scale(q, k, v, sel, g, query_blocks=None, return_rowsums=False, gk=None):
    # logits left unscaled (the head_dim ** -0.5 factor dropped)
    return O.__dict__["_orig_attend"](q * math.sqrt(q.shape[1]), k, v, sel, g,
                                      query_blocks, return_rowsums, gk=gk)


def _attend_query_prefix_count(q, k, v, sel, g, query_blocks=None, return_rowsums=False, gk=None):
    # key blocks numbered with the query grid's prefix-block count
    gk = g if gk is None else gk
    out = np.full((q.shape[0], v.shape[1]), np.nan)
    for i in (range(g.num_q_blocks) if query_blocks is None else query_blocks):
        ids = list(range(g.num_prefix_blocks)) + [g.num_prefix_blocks + int(j) for j in sel[i]]
        keep = np.isin(gk.block_of_token, ids)
        L = (q[g.members[i]] @ k.T) / math.sqrt(q.shape[1])
        L[:, ~keep] = -np.inf
        Pm = np.exp(L - L.max(axis=1, keepdims=True))
        out[g.members[i]] = (Pm / Pm.sum(axis=1, keepdims=True)) @ v
    return out


def _sparsity_nearest(num_blocks, sparsity):
    # nearest integer, halves up, instead of floor
    return int(min(max(math.floor(num_blocks * (1.0 - sparsity) + 0.5 + 1e-9), 1), num_blocks))


def _sparsity_plain_floor(num_blocks, sparsity):
    # floor of the binary product, with no allowance for decimal sparsities
    return int(min(max(math.floor(num_blocks * (1.0 - sparsity)), 1), num_blocks))


def _norms_by_out(out, ref):
    # normalised by the output instead of the reference
    d = np.asarray(out, dtype=np.float64) - np.asarray(ref, dtype=np.float64)
    return {"max_abs": float(np.max(np.abs(d))), "rel_l2": float(np.linalg.norm(d) / np.linalg.norm(out))}


def _norms_signed_max(out, ref):
    # signed maximum of the difference instead of the maximum magnitude
    d = np.asarray(out, dtype=np.float64) - np.asarray(ref, dtype=np.float64)
    return {"max_abs": float(np.max(d)), "rel_l2": float(np.linalg.norm(d) / np.linalg.norm(ref))}


def _f16_bias_16(bits):
    # exponent bias off by one
    return O.__dict__["_orig_decode_f16"](bits) * 0.5


def _f16_subnormals_as_normals(bits):
    # exponent 0 given the implicit leading one
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    out = O.__dict__["_orig_decode_f16"](bits)
    e0 = ((b >> 10) & 0x1F) == 0
    out[e0] = np.where((b[e0] >> 15) & 1, -1.0, 1.0) * np.ldexp(1.0 + (b[e0] & 0x3FF) / 1024.0, -14)
    return out


@pytest.mark.parametrize("target,mutant,pin", [
    ("attend_dense_masked", _attend_query_prefix_count, "brute_cross_prefix"),
    ("topk_for_sparsity", _sparsity_nearest, "sparsity"),
    ("topk_for_sparsity", _sparsity_plain_floor, "sparsity_exact"),
    ("error_norms", _norms_by_out, "norms"),
    ("error_norms", _norms_signed_max, "norms"),
    ("decode_f16", _f16_bias_16, "f16_closed"),
    ("decode_f16", _f16_subnormals_as_normals, "f16_numpy"),
    ("pool", _pool_zero_padded, "centroid"),
    ("select_topk", _select_ties_high, "ties"),
    ("kept_blocks", _kept_no_prefix, "brute_prefix"),
    ("block_scores", _scores_swapped, "brute_padded"),
    ("attend_dense_masked", _attend_wrong_scale, "sdpa"),
])
def test_planted_mistakes(monkeypatch, target, mutant, pin):
    monkeypatch.setitem(O.__dict__, "_orig_attend", O.attend_dense_masked)
    monkeypatch.setitem(O.__dict__, "_orig_decode_f16", O.decode_f16)
    monkeypatch.setattr(O, target, mutant)
    pins = {
        "centroid": lambda: test_pool_centroid((31, 22, 40), (4, 8, 8), 0),
        "ties": test_select_ties_go_to_lower_index,
        "brute_prefix": lambda: test_brute_force_per_token(*BRUTE_CASES[3]),
        "brute_padded": lambda: test_brute_force_per_token(*BRUTE_CASES[1]),
        "sdpa": lambda: test_all_blocks_equals_dense_sdpa((5, 6, 7), (2, 4, 4), 0, 32),
        "brute_cross_prefix": lambda: test_brute_force_cross_grids(*CROSS_CASES[1]),
        "sparsity": test_topk_for_sparsity,
        "sparsity_exact": test_topk_for_sparsity_exact_rationals,
        "norms": test_error_norms_closed_forms,
        "f16_closed": test_decode_f16_exact,
        "f16_numpy": test_decode_f16_matches_numpy_on_every_pattern,
    }
    with pytest.raises(AssertionError):
        pins[pin]()
