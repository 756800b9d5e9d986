"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: hand-worked
fixtures, a constructive enumeration of the window order, closed forms,
invariants, special cases that reduce to textbook dense attention, and brute
force on tiny inputs.  No GPU is needed.
"""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special
from hypothesis import given, settings, strategies as st

from oracle import rainfusion_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = [int(v) for v in vals]
    return out


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ---------------------------------------------------------------- permutation

@pytest.mark.parametrize("name", ["slots_T2H3W4_win1x2x2.txt",
                                  "slots_T3H2W3_win2x1x3.txt"])
def test_slots_match_hand_worked_fixture(name):
    g = _read_golden(name)
    lay = orc.Layout(g["T"][0], g["H"][0], g["W"][0], g["wt"][0], g["wh"][0],
                     g["ww"][0], sink=1)
    z = orc.sizes(lay)
    assert z["Np"] == g["Np"][0] and z["nb"] == g["nb"][0]
    assert orc.slot_of_token(lay).tolist() == g["slots"]
    assert orc.block_counts(lay).tolist() == g["counts"]
    assert orc.sink_blocks(lay).tolist() == g["sinks"]


def test_tiny_workload_slots_by_hand():
    # 3x16x16 grid, 1x8x8 windows: 2x2 blocks per frame of 64 tokens.
    lay = orc.Layout(3, 16, 16, 1, 8, 8, sink=1)
    slot = orc.slot_of_token(lay)
    n = lambda t, h, w: (t * 16 + h) * 16 + w
    assert slot[n(0, 0, 8)] == 64
    assert slot[n(0, 8, 0)] == 128
    assert slot[n(1, 0, 0)] == 256
    assert slot[n(0, 1, 0)] == 8
    assert slot[n(2, 15, 15)] == 767
    assert orc.sink_blocks(lay).tolist() == [0, 1, 2, 3]


def _enumerate_window_order(lay):
    """Slot sequence built constructively: walk the padded grid window by
    window (frames outermost), and inside each window row-major; record which
    raster token (or pad) lands in each successive slot."""
    T, H, W, wt, wh, ww = lay.T, lay.H, lay.W, lay.wt, lay.wh, lay.ww
    src = []
    for t0 in range(0, math.ceil(T / wt) * wt, wt):
        for h0 in range(0, math.ceil(H / wh) * wh, wh):
            for w0 in range(0, math.ceil(W / ww) * ww, ww):
                for t in range(t0, t0 + wt):
                    for h in range(h0, h0 + wh):
                        for w in range(w0, w0 + ww):
                            ok = t < T and h < H and w < W
                            src.append((t * H + h) * W + w if ok else -1)
    return src


@pytest.mark.parametrize("dims", [(3, 16, 16, 1, 8, 8), (2, 5, 7, 2, 2, 3),
                                  (4, 6, 9, 3, 4, 2), (1, 12, 10, 1, 8, 16)])
def test_slots_match_constructive_enumeration(dims):
    lay = orc.Layout(*dims)
    src = _enumerate_window_order(lay)
    slot = orc.slot_of_token(lay)
    assert len(src) == orc.sizes(lay)["Np"]
    for p, n in enumerate(src):
        if n >= 0:
            assert slot[n] == p
    assert sorted(n for n in src if n >= 0) == list(range(lay.T * lay.H * lay.W))


def test_whole_frame_windows_are_identity():
    for lay in (orc.Layout(3, 4, 5, 1, 4, 5), orc.Layout(2, 3, 8, 1, 1, 8)):
        assert (orc.slot_of_token(lay) == np.arange(lay.T * lay.H * lay.W)).all()


@settings(max_examples=60, deadline=None)
@given(T=st.integers(1, 5), H=st.integers(1, 9), W=st.integers(1, 9),
       wt=st.integers(1, 3), wh=st.integers(1, 4), ww=st.integers(1, 4),
       n_text=st.integers(0, 7), permute=st.integers(0, 1))
def test_permutation_is_a_bijection_and_roundtrips(T, H, W, wt, wh, ww, n_text,
                                                   permute):
    lay = orc.Layout(T, H, W, wt, wh, ww, n_text=n_text, permute=permute)
    z = orc.sizes(lay)
    slot = orc.slot_of_token(lay)
    assert len(np.unique(slot)) == z["N"]
    assert slot.min() >= 0 and slot.max() < z["Np"]
    assert z["Np"] % z["bs"] == 0 and z["Np"] >= z["N"]
    x = _rng(7).standard_normal((1, 2, z["L"], 3))
    xp = orc.permute(x, lay)
    assert xp.shape == (1, 2, z["Lp"], 3)
    assert (xp[..., ~orc.slot_valid(lay), :] == 0).all()
    assert np.array_equal(orc.unpermute(xp, lay), x)
    assert np.array_equal(np.sort(xp[0, 0, orc.slot_valid(lay), 0]),
                          np.sort(x[0, 0, :, 0]))
    counts = orc.block_counts(lay)
    assert counts.sum() == z["N"] and (counts >= 1).all()


def test_raster_mode_sizes_and_sink():
    # 21x45x80 raster with 128-token blocks: 591 blocks, last one 80 valid,
    # frame 0 (3600 tokens) touches 29 blocks.
    lay = orc.Layout(21, 45, 80, 2, 8, 8, permute=0, sink=1)
    z = orc.sizes(lay)
    assert (z["nb"], z["Np"]) == (591, 75648)
    assert orc.block_counts(lay)[-1] == 80
    assert orc.sink_blocks(lay).tolist() == list(range(29))


def test_video720_padding_profile():
    lay = orc.Layout(21, 45, 80, 2, 8, 8, sink=1)
    z = orc.sizes(lay)
    assert (z["Np"], z["nb"]) == (84480, 660)
    c = orc.block_counts(lay)
    assert {v: int((c == v).sum()) for v in np.unique(c)} == \
        {40: 10, 64: 50, 80: 100, 128: 500}
    assert len(orc.sink_blocks(lay)) == 60


# ---------------------------------------------------------------- block means

@pytest.mark.parametrize("dims", [(3, 16, 16, 1, 8, 8), (5, 7, 9, 2, 4, 4),
                                  (3, 5, 6, 2, 2, 4)])
def test_means_of_affine_field_are_centroids(dims):
    """x(t,h,w) = a + bt t + bh h + bw w  =>  block mean = x(centroid of the
    block's valid tokens); the valid set is a box, so the centroid is the
    midpoint of each clipped range."""
    lay = orc.Layout(*dims)
    T, H, W, wt, wh, ww = dims
    d = 5
    r = _rng(3)
    a, bt, bh, bw = (r.standard_normal(d) for _ in range(4))
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W),
                          indexing="ij")
    x = (a + bt * t[..., None] + bh * h[..., None] + bw * w[..., None])
    x = x.reshape(1, 1, T * H * W, d)
    means = orc.block_means(orc.permute(x, lay), lay)[0, 0]
    z = orc.sizes(lay)
    mid = lambda b, win, n: (b * win + min((b + 1) * win, n) - 1) / 2.0
    for B in range(z["nb"]):
        ib, jw = divmod(B, z["nW"])
        it, ih = divmod(ib, z["nH"])
        want = (a + bt * mid(it, wt, T) + bh * mid(ih, wh, H)
                + bw * mid(jw, ww, W))
        np.testing.assert_allclose(means[B], want, rtol=0, atol=1e-12)


def test_means_ignore_pad_slots_and_constants():
    lay = orc.Layout(3, 5, 6, 2, 2, 4)
    z = orc.sizes(lay)
    x = np.full((1, 2, z["L"], 4), 2.5)
    xp = orc.permute(x, lay)
    np.testing.assert_allclose(orc.block_means(xp, lay), 2.5, atol=1e-15)
    y = _rng(5).standard_normal((1, 2, z["L"], 4))
    yp = orc.permute(y, lay)
    poisoned = yp.copy()
    poisoned[..., ~orc.slot_valid(lay), :] = 1e6
    assert np.array_equal(orc.block_means(poisoned, lay),
                          orc.block_means(yp, lay))


def test_means_by_brute_force():
    lay = orc.Layout(3, 5, 6, 2, 2, 4)
    z = orc.sizes(lay)
    x = _rng(11).standard_normal((1, 1, z["L"], 3))
    means = orc.block_means(orc.permute(x, lay), lay)[0, 0]
    for B in range(z["nb"]):
        members = [n for n in range(z["N"])
                   if orc.slot_of_token(lay)[n] // z["bs"] == B]
        np.testing.assert_allclose(means[B], x[0, 0, members].mean(axis=0),
                                   atol=1e-14)


# ---------------------------------------------------------------- mask rule

def test_block_scores_softmax():
    r = _rng(2)
    qbar, kbar = r.standard_normal((1, 2, 7, 16)), r.standard_normal((1, 2, 7, 16))
    l, P = orc.block_scores(qbar, kbar)
    np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-14)
    ref = scipy.special.softmax(np.einsum("bhid,bhjd->bhij", qbar, kbar) / 4.0,
                                axis=-1)
    np.testing.assert_allclose(P, ref, atol=1e-14)
    np.testing.assert_allclose(l[0, 1, 3, 5], qbar[0, 1, 3] @ kbar[0, 1, 5] / 4.0,
                               atol=1e-14)


def test_keep_counts_golden():
    with open(os.path.join(GOLDEN, "keep_counts.txt")) as f:
        rows = [list(map(int, l.split())) for l in f
                if l.strip() and not l.startswith("#")]
    for n, s, ns, k, keff in rows:
        assert orc.keep_count(n, s, ns) == (k, keff), (n, s, ns)


@pytest.mark.parametrize("n", [1, 7, 12, 32, 591, 660, 960])
def test_kept_fraction_hits_target(n):
    for s in range(0, 100):
        k, _ = orc.keep_count(n, s, 0)
        assert abs(k / n - (1 - s / 100)) <= 1 / (2 * n) + 1e-12


def _planted(lay, values, d=8):
    """Tokens whose key-block means are values[j] * e0 and whose query means
    are e0, so l_ij = values[j] / sqrt(d) exactly (up to rounding)."""
    z = orc.sizes(lay)
    slot = orc.slot_of_token(lay)
    blk = slot // z["bs"]
    k = np.zeros((1, 1, z["L"], d))
    k[0, 0, :z["N"], 0] = values[blk]
    q = np.zeros((1, 1, z["L"], d))
    q[0, 0, :, 0] = 1.0
    return q, k


def test_planted_ranking_gives_expected_mask():
    lay = orc.Layout(2, 8, 12, 1, 4, 4, sink=1)
    z = orc.sizes(lay)
    nb = z["nb"]
    assert nb == 12
    values = _rng(9).permutation(nb).astype(np.float64)
    q, k = _planted(lay, values)
    qbar = orc.block_means(orc.permute(q, lay), lay)
    kbar = orc.block_means(orc.permute(k, lay), lay)
    sinks = [0, 1, 2, 3, 4, 5]
    for s in (0, 25, 50, 75, 95):
        kept, _ = orc.predict_mask(qbar, kbar, lay, s)
        _, keff = orc.keep_count(nb, s, len(sinks))
        others = sorted((j for j in range(nb) if j not in sinks),
                        key=lambda j: -values[j])
        want = sorted(sinks + others[:keff - len(sinks)])
        for row in kept[0][0]:
            assert row.tolist() == want


def test_ties_go_to_lower_index_and_sinks_only_when_budget_is_small():
    lay = orc.Layout(2, 8, 12, 1, 4, 4, sink=1)
    q, k = _planted(lay, np.ones(12))
    qbar = orc.block_means(orc.permute(q, lay), lay)
    kbar = orc.block_means(orc.permute(k, lay), lay)
    kept, _ = orc.predict_mask(qbar, kbar, lay, 50)
    assert kept[0][0][0].tolist() == [0, 1, 2, 3, 4, 5]          # k_eff = 6
    kept, _ = orc.predict_mask(qbar, kbar, lay, 25)
    assert kept[0][0][0].tolist() == list(range(9))              # 6 sinks + 6,7,8
    kept, _ = orc.predict_mask(qbar, kbar, lay, 90)
    assert kept[0][0][0].tolist() == [0, 1, 2, 3, 4, 5]          # sink-bound


def test_mask_by_brute_force_subset_search():
    """With distinct scores, the kept non-sink set is the unique k-subset of
    non-sink blocks with the largest logit sum."""
    lay = orc.Layout(3, 4, 6, 1, 2, 3, sink=1)       # 12 blocks, 4 sinks
    z = orc.sizes(lay)
    r = _rng(21)
    q = r.standard_normal((1, 2, z["L"], 6))
    k = r.standard_normal((1, 2, z["L"], 6))
    qbar = orc.block_means(orc.permute(q, lay), lay)
    kbar = orc.block_means(orc.permute(k, lay), lay)
    sinks = orc.sink_blocks(lay).tolist()
    assert sinks == [0, 1, 2, 3]
    for s in (30, 60):
        kept, l = orc.predict_mask(qbar, kbar, lay, s)
        _, keff = orc.keep_count(12, s, 4)
        for h in range(2):
            for i in range(12):
                logits = qbar[0, h, i] @ kbar[0, h].T / math.sqrt(6)
                best = max(itertools.combinations(range(4, 12), keff - 4),
                           key=lambda c: sum(logits[j] for j in c))
                assert kept[0][h][i].tolist() == sorted(sinks + list(best))


def test_text_tiles_join_every_row():
    lay = orc.Layout(2, 4, 4, 1, 2, 2, n_text=6, sink=1)
    z = orc.sizes(lay)
    assert (z["nb"], z["n_text_tiles"]) == (8, 2)
    r = _rng(4)
    qbar = r.standard_normal((1, 1, 8, 4))
    kbar = r.standard_normal((1, 1, 8, 4))
    kept, _ = orc.predict_mask(qbar, kbar, lay, 50)
    rows = kept[0][0]
    assert len(rows) == 10
    for row in rows[:8]:
        assert row[-2:].tolist() == [8, 9] and len(row) == 4 + 2
        assert set([0, 1, 2, 3]) <= set(row.tolist())
    for row in rows[8:]:
        assert row.tolist() == list(range(10))


# ---------------------------------------------------------------- attention

def _dense_attention(q, k, v):
    """Textbook softmax(q k^T / sqrt(d)) v in fp64 (RainFusion page review,
    Assumptions, Eq. (1)), written independently of the oracle."""
    s = np.einsum("bhid,bhjd->bhij", q, k) / math.sqrt(q.shape[-1])
    return np.einsum("bhij,bhjd->bhid", scipy.special.softmax(s, axis=-1), v)


@pytest.mark.parametrize("dims,n_text,permute", [((3, 16, 16, 1, 8, 8), 0, 1),
                                                 ((3, 5, 7, 2, 2, 4), 0, 1),
                                                 ((2, 6, 6, 1, 4, 4), 5, 1),
                                                 ((3, 5, 7, 2, 2, 4), 3, 0)])
def test_zero_sparsity_equals_dense_attention(dims, n_text, permute):
    lay = orc.Layout(*dims, n_text=n_text, permute=permute, sink=1)
    z = orc.sizes(lay)
    r = _rng(13)
    q, k, v = (r.standard_normal((1, 2, z["L"], 8)) for _ in range(3))
    res = orc.run(q, k, v, lay, 0)
    np.testing.assert_allclose(res["o"], _dense_attention(q, k, v),
                               rtol=0, atol=1e-12)


def test_constant_values_give_constant_output():
    lay = orc.Layout(3, 5, 7, 2, 2, 4, sink=1)
    z = orc.sizes(lay)
    r = _rng(17)
    q, k = (r.standard_normal((1, 1, z["L"], 4)) for _ in range(2))
    v = np.tile(np.array([1.5, -2.0, 0.25, 3.0]), (1, 1, z["L"], 1))
    o = orc.run(q, k, v, lay, 70)["o"]
    np.testing.assert_allclose(o, v, atol=1e-13)


def _token_block(lay, z):
    """Block of each raster token from its coordinates (brute force)."""
    out = []
    for t in range(lay.T):
        for h in range(lay.H):
            for w in range(lay.W):
                if lay.permute:
                    out.append(((t // lay.wt) * z["nH"] + h // lay.wh) * z["nW"]
                               + w // lay.ww)
                else:
                    out.append(((t * lay.H + h) * lay.W + w) // z["bs"])
    out += [z["nb"] + j // z["bs"] for j in range(lay.n_text)]
    return np.array(out)


@pytest.mark.parametrize("permute,n_text", [(1, 0), (1, 5), (0, 3)])
def test_sparse_attention_equals_masked_dense_attention(permute, n_text):
    """Arbitrary kept lists: the permuted-path output, unpermuted, equals
    dense attention in raster order under the pulled-back token mask."""
    lay = orc.Layout(3, 5, 7, 2, 2, 4, n_text=n_text, permute=permute)
    z = orc.sizes(lay)
    r = _rng(19)
    q, k, v = (r.standard_normal((1, 1, z["L"], 8)) for _ in range(3))
    nt = z["n_tiles"]
    kept = [[[np.sort(r.choice(nt, size=r.integers(1, nt + 1), replace=False))
              for _ in range(nt)]]]
    op = orc.sparse_attention(orc.permute(q, lay), orc.permute(k, lay),
                              orc.permute(v, lay), kept, lay)
    o = orc.unpermute(op, lay)
    blk = _token_block(lay, z)
    allowed = np.array([[blk[j] in set(kept[0][0][blk[i]].tolist())
                         for j in range(z["L"])] for i in range(z["L"])])
    s = q[0, 0] @ k[0, 0].T / math.sqrt(8)
    s[~allowed] = -np.inf
    want = scipy.special.softmax(s, axis=-1) @ v[0, 0]
    np.testing.assert_allclose(o[0, 0], want, atol=1e-12)
    assert (op[0, 0, ~orc.slot_valid(lay)] == 0).all()


def test_single_kept_tile_restricts_attention():
    lay = orc.Layout(2, 8, 8, 1, 4, 4)
    z = orc.sizes(lay)
    r = _rng(23)
    q, k, v = (r.standard_normal((1, 1, z["L"], 4)) for _ in range(3))
    kept = [[[np.array([5]) for _ in range(z["n_tiles"])]]]
    qp, kp, vp = (orc.permute(x, lay) for x in (q, k, v))
    op = orc.sparse_attention(qp, kp, vp, kept, lay)
    members = [n for n in range(z["N"]) if _token_block(lay, z)[n] == 5]
    want = _dense_attention(q, k[:, :, members], v[:, :, members])
    np.testing.assert_allclose(orc.unpermute(op, lay), want, atol=1e-12)


def test_query_tile_subset_marks_the_rest_nan():
    lay = orc.Layout(2, 8, 8, 1, 4, 4)
    z = orc.sizes(lay)
    r = _rng(29)
    q, k, v = (orc.permute(r.standard_normal((1, 1, z["L"], 4)), lay)
               for _ in range(3))
    kept = [[[np.arange(z["n_tiles"]) for _ in range(z["n_tiles"])]]]
    part = orc.sparse_attention(q, k, v, kept, lay, query_tiles={(0, 0): [2]})
    full = orc.sparse_attention(q, k, v, kept, lay)
    bs = z["bs"]
    assert np.array_equal(part[0, 0, 2 * bs:3 * bs], full[0, 0, 2 * bs:3 * bs])
    assert np.isnan(part[0, 0, :2 * bs]).all()


# ---------------------------------------------------------------- recall R'

def _recall_in_token_order(q, k, lay, kept, b=0, h=0):
    """Independent path: dense softmax over the raster sequence, mass summed
    over the tokens whose block is in the row's kept list."""
    z = orc.sizes(lay)
    blk = _token_block(lay, z)
    s = q[b, h] @ k[b, h].T / math.sqrt(q.shape[-1])
    p = scipy.special.softmax(s, axis=-1)
    out = np.empty(z["L"])
    for i in range(z["L"]):
        mask = np.isin(blk, kept[b][h][blk[i]])
        out[i] = p[i, mask].sum()
    return out


def _slots_to_tokens(rec, lay):
    """{(b, h, tile): per-slot recall} -> per-token array for (0, 0)."""
    z = orc.sizes(lay)
    slot = orc.slot_of_token(lay)
    text_slot = np.arange(z["Np"], z["Np"] + lay.n_text)
    slots = np.concatenate([slot, text_slot])
    bs = z["bs"]
    return np.array([rec[(0, 0, s // bs)][s % bs] for s in slots])


@pytest.mark.parametrize("permute,n_text", [(1, 0), (1, 5), (0, 3)])
def test_recall_equals_dense_mass_in_token_order(permute, n_text):
    lay = orc.Layout(3, 5, 7, 2, 2, 4, n_text=n_text, permute=permute)
    z = orc.sizes(lay)
    r = _rng(31)
    q, k = (r.standard_normal((1, 1, z["L"], 8)) for _ in range(2))
    nt = z["n_tiles"]
    kept = [[[np.sort(r.choice(nt, size=r.integers(1, nt + 1), replace=False))
              for _ in range(nt)]]]
    rec = orc.attention_recall(orc.permute(q, lay), orc.permute(k, lay), kept, lay,
                               {(0, 0): range(nt)})
    np.testing.assert_allclose(_slots_to_tokens(rec, lay),
                               _recall_in_token_order(q, k, lay, kept), atol=1e-12)
    # Pad query slots are NaN, valid ones are in [0, 1].
    valid = orc.slot_valid(lay)
    bs = z["bs"]
    for (b, h, i), v in rec.items():
        vm = valid[i * bs:(i + 1) * bs]
        vm = np.pad(vm, (0, bs - len(vm)))
        assert np.isnan(v[~vm]).all() and ((v[vm] >= 0) & (v[vm] <= 1 + 1e-12)).all()


def test_recall_zero_sparsity_is_one():
    lay = orc.Layout(3, 16, 16, 1, 8, 8, sink=1)
    z = orc.sizes(lay)
    r = _rng(37)
    q, k, v = (r.standard_normal((1, 1, z["L"], 8)) for _ in range(3))
    res = orc.run(q, k, v, lay, 0)
    rec = orc.attention_recall(res["qp"], res["kp"], res["kept"], lay,
                               {(0, 0): range(z["n_tiles"])})
    vals = np.concatenate(list(rec.values()))
    np.testing.assert_allclose(vals[~np.isnan(vals)], 1.0, atol=1e-15)


def test_recall_with_uniform_logits_is_the_kept_key_share():
    """k = 0 makes every logit 0: the recall is the number of valid kept
    keys over the number of valid keys (closed form)."""
    lay = orc.Layout(2, 6, 6, 1, 4, 4, n_text=3)
    z = orc.sizes(lay)
    r = _rng(41)
    q = orc.permute(r.standard_normal((1, 1, z["L"], 4)), lay)
    kz = np.zeros_like(q)
    nt = z["n_tiles"]
    kept = [[[np.sort(r.choice(nt, size=r.integers(1, nt + 1), replace=False))
              for _ in range(nt)]]]
    rec = orc.attention_recall(q, kz, kept, lay, {(0, 0): range(nt)})
    counts = np.concatenate([orc.block_counts(lay),
                             [min(z["bs"], lay.n_text - j * z["bs"])
                              for j in range(z["n_text_tiles"])]])
    for i in range(nt):
        want = counts[kept[0][0][i]].sum() / z["L"]
        v = rec[(0, 0, i)]
        np.testing.assert_allclose(v[~np.isnan(v)], want, atol=1e-15)


def test_recall_of_complementary_masks_sums_to_one():
    lay = orc.Layout(2, 8, 8, 1, 4, 4)
    z = orc.sizes(lay)
    r = _rng(43)
    q, k = (orc.permute(r.standard_normal((1, 1, z["L"], 4)), lay) for _ in range(2))
    nt = z["n_tiles"]
    a = [np.sort(r.choice(nt, size=3, replace=False)) for _ in range(nt)]
    c = [np.setdiff1d(np.arange(nt), x) for x in a]
    ra = orc.attention_recall(q, k, [[a]], lay, {(0, 0): range(nt)})
    rc = orc.attention_recall(q, k, [[c]], lay, {(0, 0): range(nt)})
    for key in ra:
        np.testing.assert_allclose(ra[key] + rc[key], 1.0, atol=1e-13)


def test_recall_follows_a_planted_dominant_key():
    """One key equal to a large multiple of query 0 holds almost all of that
    query's mass: recall is ~1 when its tile is kept and ~0 when not."""
    lay = orc.Layout(2, 8, 8, 1, 4, 4)
    z = orc.sizes(lay)
    r = _rng(47)
    qp = orc.permute(0.1 * r.standard_normal((1, 1, z["L"], 4)), lay)
    kp = orc.permute(0.1 * r.standard_normal((1, 1, z["L"], 4)), lay)
    qp[0, 0, 0] = [1.0, 0.0, 0.0, 0.0]
    kp[0, 0, 3 * z["bs"] + 1] = [200.0, 0.0, 0.0, 0.0]   # slot in tile 3
    nt = z["n_tiles"]
    with_t3 = [[[np.array([0, 3])] + [np.arange(nt)] * (nt - 1)]]
    without = [[[np.array([0, 1])] + [np.arange(nt)] * (nt - 1)]]
    assert orc.attention_recall(qp, kp, with_t3, lay, {(0, 0): [0]})[(0, 0, 0)][0] > 1 - 1e-12
    assert orc.attention_recall(qp, kp, without, lay, {(0, 0): [0]})[(0, 0, 0)][0] < 1e-12


# ------------------------------------------------------- v1 head patterns

def _first_token_coords(lay, z):
    """(t, h, w) of the first valid token of each video tile, by walking the
    grid token by token (brute force, no slot arithmetic)."""
    first = {}
    for t in range(lay.T):
        for h in range(lay.H):
            for w in range(lay.W):
                n = (t * lay.H + h) * lay.W + w
                if lay.permute:
                    blk = (((t // lay.wt) * z["nH"] + h // lay.wh) * z["nW"]
                           + w // lay.ww)
                    inner = ((t % lay.wt) * lay.wh + h % lay.wh) * lay.ww + w % lay.ww
                else:
                    blk, inner = divmod(n, z["bs"])
                if blk not in first or inner < first[blk][0]:
                    first[blk] = (inner, (t, h, w))
    return [first[i][1] for i in range(z["nb"])]


def test_tile_rank_in_window_order_is_bh_bw_bt():
    """With the window order, sorting tiles by (h, w, t) of their first token
    is sorting by block coordinates (bh, bw, bt): r = (bh nW + bw) nT + bt."""
    lay = orc.Layout(5, 7, 9, 2, 2, 4)
    z = orc.sizes(lay)
    r = orc.tile_rank(lay)
    for i in range(z["nb"]):
        bt, rem = divmod(i, z["nH"] * z["nW"])
        bh, bw = divmod(rem, z["nW"])
        assert r[i] == (bh * z["nW"] + bw) * z["nT"] + bt


@pytest.mark.parametrize("dims,permute", [((3, 5, 7, 2, 2, 4), 0),
                                          ((4, 6, 10, 1, 2, 8), 0),
                                          ((3, 5, 7, 2, 2, 4), 1)])
def test_tile_rank_sorts_first_tokens_spatial_major(dims, permute):
    lay = orc.Layout(*dims, permute=permute)
    z = orc.sizes(lay)
    coords = _first_token_coords(lay, z)
    r = orc.tile_rank(lay)
    assert sorted(r.tolist()) == list(range(z["nb"]))
    for i, j in itertools.combinations(range(z["nb"]), 2):
        (ti, hi, wi), (tj, hj, wj) = coords[i], coords[j]
        assert (r[i] < r[j]) == ((hi, wi, ti) < (hj, wj, tj))


def test_band_kept_count_closed_form():
    """A band |i - j| <= w on n x n keeps n (2w + 1) - w (w + 1) entries;
    the temporal band is the same band in another order, so it keeps as
    many."""
    lay = orc.Layout(5, 7, 9, 2, 2, 4)
    n = orc.sizes(lay)["nb"]
    for w in (0, 1, 5, n // 4, n - 2):
        want = n * (2 * w + 1) - w * (w + 1)
        for p in (orc.SPATIAL, orc.TEMPORAL):
            assert orc.pattern_keeps(lay, p, w, 2).sum() == want


def test_bandwidth_quarter_cuts_nine_sixteenths():
    """Bandwidth 1/4 keeps 1 - (3/4)^2 = 7/16 of the tile pairs, the 9/16
    reduction the v1 page states, up to O(1/nb)."""
    lay = orc.Layout(21, 45, 80, 2, 8, 8)
    n = orc.sizes(lay)["nb"]
    assert n == 660
    w = orc.band_halfwidth(lay, 0.25)
    assert w == 165
    for p in (orc.SPATIAL, orc.TEMPORAL):
        frac = orc.pattern_keeps(lay, p, w, 2).mean()
        assert abs(frac - 7 / 16) < 1.0 / n


def test_temporal_equals_spatial_with_one_frame_window():
    """With a single window along time the spatial-major order of the tiles
    is the block order itself, so the two bands coincide."""
    lay = orc.Layout(1, 16, 24, 1, 4, 8)
    for w in (0, 3, 7):
        np.testing.assert_array_equal(orc.pattern_keeps(lay, orc.TEMPORAL, w, 2),
                                      orc.pattern_keeps(lay, orc.SPATIAL, w, 2))


@pytest.mark.parametrize("tau", [1, 2, 3, 4])
def test_textural_checkerboard_keeps_one_residue_class(tau):
    """The union over k of {i = k and j = k (mod tau)} is j = i (mod tau):
    row i keeps ceil((nb - i mod tau) / tau) tiles."""
    lay = orc.Layout(5, 7, 9, 2, 2, 4)
    n = orc.sizes(lay)["nb"]
    m = orc.pattern_keeps(lay, orc.TEXTURAL, 0, tau)
    for i in range(n):
        assert np.flatnonzero(m[i]).tolist() == list(range(i % tau, n, tau))
    assert m.sum(axis=1).tolist() == [-(-(n - i % tau) // tau) for i in range(n)]


def test_pattern_masks_are_symmetric_and_keep_the_diagonal():
    lay = orc.Layout(3, 5, 7, 2, 2, 4, permute=0)
    for p, w, tau in [(orc.SPATIAL, 2, 2), (orc.TEMPORAL, 2, 2), (orc.TEXTURAL, 0, 3)]:
        m = orc.pattern_keeps(lay, p, w, tau)
        np.testing.assert_array_equal(m, m.T)
        assert m.diagonal().all()


def test_pattern_rows_with_text_and_full_band_is_dense_attention():
    """A band wider than the grid keeps every tile, so the attention equals
    textbook dense attention."""
    lay = orc.Layout(2, 6, 6, 1, 4, 4, n_text=5)
    z = orc.sizes(lay)
    hp = np.array([[orc.SPATIAL, orc.TEMPORAL]])
    kept = orc.pattern_mask(lay, hp, z["nb"], 2)
    for rows in kept[0]:
        assert len(rows) == z["n_tiles"]
        for row in rows:
            assert row.tolist() == list(range(z["n_tiles"]))
    r = _rng(53)
    q, k, v = (r.standard_normal((1, 2, z["L"], 8)) for _ in range(3))
    qp, kp, vp = (orc.permute(x, lay) for x in (q, k, v))
    o = orc.unpermute(orc.sparse_attention(qp, kp, vp, kept, lay), lay)
    np.testing.assert_allclose(o, _dense_attention(q, k, v), atol=1e-12)


def test_pattern_rows_append_text_tiles():
    lay = orc.Layout(3, 5, 7, 2, 2, 4, n_text=9)
    z = orc.sizes(lay)
    nb, nt = z["nb"], z["n_tiles"]
    kept = orc.pattern_mask(lay, np.array([[orc.TEXTURAL]]), 0, 2)[0][0]
    assert len(kept) == nt
    for i in range(nb):
        assert kept[i].tolist() == list(range(i % 2, nb, 2)) + list(range(nb, nt))
    for i in range(nb, nt):
        assert kept[i].tolist() == list(range(nt))


# ------------------------------------------------------------------ ARM

def test_arm_samples():
    lay = orc.Layout(3, 5, 7, 2, 2, 4)
    assert orc.arm_samples(lay, True, 4).tolist() == [0, 4, 8, 12, 16, 20, 24, 28, 32]
    g = orc.arm_samples(lay, False, 8)
    assert len(g) == -(-105 // 8) and g[-1] == 104


def test_arm_recall_two_tokens_is_a_sigmoid():
    """Two sampled tokens in different tiles, a mask that keeps only the
    query's own tile: R' = e^{s_aa} / (e^{s_aa} + e^{s_ab})."""
    lay = orc.Layout(1, 8, 8, 1, 4, 4)
    r = _rng(59)
    q, k = (r.standard_normal((1, 1, 64, 4)) for _ in range(2))
    toks = np.array([0, 63])                     # tiles 0 and 3
    rec = orc.arm_recall(q, k, lay, orc.SPATIAL, 0, 2, toks)
    s = q[0, 0, toks] @ k[0, 0, toks].T / 2.0
    np.testing.assert_allclose(rec[0, 0], scipy.special.expit(
        [s[0, 0] - s[0, 1], s[1, 1] - s[1, 0]]), atol=1e-15)


def test_arm_recall_uniform_logits_and_full_band():
    lay = orc.Layout(4, 8, 8, 2, 4, 4)
    z = orc.sizes(lay)
    r = _rng(61)
    q, k = (r.standard_normal((1, 2, z["L"], 4)) for _ in range(2))
    toks = orc.arm_samples(lay, False, 3)
    full = orc.arm_recall(q, k, lay, orc.TEMPORAL, z["nb"], 2, toks)
    np.testing.assert_allclose(full, 1.0, atol=1e-14)
    # zero keys: the recall is the share of sampled keys in kept tiles
    uni = orc.arm_recall(q, np.zeros_like(k), lay, orc.SPATIAL, 1, 2, toks)
    tile = [_token_block(lay, z)[t] for t in toks]
    for a in range(len(toks)):
        want = sum(abs(tile[a] - tb) <= 1 for tb in tile) / len(toks)
        np.testing.assert_allclose(uni[0, :, a], want, atol=1e-15)


def test_arm_recall_planted_key():
    lay = orc.Layout(4, 8, 8, 2, 4, 4)
    z = orc.sizes(lay)
    r = _rng(67)
    q, k = (0.1 * r.standard_normal((1, 1, z["L"], 4)) for _ in range(2))
    toks = orc.arm_samples(lay, False, 2)
    q[0, 0, 0] = [1.0, 0, 0, 0]
    far = toks[-1]                                # last frame, far band
    k[0, 0, far] = [300.0, 0, 0, 0]
    rec = orc.arm_recall(q, k, lay, orc.SPATIAL, 1, 2, toks)
    assert rec[0, 0, 0] < 1e-12
    rec = orc.arm_recall(q, k, lay, orc.SPATIAL, z["nb"], 2, toks)
    assert rec[0, 0, 0] > 1 - 1e-12


def test_arm_classification_order():
    """Temporal is tested first, then spatial; a mean equal to alpha reaches
    it (values chosen exact in binary)."""
    a = 0.75
    loc = np.array([[[1.0, 0.25], [0.5, 0.5], [0.5, 1.0], [0.25, 0.25]]])
    glo = np.array([[[0.25, 0.25], [1.0, 0.5], [1.0, 1.0], [0.5, 0.75]]])
    got = orc.arm_classify(loc, glo, a)
    assert got.tolist() == [[orc.TEXTURAL, orc.SPATIAL, orc.TEMPORAL, orc.TEXTURAL]]


# ------------------------------------------------------------------ FP8

def _e4m3_decode(c):
    """Value of an e4m3 bit pattern from the format's fields."""
    s = -1.0 if c & 0x80 else 1.0
    e, m = (c >> 3) & 15, c & 7
    if e == 15 and m == 7:
        return math.nan
    return s * (m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))


def test_e4m3_grid_from_the_format_fields():
    """Every finite code is a fixed point; 448 is the largest; the subnormal
    step is 2^-9; 254 finite codes give 253 distinct values (+-0 equal)."""
    vals = [_e4m3_decode(c) for c in range(256)]
    finite = np.array([v for v in vals if not math.isnan(v)])
    assert len(finite) == 254 and len(set(finite.tolist())) == 253
    np.testing.assert_array_equal(orc.e4m3(finite), finite)
    assert finite.max() == 448.0 and sorted(set(np.abs(finite)))[1] == 2.0 ** -9


def test_e4m3_rounds_to_nearest_even_like_torch():
    """Midpoints go to the even code, neighbours of a midpoint to the
    nearer value; the same as torch's CPU float8_e4m3fn conversion (a
    library routine) on the midpoints, their float32 neighbours and random
    values."""
    import torch
    pos = sorted(set(abs(v) for v in (_e4m3_decode(c) for c in range(128))
                     if not math.isnan(v)))
    x = []
    for lo, hi in zip(pos[:-1], pos[1:]):
        mid = np.float32((lo + hi) / 2)
        x += [lo, mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))]
    x = np.array(x + list(_rng(71).standard_normal(5000) * 40), np.float32)
    x = np.concatenate([x, -x])
    x = x[np.abs(x) <= 464]
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(orc.e4m3(x), want)
    # ties by hand: 1 + 1/16 lies between 1 and 1.125 -> 1 (even mantissa 0);
    # 1 + 3/16 between 1.125 and 1.25 -> 1.25 (mantissa 2)
    assert orc.e4m3(1 + 1 / 16) == 1.0 and orc.e4m3(1 + 3 / 16) == 1.25
    with pytest.raises(ValueError):
        orc.e4m3(465.0)


def test_pow2_exponent_closed_forms():
    assert orc.pow2_exponent(0.0) == 0
    assert orc.pow2_exponent(448.0) == 0 and orc.pow2_exponent(448.5) == 1
    assert orc.pow2_exponent(224.0) == -1 and orc.pow2_exponent(224.5) == 0
    assert orc.pow2_exponent(3.5) == -7 and orc.pow2_exponent(3.75) == -6
    for a in _rng(73).uniform(1e-6, 1e6, 200):
        e = orc.pow2_exponent(a)
        assert 224.0 < a / 2.0 ** e <= 448.0


def test_quantize_tiles_and_channels():
    """Scaled codes reach into (224, 448] in every nonzero tile; the
    dequantized error is within half a step (2^-4 relative above the
    subnormal range); pad slots stay 0."""
    lay = orc.Layout(3, 5, 7, 2, 2, 4, n_text=9)
    z = orc.sizes(lay)
    r = _rng(79)
    xp = orc.permute(r.standard_normal((1, 2, z["L"], 8)) * 3, lay)
    q, ex = orc.quantize_tiles(xp, lay)
    bs = z["bs"]
    for t in range(z["n_tiles"]):
        rows = slice(t * bs, min((t + 1) * bs, z["Lp"]))
        for h in range(2):
            x = xp[0, h, rows]
            amax = np.abs(x).max()
            assert 224 < amax / 2.0 ** ex[0, h, t] <= 448
            err = np.abs(q[0, h, rows] - x)
            tol = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** (ex[0, h, t] - 10))
            assert np.all(err <= tol + 1e-300)
    assert np.all(q[:, :, ~orc.slot_valid(lay)] == 0)
    v, evx = orc.quantize_channels(xp)
    amax = np.abs(xp).max(axis=2)
    assert np.all((amax / 2.0 ** evx > 224) & (amax / 2.0 ** evx <= 448))


def test_fp8_attention_is_exact_on_representable_inputs():
    """Inputs in {-2, ..., 2}: every tile and feature max is 2, the scale is
    2^-7 and 2 * 2^7 = 256 is a code, so quantization is the identity and
    the fp8 attention equals the plain one."""
    lay = orc.Layout(2, 6, 6, 1, 4, 4, n_text=5)
    z = orc.sizes(lay)
    r = _rng(83)
    x = [r.integers(-2, 3, size=(1, 1, z["L"], 8)).astype(np.float64) for _ in range(3)]
    for t in x:
        t[..., 0, :] = 2.0              # make sure every feature reaches 2
    qp, kp, vp = (orc.permute(t, lay) for t in x)
    # every query/key tile must reach 2 too
    for t in range(z["n_tiles"]):
        qp[0, 0, t * z["bs"], 0] = 2.0
        kp[0, 0, t * z["bs"], 0] = 2.0
    kept, _ = orc.predict_mask(orc.block_means(qp, lay), orc.block_means(kp, lay), lay, 50)
    a = orc.sparse_attention(qp, kp, vp, kept, lay)
    b = orc.sparse_attention_fp8(qp, kp, vp, kept, lay)
    np.testing.assert_array_equal(a, b)


def _closed_form_exponent(amax):
    """e = ceil(log2(amax / 448)) for amax > 0, checked against the defining
    inequality 224 < amax / 2^e <= 448; 0 for amax = 0."""
    if amax == 0:
        return 0
    m, ex = math.frexp(amax / 448.0)       # amax / 448 = m 2^ex, m in [1/2, 1)
    e = ex if m > 0.5 else ex - 1          # exact powers of two need no round-up
    assert 224.0 < amax / 2.0 ** e <= 448.0
    return e


def _torch_e4m3(x):
    """Round to e4m3 with torch's CPU float8_e4m3fn conversion (a library
    routine), back to fp64."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float64)).to(
        torch.float8_e4m3fn).to(torch.float64).numpy()


def _features_of_mixed_range(seed, lay, d=8):
    """A permuted tensor whose features span very different ranges (feature f
    scaled by 4^(f - 3), so its maximum ranges over some 2^12), sigma ~ 3,
    with a few values in the subnormal range of their feature's scale."""
    z = orc.sizes(lay)
    r = _rng(seed)
    x = r.standard_normal((1, 2, z["L"], d)) * 3.0 * 4.0 ** (np.arange(d) - 3)
    x[0, 0, :5, 2] *= 2.0 ** -14                       # deep in the subnormal steps
    return orc.permute(x, lay)


def test_quantize_channels_values_equal_library_e4m3_per_feature():
    """RF2 TL;DR (quantization as future work), reading R12, V operand: one
    power-of-two scale per (b, h, feature) over all slots.  Independent
    construction: the scale from the closed form of the exponent, torch's
    float8_e4m3fn conversion of x 2^-e, times 2^e.  Every dequantized value
    and exponent must match, and the error must stay within half an e4m3 step
    (2^-4 relative for normal codes, 2^(e-10) in the subnormal range)."""
    lay = orc.Layout(3, 5, 7, 2, 2, 4, n_text=9)
    xp = _features_of_mixed_range(103, lay)
    got, ex = orc.quantize_channels(xp)
    B, H, Lp, d = xp.shape
    want = np.empty_like(xp)
    for b in range(B):
        for h in range(H):
            for f in range(d):
                e = _closed_form_exponent(np.abs(xp[b, h, :, f]).max())
                assert ex[b, h, f] == e, (b, h, f)
                want[b, h, :, f] = _torch_e4m3(xp[b, h, :, f] * 2.0 ** -e) * 2.0 ** e
                err = np.abs(got[b, h, :, f] - xp[b, h, :, f])
                tol = np.maximum(np.abs(xp[b, h, :, f]) * 2.0 ** -4, 2.0 ** (e - 10))
                assert np.all(err <= tol), (b, h, f, err.max())
    np.testing.assert_array_equal(got, want)
    # pad slots (zero) stay zero
    assert np.all(got[:, :, ~orc.slot_valid(lay)] == 0)


def test_quantize_channels_pin_rejects_wrong_direction_and_grouping():
    """The data of the per-feature pin separates the two plausible mistakes:
    scaling the wrong way (e4m3(x 2^e) 2^-e) and one scale per tile (as for
    Q and K) instead of per feature both give values that differ from the
    per-feature construction, so either mistake fails the pin above."""
    lay = orc.Layout(3, 5, 7, 2, 2, 4, n_text=9)
    z = orc.sizes(lay)
    xp = _features_of_mixed_range(103, lay)
    good, ex = orc.quantize_channels(xp)
    # wrong direction; values beyond the e4m3 range saturate to keep it finite
    flipped = np.empty_like(xp)
    for f in range(xp.shape[-1]):
        s = 2.0 ** ex[:, :, None, f]
        flipped[..., f] = np.clip(_torch_e4m3(np.clip(xp[..., f] * s, -448, 448)), -448, 448) / s
    assert not np.array_equal(flipped, good)
    # per-tile grouping
    tiled = np.empty_like(xp)
    bs = z["bs"]
    for t in range(z["n_tiles"]):
        rows = slice(t * bs, min((t + 1) * bs, z["Lp"]))
        for b in range(xp.shape[0]):
            for h in range(xp.shape[1]):
                e = _closed_form_exponent(np.abs(xp[b, h, rows]).max())
                tiled[b, h, rows] = _torch_e4m3(xp[b, h, rows] * 2.0 ** -e) * 2.0 ** e
    assert not np.array_equal(tiled, good)
    # and per-tile scales break the per-feature half-step bound on the
    # features of small range, whose values fall into coarse subnormal steps
    bound = np.maximum(np.abs(xp) * 2.0 ** -4, 2.0 ** (ex[:, :, None, :] - 10))
    assert np.any(np.abs(tiled - xp) > bound)
    assert np.all(np.abs(good - xp) <= bound)


def test_fp8_attention_uses_per_tile_qk_and_per_feature_v():
    """sparse_attention_fp8 equals the plain attention on operands built
    independently: Q and K with one closed-form scale per (b, h, tile) and V
    with one per (b, h, feature), each rounded by torch's e4m3 conversion."""
    lay = orc.Layout(3, 5, 7, 2, 2, 4, n_text=9, sink=1)
    z = orc.sizes(lay)
    r = _rng(107)
    qp, kp = (orc.permute(r.standard_normal((1, 1, z["L"], 8)) * 3, lay) for _ in range(2))
    vp = _features_of_mixed_range(109, lay)[:, :1]
    kept, _ = orc.predict_mask(orc.block_means(qp, lay), orc.block_means(kp, lay), lay, 40)

    def per_tile(x):
        out = np.empty_like(x)
        bs = z["bs"]
        for t in range(z["n_tiles"]):
            rows = slice(t * bs, min((t + 1) * bs, z["Lp"]))
            e = _closed_form_exponent(np.abs(x[0, 0, rows]).max())
            out[0, 0, rows] = _torch_e4m3(x[0, 0, rows] * 2.0 ** -e) * 2.0 ** e
        return out

    def per_feature(x):
        out = np.empty_like(x)
        for f in range(x.shape[-1]):
            e = _closed_form_exponent(np.abs(x[0, 0, :, f]).max())
            out[0, 0, :, f] = _torch_e4m3(x[0, 0, :, f] * 2.0 ** -e) * 2.0 ** e
        return out

    want = orc.sparse_attention(per_tile(qp), per_tile(kp), per_feature(vp), kept, lay)
    got = orc.sparse_attention_fp8(qp, kp, vp, kept, lay)
    np.testing.assert_array_equal(got, want)
    # per-tile V would change the result on these features
    alt = orc.sparse_attention(per_tile(qp), per_tile(kp), per_tile(vp), kept, lay)
    assert not np.allclose(alt, want, atol=1e-6, equal_nan=True)


# ---------------------------------------------------------- LSE and dense mask

@pytest.mark.parametrize("n_text,permute", [(0, 1), (5, 1), (3, 0)])
def test_lse_zero_sparsity_is_dense_logsumexp(n_text, permute):
    """With every tile kept the log-sum-exp is scipy's over the dense logits
    of the raster sequence (library routine), slot by slot."""
    lay = orc.Layout(3, 5, 7, 2, 2, 4, n_text=n_text, permute=permute, sink=1)
    z = orc.sizes(lay)
    r = _rng(89)
    q, k = (r.standard_normal((1, 1, z["L"], 8)) for _ in range(2))
    qp, kp = orc.permute(q, lay), orc.permute(k, lay)
    nt = z["n_tiles"]
    kept = [[[np.arange(nt)] * nt]]
    lse = orc.attention_lse(qp, kp, kept, lay)
    want = scipy.special.logsumexp(q[0, 0] @ k[0, 0].T / math.sqrt(8), axis=1)
    got = lse[0, 0, orc.slot_of_token(lay).tolist() + list(range(z["Np"], z["Lp"]))]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    assert np.all(np.isneginf(lse[0, 0, ~orc.slot_valid(lay)]))


def test_lse_of_zero_keys_is_log_count():
    """k = 0 gives logits 0: lse = log(number of valid kept keys)."""
    lay = orc.Layout(2, 6, 6, 1, 4, 4, n_text=3)
    z = orc.sizes(lay)
    r = _rng(97)
    q = orc.permute(r.standard_normal((1, 1, z["L"], 4)), lay)
    nt = z["n_tiles"]
    kept = [[[np.sort(r.choice(nt, size=r.integers(1, nt + 1), replace=False))
              for _ in range(nt)]]]
    lse = orc.attention_lse(q, np.zeros_like(q), kept, lay)
    counts = np.concatenate([orc.block_counts(lay),
                             [min(z["bs"], lay.n_text - j * z["bs"])
                              for j in range(z["n_text_tiles"])]])
    valid = orc.slot_valid(lay)
    for i in range(nt):
        sl = slice(i * z["bs"], min((i + 1) * z["bs"], z["Lp"]))
        np.testing.assert_allclose(lse[0, 0, sl][valid[sl]],
                                   math.log(counts[kept[0][0][i]].sum()), atol=1e-14)


def test_kept_dense_matches_rows():
    lay = orc.Layout(2, 4, 4, 1, 2, 2, n_text=6, sink=1)
    r = _rng(101)
    qbar = r.standard_normal((1, 1, 8, 4))
    kbar = r.standard_normal((1, 1, 8, 4))
    kept, _ = orc.predict_mask(qbar, kbar, lay, 50)
    m = orc.kept_dense(kept, lay)
    for i, row in enumerate(kept[0][0]):
        assert np.flatnonzero(m[0, 0, i]).tolist() == row.tolist()
