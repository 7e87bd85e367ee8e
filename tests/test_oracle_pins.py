"""Pins of the CPU oracle to things other than itself.

Each test checks the oracle against a hand computation, a closed form, a
brute-force enumeration over tiny inputs or an invariant that the definitions
fix ("MISA: Mixture of Indexer Sparse Attention for Long-Context LLM
Inference", Technical Summary: Problem Statement, Methodology: MISA,
Hierarchical Variant).  Inputs are chosen so that a plausible slip (a dropped
ReLU, a wrong sign, a transposed operand, an off-by-one prefix, a partial
block averaged over B, a reversed tie rule) fails at least one of them.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import oracle as orc
from long_context_sparse_05_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_example.json")


def _bf(x):
    return synth.to_bf16_bits(np.asarray(x, np.float32))


def _one_seq_batch(keys, qs, ws, ps, Lmax=None):
    keys = np.asarray(keys, np.float32)
    L, d = keys.shape
    Lmax = Lmax or L
    kk = np.zeros((1, Lmax, d), np.float32)
    kk[0, :L] = keys
    return orc.Batch(_bf(kk), _bf(np.asarray(qs, np.float32)), np.asarray(ws, np.float32),
                     np.zeros(len(ps), np.int32), np.asarray(ps, np.int32))


# ---------------------------------------------------------------- hand example
def test_hand_worked_example():
    g = json.load(open(GOLDEN))
    qs = [e["q"] for e in g["queries"]]
    ws = [e["w"] for e in g["queries"]]
    ps = [e["p"] for e in g["queries"]]
    b = _one_seq_batch(g["keys"], qs, ws, ps)
    B = g["B"]
    sc = orc.scores(b)
    for t, e in enumerate(g["queries"]):
        n = e["p"] + 1
        np.testing.assert_array_equal(sc[t, :n], e["dsa_scores"])
        assert np.all(np.isneginf(sc[t, n:]))
    idx, _ = orc.dsa(b, 2)
    assert [list(r) for r in idx] == [e["dsa_top2"] for e in g["queries"]]
    idx3, _ = orc.dsa(b, 3)
    assert list(idx3[1]) == g["queries"][1]["dsa_top3"]
    for mode in (0, 1):
        heads, gg = orc.route(b, B, 1, mode)
        for t, e in enumerate(g["queries"]):
            np.testing.assert_array_equal(gg[t], e["g_mode%d" % mode])
            assert list(heads[t]) == e["heads_h1_mode%d" % mode]
    m = orc.misa(b, B, 1, 2, mode=0, want_scores=True)
    for t, e in enumerate(g["queries"]):
        assert list(m["idx"][t]) == e["misa_h1_mode0_top2"]
        np.testing.assert_array_equal(m["scores"][t, :e["p"] + 1], e["misa_h1_mode0_scores"])
    m1 = orc.misa(b, B, 1, 2, mode=1)
    assert list(m1["idx"][1]) == g["queries"][1]["misa_h1_mode1_top2"]
    dg = orc.misa_dagger(b, B, 1, 3, 2, mode=0)
    for t, e in enumerate(g["queries"]):
        assert list(dg["cand"][t]) == e["dagger_h1_kc3_cand"]
        assert list(dg["idx"][t]) == e["dagger_h1_kc3_top2"]


# ----------------------------------------------------------- top-k brute force
def _valid_topk_set(v, S):
    """S is the top set iff every member beats every non-member under
    (value desc, index asc), comparing -0.0 == +0.0."""
    out = [i for i in range(len(v)) if i not in S]
    for i in S:
        for j in out:
            if not (v[i] > v[j] or (v[i] == v[j] and i < j)):
                return False
    return True


@pytest.mark.parametrize("seed", range(40))
def test_topk_against_subset_enumeration(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 9))
    pool = np.array([-1.5, -0.0, 0.0, 0.25, 0.25, 1.0, 3.0, -np.inf])
    v = rng.choice(pool, size=n) if n else np.zeros(0)
    for k in range(1, n + 3):
        idx, val = orc.topk(v, k)
        m = min(k, n)
        sets = [set(c) for c in itertools.combinations(range(n), m) if _valid_topk_set(v, set(c))]
        assert len(sets) == 1, "the tie rule makes the top set unique"
        assert set(idx[:m].tolist()) == sets[0]
        assert np.all(idx[m:] == -1) and np.all(np.isneginf(val[m:]))
        # the listed order is the ranking itself
        for a, c in zip(idx[:m - 1], idx[1:m]):
            assert v[a] > v[c] or (v[a] == v[c] and a < c)
        assert np.array_equal(orc.topk_f32(v.astype(np.float32), k), idx)


# ---------------------------------------------------------- scoring closed form
def test_scores_one_hot_queries_closed_form():
    """With q_j = a_j e_{c_j}, x_j(i) = a_j K_i[c_j]; the score is read off the
    key entries with no dot product.  Distinct c_j and signs catch a
    transposed q/k operand, a dropped ReLU and a head/weight mix-up."""
    rng = np.random.default_rng(7)
    d, H, L = 16, 5, 40
    K = rng.integers(-3, 4, size=(L, d)).astype(np.float32)
    cs = [3, 0, 11, 7, 15]
    a = [1.0, -2.0, 0.5, 3.0, -1.0]
    w = [0.5, -1.0, 2.0, 0.25, 1.5]
    qs = np.zeros((1, H, d), np.float32)
    for j in range(H):
        qs[0, j, cs[j]] = a[j]
    p = 33
    b = _one_seq_batch(K, qs, [w], [p])
    sc = orc.scores(b)[0]
    for i in range(L):
        if i > p:
            assert np.isneginf(sc[i])
            continue
        expect = sum(w[j] * max(0.0, a[j] * K[i, cs[j]]) for j in range(H))
        assert sc[i] == expect
    # routed scoring over a subset of heads is the same sum over that subset
    heads = np.array([[4, 1]], np.int32)
    scr = orc.scores(b, heads)[0]
    for i in range(p + 1):
        assert scr[i] == sum(w[j] * max(0.0, a[j] * K[i, cs[j]]) for j in (1, 4))


# ------------------------------------------------------------- pooling closed form
def test_pool_closed_forms():
    """Keys K_i = i along dim 0 and -2 along dim 1: the mean of block
    [lo, hi) is (lo+hi-1)/2 and -2, for partial blocks too (count = hi-lo)."""
    S, Lmax, d, B = 2, 23, 4, 5
    K = np.zeros((S, Lmax, d), np.float32)
    K[:, :, 0] = np.arange(Lmax)
    K[:, :, 1] = -2.0
    K[1, :, 2] = 8.0
    seq_lens = np.array([23, 12], np.int32)
    b = orc.Batch(_bf(K), _bf(np.zeros((1, 1, d))), np.zeros((1, 1), np.float32),
                  np.zeros(1, np.int32), np.zeros(1, np.int32), seq_lens)
    P = orc.pool(b, B)
    assert P.shape == (S, 5, d)
    for s in range(S):
        for blk in range(5):
            lo, hi = blk * B, min(blk * B + B, seq_lens[s])
            if hi <= lo:
                assert np.all(P[s, blk] == 0)
                continue
            assert P[s, blk, 0] == (lo + hi - 1) / 2
            assert P[s, blk, 1] == -2.0
            assert P[s, blk, 2] == (8.0 if s == 1 else 0.0)


# ------------------------------------------------------------- router closed forms
def test_router_constant_keys_closed_form():
    """All prefix keys equal k0 = e_c: every block mean is k0 whatever its
    count, so g_j = w'_j * M_t * ReLU(q_j[c]) with M_t = ceil((p+1)/B).
    Lmax > n and n not a multiple of B catch a block count taken from Lmax
    and a partial block averaged over B."""
    d, H, B, Lmax, c = 8, 6, 4, 64, 5
    K = np.zeros((Lmax, d), np.float32)
    K[:, c] = 1.0
    rng = np.random.default_rng(3)
    qs = rng.integers(-3, 4, size=(3, H, d)).astype(np.float32)
    ws = np.array([[1, -2, 0.5, 3, -0.25, 2]] * 3, np.float32)
    ps = [0, 13, 30]
    b = _one_seq_batch(K, qs, ws, ps, Lmax=Lmax)
    for mode in (0, 1):
        heads, g = orc.route(b, B, 3, mode)
        for t, p in enumerate(ps):
            M = -(-(p + 1) // B)
            for j in range(H):
                wj = abs(ws[t, j]) if mode else ws[t, j]
                assert g[t, j] == wj * M * max(0.0, qs[t, j, c])
            # top-3 by (g desc, j asc) written out by hand from the closed form
            order = sorted(range(H), key=lambda j: (-g[t, j], j))
            assert list(heads[t]) == order[:3]


def test_router_single_block_and_unit_blocks():
    """B >= n: one block, g_j = w_j ReLU(q_j . mean(K[0..p])).
    B = 1: g_j = w_j * sum_i ReLU(q_j . K_i) -- the head's own token terms."""
    d, H, L = 4, 3, 9
    K = np.array([[1, 0, 2, 0], [3, 1, 0, -1], [0, 0, 1, 1], [2, -2, 0, 0],
                  [1, 1, 1, 1], [0, 4, 0, 0], [-1, 0, 0, 2], [0, 0, -3, 0],
                  [5, 5, 5, 5]], np.float32)
    qs = np.array([[[1, 0, 0, 0], [0, 1, -1, 0], [0.5, 0, 0, 2]]], np.float32)
    ws = np.array([[2.0, -1.0, 0.5]], np.float32)
    p = 7
    b = _one_seq_batch(K, qs, ws, [p])
    _, g = orc.route(b, 64, 1, 0)
    mean = K[:p + 1].astype(np.float64).mean(0)
    for j in range(H):
        assert g[0, j] == pytest.approx(ws[0, j] * max(0.0, float(qs[0, j] @ mean)), rel=1e-15)
    _, g1 = orc.route(b, 1, 1, 0)
    for j in range(H):
        dots = [float(qs[0, j] @ K[i]) for i in range(p + 1)]
        assert g1[0, j] == ws[0, j] * sum(max(0.0, x) for x in dots)


# ------------------------------------------------------------------ invariants
def _rand(seed, S=2, Lmax=300, T=6, H=8, d=32, dist="normal"):
    c = synth.random_case(S, Lmax, T, H, seed=seed, d=d, dist=dist)
    return orc.Batch.from_case(c), c


@pytest.mark.parametrize("seed", range(4))
def test_invariant_misa_all_heads_is_dsa(seed):
    b, _ = _rand(seed)
    k = 17
    d_idx, d_val, d_sc = orc.dsa(b, k, want_scores=True)
    m = orc.misa(b, 16, b.H, k, want_scores=True)
    assert np.array_equal(np.sort(m["heads"], 1), np.tile(np.arange(b.H), (b.T, 1)))
    assert np.array_equal(m["scores"], d_sc)      # same sum in the same order
    assert np.array_equal(m["idx"], d_idx)


@pytest.mark.parametrize("seed", range(4))
def test_invariant_dagger_full_candidates_is_dsa(seed):
    b, _ = _rand(seed)
    k = 13
    d_idx, _ = orc.dsa(b, k)
    dg = orc.misa_dagger(b, 16, 2, b.Lmax, k)      # k' >= every prefix
    assert np.array_equal(dg["idx"], d_idx)
    dg2 = orc.misa_dagger(b, 16, b.H, 40, k)       # h = H, any k' >= k
    assert np.array_equal(dg2["idx"], d_idx)


@pytest.mark.parametrize("seed", range(4))
def test_invariant_dagger_kc_equal_k_and_recovery(seed):
    b, _ = _rand(seed)
    k, kc, B, h = 12, 48, 16, 2
    m = orc.misa(b, B, h, k)
    dg_same = orc.misa_dagger(b, B, h, k, k)
    for t in range(b.T):
        assert set(dg_same["idx"][t]) == set(m["idx"][t])
    dg = orc.misa_dagger(b, B, h, kc, k)
    D, _ = orc.dsa(b, k)
    for t in range(b.T):
        Dt = set(D[t]) - {-1}
        Ct = set(dg["cand"][t]) - {-1}
        Ft = set(dg["idx"][t]) - {-1}
        assert Ft <= Ct
        assert Ft & Dt == Ct & Dt                   # the rerank keeps every DSA token it was given
        assert len(Ft & Dt) >= len((set(m["idx"][t]) - {-1}) & Dt)


@pytest.mark.parametrize("seed", range(3))
def test_invariant_causality(seed):
    b, c = _rand(seed)
    k = 20
    ref = orc.misa(b, 16, 3, k)
    refd = orc.misa_dagger(b, 16, 3, 50, k)
    keys = c["keys"].copy()
    rng = np.random.default_rng(100 + seed)
    for t in range(b.T):
        s, p = c["q_seq"][t], c["q_pos"][t]
        # scramble only tokens beyond the earliest query of this sequence
        pmin = c["q_pos"][c["q_seq"] == s].min()
        keys[s, pmin + 1:] = rng.integers(0, 65535, size=keys[s, pmin + 1:].shape, dtype=np.uint16) & 0xBFFF
    c2 = dict(c, keys=keys)
    b2 = orc.Batch.from_case(c2)
    out = orc.misa(b2, 16, 3, k)
    outd = orc.misa_dagger(b2, 16, 3, 50, k)
    for t in range(b.T):
        s = c["q_seq"][t]
        if c["q_pos"][t] == c["q_pos"][c["q_seq"] == s].min():
            assert np.array_equal(out["idx"][t], ref["idx"][t])
            assert np.array_equal(out["heads"][t], ref["heads"][t])
            assert np.array_equal(outd["idx"][t], refd["idx"][t])


@pytest.mark.parametrize("seed", range(3))
def test_invariant_nested_topk(seed):
    b, _ = _rand(seed)
    small, _ = orc.dsa(b, 9)
    big, _ = orc.dsa(b, 31)
    for t in range(b.T):
        assert set(small[t]) - {-1} <= set(big[t]) - {-1}
        assert np.array_equal(big[t][:9], small[t])


@pytest.mark.parametrize("seed", range(3))
def test_invariant_head_permutation_and_scaling(seed):
    """Integer inputs keep every sum exact, so reordering heads changes no bit."""
    b, c = _rand(seed, dist="int")
    perm = np.random.default_rng(seed).permutation(b.H)
    c2 = dict(c, q=c["q"][:, perm], w=c["w"][:, perm])
    b2 = orc.Batch.from_case(c2)
    assert np.array_equal(orc.scores(b), orc.scores(b2))
    h1, g1 = orc.route(b, 16, 3, 0)
    h2, g2 = orc.route(b2, 16, 3, 0)
    assert np.array_equal(g1[:, perm], g2)
    # same sets of heads, named through the permutation (ties may reorder ids)
    for t in range(b.T):
        assert set(perm[h2[t]]) == set(h1[t]) or np.any(
            np.sort(g1[t])[::-1][2] == np.sort(g1[t])[::-1][3])
    # w scaled by 4 (exact): scores scale by 4, selections do not move
    c3 = dict(c, w=c["w"] * np.float32(4))
    b3 = orc.Batch.from_case(c3)
    assert np.array_equal(orc.scores(b3), 4 * orc.scores(b))
    assert np.array_equal(orc.misa(b3, 16, 3, 11)["idx"], orc.misa(b, 16, 3, 11)["idx"])


def test_prefix_shorter_than_k_pads():
    b, c = _rand(0, S=1, Lmax=50, T=3)
    k = 64
    idx, val = orc.dsa(b, k)
    for t in range(b.T):
        n = c["q_pos"][t] + 1
        assert sorted(idx[t][:n]) == list(range(n))
        assert np.all(idx[t][n:] == -1) and np.all(np.isneginf(val[t][n:]))


def test_needles_are_selected():
    """Generator sanity: on the tiny decode workload most needles planted
    along the last query's heads (unit direction, strength 1) rank in that
    query's dense top-k."""
    case, cfg = synth.make_workload("tiny_dsa_vs_misa_decode_L4096")
    b = orc.Batch.from_case(case)
    idx, _ = orc.dsa(b, cfg["k"])
    # needles: the keys whose bf16 norm stands out from the N(0,1/d) bulk
    kf = synth.bf16_bits_to_f32(case["keys"][0]).astype(np.float64)
    norms = np.linalg.norm(kf, axis=1)
    needles = np.argsort(-norms)[:16]
    assert np.isin(needles, idx[b.T - 1]).mean() > 0.5


# ------------------------------------------------- hierarchical indexer (HISA)
def test_hisa_hand_worked_example():
    g = json.load(open(GOLDEN))
    e0, e1 = g["queries"]
    b = _one_seq_batch(g["keys"], [e0["q"], e1["q"]], [e0["w"], e1["w"]], [e0["p"], e1["p"]])
    B = g["B"]
    r = orc.hisa(b, B, 1, 3)
    np.testing.assert_array_equal(r["bscore"][0, :3], e0["hisa_block_scores"])
    np.testing.assert_array_equal(r["bscore"][1, :3], e1["hisa_block_scores"])
    assert list(r["blocks"][0]) == e0["hisa_m1_blocks"] and list(r["blocks"][1]) == e1["hisa_m1_blocks"]
    assert list(r["idx"][0]) == e0["hisa_m1_top3"]
    assert list(orc.hisa(b, B, 1, 2)["idx"][1]) == e1["hisa_m1_top2"]
    r2 = orc.hisa(b, B, 2, 3)
    assert list(r2["blocks"][0]) == e0["hisa_m2_blocks"] and list(r2["blocks"][1]) == e1["hisa_m2_blocks"]
    assert list(r2["idx"][0]) == e0["hisa_m2_top3"]
    assert list(orc.hisa(b, B, 2, 2)["idx"][1]) == e1["hisa_m2_top2"]
    # routed heads in both stages
    rh = orc.hisa(b, B, 1, 2, heads=np.array([[0], [1]], np.int32))
    assert list(rh["idx"][0][:1]) == e0["misa_hisa_head0_m1_top1"]
    assert list(rh["idx"][1]) == e1["misa_hisa_head1_m1_top2"]


@pytest.mark.parametrize("seed", range(4))
def test_hisa_keeping_every_block_is_dsa(seed):
    """m >= the query's block count: the refinement sees the whole prefix, so
    HISA is the dense indexer, bit for bit."""
    b, _ = _rand(seed)
    for B in (1, 7, 64):
        M = (b.Lmax + B - 1) // B
        r = orc.hisa(b, B, M, 50)
        idx, val = orc.dsa(b, 50)
        assert np.array_equal(r["idx"], idx) and np.array_equal(r["val"], val)


@pytest.mark.parametrize("seed", range(3))
def test_hisa_unit_blocks_is_dsa(seed):
    """B = 1: a block's mean is its one key, so block scores are token scores
    and the m >= k best blocks contain the dense top-k."""
    b, _ = _rand(seed)
    for k, m in ((10, 10), (20, 37)):
        r = orc.hisa(b, 1, m, k)
        idx, val = orc.dsa(b, k)
        assert np.array_equal(r["idx"], idx) and np.array_equal(r["val"], val)
        sc = orc.scores(b)
        for t in range(b.T):
            n = b.q_pos[t] + 1
            np.testing.assert_array_equal(r["bscore"][t, :n], sc[t, :n])


@pytest.mark.parametrize("seed", range(3))
def test_hisa_with_every_head_routed_is_hisa(seed):
    """Routing every head (in any order) changes nothing."""
    b, _ = _rand(seed)
    rng = np.random.default_rng(seed)
    heads = np.stack([rng.permutation(b.H) for _ in range(b.T)]).astype(np.int32)
    for B, m in ((8, 3), (32, 2)):
        a = orc.hisa(b, B, m, 40)
        c = orc.hisa(b, B, m, 40, heads=heads)
        for key in ("idx", "val", "blocks", "bscore"):
            assert np.array_equal(a[key], c[key]), key


@pytest.mark.parametrize("seed", range(3))
def test_hisa_single_head_block_scores_sum_to_router_importance(seed):
    """With one head j in both stages and w_j > 0, the block scores are
    w_j * ReLU(q_j . Kbar_b); their sum over the query's blocks is the
    router's importance g_j (mode 0), computed by the router's own code."""
    b, _ = _rand(seed)
    B = 16
    _, g = orc.route(b, B, 1, 0)
    for j in range(b.H):
        heads = np.full((b.T, 1), j, np.int32)
        r = orc.hisa(b, B, 1, 5, heads=heads)
        for t in range(b.T):
            M = (b.q_pos[t] + 1 + B - 1) // B
            assert np.isclose(r["bscore"][t, :M].sum(), g[t, j], rtol=1e-12, atol=1e-12)
            assert np.all(np.isneginf(r["bscore"][t, M:]))


def test_hisa_constant_keys_closed_form():
    """All keys equal: every block and every token score is the same, so the
    first m blocks are kept and the top-k is the first k tokens."""
    L, d, B, m, k = 200, 4, 16, 3, 20
    keys = np.tile(np.array([1.0, -0.5, 0.25, 2.0], np.float32), (L, 1))
    b = _one_seq_batch(keys, [[[0.5, 1.0, -1.0, 0.25], [1.0, 0.0, 0.0, 0.0]]], [[0.7, -0.2]], [150])
    r = orc.hisa(b, B, m, k)
    assert list(r["blocks"][0]) == [0, 1, 2]
    assert list(r["idx"][0]) == list(range(k))
    x0, x1 = 0.5 - 0.5 - 0.25 + 0.5, 1.0
    assert np.allclose(r["val"][0], 0.7 * max(x0, 0) - 0.2 * max(x1, 0))
