"""Parity at the full workload sizes, in the launch configuration the
benchmark times: the same calls over every query row of each workload
(16 x 128K decode, 32 x 32K dense, MISA-dagger, the 4096-query prefill
chunk, HISA and MISA composed with HISA), then the oracle on every query row
of the decode workloads and on at least 256 rows of the prefill chunk (the
edges of every query workgroup and random rows), computed for those rows
alone.  Routed heads and kept blocks must be the oracle's (up to a near-tie),
selected sets the oracle's up to swaps at the k-th score, and every reported
score within the score tolerance of the oracle's fp64 score (parity.py)."""
import numpy as np
import pytest

from oracle import oracle as orc
from long_context_sparse_05_amd import synth
import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from long_context_sparse_05_amd import abi
    abi.load()  # raises if the HIP library is missing: no silent fallback
    return abi


def _abi():
    from long_context_sparse_05_amd import abi
    return abi


def np_(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


QWG = 64  # queries per workgroup of the prefill tiling at h = 8


def _sample_rows(T):
    """Every row of the decode workloads; for the 4096-query prefill chunk the
    first and last row of every 64-query workgroup (which also puts rows on
    both sides of every 128-key tile edge of the causal boundary) plus
    seeded random rows, at least 256 in all."""
    if T <= 64:
        return list(range(T))
    rows = set()
    for q0 in range(0, T, QWG):
        rows.update((q0, min(q0 + QWG, T) - 1))
    rng = np.random.default_rng(2024)
    while len(rows) < 256:
        rows.add(int(rng.integers(0, T)))
    return sorted(rows)


def _allowed_skips(n_rows):
    """Rows whose routed heads differ from the oracle's on a near-tie are
    skipped (their selection is a different, equally valid set)."""
    return max(1, n_rows // 50)


def _sub(case, rows):
    """The sampled query rows with the whole key cache: the oracle's batch."""
    sub = dict(case)
    for key in ("q", "w", "q_seq", "q_pos"):
        sub[key] = np.ascontiguousarray(case[key][rows])
    return orc.Batch.from_case(sub)


def _heads_agree(g_heads, o_heads, o_g):
    """Routed heads: the same set as the oracle's, or a near-tie there."""
    if set(int(x) for x in g_heads) == set(int(x) for x in o_heads):
        return True
    assert parity.head_margin(o_g, len(o_heads)) < 1e-4, (sorted(g_heads), sorted(o_heads))
    return False


def _check_row(g_idx, g_val, o_idx, o_row, n, k, n_cand=None):
    sb = parity.row_sbar(o_row, n)
    parity.check_set(g_idx, o_idx, lambda i: o_row[i], n if n_cand is None else n_cand, k, sb)
    for i, v in zip(g_idx, g_val):
        if i >= 0:
            assert abs(float(v) - o_row[i]) <= parity.REL * (abs(o_row[i]) + sb), (int(i), v, o_row[i])


def _load(name):
    case, cfg = synth.make_workload(name)
    print("workload %s: %s" % (name, {k: v for k, v in cfg.items()}), flush=True)
    return case, cfg, _abi().Batch.from_numpy(case)


@pytest.mark.parametrize("name", ["tiny_dsa_vs_misa_decode_L4096", "misa_decode_16x128K",
                                  "misa_multiquery_decode_8x8x32K", "misa_prefill_chunk_4096q_L65536"])
def test_workload_misa(name):
    """The fused MISA call (router, routed scoring, top-k); the prefill chunk
    takes the tiled router, the 32x32 MFMA scoring and the threshold-list
    select, the multi-query decode batch the MFMA tiling over its tile table."""
    abi = _abi()
    case, cfg, b = _load(name)
    B, h, k = cfg["B"], cfg["h"], cfg["k"]
    pooled = abi.pool(b, B)
    heads, idx, val = abi.indexer(b, pooled, B, h, k)
    heads, idx, val = np_(heads), np_(idx), np_(val)
    rows = _sample_rows(b.T)
    o = orc.misa(_sub(case, rows), B, h, k, want_scores=True)
    checked = 0
    for j, r in enumerate(rows):
        if not _heads_agree(heads[r], o["heads"][j], o["g"][j]):
            continue
        n = int(case["q_pos"][r]) + 1
        _check_row(idx[r], val[r], o["idx"][j], o["scores"][j], n, k)
        checked += 1
    assert checked >= len(rows) - _allowed_skips(len(rows))


def test_workload_dsa_dense():
    abi = _abi()
    case, cfg, b = _load("dsa_dense_decode_32x32K")
    k = cfg["k"]
    idx, val = abi.score_topk(b, None, k)
    idx, val = np_(idx), np_(val)
    rows = _sample_rows(b.T)
    oidx, _, osc = orc.dsa(_sub(case, rows), k, want_scores=True)
    for j, r in enumerate(rows):
        _check_row(idx[r], val[r], oidx[j], osc[j], int(case["q_pos"][r]) + 1, k)


def test_workload_misa_dagger():
    """Coarse stage against the oracle's routed top-k'; fine stage against
    the oracle's all-head rerank of the GPU's own candidate list."""
    abi = _abi()
    case, cfg, b = _load("misa_dagger_decode_16x128K")
    B, h, kc, k = cfg["B"], cfg["h"], cfg["kc"], cfg["k"]
    pooled = abi.pool(b, B)
    heads, cidx, cval = abi.indexer(b, pooled, B, h, kc)
    fin, fval = abi.rerank(b, cidx, k)
    heads, cidx, cval, fin, fval = np_(heads), np_(cidx), np_(cval), np_(fin), np_(fval)
    rows = _sample_rows(b.T)
    ob = _sub(case, rows)
    o = orc.misa(ob, B, h, kc, want_scores=True)
    full = orc.scores(ob)
    ofin, _ = orc.rerank(ob, np.ascontiguousarray(cidx[rows]), k)
    for j, r in enumerate(rows):
        n = int(case["q_pos"][r]) + 1
        if _heads_agree(heads[r], o["heads"][j], o["g"][j]):
            _check_row(cidx[r], cval[r], o["idx"][j], o["scores"][j], n, kc)
        nv = int((cidx[r] >= 0).sum())
        _check_row(fin[r], fval[r], ofin[j], full[j], n, k, n_cand=nv)
        assert set(int(x) for x in fin[r] if x >= 0) <= set(int(x) for x in cidx[r])


@pytest.mark.parametrize("name", ["hisa_decode_16x128K", "misa_hisa_decode_16x128K"])
def test_workload_hisa(name):
    """Kept blocks the oracle's (up to a near-tie in the block scores) and
    the refinement's tokens the oracle's among those blocks."""
    abi = _abi()
    case, cfg, b = _load(name)
    B, m, k = cfg["B"], cfg["m"], cfg["k"]
    pooled = abi.pool(b, B)
    rows = _sample_rows(b.T)
    ob = _sub(case, rows)
    th = oh = None
    if "h" in cfg:
        th = abi.route(b, pooled, B, cfg["h"], 0)
        oh, og = orc.route(ob, B, cfg["h"])
    gs, gb = abi.hisa_blocks(b, pooled, B, m, heads=th)
    gi, gv = abi.hisa_indexer(b, pooled, B, m, k, heads=th)
    gs, gb, gi, gv = np_(gs), np_(gb), np_(gi), np_(gv)
    gh = np_(th) if th is not None else None
    o = orc.hisa(ob, B, m, k, heads=oh)
    osc = orc.scores(ob, oh)
    checked = 0
    for j, r in enumerate(rows):
        if gh is not None and not _heads_agree(gh[r], oh[j], og[j]):
            continue
        M = int(case["q_pos"][r]) // B + 1
        ob_s = o["bscore"][j, :M]
        sb = float(np.mean(np.abs(ob_s))) + 1e-30
        assert np.all(np.abs(gs[r, :M] - ob_s) <= 1e-4 * (np.abs(ob_s) + sb)), r
        if set(int(x) for x in gb[r]) != set(int(x) for x in o["blocks"][j]):
            assert parity.head_margin(ob_s, min(m, M)) < 1e-4, r
            continue
        n = int(case["q_pos"][r]) + 1
        allowed = np.zeros(n, bool)
        for blk in gb[r]:
            if blk >= 0:
                allowed[blk * B:min(blk * B + B, n)] = True
        assert all(allowed[i] for i in gi[r] if i >= 0)
        masked = np.where(allowed, osc[j, :n], -np.inf)
        sbt = parity.row_sbar(osc[j], n)
        parity.check_set(gi[r], o["idx"][j], lambda i: masked[i], int(allowed.sum()), k, sbt)
        for i, v in zip(gi[r], gv[r]):
            if i >= 0:
                assert abs(float(v) - osc[j, i]) <= parity.REL * (abs(osc[j, i]) + sbt)
        checked += 1
    assert checked >= len(rows) - _allowed_skips(len(rows))
