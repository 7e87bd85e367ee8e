"""GPU parity of every C-ABI call against the CPU oracle, on seeded inputs
small enough for the oracle, spanning several tiles, ragged tails and the
degenerate cases (prefix shorter than k, k = prefix, h = 1, h = H, ties,
-0.0, candidate lists with empty slots, too many tied candidates for LDS).
Comparison rules are in parity.py."""
import json
import os

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


def upload(case):
    return _abi().Batch.from_numpy(case)


def n_valid(case):
    return case["q_pos"] + 1


CASES = [
    # S, Lmax, T, H, seed
    (1, 300, 5, 64, 0),
    (3, 1000, 7, 32, 1),
    (2, 4133, 6, 8, 2),
    (2, 2500, 9, 20, 3),
    (1, 17, 3, 64, 4),
    (2, 1500, 4, 128, 5),  # the largest head count the kernels take (MISA_MAX_HEADS)
]


def make(S, Lmax, T, H, seed, dist="normal", ragged=True):
    seq_lens = None
    if ragged and S > 1:
        rng = np.random.default_rng(seed + 77)
        seq_lens = rng.integers(max(1, Lmax // 3), Lmax + 1, size=S).astype(np.int32)
        seq_lens[0] = Lmax
    return synth.random_case(S, Lmax, T, H, seed=seed, dist=dist, seq_lens=seq_lens)


# ----------------------------------------------------------------------- pool
@pytest.mark.parametrize("B", [1, 7, 64, 128])
def test_pool(B):
    abi = _abi()
    case = make(3, 1000, 2, 8, 5)
    b = upload(case)
    got = np_(abi.pool(b, B))
    ref = orc.pool(orc.Batch.from_case(case), B)
    # fp32 sums of <= B bf16 values against fp64: a few ulps of the block's magnitude
    scale = np.abs(ref).mean() + 1e-30
    assert np.allclose(got, ref, rtol=1e-5, atol=1e-6 * scale)


# --------------------------------------------------------------------- scores
@pytest.mark.parametrize("S,Lmax,T,H,seed", CASES)
def test_score_dense_and_routed(S, Lmax, T, H, seed):
    abi = _abi()
    case = make(S, Lmax, T, H, seed)
    b = upload(case)
    ob = orc.Batch.from_case(case)
    parity.check_scores(np_(abi.score(b)), orc.scores(ob), n_valid(case))
    rng = np.random.default_rng(seed)
    for h in sorted({1, min(8, H), H}):
        heads = np.stack([rng.permutation(H)[:h] for _ in range(T)]).astype(np.int32)
        got = np_(abi.score(b, torch.from_numpy(heads).cuda()))
        parity.check_scores(got, orc.scores(ob, heads), n_valid(case))


# ---------------------------------------------------------------------- top-k
def _topk_rows(rng, rows, ld, kind):
    if kind == "ties":
        v = rng.choice(np.array([-1.5, -0.0, 0.0, 0.25, 1.0, 3.0], np.float32), size=(rows, ld))
    elif kind == "equal":
        v = np.full((rows, ld), 0.5, np.float32)
    elif kind == "spread":
        v = (rng.standard_normal((rows, ld)) * np.exp(rng.uniform(-20, 20, (rows, ld)))).astype(np.float32)
    elif kind == "negative":   # the k-th score is negative (keys below the sign flip)
        v = (rng.standard_normal((rows, ld)) * 0.05 - 0.2).astype(np.float32)
    elif kind == "straddle":   # the top k spans zero: positive and negative keys
        v = (rng.standard_normal((rows, ld)) * 0.05 - 0.1).astype(np.float32)
    else:
        v = rng.standard_normal((rows, ld)).astype(np.float32) * 0.05
    return v


@pytest.mark.parametrize("kind,rows,ld,k", [
    ("normal", 6, 5000, 300), ("ties", 5, 3000, 257), ("spread", 4, 70000, 2048),
    ("equal", 2, 20000, 100), ("normal", 3, 100, 100), ("ties", 2, 40000, 1),
    ("normal", 3, 33000, 16384), ("negative", 3, 40000, 2048), ("straddle", 4, 131072, 2048),
])
def test_topk_exact(kind, rows, ld, k):
    abi = _abi()
    rng = np.random.default_rng(hash(kind) % 1000 + rows)
    v = _topk_rows(rng, rows, ld, kind)
    row_len = rng.integers(0, ld + 1, size=rows).astype(np.int32)
    row_len[0] = ld
    if rows > 2:
        row_len[1] = min(ld, k // 2)    # prefix shorter than k
        row_len[2] = 0
    idx, val = abi.topk(torch.from_numpy(v).cuda(), torch.from_numpy(row_len).cuda(), k)
    idx, val = np_(idx), np_(val)
    for r in range(rows):
        n = int(row_len[r])
        parity.check_exact_topk(idx[r], val[r], v[r], n, k, orc.topk_f32)
        assert np.all(idx[r][idx[r] >= 0] < n)


@pytest.mark.parametrize("k", [1, 200, 3000])
def test_topk_exact_row_mode(k):
    """Enough rows to fill the GPU take the one-workgroup-per-row select;
    rows mix ties, all-equal (more tied candidates than fit in LDS), wide
    dynamic range, short and empty prefixes."""
    abi = _abi()
    rows, ld = 300, 20000
    rng = np.random.default_rng(k)
    kinds = ["equal", "ties", "normal", "spread"]
    v = np.stack([_topk_rows(rng, 1, ld, kinds[r % 4])[0] for r in range(rows)])
    row_len = rng.integers(0, ld + 1, size=rows).astype(np.int32)
    row_len[:8] = ld
    row_len[8] = 0
    row_len[9] = min(ld, k // 2)
    idx, val = abi.topk(torch.from_numpy(v).cuda(), torch.from_numpy(row_len).cuda(), k)
    idx, val = np_(idx), np_(val)
    for r in range(rows):
        n = int(row_len[r])
        parity.check_exact_topk(idx[r], val[r], v[r], n, k, orc.topk_f32)
        assert np.all(idx[r][idx[r] >= 0] < n)


def _skewed_rows(rng, rows, ld, kind):
    """Rows whose columns = 0 mod 4 differ from the rest, so that an estimate
    drawn from such columns misjudges the k-th score (both ways), plus
    needles and a ramp along the row."""
    v = rng.standard_normal((rows, ld)).astype(np.float32)
    c = np.arange(ld)
    if kind == "mod4_hi":
        v[:, c % 4 == 0] += 6.0
    elif kind == "mod4_lo":
        v[:, c % 4 == 0] -= 6.0
    elif kind == "needles":
        for r in range(rows):
            v[r, rng.choice(ld, 40, replace=False)] = 50.0 + rng.standard_normal(40).astype(np.float32)
    elif kind == "ramp":
        v += (c / ld * 4.0).astype(np.float32)
    elif kind == "ties":
        v = np.round(v * 4.0) / 4.0
    return v


@pytest.mark.parametrize("ld,k", [(65536, 2048), (65536, 64), (8192, 1000), (65528, 700)])
def test_topk_row_mode_long_rows(ld, k):
    """One-workgroup-per-row select on long rows: the sampled threshold is
    taken where it brackets the k-th score, and the exact histogram path
    otherwise (too few or too many columns above the estimate)."""
    abi = _abi()
    rows = 256
    rng = np.random.default_rng(ld + k)
    kinds = ["normal", "mod4_hi", "mod4_lo", "needles", "ramp", "ties"]
    v = np.concatenate([_skewed_rows(rng, (rows + 5) // 6, ld, kd) for kd in kinds])[:rows]
    row_len = np.full(rows, ld, np.int32)
    row_len[1::7] = rng.integers(k, ld + 1, size=len(row_len[1::7]))   # ragged prefixes
    row_len[2] = ld - 1
    row_len[3] = 8 * k - 3          # just below the sampled path's k <= n/8 bound
    row_len[4] = min(ld, 8 * k)     # just at it
    idx, val = abi.topk(torch.from_numpy(v).cuda(), torch.from_numpy(row_len).cuda(), k)
    idx, val = np_(idx), np_(val)
    for r in range(rows):
        n = int(row_len[r])
        parity.check_exact_topk(idx[r], val[r], v[r], n, k, orc.topk_f32)
        assert np.all(idx[r][idx[r] >= 0] < n)


@pytest.mark.parametrize("k", [1, 300, 2048, 4096])
def test_topk_streamed_select(k):
    """Many long rows take the streamed select (sampled threshold, one pass,
    the list resolved in LDS); rows it cannot settle -- prefixes too short,
    heavy ties that overflow its list -- go on to the row select, and a k
    whose expected list does not fit (k = 4096 here) takes the row select
    alone.  Every row is checked exactly."""
    abi = _abi()
    rows, ld = 512, 32768
    rng = np.random.default_rng(k + 7)
    kinds = ["normal", "needles", "ramp", "ties", "mod4_hi"]
    v = np.concatenate([_skewed_rows(rng, (rows + 4) // 5, ld, kd) for kd in kinds])[:rows]
    v[5::11] = _topk_rows(rng, len(v[5::11]), ld, "spread")
    v[6::13] = _topk_rows(rng, len(v[6::13]), ld, "ties")
    row_len = np.full(rows, ld, np.int32)
    row_len[1::3] = rng.integers(0, ld + 1, size=len(row_len[1::3]))  # some below the streamed minimum
    row_len[2] = 16384
    row_len[3] = 16383
    row_len[4] = min(ld, k)
    idx, val = abi.topk(torch.from_numpy(v).cuda(), torch.from_numpy(row_len).cuda(), k)
    idx, val = np_(idx), np_(val)
    for r in range(rows):
        n = int(row_len[r])
        parity.check_exact_topk(idx[r], val[r], v[r], n, k, orc.topk_f32)
        assert np.all(idx[r][idx[r] >= 0] < n)


def test_topk_streamed_select_wide_rows_and_infinities():
    """The streamed select at its widest rows (131072 columns) on value
    patterns a caller's score rows can hold: -inf tails (a prefix shorter
    than the row), all -inf, a few +inf, signed zeros around the k-th score
    (-0 ranks equal to +0, so the lower index wins), values spanning many
    binades, all-negative rows.  Every row is checked exactly."""
    abi = _abi()
    rows, ld, k = 256, 131072, 2048
    rng = np.random.default_rng(131)
    v = rng.standard_normal((rows, ld)).astype(np.float32)
    for r in range(rows):
        kind = r % 8
        if kind == 1:                      # -inf tail after a random prefix
            v[r, rng.integers(k, ld):] = -np.inf
        elif kind == 2 and r % 16 == 2:    # the whole row -inf
            v[r, :] = -np.inf
        elif kind == 3:                    # a few +inf
            v[r, rng.choice(ld, 5, replace=False)] = np.inf
        elif kind == 4:                    # signed zeros straddle the k-th score
            v[r] = np.abs(v[r])
            z = rng.choice(ld, ld - k // 2, replace=False)
            v[r, z] = np.where(rng.random(z.size) < 0.5, np.float32(0.0), np.float32(-0.0))
        elif kind == 5:                    # many binades
            v[r] = (rng.standard_normal(ld) * 10.0 ** rng.uniform(-30, 30, ld)).astype(np.float32)
        elif kind == 6:                    # all negative
            v[r] = -np.abs(v[r]) - 1.0
    row_len = np.full(rows, ld, np.int32)
    row_len[7::8] = rng.integers(16384, ld + 1, size=len(row_len[7::8]))
    idx, val = abi.topk(torch.from_numpy(v).cuda(), torch.from_numpy(row_len).cuda(), k)
    idx, val = np_(idx), np_(val)
    for r in range(rows):
        n = int(row_len[r])
        parity.check_exact_topk(idx[r], val[r], v[r], n, k, orc.topk_f32)
        assert np.all(idx[r][idx[r] >= 0] < n)


@pytest.mark.parametrize("rows,ld,k", [(300, 32768, 512), (4, 65536, 2048)])
def test_topk_unaligned_score_rows(rows, ld, k):
    """Score rows that start 4 bytes past a 16-byte boundary (a view into a
    larger buffer): the selects read them with scalar loads."""
    abi = _abi()
    rng = np.random.default_rng(rows + k)
    v = rng.standard_normal((rows, ld)).astype(np.float32)
    row_len = np.full(rows, ld, np.int32)
    row_len[1::5] = rng.integers(k, ld + 1, size=len(row_len[1::5]))
    buf = torch.empty(rows * ld + 1, dtype=torch.float32, device="cuda")
    sc = buf[1:].view(rows, ld)
    sc.copy_(torch.from_numpy(v))
    assert sc.data_ptr() % 16 == 4
    idx, val = abi.topk(sc, torch.from_numpy(row_len).cuda(), k)
    idx, val = np_(idx), np_(val)
    for r in range(rows):
        n = int(row_len[r])
        parity.check_exact_topk(idx[r], val[r], v[r], n, k, orc.topk_f32)


# ---------------------------------------------------------- score + top-k
@pytest.mark.parametrize("S,Lmax,T,H,seed", CASES)
@pytest.mark.parametrize("k", [1, 64, 600])
def test_score_topk(S, Lmax, T, H, seed, k):
    abi = _abi()
    k = min(k, Lmax)
    case = make(S, Lmax, T, H, seed)
    b = upload(case)
    ob = orc.Batch.from_case(case)
    rng = np.random.default_rng(seed + k)
    h = min(8, H)
    heads = np.stack([rng.permutation(H)[:h] for _ in range(T)]).astype(np.int32)
    for hh in (None, heads):
        th = None if hh is None else torch.from_numpy(hh).cuda()
        idx, val = abi.score_topk(b, th, k)
        idx, val = np_(idx), np_(val)
        osc = orc.scores(ob, hh)
        oidx = np.stack([orc.topk(osc[t, :n_valid(case)[t]], k)[0] for t in range(T)])
        # misa_score computes the same fp32 scores unless score_topk took the
        # multi-query MFMA tiling (S > 1, two rows a sequence): then only the
        # oracle comparison applies
        nh = H if hh is None else hh.shape[1]
        same_kernel = not (S > 1 and T >= 2 * S and nh <= 64)
        rows = np_(abi.score(b, th)) if same_kernel else None
        for t in range(T):
            n = int(n_valid(case)[t])
            sb = parity.row_sbar(osc[t], n)
            if same_kernel:
                parity.check_exact_topk(idx[t], val[t], rows[t], n, k, orc.topk_f32)
            else:
                for i, v in zip(idx[t], val[t]):
                    if i >= 0:
                        assert abs(float(v) - osc[t, i]) <= parity.REL * (abs(osc[t, i]) + sb)
            parity.check_set(idx[t], oidx[t], lambda i: osc[t, i], n, k, sb)
    # indexer_dense is the all-head call
    di, _ = abi.indexer_dense(b, k)
    di = np_(di)
    dref, _ = abi.score_topk(b, None, k)
    assert np.array_equal(np.sort(di, 1), np.sort(np_(dref), 1))


@pytest.mark.parametrize("k", [2048, 6000])
@pytest.mark.parametrize("concentrated", [False, True])
def test_two_stage_select_on_scored_rows(concentrated, k):
    """Few long rows take the two-stage select: each scoring workgroup keeps
    its chunk's share of the row's top-k, and the merge takes the top-k of
    the union.  With the top-k spread over the row the union proves the
    result; with most of it packed into a few chunks (keys aligned with a
    positive-weight head along one stretch of the sequence) those chunks
    drop entries of the true top-k, the merge detects it and selects from
    the whole score row.  Both are checked exactly against the kernel's own
    scores and against the oracle's selection."""
    abi = _abi()
    S, Lmax, T, H = 3, 40000, 5, 16
    q_seq = np.array([0, 1, 2, 0, 1], np.int32)
    q_pos = np.array([Lmax - 1, 39000, 17000, 25000, Lmax - 1], np.int32)
    case = synth.random_case(S, Lmax, T, H, seed=41, q_pos=q_pos, q_seq=q_seq)
    if concentrated:
        keys = synth.bf16_bits_to_f32(case["keys"]).copy()
        for t in range(T):
            j = int(np.argmax(case["w"][t]))
            qd = synth.bf16_bits_to_f32(case["q"][t, j])
            lo = 3000 + 1000 * t
            keys[q_seq[t], lo:lo + 2500] += 0.5 * qd / np.linalg.norm(qd)
        case["keys"] = synth.to_bf16_bits(keys)
    b = upload(case)
    ob = orc.Batch.from_case(case)
    rng = np.random.default_rng(3)
    heads = np.stack([rng.permutation(H)[:4] for _ in range(T)]).astype(np.int32)
    for hh in (None, heads):
        th = None if hh is None else torch.from_numpy(hh).cuda()
        idx, val = abi.score_topk(b, th, k)
        idx, val = np_(idx), np_(val)
        rows = np_(abi.score(b, th))
        osc = orc.scores(ob, hh)
        for t in range(T):
            n = int(q_pos[t]) + 1
            parity.check_exact_topk(idx[t], val[t], rows[t], n, k, orc.topk_f32)
            oi = orc.topk(osc[t, :n], k)[0]
            parity.check_set(idx[t], oi, lambda i: osc[t, i], n, k, parity.row_sbar(osc[t], n))


@pytest.mark.parametrize("heavy_chunk", [0, 3])
def test_two_stage_merge_list_longer_than_first_load_round(heavy_chunk):
    """A chunk list longer than the merge's first round of loads (four
    entries a lane, 256 a list, when the expected list is short): 2 rows of
    40960 columns, k = 512, ten lists of 4096 columns whose quota is 111.
    Every score is 0 except 280 columns of one chunk and 30 of each other
    chunk at 1.0: the heavy chunk keeps its 280 tied entries (at most
    2 quota + 64 = 286), the others their 30, and the top-512 -- the 512
    lowest columns scoring 1.0 -- is proven by the lists, so the merge
    itself, with the tail of the long list loaded in a second round, writes
    it (checked exactly against the oracle's fp32 top-k)."""
    abi = _abi()
    rows, ld, k, chunk = 2, 40960, 512, 4096
    rng = np.random.default_rng(17 + heavy_chunk)
    v = np.zeros((rows, ld), np.float32)
    for r in range(rows):
        for c in range(ld // chunk):
            m = 280 if c == heavy_chunk else 30
            v[r, c * chunk + rng.choice(chunk, m, replace=False)] = 1.0
    row_len = np.full(rows, ld, np.int32)
    idx, val = abi.topk(torch.from_numpy(v).cuda(), torch.from_numpy(row_len).cuda(), k)
    idx, val = np_(idx), np_(val)
    for r in range(rows):
        parity.check_exact_topk(idx[r], val[r], v[r], ld, k, orc.topk_f32)
        ones = np.flatnonzero(v[r] == 1.0)
        assert np.array_equal(np.sort(idx[r]), ones[:k])


# ------------------------------------------------------- pooled-cache append
@pytest.mark.parametrize("B", [1, 16, 64, 128])
def test_pool_append_matches_fresh_pool(B):
    """After keys are appended, misa_pool_append rewrites only the blocks
    that hold them; the cache then equals a fresh misa_pool bit for bit and
    the oracle's pooling to fp32 accuracy, and blocks past the new lengths
    are left untouched."""
    abi = _abi()
    S, Lmax = 3, 1000
    case = synth.random_case(S, Lmax, 2, 8, seed=B)
    old = np.array([100, 383, 700], np.int32)
    new = old + np.array([1, 50, 129], np.int32)
    case["seq_lens"] = old.copy()
    b = upload(case)
    pooled = abi.pool(b, B)
    sentinel = 12345.0
    M = (Lmax + B - 1) // B
    nb_new = (new + B - 1) // B
    for s_ in range(S):  # blocks past the new length must not be written
        pooled[s_, nb_new[s_]:] = sentinel
    b.seq_lens.copy_(torch.from_numpy(new))
    abi.pool_append(b, B, torch.from_numpy(old).cuda(), int((new - old).max()), pooled)
    fresh = abi.pool(b, B)
    got, ref = np_(pooled), np_(fresh)
    for s_ in range(S):
        n = nb_new[s_]
        assert np.array_equal(got[s_, :n], ref[s_, :n])
        assert np.all(got[s_, n:] == sentinel)
    case["seq_lens"] = new
    opool = orc.pool(orc.Batch.from_case(case), B)
    for s_ in range(S):
        n = nb_new[s_]
        assert np.allclose(got[s_, :n], opool[s_, :n], rtol=1e-5, atol=1e-6)


def test_pool_append_streaming_decode():
    """One key per step for 300 steps (the decode loop the append serves):
    the cache stays equal to a fresh pool, and so does the router."""
    abi = _abi()
    S, Lmax, B, H = 2, 700, 16, 16
    case = synth.random_case(S, Lmax, S, H, seed=7, q_seq=np.arange(S, dtype=np.int32),
                             q_pos=np.full(S, 399, np.int32))
    lens = np.array([100, 250], np.int32)
    case["seq_lens"] = lens.copy()
    b = upload(case)
    pooled = abi.pool(b, B)
    for _ in range(300):
        old = torch.from_numpy(lens.copy()).cuda()
        lens = lens + 1
        b.seq_lens.copy_(torch.from_numpy(lens))
        abi.pool_append(b, B, old, 1, pooled)
    fresh = abi.pool(b, B)
    assert np.array_equal(np_(pooled), np_(fresh))
    h1 = np_(abi.route(b, pooled, B, 4, 0))
    h2 = np_(abi.route(b, fresh, B, 4, 0))
    assert np.array_equal(h1, h2)


# --------------------------------------------------------------------- router
@pytest.mark.parametrize("S,Lmax,T,H,seed", CASES)
@pytest.mark.parametrize("B", [1, 16, 64, 128])
@pytest.mark.parametrize("mode", [0, 1])
def test_route(S, Lmax, T, H, seed, B, mode):
    abi = _abi()
    B = min(B, Lmax)
    case = make(S, Lmax, T, H, seed)
    b = upload(case)
    ob = orc.Batch.from_case(case)
    pooled = abi.pool(b, B)
    for h in sorted({1, min(8, H), H}):
        heads, g = abi.route(b, pooled, B, h, mode, want_score=True)
        heads, g = np_(heads), np_(g)
        oheads, og = orc.route(ob, B, h, mode)
        for t in range(T):
            sb = float(np.mean(np.abs(og[t])))
            assert np.all(np.abs(g[t] - og[t]) <= 1e-4 * (np.abs(og[t]) + sb)), (t, g[t], og[t])
            # the decision, taken on the GPU's own fp32 importances, in rank order
            assert list(heads[t]) == list(orc.topk_f32(g[t], h)), t
            if list(heads[t]) != list(oheads[t]):
                assert parity.head_margin(og[t], h) < 1e-4 or sorted(heads[t]) == sorted(oheads[t]), \
                    "router heads differ at margin %g" % parity.head_margin(og[t], h)


ROUTE_TILE_CASES = [
    # Lmax, T, H, B, positions, mode
    (3000, 200, 32, 64, "tail", 0),
    (1100, 97, 8, 16, "random", 1),
    (2500, 130, 64, 128, "random", 0),
    (700, 64, 16, 1, "tail", 0),
    (4200, 256, 64, 128, "tail", 1),
    (5000, 70, 32, 128, "early", 0),
]


@pytest.mark.parametrize("Lmax,T,H,B,positions,mode", ROUTE_TILE_CASES)
def test_route_prefill_tiles(Lmax, T, H, B, positions, mode):
    """Many queries of one sequence take the tiled one-kernel router: the
    importances and the routed heads match the oracle, including queries
    whose prefix is shorter than one block and prefixes ending on a block
    boundary."""
    abi = _abi()
    rng = np.random.default_rng(Lmax + T + B)
    if positions == "tail":
        q_pos = np.arange(Lmax - T, Lmax, dtype=np.int32)
    elif positions == "early":
        q_pos = np.concatenate([np.arange(0, 40), rng.integers(0, Lmax, T - 42), [B - 1, 2 * B - 1]])
        q_pos = q_pos.astype(np.int32)
    else:
        q_pos = np.sort(rng.integers(0, Lmax, size=T)).astype(np.int32)
    case = synth.random_case(1, Lmax, T, H, seed=Lmax % 97, q_pos=q_pos, q_seq=np.zeros(T, np.int32))
    b = upload(case)
    ob = orc.Batch.from_case(case)
    pooled = abi.pool(b, B)
    for h in sorted({1, min(8, H), H}):
        heads, g = abi.route(b, pooled, B, h, mode, want_score=True)
        heads, g = np_(heads), np_(g)
        oheads, og = orc.route(ob, B, h, mode)
        for t in range(T):
            sb = float(np.mean(np.abs(og[t])))
            assert np.all(np.abs(g[t] - og[t]) <= 1e-4 * (np.abs(og[t]) + sb)), (t, g[t], og[t])
            assert list(heads[t]) == list(orc.topk_f32(g[t], h)), t
            if list(heads[t]) != list(oheads[t]):
                assert parity.head_margin(og[t], h) < 1e-4 or sorted(heads[t]) == sorted(oheads[t]), \
                    "router heads differ at margin %g" % parity.head_margin(og[t], h)


# ------------------------------------------------------- selection fidelity
def test_fidelity_sweep_matches_oracle_selections():
    """The GPU sweep's recall / IoU against the dense set equal the same
    metrics taken on the oracle's selections, and the invariants hold:
    MISA with h = H and MISA-dagger with k' >= L reproduce DSA exactly."""
    from long_context_sparse_05_amd import fidelity
    S, L, H, k = 4, 3000, 16, 100
    case = synth.decode_case(S, L, H, seed=5, n_needles=8)
    rows = fidelity.sweep(case, k, hs=[1, 4, H], kps=[400, L], Bs=[16, 64], ms=[3, 200], hisa_h=4)
    ob = orc.Batch.from_case(case)
    dense, _ = orc.dsa(ob, k)
    for r in rows:
        if r["method"] == "MISA":
            sel = orc.misa(ob, r["B"], r["h"], k)["idx"]
        elif r["method"] == "MISA-dagger":
            sel = orc.misa_dagger(ob, r["B"], r["h"], r["kp"], k)["idx"]
        elif r["method"] == "HISA":
            sel = orc.hisa(ob, r["B"], r["kp"] // r["B"], k)["idx"]
        else:
            heads, _ = orc.route(ob, r["B"], r["h"])
            sel = orc.hisa(ob, r["B"], r["kp"] // r["B"], k, heads=heads)["idx"]
        orr, ori = fidelity.set_metrics(sel, dense)
        # a near-tie at the k-th boundary may swap one token of a row
        assert abs(r["recall"] - orr) <= 1.5 / k and abs(r["iou"] - ori) <= 3.0 / k, (r, orr, ori)
        full = r["kp"] >= L if r["method"] in ("MISA-dagger", "HISA") else False
        if (r["method"] in ("MISA", "MISA-dagger") and r["h"] == H) or full:
            assert r["recall"] == 1.0 and r["iou"] == 1.0, r


# ------------------------------------------------ hierarchical indexer (HISA)
HISA_CASES = [
    # S, Lmax, T, H, B, m
    (2, 3000, 6, 16, 64, 5),
    (3, 4133, 5, 64, 128, 3),
    (1, 2500, 9, 32, 16, 40),
    (2, 1000, 4, 8, 128, 1),
]


def _hisa_heads(case, T, H, h, seed):
    rng = np.random.default_rng(seed)
    return np.stack([rng.permutation(H)[:h] for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("S,Lmax,T,H,B,m", HISA_CASES)
@pytest.mark.parametrize("routed", [False, True])
def test_hisa_matches_oracle(S, Lmax, T, H, B, m, routed):
    """Block scores within fp32 accuracy of the oracle, the kept blocks the
    top-m of the GPU's own block scores and the oracle's (up to a near-tie),
    and the selected tokens the oracle's (up to swaps at the k-th score)."""
    abi = _abi()
    case = make(S, Lmax, T, H, Lmax % 13)
    b = upload(case)
    ob = orc.Batch.from_case(case)
    heads = _hisa_heads(case, T, H, min(4, H), Lmax) if routed else None
    th = torch.from_numpy(heads).cuda() if routed else None
    k = min(200, Lmax)
    pooled = abi.pool(b, B)
    gs, gb = abi.hisa_blocks(b, pooled, B, m, heads=th)
    gs, gb = np_(gs), np_(gb)
    gi, gv = abi.hisa_indexer(b, pooled, B, m, k, heads=th)
    gi, gv = np_(gi), np_(gv)
    o = orc.hisa(ob, B, m, k, heads=heads)
    osc = orc.scores(ob, heads)
    for t in range(T):
        M = int(case["q_pos"][t]) // B + 1
        ob_s = o["bscore"][t, :M]
        sb = float(np.mean(np.abs(ob_s))) + 1e-30
        assert np.all(np.abs(gs[t, :M] - ob_s) <= 1e-4 * (np.abs(ob_s) + sb)), t
        assert np.all(np.isneginf(gs[t, M:]))
        assert sorted(x for x in gb[t] if x >= 0) == sorted(x for x in orc.topk_f32(gs[t, :M], m) if x >= 0)
        same_blocks = set(gb[t]) == set(o["blocks"][t])
        if not same_blocks:
            assert parity.head_margin(ob_s, min(m, M)) < 1e-4, (t, gb[t], o["blocks"][t])
            continue
        # the refinement: the tokens of the kept blocks, ranked by the indexer
        n = int(case["q_pos"][t]) + 1
        allowed = np.zeros(n, bool)
        for blk in gb[t]:
            if blk >= 0:
                allowed[blk * B:min(blk * B + B, n)] = True
        assert all(allowed[i] for i in gi[t] if i >= 0)
        nc = int(allowed.sum())
        masked = np.where(allowed, osc[t, :n], -np.inf)
        parity.check_set(gi[t], o["idx"][t], lambda i: masked[i], nc, k, parity.row_sbar(osc[t], n))
        for i, v in zip(gi[t], gv[t]):
            if i >= 0:
                assert abs(v - osc[t, i]) <= parity.REL * (abs(osc[t, i]) + parity.row_sbar(osc[t], n))


@pytest.mark.parametrize("S,Lmax,T,H,B,m", HISA_CASES[:3])
def test_hisa_keeping_every_block_is_the_dense_indexer(S, Lmax, T, H, B, m):
    abi = _abi()
    case = make(S, Lmax, T, H, 3)
    b = upload(case)
    pooled = abi.pool(b, B)
    M = (Lmax + B - 1) // B
    k = min(300, Lmax)
    gi, _ = abi.hisa_indexer(b, pooled, B, M, k)
    di, _ = abi.indexer_dense(b, k)
    assert [set(r) for r in np_(gi)] == [set(r) for r in np_(di)]


def test_hisa_integer_inputs_bit_exact():
    """Integer q, keys and w with unit blocks: every block and token score is
    an exact integer on both sides, so blocks, ties and tokens match the
    oracle exactly, for all heads and for routed heads."""
    abi = _abi()
    S, Lmax, T, H = 2, 700, 5, 16
    case = synth.random_case(S, Lmax, T, H, seed=4, dist="int")
    b = upload(case)
    ob = orc.Batch.from_case(case)
    pooled = abi.pool(b, 1)
    for heads in (None, _hisa_heads(case, T, H, 3, 1)):
        th = torch.from_numpy(heads).cuda() if heads is not None else None
        for m, k in ((40, 30), (7, 20)):
            gs, gb = abi.hisa_blocks(b, pooled, 1, m, heads=th)
            gi, gv = abi.hisa_indexer(b, pooled, 1, m, k, heads=th)
            o = orc.hisa(ob, 1, m, k, heads=heads)
            gs, gb, gi, gv = np_(gs), np_(gb), np_(gi), np_(gv)
            for t in range(T):
                n = int(case["q_pos"][t]) + 1
                assert np.array_equal(gs[t, :n].astype(np.float64), o["bscore"][t, :n])
                assert set(gb[t]) == set(o["blocks"][t])
                assert set(gi[t]) == set(o["idx"][t])


# --------------------------------------------------------------------- rerank
@pytest.mark.parametrize("S,Lmax,T,H,seed", CASES[:4])
def test_rerank(S, Lmax, T, H, seed):
    abi = _abi()
    case = make(S, Lmax, T, H, seed)
    b = upload(case)
    ob = orc.Batch.from_case(case)
    B, h, kc, k = 16, min(8, H), min(300, Lmax), min(100, Lmax)
    od = orc.misa_dagger(ob, B, h, kc, k)
    cand = od["cand"].copy()
    # punch a few empty slots into the candidate lists
    cand[:, ::7] = -1
    idx, val = abi.rerank(b, torch.from_numpy(cand).cuda(), k)
    idx, val = np_(idx), np_(val)
    oidx, _ = orc.rerank(ob, cand, k)
    full = orc.scores(ob)
    for t in range(T):
        nv = int((cand[t] >= 0).sum())
        sb = parity.row_sbar(full[t], int(n_valid(case)[t]))
        parity.check_set(idx[t], oidx[t], lambda i: full[t, i], nv, k, sb)
        for i, v in zip(idx[t], val[t]):
            if i >= 0:
                assert abs(v - full[t, i]) <= parity.REL * (abs(full[t, i]) + sb)
                assert i in set(cand[t])


# ------------------------------------------------ exact-arithmetic end to end
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_integer_inputs_bit_exact(seed):
    """Small-integer q, k, w: every product and sum is an exact integer in
    bf16, fp32 and fp64, so scores, ties, router importances (B=1), routed
    heads and selected sets must equal the oracle bit for bit."""
    abi = _abi()
    S, Lmax, T, H = 2, 700, 6, 16
    case = make(S, Lmax, T, H, seed, dist="int")
    b = upload(case)
    ob = orc.Batch.from_case(case)
    sc = np_(abi.score(b))
    osc = orc.scores(ob)
    for t in range(T):
        n = int(n_valid(case)[t])
        assert np.array_equal(sc[t, :n].astype(np.float64), osc[t, :n])
    for k in (1, 50, 333):
        idx, _ = abi.indexer_dense(b, k)
        oidx, _ = orc.dsa(ob, k)
        assert [set(r) for r in np_(idx)] == [set(r) for r in oidx]
    pooled = abi.pool(b, 1)
    for mode in (0, 1):
        heads, g = abi.route(b, pooled, 1, 4, mode, want_score=True)
        oheads, og = orc.route(ob, 1, 4, mode)
        assert np.array_equal(np_(g).astype(np.float64), og)
        assert np.array_equal(np_(heads), oheads)
    heads = abi.route(b, pooled, 1, 4, 0)
    idx, _ = abi.score_topk(b, heads, 77)
    om = orc.misa(ob, 1, 4, 77)
    assert [set(r) for r in np_(idx)] == [set(r) for r in om["idx"]]
    cand, _ = abi.score_topk(b, heads, 200)
    fin, _ = abi.rerank(b, cand, 77)
    od = orc.misa_dagger(ob, 1, 4, 200, 77)
    assert [set(r) for r in np_(fin)] == [set(r) for r in od["idx"]]


def test_hand_worked_example_on_gpu():
    """The golden example, zero-padded from d=2 to d=128."""
    abi = _abi()
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_example.json")))
    L = len(g["keys"])
    keys = np.zeros((1, L, 128), np.float32)
    keys[0, :, :2] = g["keys"]
    qs = np.zeros((2, 2, 128), np.float32)
    qs[:, :, :2] = [e["q"] for e in g["queries"]]
    case = dict(keys=synth.to_bf16_bits(keys), seq_lens=np.array([L], np.int32),
                q=synth.to_bf16_bits(qs), w=np.array([e["w"] for e in g["queries"]], np.float32),
                q_seq=np.zeros(2, np.int32), q_pos=np.array([e["p"] for e in g["queries"]], np.int32))
    b = upload(case)
    sc = np_(abi.score(b))
    for t, e in enumerate(g["queries"]):
        assert list(sc[t, :e["p"] + 1]) == e["dsa_scores"]
    idx, _ = abi.indexer_dense(b, 2)
    assert [set(r) for r in np_(idx)] == [set(e["dsa_top2"]) for e in g["queries"]]
    pooled = abi.pool(b, g["B"])
    for mode in (0, 1):
        heads, gg = abi.route(b, pooled, g["B"], 1, mode, want_score=True)
        assert [list(r) for r in np_(heads)] == [e["heads_h1_mode%d" % mode] for e in g["queries"]]
        assert [list(r) for r in np_(gg)] == [e["g_mode%d" % mode] for e in g["queries"]]
    heads = abi.route(b, pooled, g["B"], 1, 0)
    idx, _ = abi.score_topk(b, heads, 2)
    assert [set(r) for r in np_(idx)] == [set(e["misa_h1_mode0_top2"]) for e in g["queries"]]
    cand, _ = abi.score_topk(b, heads, 3)
    assert [set(r) for r in np_(cand)] == [set(e["dagger_h1_kc3_cand"]) for e in g["queries"]]
    fin, _ = abi.rerank(b, cand, 2)
    assert [set(r) for r in np_(fin)] == [set(e["dagger_h1_kc3_top2"]) for e in g["queries"]]


# ------------------------------------------------------------- GPU invariants
@pytest.mark.parametrize("seed", [0, 1])
def test_gpu_invariants(seed):
    """MISA with h = H (heads in id order) is the dense indexer bit for bit;
    MISA-dagger with k' covering every prefix is the dense indexer."""
    abi = _abi()
    case = make(2, 3000, 5, 32, seed)
    b = upload(case)
    k = 128
    dense, dval = abi.indexer_dense(b, k)
    allh = torch.arange(32, dtype=torch.int32, device="cuda").repeat(5, 1).contiguous()
    m, mval = abi.score_topk(b, allh, k)
    assert [set(r) for r in np_(dense)] == [set(r) for r in np_(m)]
    assert np.array_equal(np.sort(np_(dval), 1), np.sort(np_(mval), 1))
    pooled = abi.pool(b, 64)
    heads = abi.route(b, pooled, 64, 4, 0)
    cand, _ = abi.score_topk(b, heads, 3000)
    fin, _ = abi.rerank(b, cand, k)
    assert [set(r) for r in np_(dense)] == [set(r) for r in np_(fin)]


# ------------------------------------------------------------ fused indexer
# (H = 128: the fused scoring prologue reads the routed query rows from
# memory instead of staging the row's heads in LDS)
@pytest.mark.parametrize("S,Lmax,T,H,seed", CASES[:4] + [CASES[5]])
@pytest.mark.parametrize("mode", [0, 1])
def test_indexer_fused_equals_separate_calls(S, Lmax, T, H, seed, mode):
    """misa_indexer = misa_route then misa_score_topk, bit for bit; its
    selection also passes the oracle comparison."""
    abi = _abi()
    case = make(S, Lmax, T, H, seed)
    b = upload(case)
    B, h, k = 64, min(8, H), min(300, Lmax)
    pooled = abi.pool(b, B)
    heads_sep = abi.route(b, pooled, B, h, mode)
    idx_sep, val_sep = abi.score_topk(b, heads_sep, k)
    for rep in range(2):  # the workspace holds the previous call's contents the second time
        ws = b.workspace(abi.MISA_OP_INDEXER, B=B, h=h, k=k)
        heads, idx, val = abi.indexer(b, pooled, B, h, k, mode=mode, ws=ws)
        assert np.array_equal(np_(heads), np_(heads_sep))
        gi, gv = np_(idx), np_(val)
        si, sv = np_(idx_sep), np_(val_sep)
        for t in range(T):
            assert set(gi[t]) == set(si[t])
            assert np.array_equal(np.sort(gv[t]), np.sort(sv[t]))
    ob = orc.Batch.from_case(case)
    om = orc.misa(ob, B, h, k, mode=mode, want_scores=True)
    for t in range(T):
        n = int(n_valid(case)[t])
        if sorted(gi[t]) != sorted(om["idx"][t]):
            parity.check_set(gi[t], om["idx"][t], lambda i: om["scores"][t, i], n, k,
                             parity.row_sbar(om["scores"][t], n))


def test_indexer_many_decode_rows_take_the_streamed_select():
    """Per-row decode scoring of 256 query rows over two sequences, prefixes
    of 16384..20000 keys: the fused call scores the rows and selects them
    with the streamed select (rows at or past 16384 columns); heads and
    selections match the oracle for every row."""
    abi = _abi()
    S, Lmax, T, H = 2, 20000, 256, 16
    rng = np.random.default_rng(77)
    q_seq = np.repeat(np.arange(S, dtype=np.int32), T // S)
    q_pos = rng.integers(16383, Lmax, size=T).astype(np.int32)
    q_pos[:4] = [16383, 16384, Lmax - 1, 16390]
    case = synth.random_case(S, Lmax, T, H, seed=13, q_pos=q_pos, q_seq=q_seq)
    b = upload(case)
    B, h, k = 128, 4, 300
    pooled = abi.pool(b, B)
    heads, idx, val = abi.indexer(b, pooled, B, h, k)
    heads, idx, val = np_(heads), np_(idx), np_(val)
    om = orc.misa(orc.Batch.from_case(case), B, h, k, want_scores=True)
    checked = 0
    for t in range(T):
        if set(heads[t]) != set(om["heads"][t]):
            assert parity.head_margin(om["g"][t], h) < 1e-4, t
            continue
        n = int(q_pos[t]) + 1
        sb = parity.row_sbar(om["scores"][t], n)
        parity.check_set(idx[t], om["idx"][t], lambda i: om["scores"][t, i], n, k, sb)
        for i, v in zip(idx[t], val[t]):
            assert abs(float(v) - om["scores"][t, i]) <= parity.REL * (abs(om["scores"][t, i]) + sb)
        checked += 1
    assert checked >= T - 4


# ------------------------------------------------------- prefill tiling path
PREFILL_CASES = [
    # Lmax, T, H, h, positions
    (3000, 200, 32, 8, "tail"),
    (1100, 97, 8, 3, "random"),
    (2500, 130, 32, 16, "random"),
    (700, 64, 16, 1, "tail"),
    (4200, 256, 64, 8, "tail"),
    # whole query tiles and key tiles only (no ragged workgroup)
    (4096, 128, 32, 8, "tail"),
    (2048, 128, 16, 4, "random"),
    (2560, 256, 8, 2, "tail"),
    # ragged only in the keys, or only in the queries
    (3000, 128, 32, 8, "tail"),
    (2048, 100, 32, 4, "tail"),
    # wide head sets: a tile per query (h <= 32) or two (h <= 64)
    (3000, 100, 64, 24, "random"),
    (2100, 80, 32, 32, "tail"),
    (2600, 72, 64, 40, "tail"),
    (2048, 64, 64, 64, "random"),
]


def make_prefill(Lmax, T, H, seed, positions):
    rng = np.random.default_rng(seed + 5)
    if positions == "tail":
        q_pos = np.arange(Lmax - T, Lmax, dtype=np.int32)
    else:
        q_pos = np.sort(rng.integers(0, Lmax, size=T)).astype(np.int32)
    return synth.random_case(1, Lmax, T, H, seed=seed, q_pos=q_pos,
                             q_seq=np.zeros(T, np.int32))


@pytest.mark.parametrize("Lmax,T,H,h,positions", PREFILL_CASES)
def test_prefill_scores_and_selection(Lmax, T, H, h, positions):
    """Many queries of one sequence with h <= 16 routed heads take the
    32x32 MFMA tiling; scores, selections and the fused call all match the
    oracle."""
    abi = _abi()
    case = make_prefill(Lmax, T, H, 11, positions)
    b = upload(case)
    ob = orc.Batch.from_case(case)
    rng = np.random.default_rng(Lmax + T)
    heads = np.stack([rng.permutation(H)[:h] for _ in range(T)]).astype(np.int32)
    th = torch.from_numpy(heads).cuda()
    got = np_(abi.score(b, th))
    osc = orc.scores(ob, heads)
    parity.check_scores(got, osc, n_valid(case))
    k = min(257, Lmax)
    idx, val = abi.score_topk(b, th, k)
    idx, val = np_(idx), np_(val)
    oidx = np.stack([orc.topk(osc[t, :n_valid(case)[t]], k)[0] for t in range(T)])
    for t in range(T):
        n = int(n_valid(case)[t])
        parity.check_exact_topk(idx[t], val[t], got[t], n, k, orc.topk_f32)
        parity.check_set(idx[t], oidx[t], lambda i: osc[t, i], n, k, parity.row_sbar(osc[t], n))
    # the fused call routes first; compare with route + score_topk
    B = 64
    pooled = abi.pool(b, B)
    rh = abi.route(b, pooled, B, h, 0)
    ri, rv = abi.score_topk(b, rh, k)
    fh, fi, fv = abi.indexer(b, pooled, B, h, k)
    assert np.array_equal(np_(fh), np_(rh))
    assert [set(r) for r in np_(fi)] == [set(r) for r in np_(ri)]


DENSE_PREFILL_CASES = [
    # Lmax, T, H, positions
    (3000, 200, 32, "tail"),
    (2500, 130, 64, "random"),
    (4096, 128, 64, "tail"),   # whole query and key tiles
    (1800, 96, 16, "tail"),
    (2200, 70, 48, "random"),
]


@pytest.mark.parametrize("Lmax,T,H,positions", DENSE_PREFILL_CASES)
def test_prefill_dense_all_heads(Lmax, T, H, positions):
    """The dense indexer (every head, no routing) on a prefill chunk takes
    the MFMA tiling too (up to 64 heads a query): scores and selections
    match the oracle's DSA indexer."""
    abi = _abi()
    case = make_prefill(Lmax, T, H, 23, positions)
    b = upload(case)
    ob = orc.Batch.from_case(case)
    got = np_(abi.score(b, None))
    osc = orc.scores(ob)
    parity.check_scores(got, osc, n_valid(case))
    k = min(300, Lmax)
    idx, val = abi.indexer_dense(b, k)
    idx, val = np_(idx), np_(val)
    for t in range(T):
        n = int(n_valid(case)[t])
        parity.check_exact_topk(idx[t], val[t], got[t], n, k, orc.topk_f32)
        oidx = orc.topk(osc[t, :n], k)[0]
        parity.check_set(idx[t], oidx, lambda i: osc[t, i], n, k, parity.row_sbar(osc[t], n))


def test_prefill_integer_inputs_bit_exact():
    abi = _abi()
    T, Lmax, H, h = 96, 1500, 16, 8
    q_pos = np.arange(Lmax - T, Lmax, dtype=np.int32)
    case = synth.random_case(1, Lmax, T, H, seed=3, dist="int", q_pos=q_pos,
                             q_seq=np.zeros(T, np.int32))
    b = upload(case)
    ob = orc.Batch.from_case(case)
    rng = np.random.default_rng(9)
    heads = np.stack([rng.permutation(H)[:h] for _ in range(T)]).astype(np.int32)
    th = torch.from_numpy(heads).cuda()
    got = np_(abi.score(b, th))
    osc = orc.scores(ob, heads)
    for t in range(T):
        n = int(q_pos[t]) + 1
        assert np.array_equal(got[t, :n].astype(np.float64), osc[t, :n])
        assert np.all(np.isneginf(got[t, n:]))
    idx, _ = abi.score_topk(b, th, 300)
    oidx = np.stack([orc.topk(osc[t, :q_pos[t] + 1], 300)[0] for t in range(T)])
    assert [set(r) for r in np_(idx)] == [set(r) for r in oidx]


# ------------------------------------------------- multi-query decode (S > 1)
GROUPED_CASES = [
    # S, Lmax, Q (queries per sequence), H, h (None: dense), layout
    (4, 3000, 2, 32, 8, "grouped"),
    (6, 2500, 4, 64, 8, "grouped"),
    (4, 4096, 8, 64, None, "grouped"),
    (5, 2200, 8, 32, 24, "grouped"),
    (8, 1800, 3, 16, None, "grouped"),
    (4, 2600, 4, 64, 8, "interleaved"),   # rows of a sequence not contiguous
]


def make_grouped(S, Lmax, Q, H, seed, layout):
    rng = np.random.default_rng(seed + 11)
    seq_lens = rng.integers(max(Q, Lmax // 3), Lmax + 1, size=S).astype(np.int32)
    seq_lens[0] = Lmax
    q_seq = np.repeat(np.arange(S, dtype=np.int32), Q)
    if layout == "interleaved":
        q_seq = np.tile(np.arange(S, dtype=np.int32), Q)
    # the sequence's last Q positions (draft tokens after its cache), in order
    j = np.zeros(S, np.int32)
    q_pos = np.empty(S * Q, np.int32)
    for t, s in enumerate(q_seq):
        q_pos[t] = seq_lens[s] - Q + j[s]
        j[s] += 1
    return synth.random_case(S, Lmax, S * Q, H, seed=seed, seq_lens=seq_lens, q_seq=q_seq, q_pos=q_pos)


@pytest.mark.parametrize("S,Lmax,Q,H,h,layout", GROUPED_CASES)
def test_multi_query_decode_shares_the_key_stream(S, Lmax, Q, H, h, layout):
    """Several query rows per sequence (S > 1) take the MFMA tiling over a
    tile table built on the device (routed or dense heads); rows of a
    sequence that are not contiguous are each scored on their own.  Either
    way the selections are the oracle's, and the fused call equals route +
    score_topk."""
    abi = _abi()
    case = make_grouped(S, Lmax, Q, H, 5 + S * Q, layout)
    T = S * Q
    b = upload(case)
    ob = orc.Batch.from_case(case)
    rng = np.random.default_rng(T + H)
    heads = None if h is None else np.stack([rng.permutation(H)[:h] for _ in range(T)]).astype(np.int32)
    th = None if heads is None else torch.from_numpy(heads).cuda()
    k = min(250, Lmax // 4)
    idx, val = abi.score_topk(b, th, k)
    idx, val = np_(idx), np_(val)
    osc = orc.scores(ob, heads)
    for t in range(T):
        n = int(n_valid(case)[t])
        sb = parity.row_sbar(osc[t], n)
        parity.check_set(idx[t], orc.topk(osc[t, :n], k)[0], lambda i: osc[t, i], n, k, sb)
        for i, v in zip(idx[t], val[t]):
            if i >= 0:
                assert abs(float(v) - osc[t, i]) <= parity.REL * (abs(osc[t, i]) + sb)
    if h is not None:
        B = 64
        pooled = abi.pool(b, B)
        rh = abi.route(b, pooled, B, h, 0)
        ri, _ = abi.score_topk(b, rh, k)
        fh, fi, _ = abi.indexer(b, pooled, B, h, k)
        assert np.array_equal(np_(fh), np_(rh))
        assert [set(r) for r in np_(fi)] == [set(r) for r in np_(ri)]
