"""Comparison rules between the GPU path and the CPU oracle.

Tolerance (bf16 inputs, fp32 accumulation on the GPU, fp64 in the oracle):
a GPU score s_gpu of token i in query row t must satisfy
    |s_gpu - s_orc| <= REL * (|s_orc| + sbar_t),
where sbar_t is the mean |score| over the row's prefix (a pure relative test
is meaningless at the exact zeros a ReLU produces).  A selected set G may
differ from the oracle's O only by swaps across the k-th boundary: with
tau = the oracle's k-th score and tol = REL * (|tau| + sbar_t), every
x in G\\O has s_orc(x) >= tau - tol and every y in O\\G has s_orc(y) <= tau + tol.
Integer decisions taken on the GPU's own fp32 values (top-k, top-h) must
match the oracle's ranking applied to those same values exactly.
"""
import numpy as np

REL = 1e-2


def row_sbar(orc_row, n):
    v = orc_row[:n]
    return float(np.mean(np.abs(v))) if n else 0.0


def check_scores(gpu, orc, n_valid, rel=REL):
    """gpu fp32 [T][L], orc fp64 [T][L]; columns >= n_valid[t] must be -inf."""
    worst = 0.0
    for t in range(gpu.shape[0]):
        n = int(n_valid[t])
        g = gpu[t, :n].astype(np.float64)
        o = orc[t, :n]
        sb = row_sbar(orc[t], n)
        err = np.abs(g - o)
        lim = rel * (np.abs(o) + sb)
        bad = np.nonzero(err > lim)[0]
        assert bad.size == 0, "row %d: %d scores off, first col %d gpu %r orc %r" % (
            t, bad.size, bad[0], g[bad[0]], o[bad[0]])
        if n:
            worst = max(worst, float(np.max(err / np.maximum(np.abs(o) + sb, 1e-300))))
        assert np.all(np.isneginf(gpu[t, n:])), "row %d: columns past the prefix not -inf" % t
    return worst


def check_set(gpu_idx, orc_idx, orc_score_of, n, k, sbar, rel=REL):
    """One row.  orc_score_of(i) -> oracle fp64 score of token i.  Returns the
    number of boundary swaps (0 when the sets are identical)."""
    m = min(k, n)
    g = [int(x) for x in gpu_idx]
    o = [int(x) for x in orc_idx]
    G = set(x for x in g if x >= 0)
    O = set(x for x in o if x >= 0)
    assert len(G) == m and len(O) == m, "set sizes %d/%d, expected %d" % (len(G), len(O), m)
    assert sum(1 for x in g if x >= 0) == m, "duplicate ids in the GPU set"
    assert all(x == -1 for x in g if x < 0)
    if G == O:
        return 0
    tau = orc_score_of(o[m - 1])
    tol = rel * (abs(tau) + sbar)
    for x in G - O:
        assert orc_score_of(x) >= tau - tol, "token %d (%r) selected, k-th %r" % (x, orc_score_of(x), tau)
    for y in O - G:
        assert orc_score_of(y) <= tau + tol, "token %d (%r) dropped, k-th %r" % (y, orc_score_of(y), tau)
    return len(G - O)


def check_exact_topk(gpu_idx, gpu_val, scores_f32_row, n, k, topk_f32):
    """The GPU's selection equals the oracle ranking taken on the GPU's own
    fp32 scores, as a set, and the reported values are those scores."""
    ref = topk_f32(scores_f32_row[:n], k)
    assert set(int(x) for x in gpu_idx) == set(int(x) for x in ref)
    if gpu_val is not None:
        for i, v in zip(gpu_idx, gpu_val):
            if i < 0:
                assert np.isneginf(v)
            else:
                assert v == scores_f32_row[i]  # -0.0 == +0.0 here


def head_margin(g_row, h):
    """Relative gap between the h-th and (h+1)-th router importances."""
    s = np.sort(np.asarray(g_row, np.float64))[::-1]
    if h >= s.size:
        return np.inf
    return float((s[h - 1] - s[h]) / max(np.max(np.abs(s)), 1e-300))
