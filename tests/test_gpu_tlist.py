"""The prefill chunk's select from threshold lists (many long rows, a few
routed heads per query): the scores of keys sampled evenly over the shortest
prefix give each row a lower bound tau of its k-th score, the scoring kernel
lists every score >= tau (and writes no score rows), and the top-k is taken
from those lists; a row whose lists cannot prove its top-k (fewer than k
entries reach tau, a list overflowed) is rescored on its own and takes the
row select.

Parity on every row: a row settled from its lists selects exactly the top-k
of the score matrix misa_score computes (the same MFMA tiling, so the same
fp32 scores) and reports those scores; a rescored row matches it up to swaps
at the k-th score within the score tolerance; on sampled rows the selection
is the oracle's (parity.py).  Inputs built to defeat the sample -- the
sampled keys scoring far above the rest for half the rows, or scoring zero
for all -- drive those rows through the fallback, and the per-row flags the
merge leaves in the workspace confirm which path each row took."""
import numpy as np
import pytest

from oracle import oracle as orc
from long_context_sparse_05_amd import synth
import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

NS = 2048           # sampled keys (tlist.hip): positions floor(j n / NS), n = shortest prefix
ROW_COUNTERS = 8    # per-row counters after the score rows; counter 7 = the row's flag


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


def _align(x):
    return (x + 255) // 256 * 256


def _sampled_positions(q_pos, Lmax):
    n = int(min(max(int(q_pos.min()) + 1, 1), Lmax))
    return (np.arange(NS, dtype=np.int64) * n) // NS


def _case(Lmax, T, H, seed, positions, structure):
    rng = np.random.default_rng(seed + 3)
    if positions == "tail":
        q_pos = np.arange(Lmax - T, Lmax, dtype=np.int32)
    elif positions == "spread":  # short rows (n < k: every score listed), medium rows (lists overflow), long rows
        q_pos = np.sort(rng.integers(0, Lmax, size=T)).astype(np.int32)
    else:
        q_pos = np.sort(rng.integers(Lmax // 2, Lmax, size=T)).astype(np.int32)
    case = synth.random_case(1, Lmax, T, H, seed=seed, q_pos=q_pos, q_seq=np.zeros(T, np.int32))
    if structure == "plain":
        return case
    keys = synth.bf16_bits_to_f32(case["keys"]).copy()
    sp = np.unique(_sampled_positions(q_pos, Lmax))
    if structure == "sample_zero":  # every sampled key scores 0: tau = 0, the lists overflow
        keys[0, sp] = 0.0
        case["keys"] = synth.to_bf16_bits(keys)
        return case
    assert structure == "sample_high"
    # the sampled keys get a shared direction v; even rows' queries point
    # along it (their sampled scores tower over the rest: fewer than k scores
    # reach tau), odd rows' queries are orthogonal to it (ordinary rows)
    v = rng.standard_normal(keys.shape[-1]).astype(np.float32)
    v /= np.linalg.norm(v)
    keys[0, sp] += 3.0 * v
    q = synth.bf16_bits_to_f32(case["q"]).copy()
    q[0::2] += 2.0 * v
    q[1::2] -= (q[1::2] @ v)[..., None] * v
    case["keys"] = synth.to_bf16_bits(keys)
    case["q"] = synth.to_bf16_bits(q)
    case["w"] = np.abs(case["w"]).astype(np.float32)
    return case


TLIST_CASES = [
    # Lmax, T, H, h, k, positions, structure
    (32768, 1024, 16, 8, 512, "tail", "plain"),
    (30001, 1000, 16, 5, 300, "random", "plain"),     # ragged keys and queries, h < the tile's slots
    (20000, 2048, 8, 6, 128, "tail", "plain"),
    (24576, 1024, 32, 16, 1024, "tail", "plain"),
    (49152, 2048, 16, 8, 2500, "tail", "plain"),     # k past the merge's LDS staging: written directly
    (32768, 1024, 16, 8, 512, "spread", "plain"),     # prefixes from 1 key to the whole sequence
    (32768, 1024, 16, 8, 512, "tail", "sample_high"),
    (24000, 1024, 16, 8, 256, "tail", "sample_zero"),
]


@pytest.mark.parametrize("Lmax,T,H,h,k,positions,structure", TLIST_CASES)
def test_prefill_threshold_list_select(Lmax, T, H, h, k, positions, structure):
    abi = _abi()
    print("tlist case", Lmax, T, H, h, k, positions, structure, flush=True)
    case = _case(Lmax, T, H, 31 + h, positions, structure)
    b = abi.Batch.from_numpy(case)
    rng = np.random.default_rng(Lmax + T + h)
    heads = np.stack([rng.permutation(H)[:h] for _ in range(T)]).astype(np.int32)
    th = torch.from_numpy(heads).cuda()
    # the list path needs its own workspace: more than the score rows and counters alone
    wsz = b.workspace_bytes(abi.MISA_OP_SCORE_TOPK, h=h, k=k)
    base = _align(T * Lmax * 4) + _align(T * ROW_COUNTERS * 4)
    assert wsz > base, "the threshold-list select is not taken for this shape"
    ws = torch.empty(wsz, dtype=torch.uint8, device="cuda")
    idx, val = abi.score_topk(b, th, k, ws=ws)
    idx, val = np_(idx), np_(val)
    off = _align(T * Lmax * 4)
    flags = np_(ws[off:off + T * ROW_COUNTERS * 4]).view(np.uint32).reshape(T, ROW_COUNTERS)[:, 7]
    assert set(np.unique(flags)) <= {0, 1}
    sc = np_(abi.score(b, th))  # the full score matrix of the same tiling
    n_valid = np.minimum(case["q_pos"].astype(np.int64) + 1, Lmax)
    for t in range(T):
        n = int(n_valid[t])
        if flags[t] == 0:
            parity.check_exact_topk(idx[t], val[t], sc[t], n, k, orc.topk_f32)
        else:
            sb = parity.row_sbar(sc[t], n)
            parity.check_set(idx[t], orc.topk_f32(sc[t, :n], k), lambda i: float(sc[t, i]), n, k, sb)
            for i, v in zip(idx[t], val[t]):
                if i >= 0:
                    assert abs(float(v) - sc[t, i]) <= parity.REL * (abs(float(sc[t, i])) + sb)
    if structure == "plain" and positions == "spread":
        # rows too short for the sample to bound (r >= NS: tau = -inf, among
        # them every row with at most k keys) go to the rescoring.  The
        # sample spans only the shortest prefix (a few keys here), so a long
        # row's tau may miss too and take the rescoring (every row was
        # checked above); most long rows are still settled by their lists
        m = k * NS / n_valid.astype(np.float64)
        short = np.ceil(m + 4.0 * np.sqrt(m) + 8.0) >= NS
        assert short.any() and np.all(flags[short] == 1)
        assert flags[n_valid >= Lmax // 2].mean() <= 0.25
    elif structure == "plain":
        # every row is settled by its lists (ties at the k-th score -- the
        # exact zeros of rows whose weights are all negative -- included)
        assert flags.mean() <= 0.01, flags.mean()
    elif structure == "sample_zero":
        # tau = 0: a row with more positive scores than the merge holds
        # (8192) cannot be settled from its lists; rows with mostly negative
        # weights have few and may be
        big = np.array([(sc[t, :n_valid[t]] > 0).sum() > 8192 for t in range(T)])
        assert big.mean() >= 0.5 and np.all(flags[big] == 1), (big.mean(), flags[big].mean())
    else:
        assert flags[0::2].mean() >= 0.9, flags[0::2].mean()
        assert flags[1::2].mean() <= 0.05, flags[1::2].mean()
    # sampled rows against the oracle: both ends, flagged and settled rows
    rows = set(range(8)) | set(range(T - 8, T))
    rows |= set(int(r) for r in np.flatnonzero(flags)[:8]) | set(int(r) for r in np.flatnonzero(flags == 0)[:8])
    rows |= set(int(r) for r in rng.choice(T, 8, replace=False))
    rows = sorted(rows)
    sub = dict(case)
    for key in ("q", "w", "q_seq", "q_pos"):
        sub[key] = np.ascontiguousarray(case[key][rows])
    osc = orc.scores(orc.Batch.from_case(sub), heads[rows])
    for j, t in enumerate(rows):
        n = int(n_valid[t])
        sb = parity.row_sbar(osc[j], n)
        oidx = orc.topk(osc[j, :n], k)[0]
        parity.check_set(idx[t], oidx, lambda i: osc[j, i], n, k, sb)
        for i, v in zip(idx[t], val[t]):
            if i >= 0:
                assert abs(float(v) - osc[j, i]) <= parity.REL * (abs(osc[j, i]) + sb)


def test_threshold_list_select_in_the_fused_call():
    """misa_indexer on a prefill chunk routes, then takes the same list
    select: its selection equals route + score_topk's."""
    abi = _abi()
    Lmax, T, H, h, k = 32768, 1024, 16, 8, 512
    case = _case(Lmax, T, H, 5, "tail", "plain")
    b = abi.Batch.from_numpy(case)
    pooled = abi.pool(b, 64)
    rh = abi.route(b, pooled, 64, h, 0)
    ri, _ = abi.score_topk(b, rh, k)
    fh, fi, _ = abi.indexer(b, pooled, 64, h, k)
    assert np.array_equal(np_(fh), np_(rh))
    assert [set(r) for r in np_(fi)] == [set(r) for r in np_(ri)]
