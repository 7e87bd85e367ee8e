"""The entry points enqueue kernels only (no allocation, no memset node, no
host synchronisation), so a caller may capture them in a graph.  Each case
captures one call sequence, replays the graph several times with eager
library work and synchronisations between the replays, and checks every
replay against the eager result (selected sets: the order inside a row is
unspecified)."""
import ctypes

import numpy as np
import pytest

from long_context_sparse_05_amd import synth

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


def _sets(t):
    torch.cuda.synchronize()
    return [set(int(x) for x in row) for row in t.cpu().numpy()]


def _replay_and_check(capture, outputs, eager, disturb, reps=4):
    """capture(): the call sequence; outputs: tensors it writes; eager: the
    expected sets per output; disturb(): eager library work between replays."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        capture()  # warm-up on the side stream, outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        capture()
    for rep in range(reps):
        for o in outputs:
            o.fill_(-7)  # stale values must be overwritten by the replay
        g.replay()
        torch.cuda.synchronize()
        for o, want in zip(outputs, eager):
            assert _sets(o) == want, "replay %d differs from the eager call" % rep
        disturb()
        torch.cuda.synchronize()


def test_graph_fused_decode_indexer():
    """Router (partial + final, which clears the select workspace),
    routed scoring with the histogram epilogue, filter and finish."""
    abi = _abi()
    case = synth.random_case(3, 5000, 3, 16, seed=21)
    b = abi.Batch.from_numpy(case)
    B, h, k = 64, 4, 300
    pooled = abi.pool(b, B)
    ws = b.workspace(abi.MISA_OP_INDEXER, B=B, h=h, k=k)
    heads = torch.empty((b.T, h), dtype=torch.int32, device="cuda")
    idx = torch.empty((b.T, k), dtype=torch.int32, device="cuda")
    val = torch.empty((b.T, k), dtype=torch.float32, device="cuda")
    eh, ei, _ = abi.indexer(b, pooled, B, h, k)
    eager = [_sets(eh), _sets(ei)]
    other = synth.random_case(2, 3000, 2, 16, seed=5)
    ob = abi.Batch.from_numpy(other)

    def capture():
        abi.indexer(b, pooled, B, h, k, heads=heads, idx=idx, val=val, ws=ws)

    def disturb():
        abi.score_topk(ob, None, 100)  # eager work on its own workspace

    _replay_and_check(capture, [heads, idx], eager, disturb)


def test_graph_separate_calls_and_many_row_select():
    """misa_score_topk (the select workspace cleared by a fill kernel) and
    misa_topk over enough long rows to take the streamed select."""
    abi = _abi()
    case = synth.random_case(2, 4000, 4, 16, seed=9)
    b = abi.Batch.from_numpy(case)
    k = 200
    ws = b.workspace(abi.MISA_OP_SCORE_TOPK, h=16, k=k)
    idx = torch.empty((b.T, k), dtype=torch.int32, device="cuda")
    val = torch.empty((b.T, k), dtype=torch.float32, device="cuda")
    ei, _ = abi.score_topk(b, None, k)
    rows, ld, kt = 300, 16384, 512
    rng = np.random.default_rng(3)
    sc = torch.from_numpy(rng.standard_normal((rows, ld)).astype(np.float32)).cuda()
    rl = torch.from_numpy(rng.integers(kt, ld + 1, size=rows).astype(np.int32)).cuda()
    eti, _ = abi.topk(sc, rl, kt)
    shape = abi.MisaBatch(1, 0, 0, 0, 0, 0, 1, ld, 128, rows, 1)
    n = abi._SZ(0)
    abi.load().misa_workspace_bytes(ctypes.byref(shape), abi.MISA_OP_TOPK, 1, 1, kt, 1, ctypes.byref(n))
    tws = torch.empty(n.value, dtype=torch.uint8, device="cuda")
    tidx = torch.empty((rows, kt), dtype=torch.int32, device="cuda")
    tval = torch.empty((rows, kt), dtype=torch.float32, device="cuda")
    eager = [_sets(ei), _sets(eti)]

    def capture():
        abi.score_topk(b, None, k, idx=idx, val=val, ws=ws)
        abi.topk(sc, rl, kt, idx=tidx, val=tval, ws=tws)

    def disturb():
        abi.topk(sc[:8], rl[:8], 64)

    _replay_and_check(capture, [idx, tidx], eager, disturb)


def test_graph_prefill_chunk():
    """Many queries of one sequence: the tiled router, the 32x32 MFMA
    scoring and the one-workgroup-per-row select."""
    abi = _abi()
    T, L, H = 96, 3000, 16
    case = synth.random_case(1, L, T, H, seed=4, q_pos=np.arange(L - T, L, dtype=np.int32),
                             q_seq=np.zeros(T, np.int32))
    b = abi.Batch.from_numpy(case)
    B, h, k = 64, 8, 257
    pooled = abi.pool(b, B)
    ws = b.workspace(abi.MISA_OP_INDEXER, B=B, h=h, k=k)
    heads = torch.empty((T, h), dtype=torch.int32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    val = torch.empty((T, k), dtype=torch.float32, device="cuda")
    eh, ei, _ = abi.indexer(b, pooled, B, h, k)
    eager = [_sets(eh), _sets(ei)]

    def capture():
        abi.indexer(b, pooled, B, h, k, heads=heads, idx=idx, val=val, ws=ws)

    def disturb():
        abi.indexer(b, pooled, B, h, 64)

    _replay_and_check(capture, [heads, idx], eager, disturb)
