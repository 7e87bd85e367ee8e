"""Seeded synthetic inputs for the indexer (shared by the GPU path's tests,
the benchmark and the oracle's tests).

This module holds input construction only -- random draws, bf16 rounding and
needle planting -- and none of the indexer's arithmetic (no scoring, pooling,
routing or selection).  Both sides of every parity test read the same arrays
from here.

Shapes follow the pages' workloads: DeepSeek-V3.2-like indexers with
H_I = 64 heads and GLM-5-like ones with H_I = 32 ("MISA: Mixture of Indexer
Sparse Attention for Long-Context LLM Inference", Technical Summary,
Experimental Results), a 128K-token context and k' = 8192 candidates
(Hierarchical Variant).  Distributions: q, k ~ N(0, 1)/sqrt(d), w ~ N(0, 1/H),
drawn in fp32, then q and k rounded to bf16 (round to nearest even).

Layout of a case (a dict of numpy arrays):
  keys      uint16 [S][Lmax][d]   bf16 bits, one shared indexing key per token
  seq_lens  int32  [S]
  q         uint16 [T][H][d]      bf16 bits
  w         float32 [T][H]
  q_seq     int32  [T]            sequence of each query row
  q_pos     int32  [T]            position p; the prefix is tokens 0..p
"""
from __future__ import annotations

import numpy as np

D = 128


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest, ties to even (no NaN inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _streams(seed: int, n: int = 5):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def _normal_f32(rng, shape, scale):
    """N(0, scale^2) in fp32, drawn in chunks to bound host memory."""
    out = np.empty(shape, np.float32)
    flat = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat.size, step):
        e = min(flat.size, s + step)
        flat[s:e] = rng.standard_normal(e - s, dtype=np.float32)
    flat *= np.float32(scale)
    return out


def _unit(v):
    n = float(np.linalg.norm(v))
    return v / n if n > 0 else v


def decode_case(S, L, H, seed=0, n_needles=0, queries_per_seq=1, d=D,
                seq_lens=None, keep_f32_q=False):
    """S sequences of L keys, `queries_per_seq` queries at each sequence's last
    positions, i.i.d. q/k/w, plus `n_needles` planted keys per sequence.

    Needle recipe (a reading; the configs give no strength): for each sequence
    take its last query t*, draw 3 distinct heads J among those with
    w[t*, j] > 0, draw distinct positions uniformly in the shortest prefix of
    the sequence's queries, and add 1.0 * q[t*, J[i mod 3]] / |q[t*, J[i mod 3]]|
    to needle i's key (before bf16 rounding).  keep_f32_q: also return the
    queries as drawn, before bf16 rounding ("q_f32", float32 [T][H][d])."""
    r_q, r_k, r_w, r_pos, r_head = _streams(seed)
    if seq_lens is None:
        seq_lens = np.full(S, L, np.int32)
    seq_lens = np.asarray(seq_lens, np.int32)
    T = S * queries_per_seq
    keys = _normal_f32(r_k, (S, L, d), 1.0 / np.sqrt(d))
    q = _normal_f32(r_q, (T, H, d), 1.0 / np.sqrt(d))
    w = _normal_f32(r_w, (T, H), 1.0 / np.sqrt(H))
    q_seq = np.repeat(np.arange(S, dtype=np.int32), queries_per_seq)
    q_pos = np.concatenate([
        np.arange(seq_lens[s] - queries_per_seq, seq_lens[s], dtype=np.int32)
        for s in range(S)])
    if n_needles:
        for s in range(S):
            rows = np.nonzero(q_seq == s)[0]
            tstar = rows[-1]
            pos_heads = np.nonzero(w[tstar] > 0)[0]
            J = r_head.choice(pos_heads, size=min(3, pos_heads.size), replace=False)
            nmin = int(q_pos[rows].min()) + 1
            P = r_pos.choice(nmin, size=min(n_needles, nmin), replace=False)
            for i, p in enumerate(P):
                keys[s, p] += _unit(q[tstar, J[i % len(J)]])
    out = dict(keys=to_bf16_bits(keys), seq_lens=seq_lens, q=to_bf16_bits(q), w=w,
               q_seq=q_seq, q_pos=q_pos.astype(np.int32))
    if keep_f32_q:
        out["q_f32"] = q
    return out


def clustered_case(S, L, H, seed=0, seg=128, center=1.0, noise=0.5, d=D):
    """Decode inputs whose keys have segment structure: the sequence is cut
    into segments of `seg` tokens, each with its own center direction
    c ~ N(0, center^2/d), and every key is its segment's center plus
    N(0, noise^2/d) token noise.  One query per sequence at its last position,
    i.i.d. q and w.  The pages measure the hierarchical indexer on real model
    activations, which have block-level structure that i.i.d. keys lack; this
    recipe (a reading: the pages give no synthetic model of it) stands in
    for that structure when the selection fidelity is swept."""
    r_q, r_k, r_w, _, _ = _streams(seed)
    nseg = (L + seg - 1) // seg
    centers = _normal_f32(r_k, (S, nseg, d), center / np.sqrt(d))
    keys = _normal_f32(r_k, (S, L, d), noise / np.sqrt(d))
    keys += np.repeat(centers, seg, axis=1)[:, :L]
    q = _normal_f32(r_q, (S, H, d), 1.0 / np.sqrt(d))
    w = _normal_f32(r_w, (S, H), 1.0 / np.sqrt(H))
    return dict(keys=to_bf16_bits(keys), seq_lens=np.full(S, L, np.int32), q=to_bf16_bits(q), w=w,
                q_seq=np.arange(S, dtype=np.int32), q_pos=np.full(S, L - 1, np.int32))


def dagger_case(S, L, H, h, k, seed=0, d=D, frac_outside=0.1,
                a_coef=0.8, b_coef=0.0, n_coef=1.2):
    """MISA-dagger decode input: needles planted so that a share of the dense
    indexer's top-k sits on heads a router is unlikely to pick.

    Heads are split by the weights alone (no indexer arithmetic): A = the h
    heads with the largest w, N = the other heads with w > 0.  With
    u_A = unit(sum_{j in A} w_j q_j) and u_N = unit(sum_{j in N} w_j q_j),
    (1-frac)k keys get + a_coef*u_A and frac*k keys get
    + b_coef*u_A + n_coef*u_N.  The share that actually lands outside the
    routed top-k is not assumed: on the 16 x 131072 workload (h = 8, B = 128,
    k = 2048, seed 0) the oracle puts 9.9% of the dense top-k outside the
    routed top-k on average (7.6% to 13.3% per query), which
    tests/test_workload_calibration.py checks; b_coef = 0 was chosen for that
    (0.15 gave 8.0%, 0.05 gave 9.4%)."""
    r_q, r_k, r_w, r_pos, _ = _streams(seed)
    keys = _normal_f32(r_k, (S, L, d), 1.0 / np.sqrt(d))
    q = _normal_f32(r_q, (S, H, d), 1.0 / np.sqrt(d))
    w = _normal_f32(r_w, (S, H), 1.0 / np.sqrt(H))
    n_out = int(round(frac_outside * k))
    n_in = k - n_out
    for s in range(S):
        order = np.argsort(-w[s], kind="stable")
        A = order[:h]
        N = np.array([j for j in order[h:] if w[s, j] > 0], dtype=np.int64)
        uA = _unit((w[s, A, None] * q[s, A]).sum(0))
        uN = _unit((w[s, N, None] * q[s, N]).sum(0)) if N.size else np.zeros(d, np.float32)
        P = r_pos.choice(L, size=n_in + n_out, replace=False)
        keys[s, P[:n_in]] += np.float32(a_coef) * uA
        keys[s, P[n_in:]] += np.float32(b_coef) * uA + np.float32(n_coef) * uN
    return dict(keys=to_bf16_bits(keys), seq_lens=np.full(S, L, np.int32),
                q=to_bf16_bits(q), w=w, q_seq=np.arange(S, dtype=np.int32),
                q_pos=np.full(S, L - 1, np.int32))


def prefill_case(L, T, H, seed=0, d=D):
    """One sequence of L keys and a chunk of T causal queries at positions
    L-T .. L-1 (a prefill chunk), i.i.d. q/k/w, no needles."""
    r_q, r_k, r_w, _, _ = _streams(seed)
    keys = _normal_f32(r_k, (1, L, d), 1.0 / np.sqrt(d))
    q = _normal_f32(r_q, (T, H, d), 1.0 / np.sqrt(d))
    w = _normal_f32(r_w, (T, H), 1.0 / np.sqrt(H))
    return dict(keys=to_bf16_bits(keys), seq_lens=np.array([L], np.int32),
                q=to_bf16_bits(q), w=w, q_seq=np.zeros(T, np.int32),
                q_pos=np.arange(L - T, L, dtype=np.int32))


def random_case(S, Lmax, T, H, seed=0, d=D, dist="normal", seq_lens=None,
                q_pos=None, q_seq=None, int_range=2):
    """Small random case with arbitrary query placement.

    dist="normal": the standard distributions above.
    dist="int": q, k and w are small integers in [-int_range, int_range]; every
    product and sum in the indexer is then an exact integer in bf16, fp32 and
    fp64, so results can be compared bit for bit, ties included."""
    r_q, r_k, r_w, r_pos, r_seq = _streams(seed)
    if seq_lens is None:
        seq_lens = np.full(S, Lmax, np.int32)
    seq_lens = np.asarray(seq_lens, np.int32)
    if q_seq is None:
        q_seq = r_seq.integers(0, S, size=T).astype(np.int32)
    q_seq = np.asarray(q_seq, np.int32)
    if q_pos is None:
        q_pos = np.array([r_pos.integers(0, seq_lens[s]) for s in q_seq], np.int32)
    q_pos = np.asarray(q_pos, np.int32)
    if dist == "int":
        keys = r_k.integers(-int_range, int_range + 1, size=(S, Lmax, d)).astype(np.float32)
        q = r_q.integers(-int_range, int_range + 1, size=(T, H, d)).astype(np.float32)
        w = r_w.integers(-int_range, int_range + 1, size=(T, H)).astype(np.float32)
    else:
        keys = _normal_f32(r_k, (S, Lmax, d), 1.0 / np.sqrt(d))
        q = _normal_f32(r_q, (T, H, d), 1.0 / np.sqrt(d))
        w = _normal_f32(r_w, (T, H), 1.0 / np.sqrt(H))
    return dict(keys=to_bf16_bits(keys), seq_lens=seq_lens, q=to_bf16_bits(q), w=w,
                q_seq=q_seq, q_pos=q_pos)


# The five benchmark workloads, by what they are.
WORKLOADS = {
    "tiny_dsa_vs_misa_decode_L4096": dict(
        kind="decode", S=1, L=4096, H=64, queries_per_seq=8, n_needles=16,
        B=64, h=8, k=256),
    "dsa_dense_decode_32x32K": dict(
        kind="decode", S=32, L=32768, H=64, queries_per_seq=1, n_needles=64, k=2048),
    "misa_decode_16x128K": dict(
        kind="decode", S=16, L=131072, H=64, queries_per_seq=1, n_needles=64,
        B=128, h=8, k=2048),
    "misa_dagger_decode_16x128K": dict(
        kind="dagger", S=16, L=131072, H=64, B=128, h=8, kc=8192, k=2048),
    "misa_prefill_chunk_4096q_L65536": dict(
        kind="prefill", L=65536, T=4096, H=32, B=128, h=8, k=2048),
    # several queries per sequence (speculative or batched decode): the rows
    # of a sequence share one pass over its keys (the multi-query tiling)
    "misa_multiquery_decode_8x8x32K": dict(
        kind="decode", S=8, L=32768, H=64, queries_per_seq=8, n_needles=32,
        B=128, h=8, k=2048),
    # the hierarchical indexer (all heads) and MISA composed with it (the
    # routed heads in both of its stages), on the MISA decode shape; m = 64
    # kept blocks of 128 keys = 8192 candidate tokens per query
    "hisa_decode_16x128K": dict(
        kind="hisa", S=16, L=131072, H=64, queries_per_seq=1, n_needles=64,
        B=128, m=64, k=2048),
    "misa_hisa_decode_16x128K": dict(
        kind="misa_hisa", S=16, L=131072, H=64, queries_per_seq=1, n_needles=64,
        B=128, h=8, m=64, k=2048),
}


def make_workload(name, seed=0):
    cfg = WORKLOADS[name]
    if cfg["kind"] in ("decode", "hisa", "misa_hisa"):
        case = decode_case(cfg["S"], cfg["L"], cfg["H"], seed=seed,
                           n_needles=cfg.get("n_needles", 0),
                           queries_per_seq=cfg.get("queries_per_seq", 1))
    elif cfg["kind"] == "dagger":
        case = dagger_case(cfg["S"], cfg["L"], cfg["H"], cfg["h"], cfg["k"], seed=seed)
    else:
        case = prefill_case(cfg["L"], cfg["T"], cfg["H"], seed=seed)
    return case, cfg
