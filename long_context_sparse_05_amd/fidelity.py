"""Selection fidelity of the routed indexers against the dense one.

A synthetic, reproducible analog of the pages' token-recovery measurement
("MISA: Mixture of Indexer Sparse Attention for Long-Context LLM
Inference", Technical Summary, Experimental Results: the routed indexer
recovers most of the tokens the dense DSA indexer selects per layer;
the HISA pages report the same comparison as the IoU of the selected sets).

Per query row, with D the dense (DSA) top-k set and S a method's set (the
-1 padding of short prefixes dropped from both):
    recall = |S n D| / |D|        IoU = |S n D| / |S u D|
and the sweep reports both averaged over the query rows, for MISA over the
number of routed heads h and the block size B, for MISA-dagger over h and
the candidate count k', and for the hierarchical indexer (HISA: the m best
blocks, then the indexer over their tokens) and MISA composed with it over
the number of kept blocks m.  The selections come from the GPU kernels
through the C ABI.

Run: python -m long_context_sparse_05_amd.fidelity --help
"""
import argparse
import sys

import numpy as np


def set_metrics(sel, ref):
    """Mean recall and IoU of the rows of `sel` against the rows of `ref`
    (int arrays [T][k], -1 = empty slot).  A row whose reference set is
    empty counts as recall 1 and IoU 1 when the method's set is empty too."""
    sel = np.asarray(sel)
    ref = np.asarray(ref)
    rec, iou = [], []
    for s_row, r_row in zip(sel, ref):
        s = set(int(x) for x in s_row if x >= 0)
        r = set(int(x) for x in r_row if x >= 0)
        inter = len(s & r)
        union = len(s | r)
        rec.append(inter / len(r) if r else (1.0 if not s else 0.0))
        iou.append(inter / union if union else 1.0)
    return float(np.mean(rec)), float(np.mean(iou))


def sweep(case, k, hs, kps, Bs, mode=0, ms=(), hisa_h=8):
    """GPU sweep.  Returns rows of dict(method, B, h, kp, recall, iou); for
    the hierarchical rows kp holds m * B, the candidate tokens kept."""
    import torch
    from long_context_sparse_05_amd import abi

    b = abi.Batch.from_numpy(case)
    dense, _ = abi.indexer_dense(b, k, want_val=False)
    dense = dense.cpu().numpy()
    rows = []
    for B in Bs:
        pooled = abi.pool(b, B)
        for h in hs:
            h = min(h, b.H)
            _, idx, _ = abi.indexer(b, pooled, B, h, k, mode=mode, want_val=False)
            r, i = set_metrics(idx.cpu().numpy(), dense)
            rows.append(dict(method="MISA", B=B, h=h, kp=k, recall=r, iou=i))
            for kp in kps:
                kp = min(kp, b.Lmax)
                if kp <= k:
                    continue
                _, cand, _ = abi.indexer(b, pooled, B, h, kp, mode=mode, want_val=False)
                fin, _ = abi.rerank(b, cand, k, want_val=False)
                r, i = set_metrics(fin.cpu().numpy(), dense)
                rows.append(dict(method="MISA-dagger", B=B, h=h, kp=kp, recall=r, iou=i))
        M = (b.Lmax + B - 1) // B
        hh = min(hisa_h, b.H)
        routed, _, _ = abi.indexer(b, pooled, B, hh, k, mode=mode, want_val=False) if ms else (None, 0, 0)
        for m in ms:
            m = min(m, M)
            sel, _ = abi.hisa_indexer(b, pooled, B, m, k, want_val=False)
            r, i = set_metrics(sel.cpu().numpy(), dense)
            rows.append(dict(method="HISA", B=B, h=b.H, kp=m * B, recall=r, iou=i))
            sel, _ = abi.hisa_indexer(b, pooled, B, m, k, heads=routed, want_val=False)
            r, i = set_metrics(sel.cpu().numpy(), dense)
            rows.append(dict(method="MISA+HISA", B=B, h=hh, kp=m * B, recall=r, iou=i))
    torch.cuda.synchronize()
    return rows


def to_markdown(rows, title):
    lines = ["# " + title, "",
             "| Method | B | h | k' (or m*B kept) | recall vs DSA | IoU vs DSA |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append("| %s | %d | %d | %d | %.4f | %.4f |" % (r["method"], r["B"], r["h"], r["kp"],
                                                             r["recall"], r["iou"]))
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--case", choices=("decode", "dagger", "clustered"), default="decode",
                    help="decode: i.i.d. inputs with needles; dagger: needles on unrouted heads; "
                         "clustered: keys = segment center + token noise")
    ap.add_argument("--S", type=int, default=16)
    ap.add_argument("--L", type=int, default=131072)
    ap.add_argument("--H", type=int, default=64)
    ap.add_argument("--k", type=int, default=2048)
    ap.add_argument("--hs", default="1,2,4,8,16,32,64")
    ap.add_argument("--kps", default="4096,8192,16384")
    ap.add_argument("--Bs", default="64,128")
    ap.add_argument("--ms", default="16,32,64,128", help="kept blocks of the hierarchical indexer")
    ap.add_argument("--mode", type=int, default=0)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--out", default=None, help="write the markdown table here")
    args = ap.parse_args(argv)
    from long_context_sparse_05_amd import synth

    hs = [int(x) for x in args.hs.split(",")]
    kps = [int(x) for x in args.kps.split(",")]
    Bs = [int(x) for x in args.Bs.split(",")]
    if args.case == "decode":
        case = synth.decode_case(args.S, args.L, args.H, seed=args.seed, n_needles=64)
    elif args.case == "dagger":
        case = synth.dagger_case(args.S, args.L, args.H, 8, args.k, seed=args.seed)
    else:
        case = synth.clustered_case(args.S, args.L, args.H, seed=args.seed)
    ms = [int(x) for x in args.ms.split(",")] if args.ms else []
    rows = sweep(case, args.k, hs, kps, Bs, args.mode, ms)
    title = ("Selection fidelity vs the dense indexer: %s inputs, %d sequences x %d keys, H_I = %d, "
             "k = %d, seed %d" % (args.case, args.S, args.L, args.H, args.k, args.seed))
    md = to_markdown(rows, title)
    if args.out:
        with open(args.out, "w") as f:
            f.write(md)
    print(md, end="")
    return 0


if __name__ == "__main__":
    sys.exit(main())
