"""Proxy-task evaluation of the selection modes ("DynamicRad", arXiv
2604.20470, App. C.2-C.4): Eq. 20 drift inputs at the three motion regimes,
Eq. 22's normalised attention error (through an N(0, 1) probe) plus the
sparsity penalty, for each selection mode on one workload shape.

    python -m block_sparse_attention_candidates_amd.proxy [--workload wan14b_720p] [--heads 2]
        [--regimes low,mid,high] [--modes static,dynamic,token,decay-static] [--preset mid]

Prints one JSON line per (regime, mode): normalised error, sparsity, loss and
the GPU time of one evaluation (mask, dense attention, sparse attention and
dr_proxy_error). Every step runs in the library's kernels; this module only
prepares inputs and reads back three numbers per evaluation.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="wan14b_720p")
    ap.add_argument("--heads", type=int, default=2)
    ap.add_argument("--regimes", default="low,mid,high")
    ap.add_argument("--modes", default="static,dynamic,token,decay-static")
    ap.add_argument("--preset", default="mid", help="Table 2 preset of the token and decay-static modes")
    ap.add_argument("--seed", type=int, default=11)
    args = ap.parse_args(argv)
    sys.path.insert(0, ROOT)
    import torch
    import workloads
    import block_sparse_attention_candidates_amd as dr

    base = workloads.get_workload(args.workload)
    for regime in args.regimes.split(","):
        delta = workloads.PROXY_DRIFT[regime]
        qb, kb, zb = workloads.proxy_qkz(base.num_frames, base.frame_h, base.frame_w, base.head_dim, args.heads,
                                         delta, args.seed, as_bits=True)
        q, k, z = (torch.from_numpy(x).view(torch.bfloat16).cuda() for x in (qb, kb, zb))
        del qb, kb, zb
        for mode in args.modes.split(","):
            w = base
            if mode == "token":
                w, taus = workloads.token_workload(args.workload, args.preset)
            elif mode == "decay-static":
                w, rhos = workloads.static_workload(args.workload, args.preset)
            cand = dr.build_candidates(dr.radial_cfg(w.num_frames, w.tokens_per_frame, w.block_size, w.gamma,
                                                     w.lam, w.theta_c, w.theta_m))

            def evaluate():
                if mode == "token":
                    kept = dr.token_select(q, k, cand, taus[0], taus[1])
                elif mode == "decay-static":
                    kept = dr.static_select(cand, rhos[0], rhos[1], args.seed, batch=1, heads=args.heads)
                else:
                    kept = dr.score_select(q, k, cand, mode=mode, ratio=w.static_ratio, tau=w.dynamic_tau)
                return dr.proxy_loss(q, k, z, cand, kept)

            evaluate()   # warm-up
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            res = evaluate()
            ms = (time.perf_counter() - t0) * 1e3
            setting = ({"tau_near_far": list(taus)} if mode == "token" else
                       {"rho_near_far": list(rhos), "seed": args.seed} if mode == "decay-static" else
                       {"ratio": w.static_ratio} if mode == "static" else {"tau": w.dynamic_tau})
            print(json.dumps({"workload": w.name, "heads": args.heads, "regime": regime, "delta": delta,
                              "mode": mode, **setting, "gamma": w.gamma, "lambda": w.lam,
                              "theta_c": w.theta_c, "theta_m": w.theta_m,
                              "nmse": round(res["nmse"], 6), "sparsity": round(res["sparsity"], 4),
                              "loss": round(res["loss"], 6), "ms_per_evaluation": round(ms, 2)}), flush=True)


if __name__ == "__main__":
    main()
