"""Choose the router-bias strength beta of the skewed 4096-token prefill
workload and record the load it gives under the oracle's routing.

The workload biases expert e's logit by b_e = -beta * 1.1 * ln(e + 1) (a
Zipf-like skew, s = 1.1, expert id as the rank) so that the hottest expert
receives about ten times the mean load T*k/E.  beta is bisected until the
ratio max_e n_e / (T*k/E) lies in [9.5, 10.5], where n_e counts the rows that
the ORACLE's canonical routing sends to expert e.

Candidate betas are proposed from fp64 numpy logits (a cheap stand-in that
only steers the search); every candidate is then routed by the oracle, and
only the oracle's counts decide and are written out.  Run from the
repository root:

    python tests/golden/zipf_beta.py

It writes tests/golden/zipf_beta.json: beta, the oracle's max/mean ratio,
the minimum and maximum rows per expert, and how many experts are touched.
"""
import concurrent.futures as cf
import json
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from routed_expert_mxfp4_amd import synth  # noqa: E402

LO, HI = 9.5, 10.5
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_beta.json")


def bias_of(cfg, beta):
    return synth.gen_bias(synth.Config(cfg.index, cfg.name, cfg.T, cfg.d, cfg.E, cfg.k, cfg.f,
                                       seed=cfg.seed, zipf_beta=beta, zipf_s=cfg.zipf_s))


def oracle_counts(cfg, x16, wr16, beta, threads):
    b = bias_of(cfg, beta).numpy()
    chunks = np.array_split(np.arange(cfg.T), threads)

    def route(idx):
        lg = oracle.router_logits(x16[idx], wr16, b)
        return oracle.topk_softmax(lg, cfg.k)[0]

    with cf.ThreadPoolExecutor(max_workers=threads) as pool:
        ids = np.concatenate(list(pool.map(route, chunks)))
    return np.bincount(ids.ravel(), minlength=cfg.E)


def approx_ratio(cfg, base, beta):
    lg = base + bias_of(cfg, beta).numpy().astype(np.float64)[None, :]
    top = np.argpartition(-lg, cfg.k - 1, axis=1)[:, :cfg.k]
    c = np.bincount(top.ravel(), minlength=cfg.E)
    return c.max() / (cfg.T * cfg.k / cfg.E)


def main():
    cfg = synth.CONFIGS[3]
    x, wr = synth.gen_x(cfg), synth.gen_router_w(cfg)
    x16, wr16 = synth.as_u16(x), synth.as_u16(wr)
    base = x.double().numpy() @ wr.double().numpy().T
    threads = max(1, min(16, os.cpu_count() or 1))
    lo, hi = 0.25, 0.45
    mean = cfg.T * cfg.k / cfg.E
    for _ in range(40):
        beta = round((lo + hi) / 2, 4)
        r = approx_ratio(cfg, base, beta)
        if LO + 0.1 <= r <= HI - 0.1:
            counts = oracle_counts(cfg, x16, wr16, beta, threads)
            ratio = counts.max() / mean
            print("beta %.4f: approx %.3f, oracle %.3f" % (beta, r, ratio), flush=True)
            if LO <= ratio <= HI:
                rec = {"workload": cfg.name, "zipf_s": cfg.zipf_s, "beta": beta,
                       "max_over_mean": round(float(ratio), 4),
                       "max_rows": int(counts.max()), "min_rows": int(counts.min()),
                       "experts_touched": int((counts > 0).sum()),
                       "mean_rows": mean, "routing": "oracle canonical logits, top-k"}
                with open(OUT, "w") as fh:
                    json.dump(rec, fh, indent=1)
                    fh.write("\n")
                print(json.dumps(rec))
                return
            r = ratio
        if r < (LO + HI) / 2:
            lo = beta
        else:
            hi = beta
    raise SystemExit("no beta found")


if __name__ == "__main__":
    main()
