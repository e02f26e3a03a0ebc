"""Training of the learned decode-plan selector (compiled into libw4a8).

The QFactory reading notes (6.2, "ML-based kernel selector") train a small
multilayer perceptron to predict a kernel configuration's efficiency, not the
best configuration itself: the input is the matrix shape concatenated with
the kernel's tiling parameters, the label the achieved memory bandwidth over
the device maximum, the data offline measurements of randomly drawn
configurations.  This module fits that model to the CSV written by
``w4a8_quantized_linear_amd.tuning`` and writes its weights as
``csrc/selector_weights.inc``, which selector.hip compiles in:

    python -m w4a8_quantized_linear_amd.selector data/decode_plans_mi355x_train.csv.gz \
        --eval data/decode_plans_mi355x_eval.csv.gz

The features are the ones selector.hip computes (same order, same formulas);
the network is 13 -> 32 (tanh) -> 32 (tanh) -> 1 (logistic), trained by
full-batch Adam on the squared error of the utilization, seeded.
"""
from __future__ import annotations

import argparse
import csv
import json
import math
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
INC = os.path.join(HERE, "csrc", "selector_weights.inc")
JSON = os.path.join(HERE, "data", "selector_model.json")
PLAN = ("mt", "nt", "splitk", "waves", "depth", "xstage", "wave_n")
H = 32
CUS = 256


def features(M, N, K, mt, nt, splitk, waves, depth, xstage, wave_n=0, cus=CUS):
    """The selector's 13 inputs for one (shape, plan); arrays broadcast."""
    M, N, K = (np.asarray(v, np.float64) for v in (M, N, K))
    mt, nt, splitk, waves, depth, xstage = (np.asarray(v, np.float64) for v in (mt, nt, splitk, waves, depth, xstage))
    wave_n = np.broadcast_to(np.asarray(wave_n, np.float64), M.shape)
    G = K / 128.0
    mb = np.ceil(M / (16.0 * mt))
    nb = np.ceil((N / 16.0) / nt)
    return np.stack([np.log2(M), np.log2(N), np.log2(K), np.log2(mt), np.log2(nt), np.log2(splitk),
                     np.log2(waves), np.log2(depth), xstage, np.log2(mb * nb * splitk / cus),
                     np.log2(G / splitk), M / (16.0 * mt * mb), wave_n], axis=-1)


def load(path):
    import gzip
    with (gzip.open(path, "rt") if path.endswith(".gz") else open(path)) as f:
        rows = list(csv.DictReader(f))
    cols = {k: np.array([float(r.get(k) or 0) for r in rows]) for k in ("M", "N", "K", *PLAN, "us", "util", "rules")}
    X = features(cols["M"], cols["N"], cols["K"], *(cols[k] for k in PLAN))
    return rows, cols, X


def forward(p, Z):
    h1 = np.tanh(Z @ p["w1"].T + p["b1"])
    h2 = np.tanh(h1 @ p["w2"].T + p["b2"])
    a = h2 @ p["w3"] + p["b3"]
    return 1.0 / (1.0 + np.exp(-a)), (h1, h2)


def train(X, y, seed=0, steps=4000, lr=3e-3, l2=1e-5):
    rng = np.random.default_rng(seed)
    mu, sd = X.mean(axis=0), X.std(axis=0)
    sd[sd < 1e-6] = 1.0
    Z = (X - mu) / sd
    nf = X.shape[1]
    p = {"w1": rng.standard_normal((H, nf)) / math.sqrt(nf), "b1": np.zeros(H),
         "w2": rng.standard_normal((H, H)) / math.sqrt(H), "b2": np.zeros(H),
         "w3": rng.standard_normal(H) / math.sqrt(H), "b3": np.zeros(())}
    m = {k: np.zeros_like(v) for k, v in p.items()}
    v = {k: np.zeros_like(v) for k, v in p.items()}
    n = len(y)
    for t in range(1, steps + 1):
        out, (h1, h2) = forward(p, Z)
        d = 2.0 * (out - y) / n * out * (1 - out)            # through the logistic
        g = {"w3": h2.T @ d, "b3": d.sum()}
        dh2 = np.outer(d, p["w3"]) * (1 - h2 ** 2)
        g["w2"], g["b2"] = dh2.T @ h1, dh2.sum(axis=0)
        dh1 = (dh2 @ p["w2"]) * (1 - h1 ** 2)
        g["w1"], g["b1"] = dh1.T @ Z, dh1.sum(axis=0)
        for k in p:
            gk = g[k] + (l2 * p[k] if k.startswith("w") else 0)
            m[k] = 0.9 * m[k] + 0.1 * gk
            v[k] = 0.999 * v[k] + 0.001 * gk * gk
            p[k] = p[k] - lr * (m[k] / (1 - 0.9 ** t)) / (np.sqrt(v[k] / (1 - 0.999 ** t)) + 1e-8)
    return {"mu": mu, "sd": sd, **p}


def predict(model, X):
    return forward(model, (X - model["mu"]) / model["sd"])[0]


def pick_report(model, rows, cols, X):
    """Per shape: the measured time of the model's pick and of the rule table's
    plan, over the best measured plan (geometric means)."""
    pred = predict(model, X)
    shapes = {}
    for i, r in enumerate(rows):
        shapes.setdefault((r["M"], r["N"], r["K"]), []).append(i)
    rm, rr, picks = [], [], {}
    for key, idx in shapes.items():
        us = cols["us"][idx]
        best = us.min()
        j = idx[int(np.argmax(pred[idx]))]
        rm.append(cols["us"][j] / best)
        picks[key] = tuple(int(cols[k][j]) for k in PLAN)
        rule = [cols["us"][i] for i in idx if cols["rules"][i] == 1]
        if rule:
            rr.append(rule[0] / best)
    gm = lambda a: float(math.exp(np.mean(np.log(a)))) if a else float("nan")
    return {"shapes": len(shapes), "model_over_best": gm(rm), "rules_over_best": gm(rr),
            "model_worst": float(max(rm)), "rules_worst": float(max(rr)) if rr else float("nan")}, picks


def export(model, path_inc=INC, path_json=JSON, version=2):
    def arr(a):
        return "{" + ", ".join("%.9ef" % float(x) for x in np.ravel(a)) + "}"

    def mat(a):
        return "{" + ", ".join(arr(r) for r in a) + "}"

    txt = ["// generated by w4a8_quantized_linear_amd/selector.py from measured decode-plan timings",
           "const Model kModel = {",
           "    %s," % arr(model["mu"]), "    %s," % arr(model["sd"]),
           "    %s," % mat(model["w1"]), "    %s," % arr(model["b1"]),
           "    %s," % mat(model["w2"]), "    %s," % arr(model["b2"]),
           "    %s," % arr(model["w3"]), "    %.9ef," % float(model["b3"]),
           "    %d," % version, "};", ""]
    with open(path_inc, "w") as f:
        f.write("\n".join(txt))
    os.makedirs(os.path.dirname(path_json), exist_ok=True)
    with open(path_json, "w") as f:
        json.dump({**{k: np.asarray(v, np.float32).tolist() for k, v in model.items()}, "version": version}, f)


def load_model(path_json=JSON):
    d = json.load(open(path_json))
    d.pop("version", None)
    return {k: np.asarray(v, np.float64) for k, v in d.items()}


def _train_seed(job):
    path, seed = job
    _, cols, X = load(path)
    return train(X, cols["util"], seed=seed)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("train")
    ap.add_argument("--eval")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--seeds", type=int, default=1,
                    help="train seeds seed .. seed + n - 1 in parallel and keep the one whose picks on the "
                         "training set are closest to the best measured plans")
    ap.add_argument("--no-export", action="store_true")
    args = ap.parse_args(argv)
    rows, cols, X = load(args.train)
    if args.seeds > 1:
        import concurrent.futures as cf
        seeds = list(range(args.seed, args.seed + args.seeds))
        with cf.ProcessPoolExecutor(max_workers=min(len(seeds), os.cpu_count() or 1)) as ex:
            models = list(ex.map(_train_seed, [(args.train, sd) for sd in seeds]))
        scores = [pick_report(m, rows, cols, X)[0]["model_over_best"] for m in models]
        for sd, sc in zip(seeds, scores):
            print("seed %d: training-set picks %.4f x the best" % (sd, sc))
        model = models[int(np.argmin(scores))]
    else:
        model = train(X, cols["util"], seed=args.seed)
    pred = predict(model, X)
    print("train rows %d  rmse %.4f" % (len(rows), float(np.sqrt(np.mean((pred - cols["util"]) ** 2)))))
    print("train", pick_report(model, rows, cols, X)[0])
    if args.eval:
        er, ec, EX = load(args.eval)
        ep = predict(model, EX)
        print("eval rows %d  rmse %.4f" % (len(er), float(np.sqrt(np.mean((ep - ec["util"]) ** 2)))))
        print("eval", pick_report(model, er, ec, EX)[0])
    if not args.no_export:
        export(model)
        print("wrote", INC, JSON)
    return 0


if __name__ == "__main__":
    sys.exit(main())
