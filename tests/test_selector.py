"""The learned decode-plan selector (QFactory reading notes, 6.2): the oracle's
plain MLP pinned by closed forms, and the library's compiled-in model checked
against it (host code only, no GPU)."""
import json
import math
import os

import pytest

from oracle import selector_oracle as so

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MODEL = os.path.join(ROOT, "w4a8_quantized_linear_amd", "data", "selector_model.json")
FIELDS = ("mt", "nt", "splitk", "waves", "depth", "xstage", "wave_n")
MARGIN = 0.0


def tiny(nf=13, h=32, **kw):
    m = {"mu": [0.0] * nf, "sd": [1.0] * nf, "w1": [[0.0] * nf for _ in range(h)], "b1": [0.0] * h,
         "w2": [[0.0] * h for _ in range(h)], "b2": [0.0] * h, "w3": [0.0] * h, "b3": 0.0}
    m.update(kw)
    return m


def test_oracle_zero_network_is_the_logistic_of_the_bias():
    for b3 in (-2.0, 0.0, 0.7):
        assert so.mlp_utilization(tiny(b3=b3), [1.0] * 13) == 1 / (1 + math.exp(-b3))


def test_oracle_single_path_closed_form():
    """One unit per layer on one input: u = logistic(w3 tanh(w2 tanh(w1 (x - mu) / sd)))."""
    m = tiny()
    m["mu"][4], m["sd"][4] = 1.5, 2.0
    m["w1"][0][4], m["w2"][0][0], m["w3"][0] = 0.8, -1.3, 2.0
    for x4 in (-3.0, 0.0, 1.5, 4.0):
        x = [0.0] * 13
        x[4] = x4
        want = 1 / (1 + math.exp(-2.0 * math.tanh(-1.3 * math.tanh(0.8 * (x4 - 1.5) / 2.0))))
        assert abs(so.mlp_utilization(m, x) - want) < 1e-15


def test_oracle_inputs_of_a_worked_plan():
    """M=20, N=1024, K=4096, 2 m-tiles, 4 n-tiles, split 2, 4 waves, depth 2, no staging:
    one m-block of 32 rows (20 filled), 16 n-blocks, 32 workgroups on 256 CUs, 16 groups per split."""
    x = so.plan_inputs(20, 1024, 4096, 2, 4, 2, 4, 2, 0, 1)
    want = [math.log2(20), 10, 12, 1, 2, 1, 2, 1, 0.0, math.log2(32 / 256), 4, 20 / 32, 1.0]
    assert all(abs(a - b) < 1e-12 for a, b in zip(x, want))


def test_oracle_choice_keeps_the_rule_plan_inside_the_margin():
    m = tiny()
    m["w1"][0][4], m["w2"][0][0], m["w3"][0] = 1.0, 1.0, 1.0   # score grows with log2 n-tiles
    cands = [(1, 1, 1, 4, 2, 0, 0), (1, 4, 1, 4, 2, 0, 0)]
    pick, best, ref = so.choose(m, cands, (1, 1, 1, 4, 2, 0, 0), (8, 4096, 4096), margin=0.05)
    assert pick == (1, 4, 1, 4, 2, 0, 0) and best > ref * 1.05
    pick, _, _ = so.choose(m, cands, (1, 1, 1, 4, 2, 0, 0), (8, 4096, 4096), margin=10.0)
    assert pick == (1, 1, 1, 4, 2, 0, 0)


@pytest.fixture(scope="module")
def lib_model():
    from w4a8_quantized_linear_amd import _lib
    _lib.load()
    return json.load(open(MODEL))


SHAPES = [(1, 11008, 4096), (8, 11008, 4096), (16, 12288, 4096), (32, 57344, 8192), (64, 4096, 28672),
          (3, 560, 640), (47, 544, 25216), (13, 56592, 2432)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_library_scores_match_the_oracle(lib_model, M, N, K):
    import w4a8_quantized_linear_amd as w
    cands = w.gemm_w4a8_decode_candidates(M, N, K)
    lib_model = {k: v for k, v in lib_model.items() if k != "version"}
    assert 40 <= len(cands) <= 256
    for c in cands:
        got = w.gemm_w4a8_selector_score(M, N, K, c)
        want = so.mlp_utilization(lib_model, so.plan_inputs(M, N, K, *c))
        assert abs(got - want) < 2e-5, (c, got, want)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_library_choice_follows_the_margin_rule(lib_model, M, N, K, monkeypatch):
    import w4a8_quantized_linear_amd as w
    monkeypatch.setenv("W4A8_SELECTOR", "0")
    rules = w.gemm_w4a8_plan(M, N, K)
    monkeypatch.delenv("W4A8_SELECTOR")
    chosen = w.gemm_w4a8_plan(M, N, K)
    if rules["kind"] != 0:
        assert chosen == rules
        return
    cands = w.gemm_w4a8_decode_candidates(M, N, K)
    if lib_model.get("version", 1) < 2:          # a model that has not seen N-split plans does not rank them
        cands = [c for c in cands if not c[6]]
    rt = tuple(rules[f] for f in FIELDS)
    pick, best, ref = so.choose({k: v for k, v in lib_model.items() if k != "version"}, cands, rt, (M, N, K), MARGIN)
    if abs(best - ref * (1 + MARGIN)) < 1e-4:
        pytest.skip("score within rounding of the margin")
    assert tuple(chosen[f] for f in FIELDS) == pick


def test_rule_plans_are_candidates():
    import w4a8_quantized_linear_amd as w
    os.environ["W4A8_SELECTOR"] = "0"
    try:
        for (M, N, K) in SHAPES:
            p = w.gemm_w4a8_plan(M, N, K)
            if p["kind"] == 0:
                assert tuple(p[f] for f in FIELDS) in w.gemm_w4a8_decode_candidates(M, N, K)
    finally:
        del os.environ["W4A8_SELECTOR"]


def test_training_is_deterministic():
    import numpy as np
    from w4a8_quantized_linear_amd import selector as S
    rng = np.random.default_rng(3)
    X = rng.standard_normal((64, 12))
    y = 1 / (1 + np.exp(-X[:, 0]))
    a = S.train(X, y, seed=5, steps=50)
    b = S.train(X, y, seed=5, steps=50)
    assert all(np.array_equal(a[k], b[k]) for k in a)
    assert np.mean((S.predict(a, X) - y) ** 2) < np.mean((0.5 - y) ** 2)
