"""Plain reference of the learned decode-plan selector's arithmetic.

TEST INFRASTRUCTURE ONLY (see the oracle package docstring): the tests compare
the library's compiled-in selector with this, on the library's exported model.

QFactory reading notes, 6.2 ("ML-based kernel selector"): a light multilayer
perceptron maps the matrix shape concatenated with a kernel configuration's
tiling parameters to the configuration's predicted memory-bandwidth
utilization (achieved bandwidth over the device maximum); the configuration
with the best prediction is kept.  Here, written out element by element in
Python floats (double precision):
  z_i  = (x_i - mu_i) / sd_i
  h1_j = tanh(b1_j + sum_i w1_ji z_i)
  h2_j = tanh(b2_j + sum_i w2_ji h1_i)
  u    = 1 / (1 + exp(-(b3 + sum_i w3_i h2_i)))
The input vector is the library's documented feature list: log2 M, log2 N,
log2 K, log2 m-tiles, log2 n-tiles, log2 split-K, log2 waves, log2 depth,
staged activations (0/1), log2(workgroups / compute units), log2(groups per
split), filled fraction of the last m-block's rows, waves splitting N (0/1).
"""
import math


def plan_inputs(M, N, K, mt, nt, splitk, waves, depth, xstage, wave_n=0, cus=256):
    groups = K / 128
    m_blocks = -(-M // (16 * mt))
    n_blocks = -(-(N // 16) // nt)
    return [math.log2(M), math.log2(N), math.log2(K), math.log2(mt), math.log2(nt), math.log2(splitk),
            math.log2(waves), math.log2(depth), 1.0 if xstage else 0.0,
            math.log2(m_blocks * n_blocks * splitk / cus), math.log2(groups / splitk), M / (16 * mt * m_blocks),
            1.0 if wave_n else 0.0]


def mlp_utilization(model, x):
    z = [(xi - m) / s for xi, m, s in zip(x, model["mu"], model["sd"])]
    h1 = [math.tanh(b + sum(w * zi for w, zi in zip(row, z))) for row, b in zip(model["w1"], model["b1"])]
    h2 = [math.tanh(b + sum(w * hi for w, hi in zip(row, h1))) for row, b in zip(model["w2"], model["b2"])]
    a = float(model["b3"]) + sum(w * hi for w, hi in zip(model["w3"], h2))
    return 1.0 / (1.0 + math.exp(-a))


def choose(model, candidates, rules_plan, shape, margin, cus=256):
    """The kept plan: the best-scored candidate when its score beats the rule
    plan's by more than `margin` (relative), else the rule plan."""
    M, N, K = shape
    scores = [mlp_utilization(model, plan_inputs(M, N, K, *c, cus=cus)) for c in candidates]
    best = max(range(len(candidates)), key=lambda i: scores[i])
    ref = mlp_utilization(model, plan_inputs(M, N, K, *rules_plan, cus=cus))
    return (candidates[best] if scores[best] > ref * (1 + margin) else tuple(rules_plan)), scores[best], ref
