// selector.hip -- learned choice among the decode GEMM plans (host code).
//
// The QFactory reading notes (6.2, "ML-based kernel selector") do not train a
// model to output the best configuration.  They train a light multilayer
// perceptron to predict how efficient a given configuration is: the input is
// the matrix shape concatenated with the kernel's tiling parameters, the label
// is the achieved memory bandwidth over the device maximum (a bounded target,
// unlike latency), and the data comes from offline profiling of randomly
// drawn configurations.  Here the configurations are the decode kernel's
// instantiated plans (m-tiles, n-tiles, split-K, waves, pipeline depth,
// staged activations); the model is trained by
// w4a8_quantized_linear_amd/selector.py from measured timings and compiled in
// through selector_weights.inc.  plan_gemm ranks every candidate of a decode
// shape by the prediction and takes the best when the selector is enabled.
//
// Features (each standardized with the training set's mean and spread):
//   log2 M, log2 N, log2 K, log2 m-tiles, log2 n-tiles, log2 split-K,
//   log2 waves, log2 depth, staged activations (0/1),
//   log2(workgroups / compute units), log2(groups per split),
//   filled fraction of the last m-block's rows (M / (16 m-tiles m-blocks)),
//   waves splitting N instead of K (0/1).
// Network: 13 -> 32 (tanh) -> 32 (tanh) -> 1 (logistic), fp32.
#include <cmath>
#include <cstdlib>
#include <cstring>

#include "w4a8_internal.h"

namespace w4a8 {
namespace {

constexpr int kH = 32;

struct Model {
    float mu[kSelFeatures], sd[kSelFeatures];
    float w1[kH][kSelFeatures], b1[kH];
    float w2[kH][kH], b2[kH];
    float w3[kH], b3;
    int trained;    // 0: no model; 1: trained without N-split plans; 2: with them
};

#if __has_include("selector_weights.inc")
#include "selector_weights.inc"   // defines `const Model kModel = {...};`
#else
const Model kModel = {};
#endif

}  // namespace

void selector_features(const GemmPlan &p, int64_t M, int64_t N, int64_t K, int64_t cus, float *x)
{
    const double G = (double)num_groups(K);
    const double wgs = (double)p.m_blocks * (double)p.n_blocks * (double)p.splitk;
    x[0] = (float)std::log2((double)M);
    x[1] = (float)std::log2((double)N);
    x[2] = (float)std::log2((double)K);
    x[3] = (float)std::log2((double)p.mt);
    x[4] = (float)std::log2((double)p.nt);
    x[5] = (float)std::log2((double)p.splitk);
    x[6] = (float)std::log2((double)p.waves);
    x[7] = (float)std::log2((double)p.depth);
    x[8] = p.xstage ? 1.0f : 0.0f;
    x[9] = (float)std::log2(wgs / (double)cus);
    x[10] = (float)std::log2(G / (double)p.splitk);
    x[11] = (float)((double)M / (16.0 * (double)p.mt * (double)p.m_blocks));
    x[12] = (float)p.wave_n;
}

float selector_predict(const float *x)
{
    const Model &m = kModel;
    if (!m.trained)
        return -1.0f;
    float z[kSelFeatures], h1[kH], h2[kH];
    for (int i = 0; i < kSelFeatures; i++)
        z[i] = (x[i] - m.mu[i]) / m.sd[i];
    for (int j = 0; j < kH; j++) {
        float a = m.b1[j];
        for (int i = 0; i < kSelFeatures; i++)
            a += m.w1[j][i] * z[i];
        h1[j] = std::tanh(a);
    }
    for (int j = 0; j < kH; j++) {
        float a = m.b2[j];
        for (int i = 0; i < kH; i++)
            a += m.w2[j][i] * h1[i];
        h2[j] = std::tanh(a);
    }
    float a = m.b3;
    for (int i = 0; i < kH; i++)
        a += m.w3[i] * h2[i];
    return 1.0f / (1.0f + std::exp(-a));
}

// Whether the model has seen N-split plans (else they are not ranked).
bool selector_knows_wave_n(int wave_n) { return wave_n == 0 || (wave_n == 1 && kModel.trained >= 2); }

// On when a model is compiled in, unless W4A8_SELECTOR=0.
bool selector_enabled()
{
    if (!kModel.trained)
        return false;
    const char *env = std::getenv("W4A8_SELECTOR");
    return !(env && std::strcmp(env, "0") == 0);
}

}  // namespace w4a8
