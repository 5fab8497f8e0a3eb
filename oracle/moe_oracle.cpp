// fp64 CPU oracle of one sparse MoE layer with int4/int8 group-quantized
// experts, in plain C++17 with OpenMP over the host cores.
//
// TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
// benchmark's CPU-baseline leg load this library.  The HIP product path never
// links, loads or calls it, and it includes nothing from that path: no header,
// no helper, no table.  Its inputs are the logical arrays of the seeded
// generator (one code per byte, bf16 scale/bias bit patterns, fp32 router and
// gate weights, activations widened to double), never a packed expert blob.
//
// What it computes is the plain definition of the layer, step by step, in
// double precision:
//  * every token is routed to the top-k of E experts by a resident router
//    (8 of 256 for the 35B-A3B family, 10 of 512 for the 80B-A3B family) and
//    an always-active shared expert is added: page "Paquets Swiftlet 80B Qwen
//    dans Mac avec 4,3 Go de mémoire ; iPhone 17 exécutera nativement 35B"
//    (xix.ai), 4th paragraph; Swiftlet item on news.bugfactory.tech,
//    3rd paragraph;
//  * the experts' weights are MLX-style int4/int8 group-quantized: xix.ai
//    page, last paragraph; page "Swiftlet: 在 Mac 和 iPhone 上執行 80B 與 35B
//    Qwen 模型" (agentlenshq.com), section "記憶體管理與權重串流";
//  * the affine form w = scale * q + bias per group of 64 input columns,
//    SwiGLU experts, the sigmoid-gated shared expert, softmax -> top-k ->
//    renormalise and the pre-RMSNorm chain are the workload definition of
//    this project (the pages do not print them); the readings are:
//      R1 codes unsigned (0..15 / 0..255), groups along the input axis;
//      R2 scale and bias bf16, widened exactly;
//      R5 softmax over all E, top-k, renormalise over the k selected;
//      R6 top-k by logit descending, ties to the lower expert index;
//      R7 stored activations are round-to-nearest-even in the act dtype;
//      R9 chain: x_hat = act(rmsnorm(x)) (unit weight), x_next = act(x + out).
//
// Loops are the definitions written out.  Each output element is computed by
// exactly one thread, with its sum taken over the input index in ascending
// order, so results do not depend on the number of threads.  Every function
// is pinned by tests/test_oracle_pins.py, which runs the same pins against
// this library and against the numpy oracle.
//
// A test may rebuild this file with -DORACLE_PLANT=<n> to plant one known
// mistake and check that a pin catches it (see plant() below); the normal
// build defines no ORACLE_PLANT.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef ORACLE_PLANT
#define ORACLE_PLANT 0
#endif

namespace {

constexpr int kPlantGroupIndex = 1;   // dequantize: group c % G instead of c / 64
constexpr int kPlantDroppedBias = 2;  // dequantize: bias term left out
constexpr int kPlantSiluSign = 3;     // silu: g / (1 + exp(+g))
constexpr int kPlantTiesHigh = 4;     // top-k: ties to the higher index
constexpr int kPlantNoRenorm = 5;     // renormalise: weights not divided by their sum
constexpr int kPlantRmsMean = 6;      // rmsnorm: sum instead of mean of squares

constexpr bool plant(int n) { return ORACLE_PLANT == n; }

}  // namespace

extern "C" {

// One expert's logical arrays (host memory, row-major).
//   qg, qu  [inter x hidden] codes, one per byte
//   qd      [hidden x inter] codes
//   sg, bg, su, bu  [inter x hidden/group] bf16 bit patterns
//   sd, bd          [hidden x inter/group] bf16 bit patterns
struct orc_expert {
  const uint8_t* qg;
  const uint8_t* qu;
  const uint8_t* qd;
  const uint16_t* sg;
  const uint16_t* bg;
  const uint16_t* su;
  const uint16_t* bu;
  const uint16_t* sd;
  const uint16_t* bd;
  int64_t inter;
};

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

// ---------------------------------------------------------------------------
// number formats

// Exact value of a bf16 bit pattern: the upper 16 bits of an IEEE binary32
// whose lower 16 bits are zero (R2).
double orc_bf16_value(uint16_t bits) {
  const uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

void orc_bf16_to_f64(const uint16_t* bits, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_value(bits[i]);
}

// Nearest bf16 value to v (8 significant bits, ties to even), for finite v in
// the normal range: v = m 2^e with 0.5 <= |m| < 1, and m 2^8 rounded to an
// integer under the default round-to-nearest-even mode (R7).
double orc_round_bf16(double v) {
  if (v == 0.0) return v;
  int e = 0;
  const double m = frexp(v, &e);
  return ldexp(nearbyint(m * 256.0) / 256.0, e);
}

// Store in the activation dtype and widen back: act 0 = fp32, 1 = bf16.
void orc_round_act(const double* v, int64_t n, int act, double* out) {
  for (int64_t i = 0; i < n; ++i)
    out[i] = act == 1 ? orc_round_bf16(v[i]) : (double)(float)v[i];
}

// ---------------------------------------------------------------------------
// the layer, step by step

// W[r][c] = s[r][c / group] * q[r][c] + b[r][c / group]   (R1, R2)
void orc_dequantize(const uint8_t* q, const uint16_t* s, const uint16_t* b, int64_t rows,
                    int64_t cols, int64_t group, double* W) {
  const int64_t G = cols / group;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t c = 0; c < cols; ++c) {
      const int64_t g = plant(kPlantGroupIndex) ? c % G : c / group;
      const double sc = orc_bf16_value(s[r * G + g]);
      const double bi = orc_bf16_value(b[r * G + g]);
      W[r * cols + c] = plant(kPlantDroppedBias) ? sc * (double)q[r * cols + c]
                                                 : sc * (double)q[r * cols + c] + bi;
    }
  }
}

// l[t][e] = sum_c Wr[e][c] * x[t][c]  (+ bias[e])
// (router weights and bias are given as doubles: the fp32 values widened exactly)
void orc_router_logits(const double* x, const double* Wr, const double* bias, int64_t T,
                       int64_t E, int64_t H, double* l) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int64_t c = 0; c < H; ++c) acc += Wr[e * H + c] * x[t * H + c];
      if (bias) acc += bias[e];
      l[t * E + e] = acc;
    }
  }
}

// p[t][e] = exp(l[t][e] - max_e l[t]) / sum_e' exp(l[t][e'] - max_e l[t])
void orc_softmax(const double* l, int64_t T, int64_t E, double* p) {
  for (int64_t t = 0; t < T; ++t) {
    double m = l[t * E];
    for (int64_t e = 1; e < E; ++e) m = std::max(m, l[t * E + e]);
    double den = 0.0;
    for (int64_t e = 0; e < E; ++e) den += exp(l[t * E + e] - m);
    for (int64_t e = 0; e < E; ++e) p[t * E + e] = exp(l[t * E + e] - m) / den;
  }
}

// The k largest logits of one token, ordered by logit descending, ties to
// the lower expert index (R6); gap = l_(k) - l_(k+1), +inf when k == E.
void orc_topk(const double* l, int64_t E, int64_t k, int64_t* sel, double* gap) {
  std::vector<int64_t> order(E);
  for (int64_t e = 0; e < E; ++e) order[e] = e;
  std::stable_sort(order.begin(), order.end(), [&](int64_t a, int64_t b) {
    if (l[a] != l[b]) return l[a] > l[b];
    return plant(kPlantTiesHigh) ? a > b : a < b;
  });
  for (int64_t j = 0; j < k; ++j) sel[j] = order[j];
  *gap = k == E ? INFINITY : l[order[k - 1]] - l[order[k]];
}

// w_j = p[S_j] / sum_{i in S} p[i]
void orc_renormalize(const double* p, const int64_t* sel, int64_t k, double* w) {
  double den = 0.0;
  for (int64_t j = 0; j < k; ++j) den += p[sel[j]];
  for (int64_t j = 0; j < k; ++j) w[j] = plant(kPlantNoRenorm) ? p[sel[j]] : p[sel[j]] / den;
}

// silu(g) = g * sigmoid(g), written g / (1 + exp(-g)) so that g -> -inf gives 0
double orc_silu(double g) {
  return plant(kPlantSiluSign) ? g / (1.0 + exp(g)) : g / (1.0 + exp(-g));
}

double orc_sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

void orc_silu_array(const double* g, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_silu(g[i]);
}

void orc_sigmoid_array(const double* v, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_sigmoid(v[i]);
}

// SwiGLU expert on the logical arrays: g = Wg x, u = Wu x, h = silu(g) u,
// y = Wd h, for n tokens x [n x H] -> y [n x H].
void orc_expert_ffn(const double* x, int64_t n, int64_t H, const orc_expert* a, int64_t group,
                    double* y) {
  const int64_t I = a->inter;
  std::vector<double> Wg(I * H), Wu(I * H), Wd(H * I), h(n * I);
  orc_dequantize(a->qg, a->sg, a->bg, I, H, group, Wg.data());
  orc_dequantize(a->qu, a->su, a->bu, I, H, group, Wu.data());
  orc_dequantize(a->qd, a->sd, a->bd, H, I, group, Wd.data());
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < I; ++r) {
    for (int64_t t = 0; t < n; ++t) {
      double g = 0.0, u = 0.0;
      for (int64_t c = 0; c < H; ++c) {
        g += Wg[r * H + c] * x[t * H + c];
        u += Wu[r * H + c] * x[t * H + c];
      }
      h[t * I + r] = orc_silu(g) * u;
    }
  }
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < H; ++r) {
    for (int64_t t = 0; t < n; ++t) {
      double acc = 0.0;
      for (int64_t c = 0; c < I; ++c) acc += Wd[r * I + c] * h[t * I + c];
      y[t * H + r] = acc;
    }
  }
}

// gamma[t] = sigmoid(w_sg . x[t])   (R4)
void orc_shared_gate(const double* x, const double* wsg, int64_t T, int64_t H, double* gamma) {
  for (int64_t t = 0; t < T; ++t) {
    double acc = 0.0;
    for (int64_t c = 0; c < H; ++c) acc += wsg[c] * x[t * H + c];
    gamma[t] = orc_sigmoid(acc);
  }
}

// Router, softmax, top-k and renormalisation of every token (R5, R6).
// logits [T x E], idx [T x k], w [T x k], gap [T].
void orc_route(const double* x, const double* Wr, const double* bias, int64_t T, int64_t E,
               int64_t H, int64_t k, double* logits, int64_t* idx, double* w, double* gap) {
  orc_router_logits(x, Wr, bias, T, E, H, logits);
  std::vector<double> p(T * E);
  orc_softmax(logits, T, E, p.data());
  for (int64_t t = 0; t < T; ++t) {
    orc_topk(logits + t * E, E, k, idx + t * k, gap + t);
    orc_renormalize(p.data() + t * E, idx + t * k, k, w + t * k);
  }
}

// out[t] = sum_j w[t][j] FFN_{idx[t][j]}(x[t]) + gamma[t] FFN_shared(x[t]).
// experts[e] holds routed expert e (entries of experts no token selects may
// be empty); shared may be NULL (no shared expert; gamma is then ignored).
// Each routed expert is applied once, to the tokens that selected it, in
// ascending expert order; the shared expert last.
void orc_combine(const double* x, int64_t T, int64_t H, const int64_t* idx, const double* w,
                 int64_t k, const orc_expert* experts, int64_t E, int64_t group,
                 const double* gamma, const orc_expert* shared, double* out) {
  for (int64_t i = 0; i < T * H; ++i) out[i] = 0.0;
  for (int64_t e = 0; e < E; ++e) {
    std::vector<int64_t> tok, jj;
    for (int64_t t = 0; t < T; ++t)
      for (int64_t j = 0; j < k; ++j)
        if (idx[t * k + j] == e) {
          tok.push_back(t);
          jj.push_back(j);
        }
    if (tok.empty()) continue;
    const int64_t n = (int64_t)tok.size();
    std::vector<double> xs(n * H), ys(n * H);
    for (int64_t i = 0; i < n; ++i) memcpy(&xs[i * H], x + tok[i] * H, sizeof(double) * H);
    orc_expert_ffn(xs.data(), n, H, &experts[e], group, ys.data());
    for (int64_t i = 0; i < n; ++i) {
      const double wt = w[tok[i] * k + jj[i]];
      for (int64_t c = 0; c < H; ++c) out[tok[i] * H + c] += wt * ys[i * H + c];
    }
  }
  if (shared != nullptr) {
    std::vector<double> ys(T * H);
    orc_expert_ffn(x, T, H, shared, group, ys.data());
    for (int64_t t = 0; t < T; ++t)
      for (int64_t c = 0; c < H; ++c) out[t * H + c] += gamma[t] * ys[t * H + c];
  }
}

// ---------------------------------------------------------------------------
// the chain around the layer (R9)

// x / sqrt(mean(x^2) + eps) per token, unit weight
void orc_rmsnorm(const double* x, int64_t T, int64_t H, double eps, double* out) {
  for (int64_t t = 0; t < T; ++t) {
    double ss = 0.0;
    for (int64_t c = 0; c < H; ++c) ss += x[t * H + c] * x[t * H + c];
    const double ms = plant(kPlantRmsMean) ? ss : ss / (double)H;
    const double r = sqrt(ms + eps);
    for (int64_t c = 0; c < H; ++c) out[t * H + c] = x[t * H + c] / r;
  }
}

// x_hat = act(rmsnorm(x))
void orc_chain_prologue(const double* x, int64_t T, int64_t H, double eps, int act,
                        double* x_hat) {
  orc_rmsnorm(x, T, H, eps, x_hat);
  orc_round_act(x_hat, T * H, act, x_hat);
}

// x_next = act(x + out)
void orc_chain_epilogue(const double* x, const double* out, int64_t n, int act, double* x_next) {
  for (int64_t i = 0; i < n; ++i) x_next[i] = x[i] + out[i];
  orc_round_act(x_next, n, act, x_next);
}

// ---------------------------------------------------------------------------
// token -> expert bucketing of a batch

// counts [E], offsets [E+1] (exclusive prefix sum), pairs [T*k x 2] of
// (token, j) sorted by expert, then by token.
void orc_bucket(const int64_t* idx, int64_t T, int64_t k, int64_t E, int64_t* counts,
                int64_t* offsets, int64_t* pairs) {
  for (int64_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t i = 0; i < T * k; ++i) counts[idx[i]] += 1;
  offsets[0] = 0;
  for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int64_t n = 0;
  for (int64_t e = 0; e < E; ++e)
    for (int64_t t = 0; t < T; ++t)
      for (int64_t j = 0; j < k; ++j)
        if (idx[t * k + j] == e) {
          pairs[2 * n] = t;
          pairs[2 * n + 1] = j;
          ++n;
        }
}

}  // extern "C"
