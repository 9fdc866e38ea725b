/*
 * Lightning Attention CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, fp64 statement of what the Lightning Attention layer computes.
 * Only tests/, the smoke check and the bench's cpu_baseline leg may load it;
 * the GPU library shares no code with it and never calls it.
 *
 * Source of the method: "Diving into MiniMax01 405B MoE" (Hugging Face blog),
 * section "Hybrid Modeling", 7/8 Linear Attention (Lightning Attention-2),
 * Mechanism steps 1-4:  Q, K, V = SiLU(input); Y = Q (K^T V) at O(d^2) per
 * token; output = RMSNorm(Y) * sigmoid(gate input).  The model card
 * ("2. Model Architecture") fixes 64 heads of dimension 128.
 *
 * Readings taken where the page is silent:
 *  - causal, the current token included: the state after token t holds
 *    sum_{u<=t} k~_u^T v~_u and y_t = q~_t S_t (decode order "kv += k^T v,
 *    then y = q kv");
 *  - no 1/sqrt(d) scale, no decay, no normaliser (NormAttention family: the
 *    output norm replaces the softmax denominator);
 *  - RMSNorm over all H*D values of a token: mean of squares, eps inside the
 *    square root, then the weight w[h*D+d], then the elementwise sigmoid gate;
 *  - the state S is D_k x D_v, row = key dimension: S[i][j] += k~_i v~_j.
 *
 * The file ends with the hybrid's softmax attention layer (rotary embedding
 * and causal softmax attention), stated the same way.
 *
 * Layouts: activations token-major [T][H][D]; states [nseq][H][D][D].
 * Segments (batch rows or packed varlen sequences) are given by seg[0..nseq],
 * seg[0] = 0, nondecreasing, seg[nseq] = T; each starts from its own state.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* logistic function, 1 / (1 + e^-x), straight from its definition */
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }
/* SiLU(x) = x * sigmoid(x)  (Mechanism step 2) */
static double silu(double x) { return x * sigmoid(x); }

double la_oracle_sigmoid(double x) { return sigmoid(x); }
double la_oracle_silu(double x) { return silu(x); }

/*
 * Mechanism step 4 for one token: y holds the H*D raw attention outputs of
 * the token; it is overwritten with RMSNorm(y) * w * sigmoid(g).
 */
static void norm_gate_token(double* y, const double* g, const double* w, int64_t HD, double eps) {
    double ss = 0.0;
    for (int64_t i = 0; i < HD; ++i) ss += y[i] * y[i];
    double r = 1.0 / sqrt(ss / (double)HD + eps);
    for (int64_t i = 0; i < HD; ++i) y[i] = y[i] * r * w[i] * sigmoid(g[i]);
}

/*
 * Prefill by the token recurrence (Mechanism steps 2-4, causal reading):
 *   S <- S0;  for each token t:  S <- S + k~_t^T v~_t ;  y_t = q~_t S.
 * out receives the final layer output [T][H][D]; y_raw (optional) the
 * pre-norm y; final_state (optional) the state after the last token.
 */
int la_oracle_prefill(const double* q, const double* k, const double* v, const double* g,
                      const double* w, const int64_t* seg, int64_t nseq, int64_t H, int64_t D,
                      double eps, const double* init_state, double* out, double* y_raw,
                      double* final_state) {
    const int64_t HD = H * D;
    const int64_t T = seg[nseq];
    #pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t s = 0; s < nseq; ++s) {
        for (int64_t h = 0; h < H; ++h) {
            double* S = (double*)malloc(sizeof(double) * D * D);
            double* qt = (double*)malloc(sizeof(double) * D * 3);
            double* kt = qt + D;
            double* vt = qt + 2 * D;
            if (init_state) memcpy(S, init_state + (s * H + h) * D * D, sizeof(double) * D * D);
            else memset(S, 0, sizeof(double) * D * D);
            for (int64_t t = seg[s]; t < seg[s + 1]; ++t) {
                const int64_t base = t * HD + h * D;
                for (int64_t i = 0; i < D; ++i) {
                    qt[i] = silu(q[base + i]);
                    kt[i] = silu(k[base + i]);
                    vt[i] = silu(v[base + i]);
                }
                /* state update first: the current token attends to itself */
                for (int64_t i = 0; i < D; ++i)
                    for (int64_t j = 0; j < D; ++j) S[i * D + j] += kt[i] * vt[j];
                /* y_t = q~_t S */
                for (int64_t j = 0; j < D; ++j) {
                    double acc = 0.0;
                    for (int64_t i = 0; i < D; ++i) acc += qt[i] * S[i * D + j];
                    out[base + j] = acc;
                }
            }
            if (final_state) memcpy(final_state + (s * H + h) * D * D, S, sizeof(double) * D * D);
            free(qt);
            free(S);
        }
    }
    if (y_raw) memcpy(y_raw, out, sizeof(double) * T * HD);
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) norm_gate_token(out + t * HD, g + t * HD, w, HD, eps);
    return 0;
}

/*
 * Prefill by the block-tiled form the Lightning Attention-2 design implies
 * (intra-block masked product plus inter-block product against the running
 * state), used to pin block-size invariance.  Per segment and head, with
 * blocks of `block` tokens and S the state before the block:
 *   Y_b = (Q~_b K~_b^T (.) M) V~_b + Q~_b S,   M_ij = 1 iff j <= i
 *   S  <- S + K~_b^T V~_b
 */
int la_oracle_prefill_blocked(const double* q, const double* k, const double* v, const double* g,
                              const double* w, const int64_t* seg, int64_t nseq, int64_t H,
                              int64_t D, int64_t block, double eps, const double* init_state,
                              double* out, double* final_state) {
    const int64_t HD = H * D;
    const int64_t T = seg[nseq];
    if (block < 1) return 1;
    #pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t s = 0; s < nseq; ++s) {
        for (int64_t h = 0; h < H; ++h) {
            double* S = (double*)malloc(sizeof(double) * D * D);
            double* Qb = (double*)malloc(sizeof(double) * block * D * 3);
            double* Kb = Qb + block * D;
            double* Vb = Qb + 2 * block * D;
            if (init_state) memcpy(S, init_state + (s * H + h) * D * D, sizeof(double) * D * D);
            else memset(S, 0, sizeof(double) * D * D);
            for (int64_t t0 = seg[s]; t0 < seg[s + 1]; t0 += block) {
                int64_t n = seg[s + 1] - t0;
                if (n > block) n = block;
                for (int64_t a = 0; a < n; ++a)
                    for (int64_t i = 0; i < D; ++i) {
                        const int64_t idx = (t0 + a) * HD + h * D + i;
                        Qb[a * D + i] = silu(q[idx]);
                        Kb[a * D + i] = silu(k[idx]);
                        Vb[a * D + i] = silu(v[idx]);
                    }
                for (int64_t a = 0; a < n; ++a) {
                    double* y = out + (t0 + a) * HD + h * D;
                    /* inter-block: q~_a S (state before this block) */
                    for (int64_t j = 0; j < D; ++j) {
                        double acc = 0.0;
                        for (int64_t i = 0; i < D; ++i) acc += Qb[a * D + i] * S[i * D + j];
                        y[j] = acc;
                    }
                    /* intra-block: sum over c <= a of (q~_a . k~_c) v~_c */
                    for (int64_t c = 0; c <= a; ++c) {
                        double sc = 0.0;
                        for (int64_t i = 0; i < D; ++i) sc += Qb[a * D + i] * Kb[c * D + i];
                        for (int64_t j = 0; j < D; ++j) y[j] += sc * Vb[c * D + j];
                    }
                }
                for (int64_t a = 0; a < n; ++a)
                    for (int64_t i = 0; i < D; ++i)
                        for (int64_t j = 0; j < D; ++j) S[i * D + j] += Kb[a * D + i] * Vb[a * D + j];
            }
            if (final_state) memcpy(final_state + (s * H + h) * D * D, S, sizeof(double) * D * D);
            free(Qb);
            free(S);
        }
    }
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) norm_gate_token(out + t * HD, g + t * HD, w, HD, eps);
    return 0;
}

/*
 * One decode step: every sequence receives one token; its state is read,
 * updated in place (S += k~^T v~) and used for y = q~ S, then the token's
 * output is normalised and gated (constant memory per layer, which is what
 * cached generation with a linear-attention layer requires).
 * q, k, v, g, out: [nseq][H][D]; state: [nseq][H][D][D], updated in place.
 */
int la_oracle_decode(const double* q, const double* k, const double* v, const double* g,
                     const double* w, int64_t nseq, int64_t H, int64_t D, double eps,
                     double* state, double* out) {
    const int64_t HD = H * D;
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t s = 0; s < nseq; ++s) {
        for (int64_t h = 0; h < H; ++h) {
            double* S = state + (s * H + h) * D * D;
            const int64_t base = s * HD + h * D;
            for (int64_t i = 0; i < D; ++i)
                for (int64_t j = 0; j < D; ++j) S[i * D + j] += silu(k[base + i]) * silu(v[base + j]);
            for (int64_t j = 0; j < D; ++j) {
                double acc = 0.0;
                for (int64_t i = 0; i < D; ++i) acc += silu(q[base + i]) * S[i * D + j];
                out[base + j] = acc;
            }
        }
    }
    #pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < nseq; ++s) norm_gate_token(out + s * HD, g + s * HD, w, HD, eps);
    return 0;
}

/*
 * State after a prefill without its outputs: S = S0 + sum_t k~_t^T v~_t per
 * segment and head (the decode workload's initial state is defined this way).
 */
int la_oracle_state(const double* k, const double* v, const int64_t* seg, int64_t nseq, int64_t H,
                    int64_t D, double* state) {
    const int64_t HD = H * D;
    #pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t s = 0; s < nseq; ++s) {
        for (int64_t h = 0; h < H; ++h) {
            double* S = state + (s * H + h) * D * D;
            double* kt = (double*)malloc(sizeof(double) * D * 2);
            double* vt = kt + D;
            for (int64_t t = seg[s]; t < seg[s + 1]; ++t) {
                for (int64_t i = 0; i < D; ++i) {
                    kt[i] = silu(k[t * HD + h * D + i]);
                    vt[i] = silu(v[t * HD + h * D + i]);
                }
                for (int64_t i = 0; i < D; ++i)
                    for (int64_t j = 0; j < D; ++j) S[i * D + j] += kt[i] * vt[j];
            }
            free(kt);
        }
    }
    return 0;
}

/* derivative of SiLU: sigmoid(x) (1 + x (1 - sigmoid(x))) */
static double silu_grad(double x) {
    const double s = sigmoid(x);
    return s * (1.0 + x * (1.0 - s));
}

/*
 * Gradient of the layer: the reverse-mode derivative of la_oracle_prefill
 * for a loss L whose gradient w.r.t. the output is dout [T][H][D] and, if
 * d_final is given, w.r.t. the final states [nseq][H][D][D].  Writes dq, dk,
 * dv, dg [T][H][D], dw [H*D] and, if d_init is given, dL/dS0 [nseq][H][D][D].
 * The chain rule is taken through the forward steps in reverse order:
 *  step 4, per token (out = yhat c, yhat = y r, r = (mean y^2 + eps)^-1/2,
 *    c = w sigmoid(g)):  a = dout c;  dy = r (a - yhat <a, yhat> / HD);
 *    dg = dout yhat w sigmoid(g) (1 - sigmoid(g));  dw = sum_t dout yhat sigmoid(g);
 *  step 3, per segment and head:  with dS_t = dL/dS_t, the gradient reaching
 *    S_t = S_{t-1} + k~_t^T v~_t through y_t = q~_t S_t and through S_{t+1}:
 *      dS_t = q~_t^T dy_t + dS_{t+1}  (dS after the last token = d_final);
 *      dq~_t = dy_t S_t^T;  dk~_t = v~_t dS_t^T;  dv~_t = k~_t dS_t;
 *      dL/dS0 = dS_first;
 *    a forward sweep recomputes S_t for dq~, a reverse sweep accumulates dS;
 *  step 2:  dq = dq~ SiLU'(q), and likewise for k and v.
 */
int la_oracle_backward(const double* q, const double* k, const double* v, const double* g,
                       const double* w, const double* dout, const int64_t* seg, int64_t nseq,
                       int64_t H, int64_t D, double eps, const double* init_state,
                       const double* d_final, double* dq, double* dk, double* dv, double* dg,
                       double* dw, double* d_init) {
    const int64_t HD = H * D;
    const int64_t T = seg[nseq];
    /* forward recomputation of the pre-norm y */
    double* y = (double*)malloc(sizeof(double) * (T > 0 ? T * HD : 1));
    double* outs = (double*)malloc(sizeof(double) * (T > 0 ? T * HD : 1));
    double* dy = (double*)malloc(sizeof(double) * (T > 0 ? T * HD : 1));
    double* yhat = outs;  /* reused: y r per element */
    la_oracle_prefill(q, k, v, g, w, seg, nseq, H, D, eps, init_state, outs, y, NULL);
    /* step 4 backward, per token */
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const double* yt = y + t * HD;
        double ss = 0.0;
        for (int64_t i = 0; i < HD; ++i) ss += yt[i] * yt[i];
        const double r = 1.0 / sqrt(eps + ss / (double)HD);  /* the forward's r */
        double ay = 0.0;
        for (int64_t i = 0; i < HD; ++i) {
            const int64_t e = t * HD + i;
            yhat[e] = yt[i] * r;
            const double sg = sigmoid(g[e]);
            ay += dout[e] * w[i] * sg * yhat[e];
            dg[e] = dout[e] * yhat[e] * w[i] * sg * (1.0 - sg);
        }
        for (int64_t i = 0; i < HD; ++i) {
            const int64_t e = t * HD + i;
            const double a = dout[e] * w[i] * sigmoid(g[e]);
            dy[e] = r * (a - yhat[e] * ay / (double)HD);
        }
    }
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < HD; ++i) {
        double acc = 0.0;
        for (int64_t t = 0; t < T; ++t) acc += dout[t * HD + i] * yhat[t * HD + i] * sigmoid(g[t * HD + i]);
        dw[i] = acc;
    }
    /* step 3 backward, per segment and head */
    #pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t s = 0; s < nseq; ++s) {
        for (int64_t h = 0; h < H; ++h) {
            double* S = (double*)malloc(sizeof(double) * D * D);
            double* qt = (double*)malloc(sizeof(double) * D * 3);
            double* kt = qt + D;
            double* vt = qt + 2 * D;
            /* forward sweep: S_t, then dq~_t = dy_t S_t^T */
            const double* S0 = init_state ? init_state + (s * H + h) * D * D : NULL;
            for (int64_t e = 0; e < D * D; ++e) S[e] = S0 ? S0[e] : 0.0;
            for (int64_t t = seg[s]; t < seg[s + 1]; ++t) {
                const int64_t base = t * HD + h * D;
                for (int64_t d = 0; d < D; ++d) {
                    kt[d] = silu(k[base + d]);
                    vt[d] = silu(v[base + d]);
                }
                for (int64_t i = 0; i < D; ++i)
                    for (int64_t j = 0; j < D; ++j) S[i * D + j] += kt[i] * vt[j];
                for (int64_t i = 0; i < D; ++i) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < D; ++j) acc += dy[base + j] * S[i * D + j];
                    dq[base + i] = acc * silu_grad(q[base + i]);
                }
            }
            /* reverse sweep: dS_t, then dk~_t and dv~_t */
            if (d_final) memcpy(S, d_final + (s * H + h) * D * D, sizeof(double) * D * D);
            else memset(S, 0, sizeof(double) * D * D);
            for (int64_t t = seg[s + 1] - 1; t >= seg[s]; --t) {
                const int64_t base = t * HD + h * D;
                for (int64_t d = 0; d < D; ++d) {
                    qt[d] = silu(q[base + d]);
                    kt[d] = silu(k[base + d]);
                    vt[d] = silu(v[base + d]);
                }
                for (int64_t i = 0; i < D; ++i)
                    for (int64_t j = 0; j < D; ++j) S[i * D + j] += qt[i] * dy[base + j];
                for (int64_t i = 0; i < D; ++i) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < D; ++j) acc += S[i * D + j] * vt[j];
                    dk[base + i] = acc * silu_grad(k[base + i]);
                }
                for (int64_t j = 0; j < D; ++j) {
                    double acc = 0.0;
                    for (int64_t i = 0; i < D; ++i) acc += kt[i] * S[i * D + j];
                    dv[base + j] = acc * silu_grad(v[base + j]);
                }
            }
            if (d_init) memcpy(d_init + (s * H + h) * D * D, S, sizeof(double) * D * D);
            free(qt);
            free(S);
        }
    }
    free(dy);
    free(outs);
    free(y);
    return 0;
}

/* thread control for the timed baseline (OpenMP over segments x heads) */
/*
 * ------------------------------------------------ the softmax attention layer
 * The hybrid's other attention: one softmax attention layer after every
 * seven Lightning layers ("Diving into MiniMax01 405B MoE", section "Hybrid
 * Modeling", 1/8 Softmax Attention: rotary embedding on half of the head
 * dimension; the model card, "2. Model Architecture": RoPE on half of the
 * head dimension with base frequency 10,000,000).
 *
 * Readings taken where the pages are silent:
 *  - rotary embedding as first defined (RoFormer): features (2i, 2i+1) of the
 *    first rope_dim ones form a plane rotated by the angle pos * theta_i,
 *    theta_i = base^(-2i / rope_dim); the other features pass unchanged;
 *  - pos = the token's index within its own sequence (0 at each start);
 *  - causal softmax attention, the current token included, logits scaled by
 *    `scale` (1/sqrt(head_dim) unless the caller says otherwise), as many
 *    key/value heads as query heads.
 */
static void rope_vec(const double* x, double* y, int64_t D, int64_t rope_dim, double base,
                     double pos) {
    for (int64_t i = 0; i < rope_dim / 2; ++i) {
        const double theta = pow(base, -2.0 * (double)i / (double)rope_dim);
        const double c = cos(pos * theta), s = sin(pos * theta);
        const double a = x[2 * i], b = x[2 * i + 1];
        y[2 * i] = a * c - b * s;
        y[2 * i + 1] = a * s + b * c;
    }
    for (int64_t j = rope_dim; j < D; ++j) y[j] = x[j];
}

/* rotary embedding of every head vector of x [T][H][D] at its position */
int la_oracle_rope(const double* x, double* y, const int64_t* seg, int64_t nseq, int64_t H,
                   int64_t D, int64_t rope_dim, double base) {
    for (int64_t s = 0; s < nseq; ++s)
        for (int64_t t = seg[s]; t < seg[s + 1]; ++t)
            for (int64_t h = 0; h < H; ++h) {
                const int64_t e = (t * H + h) * D;
                rope_vec(x + e, y + e, D, rope_dim, base, (double)(t - seg[s]));
            }
    return 0;
}

/*
 * out_t = sum_{u <= t} softmax_u(scale * <q^_t, k^_u>) v_u over the keys u of
 * t's own sequence, q^ and k^ rotated at their positions.  rows (optional,
 * nrows entries): compute only these tokens (others are left untouched).
 */
int la_oracle_softmax_attention(const double* q, const double* k, const double* v,
                                const int64_t* seg, int64_t nseq, int64_t H, int64_t D,
                                int64_t rope_dim, double base, double scale, const int64_t* rows,
                                int64_t nrows, double* out) {
    const int64_t T = seg[nseq];
    const int64_t n = rows ? nrows : T;
    int bad = 0;
    #pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t h = 0; h < H; ++h) {
            const int64_t t = rows ? rows[r] : r;
            int64_t s = 0;
            while (s < nseq && seg[s + 1] <= t) ++s;
            const int64_t s0 = seg[s];
            double* qh = malloc(sizeof(double) * D);
            double* kh = malloc(sizeof(double) * D);
            double* p = malloc(sizeof(double) * (t - s0 + 1));
            if (!qh || !kh || !p) {
                bad = 1;
            } else {
                rope_vec(q + (t * H + h) * D, qh, D, rope_dim, base, (double)(t - s0));
                const int64_t last = t; /* causal: the current token is its own last key */
                double m = -INFINITY;
                for (int64_t u = s0; u <= last; ++u) {
                    rope_vec(k + (u * H + h) * D, kh, D, rope_dim, base, (double)(u - s0));
                    double dot = 0.0;
                    for (int64_t j = 0; j < D; ++j) dot += qh[j] * kh[j];
                    p[u - s0] = scale * dot;
                    if (p[u - s0] > m) m = p[u - s0];
                }
                double z = 0.0;
                for (int64_t u = s0; u <= last; ++u) {
                    p[u - s0] = exp(p[u - s0] - m);
                    z += p[u - s0];
                }
                double* o = out + (t * H + h) * D;
                for (int64_t j = 0; j < D; ++j) {
                    double acc = 0.0;
                    for (int64_t u = s0; u <= last; ++u) acc += p[u - s0] * v[(u * H + h) * D + j];
                    o[j] = acc / z;
                }
            }
            free(qh);
            free(kh);
            free(p);
        }
    return bad ? -1 : 0;
}

#ifdef _OPENMP
#include <omp.h>
void la_oracle_set_threads(int n) { if (n > 0) omp_set_num_threads(n); }
int la_oracle_max_threads(void) { return omp_get_max_threads(); }
#else
void la_oracle_set_threads(int n) { (void)n; }
int la_oracle_max_threads(void) { return 1; }
#endif
