/*
 * fp64 CPU oracle for the MiMo-V2.6-Flash attention layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no code, header, table or constant with the HIP
 * library: every quantity below is computed here from its definition.
 *
 * What it computes (one query row r, query head h, KV head g = h / (Hq/Hkv)):
 *
 *   partial RoPE  — "Partial RoPE" on the model-techniques-map page: the head
 *     vector is split into its first rope_dim dims, which rotate, and the rest,
 *     which carry no position.  rope_dim = int(192 * 0.334) = 64.  The rotation
 *     is the default (non-YaRN) RoPE of the Hugging Face modeling code that the
 *     page cites (rope_type set to default), in its rotate-half form: dim i and dim
 *     i + rope_dim/2 (i < rope_dim/2) rotate together by the angle
 *     pos * base^(-2i/rope_dim).  Angles and cos/sin are fp64 (the Gaudi
 *     recipe page, section on required fixes, builds its tables in float64
 *     since the fastest frequency's angle is the position itself).
 *
 *   scores — s_j = softmax_scale * <rope(q_r), rope(k_j)> over the visible keys
 *     j: pos(j) <= pos(r) and, on sliding-window layers, pos(r) - pos(j) < W
 *     (W = 128 keys counting the query itself, the HF / Megatron-Bridge
 *     convention in "Notable quirks" of the miles recipe page).
 *
 *   sink — "Learnable attention sink" on the techniques-map page: one logit per
 *     query head joins the softmax as an extra column and is dropped after the
 *     softmax, so it enlarges the normaliser and carries no value.  It is
 *     compared with the already-scaled scores and is not scaled itself.
 *
 *   softmax — two passes: m = max(all s_j, sink), Z = sum exp(s_j - m) +
 *     exp(sink - m); output o = v_scale * sum_j exp(s_j - m) v_j / Z with
 *     v_scale = 0.707 (the value path's fixed scale, miles recipe page,
 *     section 1, model introduction).
 *     GQA: consecutive query heads share one KV head (repeat_kv).
 *
 * bf16 inputs are taken as exact values (bf16 -> fp64 is exact); nothing is
 * rounded in between.
 *
 * The backward (oracle_attention_backward) differentiates exactly that map,
 * written out by the chain rule for the trainer's path (miles recipe page,
 * section 5.4: the sink is trained through the fused attention).  With
 * p_j = exp(s_j)/Z, p_sink = exp(sink)/Z and an upstream gradient dO of the
 * output row: dp_j = v_scale <dO, v_j>; D = sum_j p_j dp_j (the sink column
 * has no value, so its dp is 0); ds_j = p_j (dp_j - D); d rope(q) = scale *
 * sum_j ds_j rope(k_j); d rope(k_j) += scale * ds_j rope(q); dv_j += v_scale
 * p_j dO; d sink = -p_sink * D summed over every row of the head; and the
 * gradients of q and k are the rotated gradients turned back by the transpose
 * of the rotation (the same angle, negated).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Rotate one head vector x[0..D) at position pos into y (fp64). */
static void rope_one(const double *x, double *y, int D, int R, double base, int64_t pos) {
    int half = R / 2;
    for (int d = 0; d < D; ++d) y[d] = x[d];
    for (int i = 0; i < half; ++i) {
        double inv_freq = pow(base, -(double)(2 * i) / (double)R);
        double angle = (double)pos * inv_freq;
        double c = cos(angle), s = sin(angle);
        y[i] = x[i] * c - x[i + half] * s;
        y[i + half] = x[i + half] * c + x[i] * s;
    }
}

/* y = R(pos)^T x: the transpose of rope_one's rotation (angle negated). */
static void rope_one_transpose(const double *x, double *y, int D, int R, double base, int64_t pos) {
    int half = R / 2;
    for (int d = 0; d < D; ++d) y[d] = x[d];
    for (int i = 0; i < half; ++i) {
        double inv_freq = pow(base, -(double)(2 * i) / (double)R);
        double angle = (double)pos * inv_freq;
        double c = cos(angle), s = sin(angle);
        y[i] = x[i] * c + x[i + half] * s;
        y[i + half] = x[i + half] * c - x[i] * s;
    }
}

/* x: [n_tok, n_heads, D] bf16 bits; out: same shape, fp64. */
void oracle_rope_partial(const uint16_t *x, int64_t n_tok, int n_heads, int D, int R,
                         const int64_t *pos, double base, double *out) {
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n_tok; ++t) {
        double buf[1024];
        for (int h = 0; h < n_heads; ++h) {
            const uint16_t *src = x + ((size_t)t * n_heads + h) * D;
            for (int d = 0; d < D; ++d) buf[d] = bf16_value(src[d]);
            rope_one(buf, out + ((size_t)t * n_heads + h) * D, D, R, base, pos[t]);
        }
    }
}

static int visible(int64_t qp, int64_t kp, int64_t window) {
    if (kp > qp) return 0;
    if (window > 0 && qp - kp >= window) return 0;
    return 1;
}

/*
 * Attention rows.
 *   q      [nq, Hq, Dqk] bf16 bits (unrotated), positions q_pos[nq]
 *   k      [nk, Hkv, Dqk] bf16 bits, positions k_pos[nk]; k_rotated != 0 means
 *          the values already carry their rotation (a decode cache)
 *   v      [nk, Hkv, Dv] bf16 bits
 *   sinks  [Hq] or NULL
 *   window 0 = causal over every earlier key, > 0 = keys with qp-kp < window
 * Outputs (fp64): out [nq, Hq, Dv]; lse [nq, Hq] = log(sum exp(s_j) + exp(sink))
 * and psink [nq, Hq] = exp(sink)/that sum, each optional (NULL).
 * A row with no visible key and no sink gets o = 0, lse = -inf.
 */
void oracle_attention(const uint16_t *q, const int64_t *q_pos, int64_t nq,
                      const uint16_t *k, int k_rotated, const int64_t *k_pos, int64_t nk,
                      const uint16_t *v, int Hq, int Hkv, int Dqk, int Dv, int R,
                      double base, const double *sinks, int64_t window,
                      double softmax_scale, double v_scale,
                      double *out, double *lse, double *psink, int n_threads) {
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    int group = Hq / Hkv;

    /* Step 1: every key, rotated once, as fp64. */
    double *kr = (double *)malloc((size_t)nk * Hkv * Dqk * sizeof(double));
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < nk; ++j) {
        double buf[1024];
        for (int g = 0; g < Hkv; ++g) {
            const uint16_t *src = k + ((size_t)j * Hkv + g) * Dqk;
            double *dst = kr + ((size_t)j * Hkv + g) * Dqk;
            for (int d = 0; d < Dqk; ++d) buf[d] = bf16_value(src[d]);
            if (k_rotated) memcpy(dst, buf, Dqk * sizeof(double));
            else rope_one(buf, dst, Dqk, R, base, k_pos[j]);
        }
    }

    /* Step 2: each (row, head) independently. */
    #pragma omp parallel
    {
        double *scores = (double *)malloc((size_t)(nk > 0 ? nk : 1) * sizeof(double));
        int64_t *keys = (int64_t *)malloc((size_t)(nk > 0 ? nk : 1) * sizeof(int64_t));
        double qraw[1024], qrot[1024], acc[1024];
        #pragma omp for schedule(dynamic, 1)
        for (int64_t idx = 0; idx < nq * Hq; ++idx) {
            int64_t r = idx / Hq;
            int h = (int)(idx % Hq);
            int g = h / group;
            const uint16_t *qs = q + ((size_t)r * Hq + h) * Dqk;
            for (int d = 0; d < Dqk; ++d) qraw[d] = bf16_value(qs[d]);
            rope_one(qraw, qrot, Dqk, R, base, q_pos[r]);

            int64_t n = 0;
            for (int64_t j = 0; j < nk; ++j) {
                if (!visible(q_pos[r], k_pos[j], window)) continue;
                const double *kj = kr + ((size_t)j * Hkv + g) * Dqk;
                double dot = 0.0;
                for (int d = 0; d < Dqk; ++d) dot += qrot[d] * kj[d];
                scores[n] = softmax_scale * dot;
                keys[n] = j;
                ++n;
            }

            /* pass 1: the largest logit, the sink column included */
            double m = -INFINITY;
            for (int64_t t = 0; t < n; ++t) if (scores[t] > m) m = scores[t];
            if (sinks && sinks[h] > m) m = sinks[h];

            double *o = out + ((size_t)r * Hq + h) * Dv;
            if (m == -INFINITY) {
                for (int d = 0; d < Dv; ++d) o[d] = 0.0;
                if (lse) lse[r * Hq + h] = -INFINITY;
                if (psink) psink[r * Hq + h] = 0.0;
                continue;
            }
            /* pass 2: normaliser and weighted values */
            double z = 0.0;
            for (int d = 0; d < Dv; ++d) acc[d] = 0.0;
            for (int64_t t = 0; t < n; ++t) {
                double p = exp(scores[t] - m);
                z += p;
                const uint16_t *vj = v + ((size_t)keys[t] * Hkv + g) * Dv;
                for (int d = 0; d < Dv; ++d) acc[d] += p * bf16_value(vj[d]);
            }
            double zsink = sinks ? exp(sinks[h] - m) : 0.0;
            z += zsink;
            for (int d = 0; d < Dv; ++d) o[d] = v_scale * acc[d] / z;
            if (lse) lse[r * Hq + h] = m + log(z);
            if (psink) psink[r * Hq + h] = zsink / z;
        }
        free(scores);
        free(keys);
    }
    free(kr);
}

/*
 * Gradients of the attention rows above (same arguments, k unrotated).
 *   dout   [nq, Hq, Dv] bf16 bits: the upstream gradient of out
 * Outputs (fp64, overwritten): dq [nq, Hq, Dqk], dk [nk, Hkv, Dqk],
 * dv [nk, Hkv, Dv], dsinks [Hq] (NULL when sinks is NULL).  Work is split over
 * KV heads, so each thread owns the dk / dv rows it accumulates.
 */
void oracle_attention_backward(const uint16_t *q, const int64_t *q_pos, int64_t nq,
                               const uint16_t *k, const int64_t *k_pos, int64_t nk,
                               const uint16_t *v, int Hq, int Hkv, int Dqk, int Dv, int R,
                               double base, const double *sinks, int64_t window,
                               double softmax_scale, double v_scale, const uint16_t *dout,
                               double *dq, double *dk, double *dv, double *dsinks, int n_threads) {
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    int group = Hq / Hkv;
    double *kr = (double *)malloc((size_t)(nk > 0 ? nk : 1) * Hkv * Dqk * sizeof(double));
    double *dkr = (double *)calloc((size_t)(nk > 0 ? nk : 1) * Hkv * Dqk, sizeof(double));
    for (int64_t j = 0; j < nk; ++j) {
        double buf[1024];
        for (int g = 0; g < Hkv; ++g) {
            const uint16_t *src = k + ((size_t)j * Hkv + g) * Dqk;
            for (int d = 0; d < Dqk; ++d) buf[d] = bf16_value(src[d]);
            rope_one(buf, kr + ((size_t)j * Hkv + g) * Dqk, Dqk, R, base, k_pos[j]);
        }
    }
    memset(dv, 0, (size_t)nk * Hkv * Dv * sizeof(double));
    if (dsinks) memset(dsinks, 0, (size_t)Hq * sizeof(double));

    #pragma omp parallel for schedule(dynamic, 1)
    for (int g = 0; g < Hkv; ++g) {
        double *scores = (double *)malloc((size_t)(nk > 0 ? nk : 1) * sizeof(double));
        double *dp = (double *)malloc((size_t)(nk > 0 ? nk : 1) * sizeof(double));
        int64_t *keys = (int64_t *)malloc((size_t)(nk > 0 ? nk : 1) * sizeof(int64_t));
        double qraw[1024], qrot[1024], dqrot[1024], dor[1024];
        for (int h = g * group; h < (g + 1) * group; ++h) {
            double dsink = 0.0;
            for (int64_t r = 0; r < nq; ++r) {
                const uint16_t *qs = q + ((size_t)r * Hq + h) * Dqk;
                for (int d = 0; d < Dqk; ++d) qraw[d] = bf16_value(qs[d]);
                rope_one(qraw, qrot, Dqk, R, base, q_pos[r]);
                const uint16_t *ds = dout + ((size_t)r * Hq + h) * Dv;
                for (int d = 0; d < Dv; ++d) dor[d] = bf16_value(ds[d]);

                int64_t n = 0;
                for (int64_t j = 0; j < nk; ++j) {
                    if (!visible(q_pos[r], k_pos[j], window)) continue;
                    const double *kj = kr + ((size_t)j * Hkv + g) * Dqk;
                    double dot = 0.0;
                    for (int d = 0; d < Dqk; ++d) dot += qrot[d] * kj[d];
                    scores[n] = softmax_scale * dot;
                    keys[n] = j;
                    ++n;
                }
                double m = -INFINITY;
                for (int64_t t = 0; t < n; ++t) if (scores[t] > m) m = scores[t];
                if (sinks && sinks[h] > m) m = sinks[h];
                double *dqr = dq + ((size_t)r * Hq + h) * Dqk;
                if (m == -INFINITY) {
                    for (int d = 0; d < Dqk; ++d) dqr[d] = 0.0;
                    continue;
                }
                double z = 0.0;
                for (int64_t t = 0; t < n; ++t) z += exp(scores[t] - m);
                double zsink = sinks ? exp(sinks[h] - m) : 0.0;
                z += zsink;
                /* dp_j and D = sum_j p_j dp_j */
                double D = 0.0;
                for (int64_t t = 0; t < n; ++t) {
                    const uint16_t *vj = v + ((size_t)keys[t] * Hkv + g) * Dv;
                    double dot = 0.0;
                    for (int d = 0; d < Dv; ++d) dot += dor[d] * bf16_value(vj[d]);
                    dp[t] = v_scale * dot;
                    scores[t] = exp(scores[t] - m) / z;      /* now p_j */
                    D += scores[t] * dp[t];
                }
                if (sinks) dsink -= (zsink / z) * D;
                for (int d = 0; d < Dqk; ++d) dqrot[d] = 0.0;
                for (int64_t t = 0; t < n; ++t) {
                    double dsj = scores[t] * (dp[t] - D);
                    const double *kj = kr + ((size_t)keys[t] * Hkv + g) * Dqk;
                    double *dkj = dkr + ((size_t)keys[t] * Hkv + g) * Dqk;
                    for (int d = 0; d < Dqk; ++d) {
                        dqrot[d] += softmax_scale * dsj * kj[d];
                        dkj[d] += softmax_scale * dsj * qrot[d];
                    }
                    double *dvj = dv + ((size_t)keys[t] * Hkv + g) * Dv;
                    for (int d = 0; d < Dv; ++d) dvj[d] += v_scale * scores[t] * dor[d];
                }
                rope_one_transpose(dqrot, dqr, Dqk, R, base, q_pos[r]);
            }
            if (dsinks) dsinks[h] = dsink;
        }
        free(scores);
        free(dp);
        free(keys);
    }
    for (int64_t j = 0; j < nk; ++j)
        for (int g = 0; g < Hkv; ++g)
            rope_one_transpose(dkr + ((size_t)j * Hkv + g) * Dqk, dk + ((size_t)j * Hkv + g) * Dqk, Dqk, R,
                               base, k_pos[j]);
    free(kr);
    free(dkr);
}

/* Nearest bf16 value of x (8 significant bits, ties to even), from the fp64
 * value directly so there is no double rounding through fp32.  Values beyond
 * bf16's normal range do not occur in the rows this is used on. */
static double bf16_round(double x) {
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    double m = frexp(x, &e);                  /* x = m * 2^e, 0.5 <= |m| < 1 */
    return ldexp(nearbyint(ldexp(m, 8)), e - 8);   /* default mode: ties to even */
}

/*
 * What holding rope(q) and rope(k) as bf16 matrix-multiply operands does to the
 * attention rows.  Only the R rotated dims change: the others are bf16 inputs
 * already.  Same arguments as oracle_attention (k unrotated).  Outputs (fp64):
 *
 *   out_rounded [nq, Hq, Dv]: the rows with every rotated element of rope(q)
 *     and rope(k_j) rounded to its nearest bf16 value before the scores.
 *
 *   bound [nq, Hq, Dv]: how far any such rounding can move the exact output.
 *     A rounded element x' of x obeys |x' - x| <= u |x| with u = 2^-8 (half an
 *     ulp is at most 2^-8 |x|; a kernel that lands a hair past a midpoint and
 *     rounds to the other neighbour stays within it too), so each score moves by
 *     at most delta_j = scale (2u + u^2) sum_{i<R} |rope(q)_i rope(k_j)_i|.
 *     With p_j = exp(s_j)/Z, w_j = v_scale v_j and the row's largest delta_bar:
 *     p'_j = p_j e^{D_j} / E with |D_j| <= delta_j and E = sum_k p_k e^{D_k} +
 *     p_sink in [e^-delta_bar, e^delta_bar], hence |p'_j - p_j| <= p_j
 *     (e^{delta_j + delta_bar} - 1) and |p'_sink - p_sink| <= p_sink (e^delta_bar
 *     - 1); and o' - o = sum_j (p'_j - p_j)(w_j - o) + (p_sink - p'_sink) o, so
 *     |o'_d - o_d| <= sum_j p_j (e^{delta_j + delta_bar} - 1) |w_jd - o_d|
 *                     + p_sink (e^delta_bar - 1) |o_d|.
 *     No first-order step: the bound holds for any rounding within u.
 */
void oracle_operand_rounding(const uint16_t *q, const int64_t *q_pos, int64_t nq,
                             const uint16_t *k, const int64_t *k_pos, int64_t nk,
                             const uint16_t *v, int Hq, int Hkv, int Dqk, int Dv, int R,
                             double base, const double *sinks, int64_t window,
                             double softmax_scale, double v_scale,
                             double *out_rounded, double *bound, int n_threads) {
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    const double u = ldexp(1.0, -8);
    int group = Hq / Hkv;
    double *kr = (double *)malloc((size_t)nk * Hkv * Dqk * sizeof(double));
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < nk; ++j) {
        double buf[1024];
        for (int g = 0; g < Hkv; ++g) {
            const uint16_t *src = k + ((size_t)j * Hkv + g) * Dqk;
            for (int d = 0; d < Dqk; ++d) buf[d] = bf16_value(src[d]);
            rope_one(buf, kr + ((size_t)j * Hkv + g) * Dqk, Dqk, R, base, k_pos[j]);
        }
    }
    #pragma omp parallel
    {
        size_t cap = (size_t)(nk > 0 ? nk : 1);
        double *s = (double *)malloc(cap * sizeof(double));    /* exact scores */
        double *sr = (double *)malloc(cap * sizeof(double));   /* scores of the rounded operands */
        double *dl = (double *)malloc(cap * sizeof(double));   /* delta_j */
        int64_t *keys = (int64_t *)malloc(cap * sizeof(int64_t));
        double qraw[1024], qrot[1024], o[1024], acc[1024];
        #pragma omp for schedule(dynamic, 1)
        for (int64_t idx = 0; idx < nq * Hq; ++idx) {
            int64_t r = idx / Hq;
            int h = (int)(idx % Hq);
            int g = h / group;
            const uint16_t *qs = q + ((size_t)r * Hq + h) * Dqk;
            for (int d = 0; d < Dqk; ++d) qraw[d] = bf16_value(qs[d]);
            rope_one(qraw, qrot, Dqk, R, base, q_pos[r]);
            int64_t n = 0;
            double dbar = 0.0;
            for (int64_t j = 0; j < nk; ++j) {
                if (!visible(q_pos[r], k_pos[j], window)) continue;
                const double *kj = kr + ((size_t)j * Hkv + g) * Dqk;
                double dot = 0.0, dotr = 0.0, mag = 0.0;
                for (int d = 0; d < Dqk; ++d) {
                    dot += qrot[d] * kj[d];
                    if (d < R) {
                        dotr += bf16_round(qrot[d]) * bf16_round(kj[d]);
                        mag += fabs(qrot[d] * kj[d]);
                    } else {
                        dotr += qrot[d] * kj[d];
                    }
                }
                s[n] = softmax_scale * dot;
                sr[n] = softmax_scale * dotr;
                dl[n] = softmax_scale * (2.0 * u + u * u) * mag;
                if (dl[n] > dbar) dbar = dl[n];
                keys[n] = j;
                ++n;
            }
            double *orr = out_rounded + ((size_t)r * Hq + h) * Dv;
            double *bd = bound + ((size_t)r * Hq + h) * Dv;
            const double *sk = sinks ? &sinks[h] : NULL;
            /* both rows by the same two-pass softmax: pass 0 the exact scores
             * (kept in o for the bound), pass 1 the rounded ones */
            for (int pass = 0; pass < 2; ++pass) {
                const double *sc = pass == 0 ? s : sr;
                double *dst = pass == 0 ? o : orr;
                double m = -INFINITY;
                for (int64_t t = 0; t < n; ++t) if (sc[t] > m) m = sc[t];
                if (sk && *sk > m) m = *sk;
                if (m == -INFINITY) {
                    for (int d = 0; d < Dv; ++d) dst[d] = 0.0;
                    continue;
                }
                double z = 0.0;
                for (int d = 0; d < Dv; ++d) acc[d] = 0.0;
                for (int64_t t = 0; t < n; ++t) {
                    double p = exp(sc[t] - m);
                    z += p;
                    const uint16_t *vj = v + ((size_t)keys[t] * Hkv + g) * Dv;
                    for (int d = 0; d < Dv; ++d) acc[d] += p * bf16_value(vj[d]);
                }
                z += sk ? exp(*sk - m) : 0.0;
                for (int d = 0; d < Dv; ++d) dst[d] = v_scale * acc[d] / z;
            }
            /* the bound, from the exact p_j, p_sink and o */
            double m = -INFINITY;
            for (int64_t t = 0; t < n; ++t) if (s[t] > m) m = s[t];
            if (sk && *sk > m) m = *sk;
            for (int d = 0; d < Dv; ++d) bd[d] = 0.0;
            if (m == -INFINITY) continue;
            double z = sk ? exp(*sk - m) : 0.0;
            for (int64_t t = 0; t < n; ++t) z += exp(s[t] - m);
            for (int64_t t = 0; t < n; ++t) {
                double p = exp(s[t] - m) / z;
                double f = p * expm1(dl[t] + dbar);
                const uint16_t *vj = v + ((size_t)keys[t] * Hkv + g) * Dv;
                for (int d = 0; d < Dv; ++d) bd[d] += f * fabs(v_scale * bf16_value(vj[d]) - o[d]);
            }
            if (sk) {
                double ps = exp(*sk - m) / z;
                for (int d = 0; d < Dv; ++d) bd[d] += ps * expm1(dbar) * fabs(o[d]);
            }
        }
        free(s);
        free(sr);
        free(dl);
        free(keys);
    }
    free(kr);
}
